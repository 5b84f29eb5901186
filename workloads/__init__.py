"""Seeded synthetic inputs for the fused attention forward.

This module only draws random numbers and lays them out (packed token-major
tensors, cu_seqlens offsets, paged pools with a page table).  It holds none of
the attention arithmetic: both the CPU oracle (``oracle/``) and the HIP path
(``attention_qk_online_amd``) consume what it produces, and neither is imported
here.

Workloads follow the shapes the pages discuss:
* "FlashInfer Attention Kernel技术解析" section 1 / 4 and the FlashInfer library
  overview (API examples, fixed-size KV pages, GQA-style head sharing);
* "FlashAttention-3 内核在最新大模型推理中的集成实践" section 二 (packed
  ``[total_tokens, heads, head_dim]`` tensors addressed by ``cu_seqlens`` of
  length batch+1, paged physical blocks, chunked prefill) and section 三
  (prefill lengths 1K..32K, batch 8).

Every draw uses ``torch.Generator().manual_seed(seed)`` on the CPU, in the
order: lengths -> page permutation -> Q -> K -> V.  Values are N(0,1) fp32,
rounded to the config dtype with ``.to(dtype)`` (round to nearest even).
Unreferenced pages and tail slots of the last page of each request are filled
with NaN ("poison"), so a kernel that reads outside the logical sequence
produces NaN instead of a plausible wrong number.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import torch

__all__ = [
    "DecodeCase", "PrefillCase", "PagedPrefillCase",
    "make_decode", "make_prefill", "make_paged_prefill",
    "make_config", "CONFIG_NAMES",
    "decode_kv_bytes", "prefill_pairs", "prefill_flops",
]


def _gen(seed: int) -> torch.Generator:
    return torch.Generator().manual_seed(int(seed))


def _randn(g: torch.Generator, shape, dtype) -> torch.Tensor:
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(dtype)


def _to_layout(pool: torch.Tensor, layout: str) -> torch.Tensor:
    """An NHD pool [pages, P, Hkv, D] as itself or as HND [pages, Hkv, P, D]."""
    if layout == "NHD":
        return pool
    if layout == "HND":
        return pool.transpose(1, 2).contiguous()
    raise ValueError(f"layout must be NHD or HND, got {layout!r}")


# ---------------------------------------------------------------------------
# Paged decode
# ---------------------------------------------------------------------------
@dataclass
class DecodeCase:
    """Batched decode over a paged KV cache (NHD pages).

    q           [B, Hq, D]                       dtype
    kv_lens     [B] int32
    page_table  [B, max_pages] int32  (entries past ceil(kv_len/P) point at a
                                       NaN-poisoned page when one exists)
    k_tok/v_tok [sum(kv_lens), Hkv, D] dtype     logical tokens, request-major
    slot_index  [sum(kv_lens)] int64             flat index page*P + slot of
                                                 each logical token in the pool
    """
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    page_size: int
    num_pages: int
    dtype: torch.dtype
    scale: float
    q: torch.Tensor
    kv_lens: torch.Tensor
    page_table: torch.Tensor
    k_tok: torch.Tensor
    v_tok: torch.Tensor
    slot_index: torch.Tensor
    poison: bool = True

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def max_kv_len(self) -> int:
        return int(self.kv_lens.max().item()) if self.B > 0 else 0

    def pools(self, device="cpu", layout="NHD"):
        """Materialise (k_pages, v_pages) on ``device``: [num_pages, P, Hkv, D]
        (NHD) or, with ``layout="HND"``, the same cache as [num_pages, Hkv, P, D]."""
        shape = (self.num_pages, self.page_size, self.Hkv, self.D)
        fill = float("nan") if self.poison else 0.0
        out = []
        idx = self.slot_index.to(device)
        for tok in (self.k_tok, self.v_tok):
            pool = torch.full(shape, fill, dtype=self.dtype, device=device)
            flat = pool.view(self.num_pages * self.page_size, self.Hkv, self.D)
            flat.index_copy_(0, idx, tok.to(device))
            out.append(_to_layout(pool, layout))
        return out[0], out[1]

    def kv_bytes(self) -> int:
        return decode_kv_bytes(self.kv_lens, self.Hkv, self.D, self.dtype)

    def fp8_pools(self, device="cpu", layout="NHD"):
        """The same cache stored as 8-bit floats E4M3 with one scale per tensor.

        Each of K and V is divided by amax/448 (448 = the largest E4M3
        value) and rounded to E4M3 by torch's float8_e4m3fn conversion; the
        pools hold the raw bytes (uint8), unreferenced slots 0x7F (NaN) when
        the case is poisoned.  Returns (k_pages, v_pages, k_scale, v_scale):
        token t's key is k_scale * E4M3(k_pages[...]).
        """
        shape = (self.num_pages, self.page_size, self.Hkv, self.D)
        idx = self.slot_index.to(device)
        out = []
        for tok in (self.k_tok, self.v_tok):
            x = tok.float()
            amax = float(x.abs().max()) if x.numel() else 0.0
            sc = amax / 448.0 if amax > 0 else 1.0
            q8 = (x / sc).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
            pool = torch.full(shape, 0x7F if self.poison else 0, dtype=torch.uint8, device=device)
            flat = pool.view(self.num_pages * self.page_size, self.Hkv, self.D)
            flat.index_copy_(0, idx, q8.to(device))
            out += [_to_layout(pool, layout), sc]
        return out[0], out[2], out[1], out[3]

    def fp8_kv_bytes(self) -> int:
        """Algorithmic K+V bytes of the E4M3 cache: 2*Hkv*D*sum(kv_len)."""
        return int(2 * self.Hkv * self.D * int(self.kv_lens.long().sum().item()))


def decode_kv_bytes(kv_lens, Hkv, D, dtype) -> int:
    """Algorithmic K+V bytes a decode call must stream: 2*Hkv*D*esize*sum(kv_len)."""
    esize = torch.empty((), dtype=dtype).element_size()
    return int(2 * Hkv * D * esize * int(torch.as_tensor(kv_lens).long().sum().item()))


def make_decode(*, B, Hq, Hkv, D, page_size, kv_lens: Sequence[int] | torch.Tensor | None = None,
                len_range=None, num_pages: Optional[int] = None, dtype=torch.bfloat16,
                seed=0, scale=None, permute_pages=True, poison=True, name="decode",
                extra_pages=1) -> DecodeCase:
    """Draw a paged decode case.

    lengths: given, or discrete-uniform in ``len_range`` (both ends inclusive).
    pages:   each request takes ceil(kv_len/P) consecutive ids of a seeded
             permutation of the pool, in request order (so ids are scattered
             over the pool).  ``num_pages`` defaults to the referenced pages
             plus ``extra_pages`` spare (poisoned) pages.
    """
    g = _gen(seed)
    if kv_lens is None:
        lo, hi = len_range
        kv_lens = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64)
    kv_lens = torch.as_tensor(kv_lens, dtype=torch.int64).reshape(B)
    n_pages_req = (kv_lens + page_size - 1) // page_size
    n_ref = int(n_pages_req.sum().item())
    if num_pages is None:
        num_pages = n_ref + extra_pages
    assert num_pages >= n_ref
    if permute_pages:
        perm = torch.randperm(num_pages, generator=g)
    else:
        perm = torch.arange(num_pages)
    max_pages = max(1, int(n_pages_req.max().item()) if B > 0 else 1)
    spare = int(perm[-1].item()) if num_pages > n_ref else 0
    table = torch.full((B, max_pages), spare, dtype=torch.int32)
    off = 0
    slot_parts = []
    for b in range(B):
        n = int(n_pages_req[b])
        ids = perm[off:off + n]
        off += n
        table[b, :n] = ids.to(torch.int32)
        L = int(kv_lens[b])
        t = torch.arange(L)
        slot_parts.append(ids[t // page_size].long() * page_size + t % page_size)
    slot_index = torch.cat(slot_parts) if slot_parts else torch.zeros(0, dtype=torch.long)
    total = int(kv_lens.sum().item())
    q = _randn(g, (B, Hq, D), dtype)
    k_tok = _randn(g, (total, Hkv, D), dtype)
    v_tok = _randn(g, (total, Hkv, D), dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return DecodeCase(name=name, seed=seed, B=B, Hq=Hq, Hkv=Hkv, D=D, page_size=page_size,
                      num_pages=num_pages, dtype=dtype, scale=float(scale), q=q,
                      kv_lens=kv_lens.to(torch.int32), page_table=table, k_tok=k_tok,
                      v_tok=v_tok, slot_index=slot_index, poison=poison)


# ---------------------------------------------------------------------------
# Ragged prefill (contiguous, cu_seqlens)
# ---------------------------------------------------------------------------
@dataclass
class PrefillCase:
    """Ragged prefill packed by cu_seqlens.

    q [Tq, Hq, D], k/v [Tk, Hkv, D]; cu_seqlens_q/k [B+1] int32.
    """
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    dtype: torch.dtype
    causal: bool
    scale: float
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    cu_seqlens_q: torch.Tensor
    cu_seqlens_k: torch.Tensor

    @property
    def lens_q(self) -> List[int]:
        c = self.cu_seqlens_q.tolist()
        return [c[i + 1] - c[i] for i in range(self.B)]

    @property
    def lens_k(self) -> List[int]:
        c = self.cu_seqlens_k.tolist()
        return [c[i + 1] - c[i] for i in range(self.B)]

    @property
    def max_seqlen_q(self) -> int:
        return max(self.lens_q) if self.B else 0

    @property
    def max_seqlen_k(self) -> int:
        return max(self.lens_k) if self.B else 0

    def flops(self) -> int:
        return prefill_flops(self.lens_q, self.lens_k, self.Hq, self.D, self.causal)

    def prefix(self, L: int, name=None) -> "PrefillCase":
        """Single-sequence prefix view (first L tokens) of a B=1 case."""
        assert self.B == 1
        cu = torch.tensor([0, L], dtype=torch.int32)
        return PrefillCase(name=name or f"{self.name}[:{L}]", seed=self.seed, B=1, Hq=self.Hq,
                           Hkv=self.Hkv, D=self.D, dtype=self.dtype, causal=self.causal,
                           scale=self.scale, q=self.q[:L], k=self.k[:L], v=self.v[:L],
                           cu_seqlens_q=cu, cu_seqlens_k=cu.clone())


def prefill_pairs(lens_q, lens_k, causal: bool) -> int:
    """Number of visible (query, key) pairs per head; causal is bottom-right aligned."""
    tot = 0
    for lq, lk in zip(lens_q, lens_k):
        lq, lk = int(lq), int(lk)
        if not causal:
            tot += lq * lk
            continue
        off = lk - lq
        # row i sees keys 0 .. min(lk-1, i+off)  -> count = clip(i+off+1, 0, lk)
        for_rows = 0
        # closed form over the three regimes, summed exactly with integers
        i0 = max(0, -off)                   # first row with >=1 visible key
        i1 = min(lq, lk - off)              # rows i < i1 see i+off+1 keys
        if i1 > i0:
            a, b = i0 + off + 1, (i1 - 1) + off + 1
            for_rows += (a + b) * (i1 - i0) // 2
        if lq > max(i1, i0):
            for_rows += (lq - max(i1, i0)) * lk
        tot += for_rows
    return tot


def prefill_flops(lens_q, lens_k, Hq, D, causal) -> int:
    """Algorithmic flops: 2*D for QK^T plus 2*D for PV per visible pair, per query head."""
    return 4 * D * Hq * prefill_pairs(lens_q, lens_k, causal)


def _cu(lens) -> torch.Tensor:
    c = [0]
    for L in lens:
        c.append(c[-1] + int(L))
    return torch.tensor(c, dtype=torch.int32)


def make_prefill(*, B, Hq, Hkv, D, lens_q=None, lens_k=None, len_range=None, dtype=torch.bfloat16,
                 seed=0, causal=True, scale=None, name="prefill") -> PrefillCase:
    """Draw a ragged prefill case.  Lengths are given or discrete-uniform in
    ``len_range`` (inclusive); when only one length list is given q and k share it."""
    g = _gen(seed)
    if lens_q is None and lens_k is None:
        lo, hi = len_range
        lens = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).tolist()
        lens_q = lens_k = lens
    elif lens_k is None:
        lens_k = lens_q
    elif lens_q is None:
        lens_q = lens_k
    lens_q = [int(x) for x in lens_q]
    lens_k = [int(x) for x in lens_k]
    assert len(lens_q) == B and len(lens_k) == B
    Tq, Tk = sum(lens_q), sum(lens_k)
    q = _randn(g, (Tq, Hq, D), dtype)
    k = _randn(g, (Tk, Hkv, D), dtype)
    v = _randn(g, (Tk, Hkv, D), dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return PrefillCase(name=name, seed=seed, B=B, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype,
                       causal=bool(causal), scale=float(scale), q=q, k=k, v=v,
                       cu_seqlens_q=_cu(lens_q), cu_seqlens_k=_cu(lens_k))


# ---------------------------------------------------------------------------
# Chunked prefill over a paged cache (optionally with a shared prefix)
# ---------------------------------------------------------------------------
@dataclass
class PagedPrefillCase:
    """Query chunks (packed by cu_seqlens_q) attending to a paged KV cache.

    The cache of request b holds kv_lens[b] logical tokens; the query chunk is
    the last lens_q[b] of them (its own K/V already appended), so causal
    masking is bottom-right aligned.  Logical pages [0, shared_pages) of every
    request map to the same physical pages (a shared prefix).
    """
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    page_size: int
    num_pages: int
    dtype: torch.dtype
    causal: bool
    scale: float
    q: torch.Tensor
    cu_seqlens_q: torch.Tensor
    kv_lens: torch.Tensor
    page_table: torch.Tensor
    pool_k: torch.Tensor            # [num_pages, P, Hkv, D] (CPU, finite where referenced)
    pool_v: torch.Tensor
    shared_pages: int = 0

    @property
    def lens_q(self) -> List[int]:
        c = self.cu_seqlens_q.tolist()
        return [c[i + 1] - c[i] for i in range(self.B)]

    @property
    def max_seqlen_q(self) -> int:
        return max(self.lens_q) if self.B else 0

    @property
    def max_kv_len(self) -> int:
        return int(self.kv_lens.max().item()) if self.B else 0

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    def pools(self, device="cpu", layout="NHD"):
        """(k_pages, v_pages) on ``device``, NHD or HND (see DecodeCase.pools)."""
        return (_to_layout(self.pool_k.to(device), layout),
                _to_layout(self.pool_v.to(device), layout))

    def flops(self) -> int:
        return prefill_flops(self.lens_q, self.kv_lens.tolist(), self.Hq, self.D, self.causal)


def make_paged_prefill(*, B, Hq, Hkv, D, page_size, chunk, cached, shared_prefix=0,
                       dtype=torch.bfloat16, seed=0, causal=True, scale=None,
                       name="paged_prefill", spare_pages=0) -> PagedPrefillCase:
    """Every request appends a ``chunk``-token query to ``cached`` tokens, so
    kv_len = cached + chunk; ``chunk`` and ``cached`` are one int for every
    request or a list of B ints.  The first ``shared_prefix`` tokens (a
    multiple of the page size, at most every request's cached length) sit on
    pages shared by all requests.

    Draw order: page permutation -> Q -> K (shared prefix, then each request's
    private tokens) -> V (same order).
    """
    assert shared_prefix % page_size == 0
    g = _gen(seed)
    chunks = [int(chunk)] * B if isinstance(chunk, int) else [int(c) for c in chunk]
    cacheds = [int(cached)] * B if isinstance(cached, int) else [int(c) for c in cached]
    assert len(chunks) == B and len(cacheds) == B and all(c >= shared_prefix for c in cacheds)
    kv_lens = [c + q for c, q in zip(cacheds, chunks)]
    n_shared = shared_prefix // page_size
    n_log = [(L + page_size - 1) // page_size for L in kv_lens]
    n_priv = [n - n_shared for n in n_log]
    num_pages = n_shared + sum(n_priv) + spare_pages
    perm = torch.randperm(num_pages, generator=g)
    table = torch.full((B, max(n_log) if B else 1), int(perm[-1]) if spare_pages else 0,
                       dtype=torch.int32)
    s = n_shared
    for b in range(B):
        table[b, :n_shared] = perm[:n_shared].to(torch.int32)
        table[b, n_shared:n_log[b]] = perm[s:s + n_priv[b]].to(torch.int32)
        s += n_priv[b]
    q = _randn(g, (sum(chunks), Hq, D), dtype)
    priv_lens = [L - shared_prefix for L in kv_lens]
    pools = []
    for _ in range(2):  # K then V
        shared = _randn(g, (shared_prefix, Hkv, D), dtype)
        priv = _randn(g, (sum(priv_lens), Hkv, D), dtype)
        pool = torch.full((num_pages, page_size, Hkv, D), float("nan"), dtype=dtype)
        flat = pool.view(num_pages * page_size, Hkv, D)
        t = torch.arange(shared_prefix)
        if shared_prefix:
            flat.index_copy_(0, perm[t // page_size].long() * page_size + t % page_size, shared)
        o = 0
        for b in range(B):
            tl = torch.arange(shared_prefix, kv_lens[b])
            pid = table[b, (tl // page_size)].long()
            flat.index_copy_(0, pid * page_size + tl % page_size, priv[o:o + priv_lens[b]])
            o += priv_lens[b]
        pools.append(pool)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return PagedPrefillCase(name=name, seed=seed, B=B, Hq=Hq, Hkv=Hkv, D=D, page_size=page_size,
                            num_pages=num_pages, dtype=dtype, causal=bool(causal),
                            scale=float(scale), q=q,
                            cu_seqlens_q=_cu(chunks),
                            kv_lens=torch.tensor(kv_lens, dtype=torch.int32),
                            page_table=table, pool_k=pools[0], pool_v=pools[1],
                            shared_pages=n_shared)


# ---------------------------------------------------------------------------
# The five named workloads
# ---------------------------------------------------------------------------
CONFIG_NAMES = {
    1: "decode_f32_b1_h4_d64_kv256",
    2: "decode_paged_bf16_b64_hq32_hkv8_d128_p16_kv512-4096",
    3: "prefill_causal_bf16_b8_l1024-4096_hq64_hkv8_d128",
    4: "prefill_causal_bf16_b1_l32768_hq64_hkv8_d128",
    5: "prefill_paged_chunk_bf16_b16_q512_kv8704_shared4096_h16_d256_p16",
}


def make_config(k: int, seed: Optional[int] = None):
    """The five named workloads; the seed defaults to the workload number."""
    seed = k if seed is None else seed
    if k == 1:
        # Single-sequence fp32 decode, MHA, contiguous KV of 256 tokens viewed
        # as 16 NHD pages of 16 with the identity page table.
        return make_decode(B=1, Hq=4, Hkv=4, D=64, page_size=16, kv_lens=[256], dtype=torch.float32,
                           seed=seed, scale=1.0 / 8.0, permute_pages=False, poison=False,
                           extra_pages=0, name=CONFIG_NAMES[1])
    if k == 2:
        return make_decode(B=64, Hq=32, Hkv=8, D=128, page_size=16, len_range=(512, 4096),
                           num_pages=300000, dtype=torch.bfloat16, seed=seed,
                           name=CONFIG_NAMES[2])
    if k == 3:
        return make_prefill(B=8, Hq=64, Hkv=8, D=128, len_range=(1024, 4096), dtype=torch.bfloat16,
                            seed=seed, causal=True, name=CONFIG_NAMES[3])
    if k == 4:
        return make_prefill(B=1, Hq=64, Hkv=8, D=128, lens_q=[32768], dtype=torch.bfloat16,
                            seed=seed, causal=True, name=CONFIG_NAMES[4])
    if k == 5:
        return make_paged_prefill(B=16, Hq=16, Hkv=16, D=256, page_size=16, chunk=512, cached=8192,
                                  shared_prefix=4096, dtype=torch.bfloat16, seed=seed,
                                  causal=True, name=CONFIG_NAMES[5])
    raise ValueError(f"unknown workload {k}")
