"""CPU oracle for the fused attention forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and
its Python binding) never calls it and shares no code with it.

What it computes is the plain definition of scaled-dot-product attention,
written out without blocking tricks: the score matrix Q.K^T * scale is built
in float64, masked, pushed through an ordinary softmax and multiplied by V.
Sources:

* "FlashAttention-3 内核在最新大模型推理中的集成实践" (gtnt.cn), introduction
  and section 一: attention is Q.K^T -> softmax -> .V; the fused kernels reach
  the same result with an online softmax, so the plain definition is the
  reference.  Section 二: packed ``[total_tokens, heads, head_dim]`` tensors,
  ``cu_seqlens`` prefix offsets of length batch+1, ``num_kv_heads`` <= heads,
  a ``causal`` flag and the default scale 1/sqrt(head_dim).  Section 四: the
  rescaling must stay, i.e. results must survive large logits.
* "FlashInfer内核库深度解析" (bxzpzcl.cn), PageAttention paragraph: the KV
  cache is cut into fixed-size pages addressed through a table; precision
  support: FP8 besides FP16/BF16.  FA-3 page section 一: with FP8 the
  quantisation scale joins the softmax's exponent scaling.  The FP8 cache is
  read as E4M3 bytes with one scale per K and V tensor.

Readings where the pages are silent:
* LSE is the natural log of the sum of exp of the *scaled* visible logits.
* Query head h reads KV head h // (Hq // Hkv) (consecutive grouping).
* Causal masking is bottom-right aligned: query i of a sequence with Lq
  queries and Lk keys sees keys j <= i + (Lk - Lq).
* A row with no visible key returns out = 0 and lse = -inf.
* varlen_fwd's ``window_size`` is a (left, right) pair: query i sees keys
  i + (Lk - Lq) - left .. i + (Lk - Lq) + right, -1 leaving that side open;
  causal is the window (-1, 0), so with causal set a right window adds nothing.
* Pages are NHD: ``pages[page, slot, kv_head, d]``; logical token t of a
  request lives at ``pages[table[t // P], t % P]``.

Everything is float64 on the CPU.  Inputs of any float dtype are converted
exactly (bf16 and fp32 are subsets of fp64), so the oracle sees the same
rounded values the GPU sees.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import torch

F64 = torch.float64
NEG_INF = float("-inf")


def softmax_attend(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float,
                   visible: Optional[torch.Tensor] = None):
    """Single-head attention by its definition.

    q [Lq, D], k [Lk, D], v [Lk, Dv] (any float dtype, converted to float64);
    ``visible`` [Lq, Lk] bool (None: every key is visible).

        s_ij   = scale * sum_d q_id k_jd            (visible j only)
        lse_i  = log sum_j exp(s_ij)                (natural log)
        out_i  = sum_j exp(s_ij - lse_i) v_j

    The exponentials are taken after subtracting the row maximum so that large
    logits do not overflow.  Rows without a visible key give out 0, lse -inf.
    Returns out [Lq, Dv], lse [Lq] in float64.
    """
    q, k, v = q.to(F64), k.to(F64), v.to(F64)
    Lq, Lk = q.shape[0], k.shape[0]
    if visible is None:
        visible = torch.ones((Lq, Lk), dtype=torch.bool)
    if Lk == 0:
        return (torch.zeros((Lq, v.shape[1]), dtype=F64),
                torch.full((Lq,), NEG_INF, dtype=F64))
    s = (q @ k.transpose(0, 1)) * scale
    s = torch.where(visible, s, torch.full_like(s, NEG_INF))
    empty = ~visible.any(dim=1)
    m = torch.where(empty, torch.zeros(Lq, dtype=F64), s.max(dim=1).values)
    lse = m + torch.log(torch.exp(s - m.unsqueeze(1)).sum(dim=1))
    lse = torch.where(empty, torch.full_like(lse, NEG_INF), lse)
    p = torch.exp(s - torch.where(empty, torch.zeros_like(lse), lse).unsqueeze(1))
    p = torch.where(visible, p, torch.zeros_like(p))
    return p @ v, lse


def causal_visible(rows: torch.Tensor, n_keys: int, offset: int) -> torch.Tensor:
    """Bottom-right causal visibility: query row r sees key j iff j <= r + offset."""
    return torch.arange(n_keys).unsqueeze(0) <= (rows.long().unsqueeze(1) + offset)


def window_visible(rows: torch.Tensor, n_keys: int, offset: int, left: int) -> torch.Tensor:
    """Sliding window (left side, aligned like the causal mask): query row r
    sees key j iff j >= r + offset - left ("FlashAttention-3 内核在最新大模型
    推理中的集成实践" section 二, window_size of varlen_fwd)."""
    return torch.arange(n_keys).unsqueeze(0) >= (rows.long().unsqueeze(1) + offset - left)


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """Grouped-query mapping: consecutive groups of Hq/Hkv query heads share one KV head."""
    return h // (Hq // Hkv)


def gather_pages(pages: torch.Tensor, table_row: torch.Tensor, length: int) -> torch.Tensor:
    """Logical tokens 0..length-1 of one request from an NHD pool.

    pages [num_pages, P, Hkv, D]; table_row holds at least ceil(length/P)
    physical page ids.  Returns [length, Hkv, D] in the pool's dtype.
    """
    P = pages.shape[1]
    t = torch.arange(length)
    ids = table_row.long()[t // P]
    return pages[ids, t % P]


def rope_rotate(x: torch.Tensor, pos: torch.Tensor, theta: float, scale: float = 1.0) -> torch.Tensor:
    """Rotary position embedding, rotate-half convention, in float64.

    x [..., n, D] with positions pos [n]: pair (x_d, x_{d+D/2}), d < D/2, is
    turned by the angle pos / scale * theta^(-2d/D).  ("FlashInfer内核库深度
    解析" names dynamic RoPE in its single-request decode kernel without
    fixing a convention; this is the rotate-half form.)
    """
    x = x.to(F64)
    D = x.shape[-1]
    h = D // 2
    freq = torch.pow(torch.tensor(float(theta), dtype=F64), -2.0 * torch.arange(h, dtype=F64) / D)
    ang = pos.to(F64).unsqueeze(-1) / scale * freq                     # [n, D/2]
    c, s = torch.cos(ang), torch.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return torch.cat([a * c - b * s, b * c + a * s], dim=-1)


def _check_heads(Hq: int, Hkv: int):
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} must be a positive multiple of Hkv={Hkv}")


def decode_window_first(L: int, window_left: int) -> int:
    """First key a decode query (the last of L tokens, position L - 1) sees
    under a left window of window_left keys (-1: no window, key 0)."""
    return max(0, L - 1 - window_left) if window_left >= 0 else 0


def ref_decode_paged(q, k_pages, v_pages, page_table, kv_lens, scale,
                     requests: Optional[Iterable[int]] = None, window_left: int = -1,
                     rope: Optional[Tuple[float, float]] = None):
    """Decode: one query token per request over its paged KV (no mask).

    q [B, Hq, D]; pools [num_pages, P, Hkv, D]; page_table [B, max_pages];
    kv_lens [B].  Returns out [B, Hq, D] and lse [B, Hq] (float64).  With
    ``requests`` only those rows are filled (the rest stay NaN).  With
    window_left >= 0 the query (the last token, position kv_len - 1) sees only
    keys kv_len - 1 - window_left .. kv_len - 1.  With rope = (theta, scale)
    the query (position kv_len - 1) and the keys (their token index) are
    rotated by :func:`rope_rotate` first.
    """
    B, Hq, D = q.shape
    Hkv = k_pages.shape[2]
    _check_heads(Hq, Hkv)
    out = torch.full((B, Hq, v_pages.shape[3]), float("nan"), dtype=F64)
    lse = torch.full((B, Hq), float("nan"), dtype=F64)
    for b in (range(B) if requests is None else requests):
        L = int(kv_lens[b])
        k = gather_pages(k_pages, page_table[b], L)
        v = gather_pages(v_pages, page_table[b], L)
        qb = q[b]
        if rope is not None:
            k = rope_rotate(k.transpose(0, 1), torch.arange(L), *rope).transpose(0, 1)
            qb = rope_rotate(q[b].unsqueeze(1), torch.tensor([L - 1]), *rope).squeeze(1)
        first = decode_window_first(L, window_left)
        k, v = k[first:], v[first:]
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            o, l = softmax_attend(qb[h:h + 1], k[:, g], v[:, g], scale)
            out[b, h] = o[0]
            lse[b, h] = l[0]
    return out, lse


def fp8_e4m3_to_float(b: torch.Tensor) -> torch.Tensor:
    """Value of each byte read as an OCP 8-bit float E4M3 (the variant without
    infinities), as float64.

    Bit 7 is the sign, bits 6..3 the exponent e (bias 7), bits 2..0 the
    mantissa m.  e = 0 is subnormal: m/8 * 2^-6.  Otherwise the value is
    (1 + m/8) * 2^(e-7), including e = 15 with m < 7 (up to 448); only
    S.1111.111 is NaN.  The pages name FP8 tensor-core arithmetic
    ("FlashInfer内核库深度解析", precision support) without fixing the
    encoding; E4M3 is the format read here.
    """
    x = b.to(torch.int64) & 0xFF
    sign = (x >> 7) & 1
    e = (x >> 3) & 0xF
    m = (x & 7).to(F64)
    sub = m / 8.0 * 2.0 ** -6
    norm = (1.0 + m / 8.0) * torch.pow(torch.full_like(m, 2.0), (e - 7).to(F64))
    mag = torch.where(e == 0, sub, norm)
    val = torch.where(sign == 1, -mag, mag)
    return torch.where((e == 15) & ((x & 7) == 7), torch.full_like(val, float("nan")), val)


def ref_decode_paged_fp8(q, k_pages, v_pages, k_scale: float, v_scale: float, page_table, kv_lens,
                         scale, requests: Optional[Iterable[int]] = None, window_left: int = -1):
    """Decode over a KV cache stored as E4M3 bytes with one scale per tensor:
    each key is k_scale times the value of its bytes, each value vector
    v_scale times the value of its bytes; then plain decode attention.  (In
    "FlashAttention-3 内核在最新大模型推理中的集成实践" section 一 the FP8
    scale is folded into the softmax's exponent scaling; mathematically that
    is this product.)

    k_pages / v_pages: uint8 [num_pages, P, Hkv, D]; other arguments (the
    sliding window included) and the result as :func:`ref_decode_paged`.
    Only the tokens a request uses are decoded.
    """
    B, Hq, D = q.shape
    Hkv = k_pages.shape[2]
    _check_heads(Hq, Hkv)
    out = torch.full((B, Hq, v_pages.shape[3]), float("nan"), dtype=F64)
    lse = torch.full((B, Hq), float("nan"), dtype=F64)
    for b in (range(B) if requests is None else requests):
        L = int(kv_lens[b])
        k = fp8_e4m3_to_float(gather_pages(k_pages, page_table[b], L)) * float(k_scale)
        v = fp8_e4m3_to_float(gather_pages(v_pages, page_table[b], L)) * float(v_scale)
        first = decode_window_first(L, window_left)
        k, v = k[first:], v[first:]
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            o, l = softmax_attend(q[b, h:h + 1], k[:, g], v[:, g], scale)
            out[b, h] = o[0]
            lse[b, h] = l[0]
    return out, lse


def upper_bound_shift(causal: bool, window_right: int) -> int:
    """How far right of its own diagonal position a query row may look: the
    right half of varlen_fwd's window_size ("FlashAttention-3 内核在最新大模型
    推理中的集成实践" section 二).  Row r sees keys j <= r + offset + shift;
    causal is the window (-1, 0), so it caps the shift at 0; -1 means no bound."""
    if causal:
        return 0
    return window_right if window_right >= 0 else -1


def _prefill_one(qs, ks, vs, Hq, Hkv, scale, causal, rows: Optional[torch.Tensor],
                 block: int = 1024, window_left: int = -1, window_right: int = -1):
    """One sequence: qs [Lq, Hq, D], ks/vs [Lk, Hkv, D]; causal is bottom-right;
    window_left >= 0 adds the sliding-window bound on the left, window_right
    >= 0 one on the right (-1: none; the causal bound is a right window of 0).

    Rows go in blocks of at most ``block`` queries; under a right bound a
    block only multiplies against the keys its last row can see, since every
    later key is masked for the whole block anyway.
    """
    Lq, Lk = qs.shape[0], ks.shape[0]
    off = Lk - Lq
    shift = upper_bound_shift(causal, window_right)
    idx = torch.arange(Lq) if rows is None else rows.long()
    out = torch.empty((idx.numel(), Hq, vs.shape[2]), dtype=F64)
    lse = torch.empty((idx.numel(), Hq), dtype=F64)
    for s0 in range(0, idx.numel(), block):
        r = idx[s0:s0 + block]
        bounded = shift >= 0
        kmax = Lk if not bounded else max(0, min(Lk, int(r.max()) + off + shift + 1))
        vis = causal_visible(r, kmax, off + shift) if bounded else None
        if window_left >= 0:
            w = window_visible(r, kmax, off, window_left)
            vis = w if vis is None else vis & w
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            o, l = softmax_attend(qs[r, h], ks[:kmax, g], vs[:kmax, g], scale, vis)
            out[s0:s0 + r.numel(), h] = o
            lse[s0:s0 + r.numel(), h] = l
    return out, lse


def ref_prefill_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, causal, scale,
                       rows: Optional[torch.Tensor] = None, window_left: int = -1,
                       window_right: int = -1):
    """Ragged prefill addressed by cu_seqlens (length B+1).

    q [Tq, Hq, D]; k, v [Tk, Hkv, D].  Returns out [Tq, Hq, D], lse [Tq, Hq]
    float64.  With ``rows`` (global query token indices) only those rows are
    computed and the rest are NaN.
    """
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    _check_heads(Hq, Hkv)
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    out = torch.full((Tq, Hq, v.shape[2]), float("nan"), dtype=F64)
    lse = torch.full((Tq, Hq), float("nan"), dtype=F64)
    want = None if rows is None else torch.as_tensor(rows).long()
    for b in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if want is None:
            local = None
        else:
            sel = want[(want >= q0) & (want < q1)]
            if sel.numel() == 0:
                continue
            local = sel - q0
        o, l = _prefill_one(q[q0:q1], k[k0:k1], v[k0:k1], Hq, Hkv, scale, causal, local,
                            window_left=window_left, window_right=window_right)
        tgt = torch.arange(q0, q1) if local is None else local + q0
        out[tgt] = o
        lse[tgt] = l
    return out, lse


def ref_prefill_paged(q, cu_seqlens_q, k_pages, v_pages, page_table, kv_lens, causal, scale,
                      rows: Optional[torch.Tensor] = None, window_left: int = -1,
                      window_right: int = -1):
    """Chunked prefill over a paged cache: request b's queries are the last
    Lq_b of its kv_lens[b] tokens (bottom-right causal)."""
    B = len(cu_seqlens_q) - 1
    ks, vs, ck = [], [], [0]
    for b in range(B):
        L = int(kv_lens[b])
        ks.append(gather_pages(k_pages, page_table[b], L))
        vs.append(gather_pages(v_pages, page_table[b], L))
        ck.append(ck[-1] + L)
    tail = tuple(k_pages.shape[2:])
    k = torch.cat(ks) if ks else k_pages.new_zeros((0,) + tail)
    v = torch.cat(vs) if vs else v_pages.new_zeros((0,) + tail)
    return ref_prefill_varlen(q, k, v, cu_seqlens_q, torch.tensor(ck), causal, scale, rows=rows,
                              window_left=window_left, window_right=window_right)


def merge_states(states: Sequence[Tuple[torch.Tensor, torch.Tensor]]):
    """Combine attention states computed over disjoint key sets.

    Each state is (o, lse) with o normalised over its own keys (o = 0 when
    lse = -inf).  With L = log sum_s exp(lse_s), the merged output is
    sum_s exp(lse_s - L) o_s and the merged lse is L.
    """
    lses = torch.stack([s[1].to(F64) for s in states])          # [S, ...]
    outs = torch.stack([s[0].to(F64) for s in states])          # [S, ..., D]
    mx = lses.max(dim=0).values
    none = torch.isneginf(mx)
    mx = torch.where(none, torch.zeros_like(mx), mx)
    w = torch.exp(lses - mx.unsqueeze(0))                        # exp(-inf) = 0
    tot = w.sum(dim=0)
    L = torch.where(none, torch.full_like(mx, NEG_INF), mx + torch.log(tot))
    wn = w / torch.where(none, torch.ones_like(tot), tot).unsqueeze(0)
    return (wn.unsqueeze(-1) * outs).sum(dim=0), L


def error_stats(got: torch.Tensor, ref: torch.Tensor) -> dict:
    """max-abs and normwise max-rel (max|d| / max|ref|) over the finite
    reference entries; where the reference is infinite the result must be
    the same infinity."""
    got = got.to(F64)
    ref = ref.to(F64)
    inf_ref = torch.isinf(ref)
    inf_ok = bool(torch.equal(got[inf_ref], ref[inf_ref])) if bool(inf_ref.any()) else True
    fin = ~inf_ref
    d = (got[fin] - ref[fin]).abs()
    if d.numel() == 0:
        return {"max_abs": 0.0, "max_rel": 0.0, "inf_match": inf_ok, "n": int(ref.numel())}
    max_abs = float("nan") if bool(torch.isnan(d).any()) else float(d.max())
    ref_max = float(ref[fin].abs().max())
    max_rel = max_abs / ref_max if ref_max > 0 else max_abs
    return {"max_abs": max_abs, "max_rel": max_rel, "inf_match": inf_ok, "n": int(ref.numel())}
