"""Seeded random configurations against the oracle.

Each case draws its options from one ``random.Random(seed)``: element type,
head_dim, grouping, page size, NHD or HND pages, lengths that include 0, 1,
page and tile multiples and their neighbours, run lengths, sliding windows,
the rotary embedding and the E4M3 cache (decode), causal or not, queries
shorter or longer than the keys (prefill), and the shared-prefix cascade.
Sizes stay small, so the oracle takes well under a second per case; the
printed line names the case before the GPU runs it.
"""
import random

import pytest
import torch

import oracle
import workloads
from helpers import assert_parity

pytestmark = pytest.mark.gpu


def _length(rng, page, lo=0, hi=2000):
    kind = rng.random()
    if kind < 0.1:
        return rng.choice([0, 1])
    if kind < 0.35:
        m = rng.randint(1, max(1, hi // page))
        return max(lo, min(hi, m * page + rng.choice([-1, 0, 1])))
    return rng.randint(max(lo, 1), hi)


@pytest.mark.parametrize("seed", range(150))
def test_random_decode(gpu, seed):
    import attention_qk_online_amd as A
    rng = random.Random(7000 + seed)
    dtype = rng.choice([torch.bfloat16, torch.float16])
    D = rng.choice([64, 128, 256])
    Hkv = rng.choice([1, 2, 4, 8])
    G = rng.choice([1, 2, 4, 8])
    P = rng.choice([16, 32, 64, 128, 256])
    B = rng.randint(1, 10)
    layout = rng.choice(["NHD", "HND"])
    window = rng.choice([-1, -1, rng.randint(0, 600)])
    split = rng.choice([0, 0, rng.randint(1, 12)])
    mode = rng.choice(["plain", "plain", "fp8"] + (["rope"] if D <= 128 else []))
    lens = [_length(rng, P, hi=rng.choice([2000, 2000, 9000])) for _ in range(B)]
    desc = (f"seed {seed}: {mode} {dtype} D{D} Hq{G * Hkv} Hkv{Hkv} P{P} {layout} B{B} "
            f"window {window} split {split} lens {lens}")
    print(desc, flush=True)
    case = workloads.make_decode(B=B, Hq=G * Hkv, Hkv=Hkv, D=D, page_size=P, kv_lens=lens,
                                 dtype=dtype, seed=7000 + seed, extra_pages=2)
    t, kl = case.page_table.to(gpu), case.kv_lens.to(gpu)
    if mode == "fp8":
        kb, vb, ks, vs = case.fp8_pools()
        kg, vg, _, _ = case.fp8_pools(gpu, layout)
        out, lse = A.decode_paged_fp8(case.q.to(gpu), kg, vg, t, kl, ks, vs, scale=case.scale,
                                      max_kv_len=case.max_kv_len, split_pages=split,
                                      kv_layout=layout, window_left=window)
        ro, rl = oracle.ref_decode_paged_fp8(case.q, kb, vb, ks, vs, case.page_table, case.kv_lens,
                                             case.scale, window_left=window)
    else:
        rope = (10000.0, rng.choice([1.0, 2.0])) if mode == "rope" else None
        kg, vg = case.pools(gpu, layout)
        out, lse = A.decode_paged(case.q.to(gpu), kg, vg, t, kl, scale=case.scale,
                                  max_kv_len=case.max_kv_len, split_pages=split, kv_layout=layout,
                                  window_left=window,
                                  rope_theta=None if rope is None else rope[0],
                                  rope_scale=1.0 if rope is None else rope[1])
        kp, vp = case.pools()
        ro, rl = oracle.ref_decode_paged(case.q, kp, vp,
                                         case.page_table, case.kv_lens, case.scale,
                                         window_left=window, rope=rope)
    torch.cuda.synchronize()
    assert_parity(out, lse, ro, rl, dtype, desc)


@pytest.mark.parametrize("seed", range(40))
def test_random_decode_fp32(gpu, seed):
    """fp32 decode (16-token pages, head_dim 64 or 128): splits, windows, HND."""
    import attention_qk_online_amd as A
    rng = random.Random(7500 + seed)
    D = rng.choice([64, 128])
    Hkv = rng.choice([1, 2, 4, 8])
    G = rng.choice([1, 2, 4, 8])
    B = rng.randint(1, 10)
    layout = rng.choice(["NHD", "HND"])
    window = rng.choice([-1, -1, rng.randint(0, 600)])
    split = rng.choice([0, 0, rng.randint(1, 40)])
    lens = [_length(rng, 16, hi=rng.choice([2000, 6000])) for _ in range(B)]
    desc = (f"seed {seed}: fp32 D{D} Hq{G * Hkv} Hkv{Hkv} {layout} B{B} window {window} "
            f"split {split} lens {lens}")
    print(desc, flush=True)
    case = workloads.make_decode(B=B, Hq=G * Hkv, Hkv=Hkv, D=D, page_size=16, kv_lens=lens,
                                 dtype=torch.float32, seed=7500 + seed, extra_pages=2)
    kg, vg = case.pools(gpu, layout)
    out, lse = A.decode_paged(case.q.to(gpu), kg, vg, case.page_table.to(gpu), case.kv_lens.to(gpu),
                              scale=case.scale, max_kv_len=case.max_kv_len, split_pages=split,
                              kv_layout=layout, window_left=window)
    torch.cuda.synchronize()
    kp, vp = case.pools()
    ro, rl = oracle.ref_decode_paged(case.q, kp, vp, case.page_table, case.kv_lens, case.scale,
                                     window_left=window)
    assert_parity(out, lse, ro, rl, torch.float32, desc)


@pytest.mark.parametrize("seed", range(100))
def test_random_prefill_varlen(gpu, seed):
    import attention_qk_online_amd as A
    rng = random.Random(8000 + seed)
    dtype = rng.choice([torch.bfloat16, torch.float16])
    D = rng.choice([128, 256])
    Hkv = rng.choice([1, 2, 4])
    G = rng.choice([1, 2, 4])
    B = rng.randint(1, 4)
    causal = rng.random() < 0.6
    hi = rng.choice([400, 400, 1200])
    lens_k = [_length(rng, 64, hi=hi) for _ in range(B)]
    lens_q = [k if rng.random() < 0.5 else _length(rng, 64, hi=hi) for k in lens_k]
    wl = rng.choice([-1, -1, rng.randint(0, 300)])
    wr = rng.choice([-1, -1, rng.randint(0, 300)])
    desc = (f"seed {seed}: {dtype} D{D} Hq{G * Hkv} Hkv{Hkv} causal {causal} window ({wl}, {wr}) "
            f"lens_q {lens_q} lens_k {lens_k}")
    print(desc, flush=True)
    case = workloads.make_prefill(B=B, Hq=G * Hkv, Hkv=Hkv, D=D, lens_q=lens_q, lens_k=lens_k,
                                  dtype=dtype, seed=8000 + seed, causal=causal)
    out, lse = A.prefill_varlen(case.q.to(gpu), case.k.to(gpu), case.v.to(gpu),
                                case.cu_seqlens_q.to(gpu), case.cu_seqlens_k.to(gpu),
                                max_seqlen_q=max(1, case.max_seqlen_q),
                                max_seqlen_k=max(1, case.max_seqlen_k), causal=causal,
                                scale=case.scale, window_left=wl, window_right=wr)
    torch.cuda.synchronize()
    ro, rl = oracle.ref_prefill_varlen(case.q, case.k, case.v, case.cu_seqlens_q, case.cu_seqlens_k,
                                       causal, case.scale, window_left=wl, window_right=wr)
    assert_parity(out, lse, ro, rl, dtype, desc)


@pytest.mark.parametrize("seed", range(80))
def test_random_prefill_paged(gpu, seed):
    import attention_qk_online_amd as A
    rng = random.Random(9000 + seed)
    dtype = rng.choice([torch.bfloat16, torch.float16])
    D = rng.choice([128, 256])
    Hkv = rng.choice([1, 2, 4])
    G = rng.choice([1, 2, 4])
    P = rng.choice([16, 32, 64, 128, 256])
    B = rng.randint(1, 4)
    layout = rng.choice(["NHD", "HND"])
    causal = rng.random() < 0.7
    cascade = rng.random() < 0.3
    shared = P * rng.randint(1, 3) if cascade else 0
    chunks = [rng.randint(1, 300) for _ in range(B)]
    cached = [shared + rng.randint(0, 400) for _ in range(B)]
    if cascade and causal:   # every query of a request sees the whole prefix
        cached = [max(c, shared) for c in cached]
    wl = -1 if cascade else rng.choice([-1, -1, rng.randint(0, 300)])
    wr = -1 if cascade else rng.choice([-1, -1, rng.randint(0, 300)])
    desc = (f"seed {seed}: {dtype} D{D} Hq{G * Hkv} Hkv{Hkv} P{P} {layout} causal {causal} "
            f"cascade {shared} window ({wl}, {wr}) chunks {chunks} cached {cached}")
    print(desc, flush=True)
    case = workloads.make_paged_prefill(B=B, Hq=G * Hkv, Hkv=Hkv, D=D, page_size=P, chunk=chunks,
                                        cached=cached, shared_prefix=shared, dtype=dtype,
                                        seed=9000 + seed, causal=causal, spare_pages=1)
    kg, vg = case.pools(gpu, layout)
    args = (case.q.to(gpu), case.cu_seqlens_q.to(gpu), kg, vg, case.page_table.to(gpu),
            case.kv_lens.to(gpu))
    if cascade:
        out, lse = A.prefill_paged_cascade(*args, max_seqlen_q=case.max_seqlen_q,
                                           max_kv_len=case.max_kv_len, shared_prefix_len=shared,
                                           causal=causal, scale=case.scale, kv_layout=layout)
    else:
        out, lse = A.prefill_paged(*args, max_seqlen_q=case.max_seqlen_q,
                                   max_kv_len=case.max_kv_len, causal=causal, scale=case.scale,
                                   kv_layout=layout, window_left=wl, window_right=wr)
    torch.cuda.synchronize()
    kp, vp = case.pools()
    ro, rl = oracle.ref_prefill_paged(case.q, case.cu_seqlens_q, kp, vp, case.page_table,
                                      case.kv_lens, causal, case.scale, window_left=wl,
                                      window_right=wr)
    assert_parity(out, lse, ro, rl, dtype, desc)


@pytest.mark.parametrize("seed", range(60))
def test_random_prefill_d256(gpu, seed):
    """head_dim 256 only (pairs of waves share 32 rows and split each tile's
    keys): varlen or paged, every page size and layout, windows, cascade,
    fp16, query and key lengths around the 32-key halves and 64-key tiles."""
    import attention_qk_online_amd as A
    rng = random.Random(9500 + seed)
    dtype = rng.choice([torch.bfloat16, torch.float16])
    Hkv = rng.choice([1, 2, 4])
    G = rng.choice([1, 2, 4])
    causal = rng.random() < 0.7
    paged = rng.random() < 0.5
    B = rng.randint(1, 4)

    def near_tile():
        return max(1, rng.choice([32, 64, 96, 128, 192]) * rng.randint(1, 4) + rng.choice([-1, 0, 1]))

    if not paged:
        lens_k = [near_tile() if rng.random() < 0.5 else rng.randint(1, 700) for _ in range(B)]
        lens_q = [k if rng.random() < 0.5 else near_tile() for k in lens_k]
        wl = rng.choice([-1, -1, rng.randint(0, 300)])
        wr = rng.choice([-1, -1, rng.randint(0, 300)])
        desc = (f"seed {seed}: varlen {dtype} Hq{G * Hkv} Hkv{Hkv} causal {causal} window ({wl}, {wr}) "
                f"lens_q {lens_q} lens_k {lens_k}")
        print(desc, flush=True)
        case = workloads.make_prefill(B=B, Hq=G * Hkv, Hkv=Hkv, D=256, lens_q=lens_q, lens_k=lens_k,
                                      dtype=dtype, seed=9500 + seed, causal=causal)
        out, lse = A.prefill_varlen(case.q.to(gpu), case.k.to(gpu), case.v.to(gpu),
                                    case.cu_seqlens_q.to(gpu), case.cu_seqlens_k.to(gpu),
                                    max_seqlen_q=max(1, case.max_seqlen_q),
                                    max_seqlen_k=max(1, case.max_seqlen_k), causal=causal,
                                    scale=case.scale, window_left=wl, window_right=wr)
        torch.cuda.synchronize()
        ro, rl = oracle.ref_prefill_varlen(case.q, case.k, case.v, case.cu_seqlens_q,
                                           case.cu_seqlens_k, causal, case.scale,
                                           window_left=wl, window_right=wr)
        assert_parity(out, lse, ro, rl, dtype, desc)
        return
    P = rng.choice([16, 32, 64, 128, 256])
    layout = rng.choice(["NHD", "HND"])
    cascade = rng.random() < 0.3
    shared = P * rng.randint(1, 3) if cascade else 0
    chunks = [near_tile() if rng.random() < 0.5 else rng.randint(1, 300) for _ in range(B)]
    cached = [shared + (near_tile() if rng.random() < 0.5 else rng.randint(0, 400)) for _ in range(B)]
    if cascade and causal:
        cached = [max(c, shared) for c in cached]
    wl = -1 if cascade else rng.choice([-1, -1, rng.randint(0, 300)])
    wr = -1 if cascade else rng.choice([-1, -1, rng.randint(0, 300)])
    desc = (f"seed {seed}: paged {dtype} Hq{G * Hkv} Hkv{Hkv} P{P} {layout} causal {causal} "
            f"cascade {shared} window ({wl}, {wr}) chunks {chunks} cached {cached}")
    print(desc, flush=True)
    case = workloads.make_paged_prefill(B=B, Hq=G * Hkv, Hkv=Hkv, D=256, page_size=P, chunk=chunks,
                                        cached=cached, shared_prefix=shared, dtype=dtype,
                                        seed=9500 + seed, causal=causal, spare_pages=1)
    kg, vg = case.pools(gpu, layout)
    args = (case.q.to(gpu), case.cu_seqlens_q.to(gpu), kg, vg, case.page_table.to(gpu),
            case.kv_lens.to(gpu))
    if cascade:
        out, lse = A.prefill_paged_cascade(*args, max_seqlen_q=case.max_seqlen_q,
                                           max_kv_len=case.max_kv_len, shared_prefix_len=shared,
                                           causal=causal, scale=case.scale, kv_layout=layout)
    else:
        out, lse = A.prefill_paged(*args, max_seqlen_q=case.max_seqlen_q,
                                   max_kv_len=case.max_kv_len, causal=causal, scale=case.scale,
                                   kv_layout=layout, window_left=wl, window_right=wr)
    torch.cuda.synchronize()
    kp, vp = case.pools()
    ro, rl = oracle.ref_prefill_paged(case.q, case.cu_seqlens_q, kp, vp, case.page_table,
                                      case.kv_lens, causal, case.scale, window_left=wl,
                                      window_right=wr)
    assert_parity(out, lse, ro, rl, dtype, desc)
