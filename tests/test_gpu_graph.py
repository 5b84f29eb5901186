"""The entry points under HIP graph capture: the library only enqueues kernels on
the caller's stream (no allocation, no synchronisation, no memset), so a captured
decode / prefill replays to the eager result bit for bit, and the replayed
results match the oracle."""
import pytest
import torch

import oracle
import workloads
from helpers import assert_parity

pytestmark = pytest.mark.gpu


def test_decode_and_prefill_replay_in_a_graph(gpu):
    import attention_qk_online_amd as A
    dec = workloads.make_decode(B=6, Hq=8, Hkv=2, D=128, page_size=16, kv_lens=[100, 1, 700, 33, 0, 256],
                                dtype=torch.bfloat16, seed=500, extra_pages=3)
    one = workloads.make_config(1)
    pre = workloads.make_prefill(B=3, Hq=8, Hkv=2, D=128, lens_q=[200, 65, 130], dtype=torch.bfloat16,
                                 seed=501, causal=True)
    d_kp, d_vp = dec.pools(gpu)
    d_in = (dec.q.to(gpu), d_kp, d_vp, dec.page_table.to(gpu), dec.kv_lens.to(gpu))
    o_kp, o_vp = one.pools(gpu)
    o_in = (one.q.to(gpu), o_kp, o_vp, one.page_table.to(gpu), one.kv_lens.to(gpu))
    p_in = (pre.q.to(gpu), pre.k.to(gpu), pre.v.to(gpu), pre.cu_seqlens_q.to(gpu), pre.cu_seqlens_k.to(gpu))
    d_out, d_lse = torch.empty_like(d_in[0]), torch.empty(dec.B, dec.Hq, device=gpu)
    o_out, o_lse = torch.empty_like(o_in[0]), torch.empty(one.B, one.Hq, device=gpu)
    p_out, p_lse = torch.empty_like(p_in[0]), torch.empty(p_in[0].shape[:2], device=gpu)
    ws_d = torch.empty(A.decode_paged_workspace_size(torch.bfloat16, dec.B, dec.Hq, dec.Hkv, dec.D, 16,
                                                     dec.max_kv_len, 0), dtype=torch.uint8, device=gpu)
    ws_o = torch.empty(max(1, A.decode_paged_workspace_size(torch.float32, one.B, one.Hq, one.Hkv, one.D,
                                                            16, one.max_kv_len, 2)),
                       dtype=torch.uint8, device=gpu)

    def run():
        A.decode_paged(*d_in, scale=dec.scale, max_kv_len=dec.max_kv_len, out=d_out, lse=d_lse,
                       workspace=ws_d)
        A.decode_paged(*o_in, scale=one.scale, max_kv_len=one.max_kv_len, split_pages=2, out=o_out,
                       lse=o_lse, workspace=ws_o)
        A.prefill_varlen(*p_in, pre.max_seqlen_q, pre.max_seqlen_k, causal=True, scale=pre.scale,
                         out=p_out, lse=p_lse)

    run()
    torch.cuda.synchronize()
    refs = [t.clone() for t in (d_out, d_lse, o_out, o_lse, p_out, p_lse)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()

    for rep in range(4):
        for t in (d_out, d_lse, o_out, o_lse, p_out, p_lse):
            t.fill_(float("nan"))
        # eager work of the program between replays, on other buffers
        A.decode_paged(*d_in, scale=dec.scale, max_kv_len=dec.max_kv_len)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip((d_out, d_lse, o_out, o_lse, p_out, p_lse), refs):
            assert torch.equal(got, ref), f"replay {rep}"

    # The replayed results against the oracle (not only against the eager run).
    kc, vc = dec.pools("cpu")
    ro, rl = oracle.ref_decode_paged(dec.q, kc, vc, dec.page_table, dec.kv_lens, dec.scale)
    assert_parity(d_out, d_lse, ro, rl, torch.bfloat16, "graph replay: bf16 decode")
    kc, vc = one.pools("cpu")
    ro, rl = oracle.ref_decode_paged(one.q, kc, vc, one.page_table, one.kv_lens, one.scale)
    assert_parity(o_out, o_lse, ro, rl, torch.float32, "graph replay: fp32 decode")
    ro, rl = oracle.ref_prefill_varlen(pre.q, pre.k, pre.v, pre.cu_seqlens_q, pre.cu_seqlens_k,
                                       True, pre.scale)
    assert_parity(p_out, p_lse, ro, rl, torch.bfloat16, "graph replay: causal prefill")


def test_more_entry_points_replay_in_a_graph(gpu):
    """E4M3 decode with a sliding window, paged prefill (HND) with a window on
    both sides, the shared-prefix cascade (two launches through a workspace)
    and the state merge, captured together: every replay equals the eager run."""
    import attention_qk_online_amd as A
    dec = workloads.make_decode(B=5, Hq=16, Hkv=4, D=128, page_size=16, kv_lens=[33, 400, 16, 1, 250],
                                dtype=torch.bfloat16, seed=510, extra_pages=3)
    kb, vb, ks, vs = dec.fp8_pools()
    f_in = (dec.q.to(gpu), kb.to(gpu), vb.to(gpu), dec.page_table.to(gpu), dec.kv_lens.to(gpu))
    f_out, f_lse = torch.empty_like(f_in[0]), torch.empty(dec.B, dec.Hq, device=gpu)
    ws_f = torch.empty(A.decode_paged_workspace_size(torch.bfloat16, dec.B, dec.Hq, dec.Hkv, dec.D, 16,
                                                     dec.max_kv_len, 0), dtype=torch.uint8, device=gpu)
    pg = workloads.make_paged_prefill(B=3, Hq=4, Hkv=2, D=128, page_size=16, chunk=90, cached=250,
                                      shared_prefix=64, dtype=torch.bfloat16, seed=511)
    h_kp, h_vp = pg.pools(gpu, layout="HND")
    n_kp, n_vp = pg.pools(gpu)
    g_in = (pg.q.to(gpu), pg.cu_seqlens_q.to(gpu))
    g_tab = (pg.page_table.to(gpu), pg.kv_lens.to(gpu))
    w_out, w_lse = torch.empty_like(g_in[0]), torch.empty(g_in[0].shape[:2], device=gpu)
    c_out, c_lse = torch.empty_like(g_in[0]), torch.empty(g_in[0].shape[:2], device=gpu)
    ws_c = torch.empty(A.prefill_paged_cascade_workspace_size(torch.bfloat16, g_in[0].shape[0], pg.Hq,
                                                              pg.D), dtype=torch.uint8, device=gpu)
    m_a = torch.randn(300, 4, 128, generator=torch.Generator().manual_seed(512)).to(torch.bfloat16).to(gpu)
    m_b = torch.randn(300, 4, 128, generator=torch.Generator().manual_seed(513)).to(torch.bfloat16).to(gpu)
    l_a = torch.randn(300, 4, generator=torch.Generator().manual_seed(514)).to(gpu)
    l_b = torch.randn(300, 4, generator=torch.Generator().manual_seed(515)).to(gpu)
    m_out, m_lse = torch.empty_like(m_a), torch.empty_like(l_a)
    outs = (f_out, f_lse, w_out, w_lse, c_out, c_lse, m_out, m_lse)

    def run():
        A.decode_paged_fp8(*f_in, ks, vs, scale=dec.scale, max_kv_len=dec.max_kv_len, out=f_out,
                           lse=f_lse, workspace=ws_f, window_left=37)
        A.prefill_paged(*g_in, h_kp, h_vp, *g_tab, pg.max_seqlen_q, pg.max_kv_len, causal=False,
                        scale=pg.scale, out=w_out, lse=w_lse, kv_layout="HND", window_left=70,
                        window_right=20)
        A.prefill_paged_cascade(*g_in, n_kp, n_vp, *g_tab, pg.max_seqlen_q, pg.max_kv_len, 64,
                                causal=True, scale=pg.scale, out=c_out, lse=c_lse, workspace=ws_c)
        A.merge_states(m_a, l_a, m_b, l_b, out=m_out, lse_out=m_lse)

    run()
    torch.cuda.synchronize()
    refs = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()

    for rep in range(4):
        for t in outs:
            t.fill_(float("nan"))
        # eager work of the program between replays, on other buffers
        A.prefill_paged(*g_in, n_kp, n_vp, *g_tab, pg.max_seqlen_q, pg.max_kv_len, causal=True,
                        scale=pg.scale)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip(outs, refs):
            assert torch.equal(got, ref), f"replay {rep}"

    # The replayed results against the oracle.
    ro, rl = oracle.ref_decode_paged_fp8(dec.q, kb, vb, ks, vs, dec.page_table, dec.kv_lens, dec.scale,
                                         window_left=37)
    assert_parity(f_out, f_lse, ro, rl, torch.bfloat16, "graph replay: E4M3 decode, window 37")
    ro, rl = oracle.ref_prefill_paged(pg.q, pg.cu_seqlens_q, pg.pool_k, pg.pool_v, pg.page_table,
                                      pg.kv_lens, False, pg.scale, window_left=70, window_right=20)
    assert_parity(w_out, w_lse, ro, rl, torch.bfloat16, "graph replay: HND paged prefill, band")
    ro, rl = oracle.ref_prefill_paged(pg.q, pg.cu_seqlens_q, pg.pool_k, pg.pool_v, pg.page_table,
                                      pg.kv_lens, True, pg.scale)
    assert_parity(c_out, c_lse, ro, rl, torch.bfloat16, "graph replay: cascade")
    ro, rl = oracle.merge_states([(m_a.cpu(), l_a.cpu()), (m_b.cpu(), l_b.cpu())])
    assert_parity(m_out, m_lse, ro, rl, torch.bfloat16, "graph replay: state merge")


def test_head_dim_256_and_long_request_merge_replay_in_a_graph(gpu):
    """head_dim 256: ragged prefill and paged-prefill cascade (pairs of waves
    exchanging P through LDS), and a one-request decode whose merge splits
    heads and d over workgroups, captured together; every replay equals the
    eager run bit for bit and the oracle."""
    import attention_qk_online_amd as A
    pre = workloads.make_prefill(B=2, Hq=4, Hkv=2, D=256, lens_q=[300, 97], dtype=torch.bfloat16,
                                 seed=505, causal=True)
    pg = workloads.make_paged_prefill(B=2, Hq=4, Hkv=4, D=256, page_size=16, chunk=[70, 33],
                                      cached=[160, 100], shared_prefix=64, dtype=torch.bfloat16, seed=506)
    dec = workloads.make_decode(B=1, Hq=32, Hkv=8, D=128, page_size=16, kv_lens=[6000],
                                dtype=torch.bfloat16, seed=507, extra_pages=2)
    p_in = (pre.q.to(gpu), pre.k.to(gpu), pre.v.to(gpu), pre.cu_seqlens_q.to(gpu), pre.cu_seqlens_k.to(gpu))
    kp, vp = pg.pools(gpu)
    g_in = (pg.q.to(gpu), pg.cu_seqlens_q.to(gpu), kp, vp, pg.page_table.to(gpu), pg.kv_lens.to(gpu))
    d_kp, d_vp = dec.pools(gpu)
    d_in = (dec.q.to(gpu), d_kp, d_vp, dec.page_table.to(gpu), dec.kv_lens.to(gpu))
    p_out, p_lse = torch.empty_like(p_in[0]), torch.empty(p_in[0].shape[:2], device=gpu)
    c_out, c_lse = torch.empty_like(g_in[0]), torch.empty(g_in[0].shape[:2], device=gpu)
    d_out, d_lse = torch.empty_like(d_in[0]), torch.empty(dec.B, dec.Hq, device=gpu)
    ws_c = torch.empty(A.prefill_paged_cascade_workspace_size(torch.bfloat16, g_in[0].shape[0], pg.Hq,
                                                              pg.D), dtype=torch.uint8, device=gpu)
    ws_d = torch.empty(A.decode_paged_workspace_size(torch.bfloat16, dec.B, dec.Hq, dec.Hkv, dec.D, 16,
                                                     dec.max_kv_len, 0), dtype=torch.uint8, device=gpu)

    def run():
        A.prefill_varlen(*p_in, pre.max_seqlen_q, pre.max_seqlen_k, causal=True, scale=pre.scale,
                         out=p_out, lse=p_lse)
        A.prefill_paged_cascade(*g_in, pg.max_seqlen_q, pg.max_kv_len, 64, causal=True,
                                scale=pg.scale, out=c_out, lse=c_lse, workspace=ws_c)
        A.decode_paged(*d_in, scale=dec.scale, max_kv_len=dec.max_kv_len, out=d_out, lse=d_lse,
                       workspace=ws_d)

    run()
    torch.cuda.synchronize()
    outs = (p_out, p_lse, c_out, c_lse, d_out, d_lse)
    refs = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(4):
        for t in outs:
            t.fill_(float("nan"))
        A.prefill_varlen(*p_in, pre.max_seqlen_q, pre.max_seqlen_k, causal=True, scale=pre.scale)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip(outs, refs):
            assert torch.equal(got, ref), f"replay {rep}"

    ro, rl = oracle.ref_prefill_varlen(pre.q, pre.k, pre.v, pre.cu_seqlens_q, pre.cu_seqlens_k, True,
                                       pre.scale)
    assert_parity(p_out, p_lse, ro, rl, torch.bfloat16, "graph replay: head_dim 256 prefill")
    ro, rl = oracle.ref_prefill_paged(pg.q, pg.cu_seqlens_q, pg.pool_k, pg.pool_v, pg.page_table,
                                      pg.kv_lens, True, pg.scale)
    assert_parity(c_out, c_lse, ro, rl, torch.bfloat16, "graph replay: head_dim 256 cascade")
    kc, vc = dec.pools("cpu")
    ro, rl = oracle.ref_decode_paged(dec.q, kc, vc, dec.page_table, dec.kv_lens, dec.scale)
    assert_parity(d_out, d_lse, ro, rl, torch.bfloat16, "graph replay: one long decode request")
