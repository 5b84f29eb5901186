"""The entry points under HIP graph capture: the library only enqueues kernels on
the caller's stream (no allocation, no synchronisation, no memset), so a captured
decode / prefill replays to the eager result bit for bit."""
import pytest
import torch

import workloads

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
