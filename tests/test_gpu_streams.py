"""Calls enqueued on two streams at once: the library keeps no state between
calls, so decode and prefill calls that overlap on the device (each with its
own buffers) give, bit for bit, what they give one at a time."""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


def test_overlapping_calls_on_two_streams(gpu):
    import attention_qk_online_amd as A
    dec = workloads.make_decode(B=16, Hq=32, Hkv=8, D=128, page_size=16, len_range=(256, 2048),
                                dtype=torch.bfloat16, seed=1500, extra_pages=3)
    dec2 = workloads.make_decode(B=7, Hq=8, Hkv=2, D=64, page_size=32, len_range=(1, 900),
                                 dtype=torch.float16, seed=1501, extra_pages=3)
    pre = workloads.make_prefill(B=3, Hq=16, Hkv=4, D=128, lens_q=[700, 129, 1000],
                                 dtype=torch.bfloat16, seed=1502, causal=True)
    kp, vp = dec.pools(gpu)
    kp2, vp2 = dec2.pools(gpu)
    d_args = (dec.q.to(gpu), kp, vp, dec.page_table.to(gpu), dec.kv_lens.to(gpu))
    d2_args = (dec2.q.to(gpu), kp2, vp2, dec2.page_table.to(gpu), dec2.kv_lens.to(gpu))
    p_args = (pre.q.to(gpu), pre.k.to(gpu), pre.v.to(gpu), pre.cu_seqlens_q.to(gpu),
              pre.cu_seqlens_k.to(gpu), pre.max_seqlen_q, pre.max_seqlen_k)

    def run_dec():
        return A.decode_paged(*d_args, scale=dec.scale, max_kv_len=dec.max_kv_len)

    def run_dec2():
        return A.decode_paged(*d2_args, scale=dec2.scale, max_kv_len=dec2.max_kv_len, split_pages=2)

    def run_pre():
        return A.prefill_varlen(*p_args, causal=True, scale=pre.scale)

    ref = [run_dec(), run_dec2(), run_pre()]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    main = torch.cuda.current_stream()
    for rep in range(3):
        s1.wait_stream(main)
        s2.wait_stream(main)
        with torch.cuda.stream(s1):
            got_pre = run_pre()
            got_dec2 = run_dec2()
        with torch.cuda.stream(s2):
            got_dec = run_dec()
        main.wait_stream(s1)
        main.wait_stream(s2)
        torch.cuda.synchronize()
        for name, got, want in (("decode", got_dec, ref[0]), ("decode fp16", got_dec2, ref[1]),
                                ("prefill", got_pre, ref[2])):
            assert torch.equal(got[0], want[0]) and torch.equal(got[1], want[1]), (rep, name)
