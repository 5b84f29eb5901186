"""GPU parity of attn_decode_paged_rope (rotary embedding applied in the
decode kernel) against the oracle's rope decode."""
import pytest
import torch

import oracle
import workloads
from helpers import assert_parity

pytestmark = pytest.mark.gpu


def _run(case, gpu, theta, scale=1.0, window=-1, layout="NHD", split_pages=0):
    import attention_qk_online_amd as A
    kp, vp = case.pools(gpu, layout=layout)
    out, lse = A.decode_paged(case.q.to(gpu), kp, vp, case.page_table.to(gpu), case.kv_lens.to(gpu),
                              scale=case.scale, max_kv_len=case.max_kv_len,
                              split_pages=split_pages, kv_layout=layout, window_left=window,
                              rope_theta=theta, rope_scale=scale)
    torch.cuda.synchronize()
    return out, lse


def _ref(case, theta, scale=1.0, window=-1):
    kp, vp = case.pools("cpu")
    return oracle.ref_decode_paged(case.q, kp, vp, case.page_table, case.kv_lens, case.scale,
                                   window_left=window, rope=(theta, scale))


@pytest.mark.parametrize("dtype,D,Hq,Hkv", [(torch.bfloat16, 128, 32, 8), (torch.bfloat16, 64, 8, 8),
                                            (torch.float16, 128, 8, 2), (torch.bfloat16, 128, 8, 1)])
@pytest.mark.parametrize("split_pages", [0, 2])
def test_rope_decode(gpu, dtype, D, Hq, Hkv, split_pages):
    lens = [1, 15, 16, 17, 300, 64, 1100, 0, 33]
    case = workloads.make_decode(B=len(lens), Hq=Hq, Hkv=Hkv, D=D, page_size=16, kv_lens=lens,
                                 dtype=dtype, seed=800 + D + Hq, extra_pages=4)
    for theta, scale in ((10000.0, 1.0), (500000.0, 4.0)):
        out, lse = _run(case, gpu, theta, scale, split_pages=split_pages)
        ro, rl = _ref(case, theta, scale)
        assert_parity(out, lse, ro, rl, dtype, f"rope {dtype} D{D} theta {theta} scale {scale}")


def test_rope_with_window_and_hnd(gpu):
    case = workloads.make_decode(B=4, Hq=16, Hkv=4, D=128, page_size=16, kv_lens=[700, 33, 2100, 1],
                                 dtype=torch.bfloat16, seed=810, extra_pages=3)
    out, lse = _run(case, gpu, 10000.0, window=300, layout="HND", split_pages=3)
    ro, rl = _ref(case, 10000.0, window=300)
    assert_parity(out, lse, ro, rl, torch.bfloat16, "rope + window 300, HND")
    o2, l2 = _run(case, gpu, 10000.0, window=300, layout="NHD", split_pages=3)
    assert torch.equal(out, o2) and torch.equal(lse, l2)


def test_rope_paged_config(gpu):
    """The batched paged GQA decode workload (B 64, Hq 32, Hkv 8, D 128, kv_len up to
    4096) with the rotary embedding (theta 10000)."""
    case = workloads.make_decode(B=64, Hq=32, Hkv=8, D=128, page_size=16, len_range=(512, 4096),
                                 dtype=torch.bfloat16, seed=2, num_pages=20000)
    out, lse = _run(case, gpu, 10000.0)
    ro, rl = _ref(case, 10000.0)
    assert_parity(out, lse, ro, rl, torch.bfloat16, "rope paged decode workload")
