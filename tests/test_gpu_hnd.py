"""GPU parity of the HND page layout ([pages, Hkv, page_size, D]).

An HND pool is the NHD pool with its middle dimensions swapped, so every
entry point must give the NHD call's result bit for bit on the permuted
cache; one case per entry point is also checked against the oracle (on the
NHD view of the same cache).
"""
import pytest
import torch

import oracle
import workloads
from helpers import assert_parity

pytestmark = pytest.mark.gpu


def _decode(case, gpu, layout, split_pages=0):
    import attention_qk_online_amd as A
    kp, vp = case.pools(gpu, layout=layout)
    out, lse = A.decode_paged(case.q.to(gpu), kp, vp, case.page_table.to(gpu), case.kv_lens.to(gpu),
                              scale=case.scale, max_kv_len=case.max_kv_len,
                              split_pages=split_pages, kv_layout=layout)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("dtype,D,Hq,Hkv", [(torch.bfloat16, 128, 32, 8), (torch.bfloat16, 256, 16, 2),
                                            (torch.float16, 64, 8, 8), (torch.float32, 128, 8, 2),
                                            (torch.float32, 64, 4, 4)])
@pytest.mark.parametrize("split_pages", [0, 3])
def test_decode_hnd_equals_nhd(gpu, dtype, D, Hq, Hkv, split_pages):
    lens = [1, 15, 16, 17, 300, 64, 1000, 0]
    case = workloads.make_decode(B=len(lens), Hq=Hq, Hkv=Hkv, D=D, page_size=16, kv_lens=lens,
                                 dtype=dtype, seed=600 + D + Hq, extra_pages=4)
    o1, l1 = _decode(case, gpu, "NHD", split_pages)
    o2, l2 = _decode(case, gpu, "HND", split_pages)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_hnd_paged_config(gpu):
    """The batched paged GQA decode workload (B 64, Hq 32, Hkv 8, D 128) in HND."""
    case = workloads.make_decode(B=64, Hq=32, Hkv=8, D=128, page_size=16, len_range=(512, 4096),
                                 dtype=torch.bfloat16, seed=2, num_pages=20000)
    out, lse = _decode(case, gpu, "HND")
    kp, vp = case.pools("cpu")
    ro, rl = oracle.ref_decode_paged(case.q, kp, vp, case.page_table, case.kv_lens, case.scale)
    assert_parity(out, lse, ro, rl, torch.bfloat16, "HND paged decode")


def test_decode_fp8_hnd_equals_nhd(gpu):
    import attention_qk_online_amd as A
    case = workloads.make_decode(B=5, Hq=16, Hkv=4, D=128, page_size=16, kv_lens=[33, 400, 16, 1, 250],
                                 dtype=torch.bfloat16, seed=610, extra_pages=3)
    res = []
    for layout in ("NHD", "HND"):
        kb, vb, ks, vs = case.fp8_pools(gpu, layout=layout)
        res.append(A.decode_paged_fp8(case.q.to(gpu), kb, vb, case.page_table.to(gpu),
                                      case.kv_lens.to(gpu), ks, vs, scale=case.scale,
                                      max_kv_len=case.max_kv_len, split_pages=2, kv_layout=layout))
    torch.cuda.synchronize()
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
    kb, vb, ks, vs = case.fp8_pools("cpu")
    ro, rl = oracle.ref_decode_paged_fp8(case.q, kb, vb, ks, vs, case.page_table, case.kv_lens,
                                         case.scale)
    assert_parity(res[1][0], res[1][1], ro, rl, torch.bfloat16, "fp8 HND decode")


def _paged(case, gpu, layout, cascade=False):
    import attention_qk_online_amd as A
    kp, vp = case.pools(gpu, layout=layout)
    args = (case.q.to(gpu), case.cu_seqlens_q.to(gpu), kp, vp, case.page_table.to(gpu),
            case.kv_lens.to(gpu), case.max_seqlen_q, case.max_kv_len)
    if cascade:
        out, lse = A.prefill_paged_cascade(*args, case.shared_pages * case.page_size,
                                           causal=case.causal, scale=case.scale, kv_layout=layout)
    else:
        out, lse = A.prefill_paged(*args, causal=case.causal, scale=case.scale, kv_layout=layout)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("D,dtype", [(128, torch.bfloat16), (256, torch.bfloat16), (128, torch.float16)])
@pytest.mark.parametrize("cascade", [False, True])
def test_prefill_paged_hnd_equals_nhd(gpu, D, dtype, cascade):
    case = workloads.make_paged_prefill(B=3, Hq=8, Hkv=2, D=D, page_size=16, chunk=90, cached=250,
                                        shared_prefix=64, dtype=dtype, seed=620 + D)
    o1, l1 = _paged(case, gpu, "NHD", cascade)
    o2, l2 = _paged(case, gpu, "HND", cascade)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    if not cascade:
        ro, rl = oracle.ref_prefill_paged(case.q, case.cu_seqlens_q, case.pool_k, case.pool_v,
                                          case.page_table, case.kv_lens, True, case.scale)
        assert_parity(o2, l2, ro, rl, dtype, f"HND paged prefill D{D}")


def test_prefill_paged_hnd_chunked_config(gpu):
    """The chunked paged workload (16 x 512 queries, 8704 keys, D 256) in HND equals NHD."""
    case = workloads.make_config(5)
    o1, l1 = _paged(case, gpu, "NHD")
    o2, l2 = _paged(case, gpu, "HND")
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
