"""GPU parity of attn_merge_states and attn_prefill_paged_cascade against the oracle.

The cascade has no oracle of its own: its contract is the result of
attn_prefill_paged on the same arguments, so every case here is checked
against oracle.ref_prefill_paged (attention over each request's whole key
range), and merge_states against oracle.merge_states.
"""
import math

import pytest
import torch

import oracle
import workloads
from helpers import TOL, assert_parity

pytestmark = pytest.mark.gpu


# ----------------------------------------------------------------- merge ---
def _merge_inputs(T, H, D, dtype, seed):
    """Two states over [T, H] rows; row classes by index mod 8: 0 -> a empty,
    1 -> b empty, 2 -> both empty, 3 -> lse_a NaN, 4 -> far-apart lse (one
    weight underflows), others random.  o of an empty side is finite garbage."""
    g = torch.Generator().manual_seed(seed)
    oa = torch.randn((T, H, D), generator=g).to(dtype)
    ob = torch.randn((T, H, D), generator=g).to(dtype)
    la = torch.rand((T, H), generator=g) * 20 - 10
    lb = torch.rand((T, H), generator=g) * 20 - 10
    cls = (torch.arange(T * H) % 8).view(T, H)
    la[cls == 0] = -math.inf
    oa[cls == 0] = 1e4
    lb[cls == 1] = -math.inf
    ob[cls == 1] = -3e3
    la[cls == 2] = -math.inf
    lb[cls == 2] = -math.inf
    la[cls == 3] = math.nan
    la[cls == 4] = 80.0
    lb[cls == 4] = -60.0
    return oa, la, ob, lb, cls


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_merge_states(gpu, dtype, D):
    import attention_qk_online_amd as A
    T, H = 37, 6
    oa, la, ob, lb, cls = _merge_inputs(T, H, D, dtype, 400 + D)
    dev = [x.to(gpu) for x in (oa, la, ob, lb)]
    out, lse = A.merge_states(*dev)
    torch.cuda.synchronize()
    nan = cls == 3
    assert torch.isnan(out[nan.to(gpu)].float()).all() and torch.isnan(lse[nan.to(gpu)]).all()
    ok = ~nan
    ro, rl = oracle.merge_states([(oa[ok], la[ok]), (ob[ok], lb[ok])])
    assert_parity(out[ok.to(gpu)], lse[ok.to(gpu)], ro, rl, dtype, f"merge {dtype} D{D}")
    both = (cls == 2).to(gpu)
    assert (out[both] == 0).all() and torch.isneginf(lse[both]).all()

    # in place on the b side, then on the a side: same bits as out of place
    ob2, lb2 = dev[2].clone(), dev[3].clone()
    A.merge_states(dev[0], dev[1], ob2, lb2, out=ob2, lse_out=lb2)
    oa2, la2 = dev[0].clone(), dev[1].clone()
    A.merge_states(oa2, la2, dev[2], dev[3], out=oa2, lse_out=la2)
    torch.cuda.synchronize()
    for o2, l2 in ((ob2, lb2), (oa2, la2)):
        assert torch.equal(o2[ok.to(gpu)], out[ok.to(gpu)])
        assert torch.equal(l2[ok.to(gpu)], lse[ok.to(gpu)])


def test_merge_states_empty_rows(gpu):
    import attention_qk_online_amd as A
    z = torch.zeros((0, 4, 128), dtype=torch.bfloat16, device=gpu)
    zl = torch.zeros((0, 4), dtype=torch.float32, device=gpu)
    out, lse = A.merge_states(z, zl, z, zl)
    assert out.shape == z.shape and lse.shape == zl.shape


def test_merge_of_split_prefill_equals_whole(gpu):
    """Attention over keys [0, n) and [n, L) (two varlen calls), merged on the
    GPU, matches the oracle's attention over [0, L)."""
    import attention_qk_online_amd as A
    case = workloads.make_prefill(B=1, Hq=8, Hkv=2, D=128, lens_q=[200], lens_k=[700],
                                  dtype=torch.bfloat16, seed=410, causal=False)
    n = 300
    parts = []
    for a, b in ((0, n), (n, 700)):
        cu_k = torch.tensor([0, b - a], dtype=torch.int32, device=gpu)
        parts.append(A.prefill_varlen(case.q.to(gpu), case.k[a:b].contiguous().to(gpu),
                                      case.v[a:b].contiguous().to(gpu),
                                      case.cu_seqlens_q.to(gpu), cu_k, 200, b - a,
                                      causal=False, scale=case.scale))
    out, lse = A.merge_states(parts[0][0], parts[0][1], parts[1][0], parts[1][1])
    torch.cuda.synchronize()
    ro, rl = oracle.ref_prefill_varlen(case.q, case.k, case.v, case.cu_seqlens_q,
                                       case.cu_seqlens_k, False, case.scale)
    assert_parity(out, lse, ro, rl, torch.bfloat16, "split keys merged")


# --------------------------------------------------------------- cascade ---
def _cascade(case, gpu, prefix=None, causal=None, q=None, cu=None, kv_lens=None, table=None,
             max_seqlen_q=None):
    import attention_qk_online_amd as A
    kp, vp = case.pools(gpu)
    prefix = case.shared_pages * case.page_size if prefix is None else prefix
    causal = case.causal if causal is None else causal
    q = case.q if q is None else q
    cu = case.cu_seqlens_q if cu is None else cu
    kv_lens = case.kv_lens if kv_lens is None else kv_lens
    table = case.page_table if table is None else table
    if max_seqlen_q is None:
        max_seqlen_q = int((cu[1:] - cu[:-1]).max())
    out, lse = A.prefill_paged_cascade(q.to(gpu), cu.to(gpu), kp, vp, table.to(gpu),
                                       kv_lens.to(gpu), max_seqlen_q, int(kv_lens.max()),
                                       prefix, causal=causal, scale=case.scale)
    torch.cuda.synchronize()
    return out, lse


def _ref(case, causal=None, q=None, cu=None, kv_lens=None, rows=None):
    causal = case.causal if causal is None else causal
    return oracle.ref_prefill_paged(case.q if q is None else q,
                                    case.cu_seqlens_q if cu is None else cu,
                                    case.pool_k, case.pool_v, case.page_table,
                                    case.kv_lens if kv_lens is None else kv_lens, causal,
                                    case.scale, rows=rows)


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_cascade_small(gpu, D, causal):
    case = workloads.make_paged_prefill(B=3, Hq=4, Hkv=2, D=D, page_size=16, chunk=70, cached=200,
                                        shared_prefix=64, dtype=torch.bfloat16, seed=420 + D,
                                        causal=causal)
    out, lse = _cascade(case, gpu)
    ro, rl = _ref(case)
    assert_parity(out, lse, ro, rl, torch.bfloat16, f"cascade D{D} causal={causal}")


@pytest.mark.parametrize("D", [128, 256])
def test_cascade_fp16_gqa(gpu, D):
    case = workloads.make_paged_prefill(B=2, Hq=16, Hkv=2, D=D, page_size=16, chunk=130,
                                        cached=300, shared_prefix=160, dtype=torch.float16,
                                        seed=430 + D)
    out, lse = _cascade(case, gpu)
    ro, rl = _ref(case)
    assert_parity(out, lse, ro, rl, torch.float16, f"cascade fp16 G8 D{D}")


def test_cascade_ragged_queries(gpu):
    """Requests with 1, 129 and 40 queries (each the last tokens of its cache)."""
    case = workloads.make_paged_prefill(B=3, Hq=4, Hkv=4, D=128, page_size=16, chunk=150,
                                        cached=250, shared_prefix=128, dtype=torch.bfloat16,
                                        seed=440)
    lens = [1, 129, 40]
    cu = torch.tensor([0, 1, 130, 170], dtype=torch.int32)
    q = torch.randn((170, 4, 128), generator=torch.Generator().manual_seed(441)).to(torch.bfloat16)
    out, lse = _cascade(case, gpu, q=q, cu=cu)
    ro, rl = _ref(case, q=q, cu=cu)
    assert_parity(out, lse, ro, rl, torch.bfloat16, f"cascade ragged {lens}")


def test_cascade_no_prefix_is_plain_paged(gpu):
    import attention_qk_online_amd as A
    case = workloads.make_paged_prefill(B=2, Hq=4, Hkv=2, D=256, page_size=16, chunk=90, cached=160,
                                        shared_prefix=32, dtype=torch.bfloat16, seed=450)
    out, lse = _cascade(case, gpu, prefix=0)
    kp, vp = case.pools(gpu)
    o2, l2 = A.prefill_paged(case.q.to(gpu), case.cu_seqlens_q.to(gpu), kp, vp,
                             case.page_table.to(gpu), case.kv_lens.to(gpu), case.max_seqlen_q,
                             case.max_kv_len, causal=True, scale=case.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2)


def test_cascade_prefix_is_whole_cache(gpu):
    """Non-causal, kv_lens equal to the prefix for one request: its own part is
    empty and the result is the prefix pass alone."""
    case = workloads.make_paged_prefill(B=2, Hq=4, Hkv=2, D=128, page_size=16, chunk=50, cached=142,
                                        shared_prefix=96, dtype=torch.bfloat16, seed=460,
                                        causal=False)
    kv = case.kv_lens.clone()
    kv[0] = 96
    out, lse = _cascade(case, gpu, kv_lens=kv)
    ro, rl = _ref(case, kv_lens=kv)
    assert_parity(out, lse, ro, rl, torch.bfloat16, "cascade, empty own part")


def test_cascade_query_inside_prefix_is_nan(gpu):
    """Causal, a request whose queries reach back into the shared prefix breaks the
    cascade's precondition: its rows are NaN, the other request is exact."""
    case = workloads.make_paged_prefill(B=2, Hq=4, Hkv=2, D=128, page_size=16, chunk=80, cached=120,
                                        shared_prefix=64, dtype=torch.bfloat16, seed=470)
    kv = case.kv_lens.clone()
    kv[1] = 64 + 79          # 79 own tokens for 80 queries
    out, lse = _cascade(case, gpu, kv_lens=kv)
    ro, rl = _ref(case, kv_lens=kv)
    n0 = int(case.cu_seqlens_q[1])
    assert_parity(out[:n0], lse[:n0], ro[:n0], rl[:n0], torch.bfloat16, "valid request")
    assert torch.isnan(out[n0:].float()).all() and torch.isnan(lse[n0:]).all()


def test_cascade_bad_prefix_page_is_nan(gpu):
    """A page id outside the pool in the shared prefix poisons every row."""
    case = workloads.make_paged_prefill(B=2, Hq=4, Hkv=2, D=128, page_size=16, chunk=40, cached=100,
                                        shared_prefix=48, dtype=torch.bfloat16, seed=480)
    table = case.page_table.clone()
    table[0, 1] = case.num_pages + 3
    out, lse = _cascade(case, gpu, table=table)
    assert torch.isnan(out.float()).all() and torch.isnan(lse).all()


def test_cascade_chunked_config_all_rows(gpu):
    """The chunked paged workload (16 requests x 512 queries over 8704 keys, the
    first 4096 shared; Hq = Hkv = 16, D 256) through the cascade: every row
    against the oracle and against the direct paged call."""
    import attention_qk_online_amd as A
    case = workloads.make_config(5)
    out, lse = _cascade(case, gpu)
    ro, rl = _ref(case)
    assert_parity(out, lse, ro, rl, torch.bfloat16, case.name + " cascade (all rows)")
    kp, vp = case.pools(gpu)
    o2, l2 = A.prefill_paged(case.q.to(gpu), case.cu_seqlens_q.to(gpu), kp, vp,
                             case.page_table.to(gpu), case.kv_lens.to(gpu), case.max_seqlen_q,
                             case.max_kv_len, causal=True, scale=case.scale)
    torch.cuda.synchronize()
    d = (out.float() - o2.float()).abs().max().item()
    dl = (lse - l2).abs().max().item()
    print(f"cascade vs direct: max|d out| {d:.3e}, max|d lse| {dl:.3e}", flush=True)
    assert d <= TOL[torch.bfloat16] and dl <= TOL[torch.bfloat16]
    assert torch.isfinite(out.float()).all()
