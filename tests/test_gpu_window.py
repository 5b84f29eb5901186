"""GPU parity of the sliding-window prefill (attn_prefill_varlen_window,
attn_prefill_paged_window) against the oracle's window_left / window_right,
and of the sliding-window decode."""
import pytest
import torch

import oracle
import workloads
from helpers import assert_parity

pytestmark = pytest.mark.gpu


def _varlen(case, gpu, window, causal=None, right=-1):
    import attention_qk_online_amd as A
    causal = case.causal if causal is None else causal
    out, lse = A.prefill_varlen(case.q.to(gpu), case.k.to(gpu), case.v.to(gpu),
                                case.cu_seqlens_q.to(gpu), case.cu_seqlens_k.to(gpu),
                                case.max_seqlen_q, case.max_seqlen_k, causal=causal,
                                scale=case.scale, window_left=window, window_right=right)
    torch.cuda.synchronize()
    return out, lse


def _ref(case, window, causal=None, rows=None, right=-1):
    causal = case.causal if causal is None else causal
    return oracle.ref_prefill_varlen(case.q, case.k, case.v, case.cu_seqlens_q, case.cu_seqlens_k,
                                     causal, case.scale, rows=rows, window_left=window,
                                     window_right=right)


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window", [0, 1, 63, 64, 100, 128, 500])
def test_window_small(gpu, D, causal, window):
    lens = [1, 17, 128, 129, 300, 64, 255]
    case = workloads.make_prefill(B=len(lens), Hq=4, Hkv=2, D=D, lens_q=lens, dtype=torch.bfloat16,
                                  seed=700 + D, causal=causal)
    out, lse = _varlen(case, gpu, window)
    ro, rl = _ref(case, window)
    assert_parity(out, lse, ro, rl, torch.bfloat16, f"window {window} D{D} causal={causal}")


@pytest.mark.parametrize("causal", [True, False])
def test_window_q_shorter_than_k(gpu, causal):
    """Lq < Lk: the window is aligned bottom-right like the causal mask."""
    case = workloads.make_prefill(B=3, Hq=4, Hkv=4, D=128, lens_q=[50, 200, 7], lens_k=[400, 333, 900],
                                  dtype=torch.bfloat16, seed=710, causal=causal)
    for window in (10, 150, 600):
        out, lse = _varlen(case, gpu, window)
        ro, rl = _ref(case, window)
        assert_parity(out, lse, ro, rl, torch.bfloat16, f"Lq<Lk window {window}")


def test_window_wider_than_keys_is_no_window(gpu):
    """A window covering every key gives the plain call's result bit for bit."""
    case = workloads.make_prefill(B=2, Hq=8, Hkv=2, D=128, lens_q=[300, 129], dtype=torch.bfloat16,
                                  seed=720, causal=True)
    o1, l1 = _varlen(case, gpu, -1)
    o2, l2 = _varlen(case, gpu, 300)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_window_paged(gpu, D, layout):
    import attention_qk_online_amd as A
    case = workloads.make_paged_prefill(B=3, Hq=4, Hkv=2, D=D, page_size=16, chunk=90, cached=250,
                                        shared_prefix=64, dtype=torch.bfloat16, seed=730 + D)
    kp, vp = case.pools(gpu, layout=layout)
    for window in (0, 77, 200):
        out, lse = A.prefill_paged(case.q.to(gpu), case.cu_seqlens_q.to(gpu), kp, vp,
                                   case.page_table.to(gpu), case.kv_lens.to(gpu), case.max_seqlen_q,
                                   case.max_kv_len, causal=True, scale=case.scale,
                                   kv_layout=layout, window_left=window)
        torch.cuda.synchronize()
        ro, rl = oracle.ref_prefill_paged(case.q, case.cu_seqlens_q, case.pool_k, case.pool_v,
                                          case.page_table, case.kv_lens, True, case.scale,
                                          window_left=window)
        assert_parity(out, lse, ro, rl, torch.bfloat16, f"paged {layout} D{D} window {window}")


def test_window_ragged_config_sampled(gpu):
    """The ragged causal workload (B 8, L in [1024, 4096], Hq 64, Hkv 8, D 128) with a
    1024-key window, sampled rows."""
    case = workloads.make_config(3)
    out, lse = _varlen(case, gpu, 1024)
    cu = [int(x) for x in case.cu_seqlens_q]
    g = torch.Generator().manual_seed(740)
    rows = set(torch.randint(0, cu[-1], (64,), generator=g).tolist())
    for a, b in zip(cu[:-1], cu[1:]):
        rows.update(r for r in (a, a + 1023, a + 1024, a + 1025, b - 1) if a <= r < b)
    rows = torch.tensor(sorted(rows))
    ro, rl = _ref(case, 1024, rows=rows)
    assert_parity(out, lse, ro, rl, torch.bfloat16, "ragged window 1024 (sampled rows)", rows=rows)
    assert torch.isfinite(out.float()).all()


def test_window_chunked_paged_config_sampled(gpu):
    """The chunked paged workload (16 x 512 queries over 8704 keys, D 256) with a 2048-key window."""
    import attention_qk_online_amd as A
    case = workloads.make_config(5)
    kp, vp = case.pools(gpu)
    out, lse = A.prefill_paged(case.q.to(gpu), case.cu_seqlens_q.to(gpu), kp, vp,
                               case.page_table.to(gpu), case.kv_lens.to(gpu), case.max_seqlen_q,
                               case.max_kv_len, causal=True, scale=case.scale, window_left=2048)
    torch.cuda.synchronize()
    cu = [int(x) for x in case.cu_seqlens_q]
    rows = torch.tensor(sorted({r for a, b in zip(cu[:-1], cu[1:]) for r in (a, a + 200, b - 1)}))
    ro, rl = oracle.ref_prefill_paged(case.q, case.cu_seqlens_q, case.pool_k, case.pool_v,
                                      case.page_table, case.kv_lens, True, case.scale, rows=rows,
                                      window_left=2048)
    assert_parity(out, lse, ro, rl, torch.bfloat16, "chunked paged window 2048 (sampled)", rows=rows)


# --------------------------------------------------- right side of the window ---
WINDOWS = [(-1, 0), (-1, 1), (-1, 63), (-1, 64), (-1, 200), (10, 5), (0, 0), (100, 30), (64, 64)]


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("left,right", WINDOWS)
def test_right_window_small(gpu, D, left, right):
    lens = [1, 17, 128, 129, 300, 64, 255]
    case = workloads.make_prefill(B=len(lens), Hq=4, Hkv=2, D=D, lens_q=lens, dtype=torch.bfloat16,
                                  seed=770 + D, causal=False)
    out, lse = _varlen(case, gpu, left, right=right)
    ro, rl = _ref(case, left, right=right)
    assert_parity(out, lse, ro, rl, torch.bfloat16, f"window ({left}, {right}) D{D}")


@pytest.mark.parametrize("D", [128, 256])
def test_right_window_q_and_k_lengths_differ(gpu, D):
    """Lq < Lk and Lq > Lk (bottom-right alignment; rows with no visible key
    get out 0 and lse -inf)."""
    case = workloads.make_prefill(B=4, Hq=4, Hkv=4, D=D, lens_q=[50, 200, 7, 300],
                                  lens_k=[400, 333, 900, 120], dtype=torch.bfloat16, seed=780 + D,
                                  causal=False)
    for left, right in ((-1, 0), (-1, 40), (20, 3), (300, 100)):
        out, lse = _varlen(case, gpu, left, right=right)
        ro, rl = _ref(case, left, right=right)
        assert_parity(out, lse, ro, rl, torch.bfloat16, f"Lq!=Lk window ({left}, {right}) D{D}")


def test_right_window_zero_is_causal_and_wide_is_none(gpu):
    """A right window of 0 gives the causal call's result bit for bit; one
    covering every key gives the plain non-causal call's; causal set, a right
    window changes nothing."""
    case = workloads.make_prefill(B=2, Hq=8, Hkv=2, D=128, lens_q=[300, 129], lens_k=[300, 200],
                                  dtype=torch.bfloat16, seed=790, causal=False)
    oc, lc = _varlen(case, gpu, -1, causal=True)
    o0, l0 = _varlen(case, gpu, -1, causal=False, right=0)
    assert torch.equal(oc, o0) and torch.equal(lc, l0)
    on, ln = _varlen(case, gpu, -1, causal=False)
    ow, lw = _varlen(case, gpu, -1, causal=False, right=100000)
    assert torch.equal(on, ow) and torch.equal(ln, lw)
    ob, lb = _varlen(case, gpu, -1, causal=True, right=50)
    assert torch.equal(oc, ob) and torch.equal(lc, lb)


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_right_window_paged(gpu, D, layout):
    import attention_qk_online_amd as A
    case = workloads.make_paged_prefill(B=3, Hq=4, Hkv=2, D=D, page_size=16, chunk=90, cached=250,
                                        shared_prefix=64, dtype=torch.bfloat16, seed=800 + D)
    kp, vp = case.pools(gpu, layout=layout)
    for left, right in ((-1, 0), (-1, 45), (77, 20), (0, 0)):
        out, lse = A.prefill_paged(case.q.to(gpu), case.cu_seqlens_q.to(gpu), kp, vp,
                                   case.page_table.to(gpu), case.kv_lens.to(gpu), case.max_seqlen_q,
                                   case.max_kv_len, causal=False, scale=case.scale,
                                   kv_layout=layout, window_left=left, window_right=right)
        torch.cuda.synchronize()
        ro, rl = oracle.ref_prefill_paged(case.q, case.cu_seqlens_q, case.pool_k, case.pool_v,
                                          case.page_table, case.kv_lens, False, case.scale,
                                          window_left=left, window_right=right)
        assert_parity(out, lse, ro, rl, torch.bfloat16,
                      f"paged {layout} D{D} window ({left}, {right})")


def test_right_window_ragged_config_sampled(gpu):
    """The ragged workload (B 8, L in [1024, 4096], Hq 64, Hkv 8, D 128), non-causal
    with the band window (512, 256), sampled rows."""
    case = workloads.make_config(3)
    out, lse = _varlen(case, gpu, 512, causal=False, right=256)
    cu = [int(x) for x in case.cu_seqlens_q]
    g = torch.Generator().manual_seed(810)
    rows = set(torch.randint(0, cu[-1], (64,), generator=g).tolist())
    for a, b in zip(cu[:-1], cu[1:]):
        rows.update(r for r in (a, a + 255, a + 256, a + 700, b - 257, b - 256, b - 1) if a <= r < b)
    rows = torch.tensor(sorted(rows))
    ro, rl = _ref(case, 512, causal=False, rows=rows, right=256)
    assert_parity(out, lse, ro, rl, torch.bfloat16, "ragged window (512, 256) (sampled rows)",
                  rows=rows)
    assert torch.isfinite(out.float()).all()


# ---------------------------------------------------------------- decode ---
def _decode(case, gpu, window, layout="NHD", split_pages=0):
    import attention_qk_online_amd as A
    kp, vp = case.pools(gpu, layout=layout)
    out, lse = A.decode_paged(case.q.to(gpu), kp, vp, case.page_table.to(gpu), case.kv_lens.to(gpu),
                              scale=case.scale, max_kv_len=case.max_kv_len,
                              split_pages=split_pages, kv_layout=layout, window_left=window)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("dtype,D,Hq,Hkv", [(torch.bfloat16, 128, 32, 8), (torch.bfloat16, 256, 16, 2),
                                            (torch.float16, 64, 8, 8), (torch.float32, 128, 8, 2)])
@pytest.mark.parametrize("split_pages", [0, 2])
def test_decode_window(gpu, dtype, D, Hq, Hkv, split_pages):
    lens = [1, 15, 16, 17, 300, 64, 1000, 0, 33]
    case = workloads.make_decode(B=len(lens), Hq=Hq, Hkv=Hkv, D=D, page_size=16, kv_lens=lens,
                                 dtype=dtype, seed=750 + D + Hq, extra_pages=4)
    kp, vp = case.pools("cpu")
    for window in (0, 5, 15, 16, 17, 100, 1000):
        out, lse = _decode(case, gpu, window, split_pages=split_pages)
        ro, rl = oracle.ref_decode_paged(case.q, kp, vp, case.page_table, case.kv_lens, case.scale,
                                         window_left=window)
        assert_parity(out, lse, ro, rl, dtype, f"decode {dtype} D{D} window {window}")


def test_decode_window_hnd_and_wide(gpu):
    """HND equals NHD bit for bit with a window; a window covering every key
    equals the plain call bit for bit."""
    case = workloads.make_decode(B=5, Hq=16, Hkv=4, D=128, page_size=16, kv_lens=[33, 400, 16, 1, 250],
                                 dtype=torch.bfloat16, seed=760, extra_pages=3)
    o1, l1 = _decode(case, gpu, 37, "NHD", 2)
    o2, l2 = _decode(case, gpu, 37, "HND", 2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o3, l3 = _decode(case, gpu, -1, "NHD", 2)
    o4, l4 = _decode(case, gpu, 400, "NHD", 2)
    assert torch.equal(o3, o4) and torch.equal(l3, l4)


def test_decode_window_paged_config(gpu):
    """The batched paged GQA decode workload (B 64, Hq 32, Hkv 8, D 128) with a
    1024-key window, every request against the oracle."""
    case = workloads.make_decode(B=64, Hq=32, Hkv=8, D=128, page_size=16, len_range=(512, 4096),
                                 dtype=torch.bfloat16, seed=2, num_pages=20000)
    out, lse = _decode(case, gpu, 1024)
    kp, vp = case.pools("cpu")
    ro, rl = oracle.ref_decode_paged(case.q, kp, vp, case.page_table, case.kv_lens, case.scale,
                                     window_left=1024)
    assert_parity(out, lse, ro, rl, torch.bfloat16, "paged decode window 1024")
