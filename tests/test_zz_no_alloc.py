"""attn_decode_paged_noalloc: the decode that allocates nothing (partial
states in the library's static per-GPU scratch array) against
attn_decode_paged with a caller workspace, both called through the C ABI.

Consecutive calls share the scratch array, so the test makes several calls
in a row, each later one smaller than the first (the array still holds the
previous call's partial states), and requires the same bits as the
workspace call and parity with the oracle each time."""
import pytest
import torch

import oracle
import workloads
from helpers import assert_parity

pytestmark = pytest.mark.gpu

DTYPE_CODE = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}


def _call(lib, noalloc, case, dev, split_pages, q, kp, vp, table, lens):
    out = torch.full_like(q, float("nan"))
    lse = torch.full((case.B, case.Hq), float("nan"), dtype=torch.float32, device=dev)
    code = DTYPE_CODE[case.dtype]
    head = (code, q.data_ptr(), kp.data_ptr(), vp.data_ptr(), table.data_ptr(), lens.data_ptr(),
            case.B, case.Hq, case.Hkv, case.D, case.page_size, kp.shape[0], table.shape[1],
            case.max_kv_len, split_pages, case.scale, out.data_ptr(), lse.data_ptr())
    stream = torch.cuda.current_stream(dev).cuda_stream
    if noalloc:
        st = lib.attn_decode_paged_noalloc(*head, stream)
    else:
        nbytes = lib.attn_decode_paged_workspace_size(code, case.B, case.Hq, case.Hkv, case.D,
                                                      case.page_size, case.max_kv_len, split_pages)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        st = lib.attn_decode_paged(*head, ws.data_ptr(), nbytes, stream)
        torch.cuda.synchronize()
        del ws
    assert st == 0, lib.attn_last_error().decode()
    torch.cuda.synchronize()
    return out, lse


# (case arguments, split_pages): the first call is the largest; the later
# ones are smaller and force several partial states per request.
CALLS = [
    (dict(B=64, Hq=32, Hkv=8, D=128, page_size=16, len_range=(512, 4096), dtype=torch.bfloat16,
          seed=700), 0),
    (dict(B=5, Hq=8, Hkv=2, D=64, page_size=16, kv_lens=[1, 300, 17, 0, 129], dtype=torch.bfloat16,
          seed=701, extra_pages=2), 2),
    (dict(B=3, Hq=4, Hkv=4, D=64, page_size=16, kv_lens=[256, 40, 100], dtype=torch.float32,
          seed=702, extra_pages=2), 2),
    (dict(B=2, Hq=16, Hkv=2, D=128, page_size=64, kv_lens=[77, 1000], dtype=torch.float16,
          seed=703, extra_pages=1), 1),
]


def test_noalloc_matches_workspace_entry_point(gpu):
    import attention_qk_online_amd as A
    lib = A.load_library()
    for i, (kw, split) in enumerate(CALLS):
        case = workloads.make_decode(**kw)
        print(f"noalloc call {i}: B={case.B} Hq={case.Hq} Hkv={case.Hkv} D={case.D} "
              f"P={case.page_size} {case.dtype} split={split}", flush=True)
        kp, vp = case.pools(gpu)
        args = (case.q.to(gpu), kp, vp, case.page_table.to(gpu), case.kv_lens.to(gpu))
        ref = _call(lib, False, case, gpu, split, *args)
        got = _call(lib, True, case, gpu, split, *args)
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), f"call {i}"
        kc, vc = case.pools("cpu")
        ro, rl = oracle.ref_decode_paged(case.q, kc, vc, case.page_table, case.kv_lens, case.scale)
        assert_parity(got[0], got[1], ro, rl, case.dtype, f"noalloc call {i}")
        del kp, vp


def test_noalloc_binding_and_size_limit(gpu):
    """The Python binding reaches the same entry point and repeated calls
    give the same bits."""
    import attention_qk_online_amd as A
    lib = A.load_library()
    case = workloads.make_decode(B=4, Hq=8, Hkv=1, D=128, page_size=16, kv_lens=[900, 2, 64, 513],
                                 dtype=torch.bfloat16, seed=704, extra_pages=2)
    kp, vp = case.pools(gpu)
    q, t, l = case.q.to(gpu), case.page_table.to(gpu), case.kv_lens.to(gpu)
    out = torch.empty_like(q)
    lse = torch.empty(case.B, case.Hq, device=gpu)
    A.decode_paged_noalloc(q, kp, vp, t, l, out, lse, case.max_kv_len, scale=case.scale)
    ro, rl = A.decode_paged(q, kp, vp, t, l, scale=case.scale, max_kv_len=case.max_kv_len)
    torch.cuda.synchronize()
    assert torch.equal(out, ro) and torch.equal(lse, rl)
    # A refused call (its partial states would exceed the static array; the
    # refusal itself is checked without a GPU in test_abi) leaves the next
    # call working.
    assert lib.attn_decode_paged_workspace_size(1, 4096, 32, 8, 128, 16, 4096, 0) > \
        A.DECODE_NOALLOC_SCRATCH_BYTES
    out2 = torch.full_like(q, float("nan"))
    A.decode_paged_noalloc(q, kp, vp, t, l, out2, lse, case.max_kv_len, scale=case.scale)
    torch.cuda.synchronize()
    assert torch.equal(out2, ro)
