"""C-ABI library checks that need no GPU: it loads, exports every function
declared in include/attn.h, and rejects bad arguments with the documented
status before touching the device."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, E_NULL, E_SHAPE, E_DTYPE, E_UNSUP, E_VALUE, E_WS, E_HIP = range(8)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import attention_qk_online_amd as A
    if not os.path.exists(A.library_path()):
        pytest.fail("libattn.so is not built (run __graft_entry__.build())")
    return A.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert len(names) >= 9, names
    raw = ctypes.CDLL(os.path.join(ROOT, "attention_qk_online_amd", "libattn.so"))
    for n in names:
        assert hasattr(raw, n), f"{n} is declared in attn.h but not exported"


def test_status_strings(lib):
    for s in range(8):
        assert lib.attn_status_string(s)
    assert lib.attn_status_string(99) == b"unknown status"
    for k in range(4):
        assert lib.attn_kernel_name(k) != b"unknown"


def _decode(lib, **kw):
    a = dict(dtype=1, q=16, k=16, v=16, table=16, lens=16, B=2, Hq=8, Hkv=2, D=128, P=16,
             num_pages=100, max_pages=8, max_kv_len=128, split=0, scale=0.1, out=16, lse=16,
             ws=16, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.attn_decode_paged(a["dtype"], a["q"], a["k"], a["v"], a["table"], a["lens"], a["B"],
                                 a["Hq"], a["Hkv"], a["D"], a["P"], a["num_pages"], a["max_pages"],
                                 a["max_kv_len"], a["split"], a["scale"], a["out"], a["lse"], a["ws"],
                                 a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), E_DTYPE),
    (dict(B=-1), E_SHAPE),
    (dict(Hq=6, Hkv=4), E_SHAPE),
    (dict(max_kv_len=129), E_SHAPE),          # above max_pages * page_size
    (dict(scale=float("inf")), E_VALUE),
    (dict(scale=float("nan")), E_VALUE),
    (dict(D=96), E_UNSUP),
    (dict(P=24, max_pages=6), E_UNSUP),       # not 16 << k
    (dict(P=48, max_pages=3), E_UNSUP),
    (dict(P=512, max_pages=1), E_UNSUP),      # above 256
    (dict(dtype=0, P=32, max_pages=4), E_UNSUP),   # fp32: 16 only
    (dict(Hq=32, Hkv=2), E_UNSUP),            # group of 16
    (dict(dtype=0, D=256), E_UNSUP),
    (dict(q=None), E_NULL),
    (dict(table=None), E_NULL),
    (dict(ws=None, split=2), E_WS),
    (dict(ws=None), E_WS),                    # bf16 always needs its run partials
    (dict(ws_bytes=8, split=2), E_WS),
    (dict(q=8), E_UNSUP),                     # misaligned
    (dict(ws=24), E_UNSUP),                   # workspace not 16-byte aligned
    (dict(num_pages=0), E_SHAPE),
    # above ATTN_MAX_TOKENS (2^30), and a batch whose unit count exceeds it
    (dict(max_kv_len=(1 << 30) + 16, max_pages=(1 << 26) + 1), E_UNSUP),
    (dict(B=1 << 20, max_kv_len=1 << 14, max_pages=1 << 10), E_UNSUP),
])
def test_decode_rejects(lib, kw, status):
    assert _decode(lib, **kw) == status
    assert lib.attn_last_error()


def _noalloc(lib, **kw):
    a = dict(dtype=1, q=16, k=16, v=16, table=16, lens=16, B=2, Hq=8, Hkv=2, D=128, P=16,
             num_pages=100, max_pages=8, max_kv_len=128, split=0, scale=0.1, out=16, lse=16,
             stream=None)
    a.update(kw)
    return lib.attn_decode_paged_noalloc(a["dtype"], a["q"], a["k"], a["v"], a["table"], a["lens"],
                                         a["B"], a["Hq"], a["Hkv"], a["D"], a["P"], a["num_pages"],
                                         a["max_pages"], a["max_kv_len"], a["split"], a["scale"],
                                         a["out"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), E_DTYPE),
    (dict(Hq=6, Hkv=4), E_SHAPE),
    (dict(D=96), E_UNSUP),
    (dict(scale=float("nan")), E_VALUE),
    (dict(q=None), E_NULL),
    # partial states above the static array: refused before any HIP call
    (dict(B=4096, Hq=32, Hkv=8, max_pages=256, max_kv_len=4096, num_pages=300000), E_WS),
])
def test_decode_noalloc_rejects(lib, kw, status):
    assert _noalloc(lib, **kw) == status
    assert lib.attn_last_error()


def test_decode_noalloc_limit_is_the_header_constant(lib):
    import attention_qk_online_amd as A
    text = open(HEADER).read()
    m = re.search(r"#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == A.DECODE_NOALLOC_SCRATCH_BYTES
    # the largest decode of 64 requests of 4096 tokens (Hq 32, Hkv 8, D 128) fits
    assert lib.attn_decode_paged_workspace_size(1, 64, 32, 8, 128, 16, 4096, 0) <= \
        A.DECODE_NOALLOC_SCRATCH_BYTES
    assert _noalloc(lib, B=0, q=None, k=None) == OK


@pytest.mark.parametrize("P", [32, 64, 128, 256])
def test_decode_larger_pages_pass_the_checks(lib, P):
    # B = 0: every argument check runs, nothing is launched
    assert _decode(lib, P=P, max_pages=max(1, 128 // P), B=0) == OK


def test_decode_empty_batch_is_noop(lib):
    assert _decode(lib, B=0, q=None, k=None) == OK


def test_workspace_size(lib):
    # fp32 split grid: one split -> no workspace; forced small splits ->
    # B*splits*Hq*(D+1) floats (two 256-byte aligned parts)
    assert lib.attn_decode_paged_workspace_size(0, 4, 8, 2, 128, 16, 100, 0) == 0
    n = lib.attn_decode_paged_workspace_size(0, 4, 8, 2, 128, 16, 160, 2)   # 10 pages -> 5 splits
    o, lse = 4 * 5 * 8 * 128 * 4, 4 * 5 * 8 * 4
    assert n == ((o + 255) // 256 + (lse + 255) // 256) * 256
    # bf16 balanced runs: B*Hkv*max_segs*G*(D+1) floats, max_segs = ceil(max_pages/run)+1,
    # and B+1 int32 (each request's first unit and the total)
    def bf16_bytes(B, Hkv, segs, G, D):
        slots = B * Hkv * segs * G
        return ((slots * D * 4 + 255) // 256 + (slots * 4 + 255) // 256 + ((B + 1) * 4 + 255) // 256) * 256
    n = lib.attn_decode_paged_workspace_size(1, 4, 8, 2, 128, 16, 160, 2)   # run 2 -> 6 segs
    assert n == bf16_bytes(4, 2, 6, 4, 128)
    n = lib.attn_decode_paged_workspace_size(1, 4, 8, 2, 128, 16, 160, 0)   # run >= 8 -> 3 segs
    assert n == bf16_bytes(4, 2, 3, 4, 128)
    n = lib.attn_decode_paged_workspace_size(1, 4, 8, 2, 128, 16, 2000, 1)  # run 1 -> 126 segs
    assert n == bf16_bytes(4, 2, 126, 4, 128)
    assert lib.attn_decode_paged_workspace_size(1, -1, 8, 2, 128, 16, 160, 2) == 0
    assert lib.attn_decode_paged_workspace_size(9, 4, 8, 2, 128, 16, 160, 2) == 0
    # f16 uses the bf16 plan
    assert (lib.attn_decode_paged_workspace_size(2, 4, 8, 2, 128, 16, 160, 2) ==
            lib.attn_decode_paged_workspace_size(1, 4, 8, 2, 128, 16, 160, 2))


def test_decode_fp8_rejects(lib):
    def call(**kw):
        a = dict(dtype=1, q=16, k=16, v=16, t=16, lens=16, B=2, Hq=8, Hkv=2, D=128, P=16,
                 num_pages=10, max_pages=4, mkv=64, split=0, scale=0.1, ks=1.0, vs=1.0, out=16,
                 lse=16, ws=256, ws_bytes=1 << 20)
        a.update(kw)
        return lib.attn_decode_paged_fp8(a["dtype"], a["q"], a["k"], a["v"], a["t"], a["lens"],
                                         a["B"], a["Hq"], a["Hkv"], a["D"], a["P"], a["num_pages"],
                                         a["max_pages"], a["mkv"], a["split"], a["scale"], a["ks"],
                                         a["vs"], a["out"], a["lse"], a["ws"], a["ws_bytes"], None)
    assert call(dtype=0) == E_UNSUP                     # fp32 queries with an E4M3 cache
    assert call(dtype=3) == E_DTYPE
    assert call(ks=float("inf")) == E_VALUE
    assert call(vs=float("nan")) == E_VALUE
    assert call(D=96) == E_UNSUP
    assert call(P=8, mkv=32) == E_UNSUP
    assert call(Hq=8, Hkv=3) == E_SHAPE
    assert call(ws=None) == E_WS
    assert call(t=None) == E_NULL
    assert call(B=0, q=None) == OK


def _prefill(lib, **kw):
    a = dict(dtype=1, q=16, k=16, v=16, cq=16, ck=16, B=2, Hq=8, Hkv=2, D=128, Tq=100, Tk=100,
             mq=64, mk=64, causal=1, scale=0.1, out=16, lse=16, stream=None)
    a.update(kw)
    return lib.attn_prefill_varlen(a["dtype"], a["q"], a["k"], a["v"], a["cq"], a["ck"], a["B"],
                                   a["Hq"], a["Hkv"], a["D"], a["Tq"], a["Tk"], a["mq"], a["mk"],
                                   a["causal"], a["scale"], a["out"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), E_DTYPE),
    (dict(dtype=0), E_UNSUP),                 # fp32 prefill is not built
    (dict(D=64), E_UNSUP),
    (dict(Hq=8, Hkv=3), E_SHAPE),
    (dict(causal=2), E_VALUE),
    (dict(scale=float("-inf")), E_VALUE),
    (dict(Tk=-1), E_SHAPE),
    (dict(cq=None), E_NULL),
    (dict(out=None), E_NULL),
    (dict(k=None), E_NULL),                   # keys to read (Tk > 0): k and v are required
    (dict(v=None), E_NULL),
    (dict(k=24), E_UNSUP),
    (dict(B=1 << 14, Hq=1 << 10, Hkv=1 << 10, mq=1 << 15), E_SHAPE),   # > INT_MAX work items
])
def test_prefill_rejects(lib, kw, status):
    assert _prefill(lib, **kw) == status


def test_window_rejects(lib):
    def call(w, wr=-1, **kw):
        a = dict(dtype=1, q=16, k=16, v=16, cq=16, ck=16, B=2, Hq=8, Hkv=2, D=128, Tq=100, Tk=100,
                 mq=64, mk=64, causal=1, scale=0.1, out=16, lse=16)
        a.update(kw)
        return lib.attn_prefill_varlen_window(a["dtype"], a["q"], a["k"], a["v"], a["cq"], a["ck"],
                                              a["B"], a["Hq"], a["Hkv"], a["D"], a["Tq"], a["Tk"],
                                              a["mq"], a["mk"], a["causal"], w, wr, a["scale"],
                                              a["out"], a["lse"], None)
    assert call(-2) == E_VALUE
    assert call(-1, -2) == E_VALUE               # right side: -1 is the only negative value
    assert call(5, D=64) == E_UNSUP
    assert call(5, B=0, q=None) == OK
    assert call(-1, 3, B=0, q=None) == OK
    assert lib.attn_prefill_paged_window(1, 2, 16, 16, 16, 16, 16, 16, 2, 4, 4, 256, 10, 16, 10, 4,
                                         5, 64, 1, 3, -1, 0.1, 16, 16, None) == E_VALUE   # layout 2
    assert lib.attn_prefill_paged_window(1, 0, 16, 16, 16, 16, 16, 16, 2, 4, 4, 256, 10, 16, 10, 4,
                                         5, 64, 0, -1, -3, 0.1, 16, 16, None) == E_VALUE


def test_decode_window_rejects(lib):
    def call(layout, w, **kw):
        a = dict(dtype=1, q=16, k=16, v=16, t=16, lens=16, B=2, Hq=8, Hkv=2, D=128, P=16,
                 num_pages=10, max_pages=4, mkv=64, split=0, scale=0.1, out=16, lse=16, ws=256,
                 ws_bytes=1 << 20)
        a.update(kw)
        return lib.attn_decode_paged_window(a["dtype"], layout, w, a["q"], a["k"], a["v"], a["t"],
                                            a["lens"], a["B"], a["Hq"], a["Hkv"], a["D"], a["P"],
                                            a["num_pages"], a["max_pages"], a["mkv"], a["split"],
                                            a["scale"], a["out"], a["lse"], a["ws"], a["ws_bytes"],
                                            None)
    assert call(0, -2) == E_VALUE
    assert call(2, 5) == E_VALUE
    assert call(0, 5, dtype=3) == E_DTYPE
    assert call(0, 5, B=0, q=None) == OK


def test_rope_rejects(lib):
    def call(theta=10000.0, scale=1.0, **kw):
        a = dict(dtype=1, layout=0, w=-1, q=16, k=16, v=16, t=16, lens=16, B=2, Hq=8, Hkv=2, D=128,
                 P=16, num_pages=10, max_pages=4, mkv=64, split=0, scale=0.1, out=16, lse=16,
                 ws=256, ws_bytes=1 << 20)
        a.update(kw)
        return lib.attn_decode_paged_rope(a["dtype"], a["layout"], a["w"], theta, scale, a["q"],
                                          a["k"], a["v"], a["t"], a["lens"], a["B"], a["Hq"],
                                          a["Hkv"], a["D"], a["P"], a["num_pages"], a["max_pages"],
                                          a["mkv"], a["split"], a["scale"], a["out"], a["lse"],
                                          a["ws"], a["ws_bytes"], None)
    assert call(theta=0.0) == E_VALUE
    assert call(theta=float("nan")) == E_VALUE
    assert call(scale=-1.0) == E_VALUE
    assert call(D=256) == E_UNSUP
    assert call(dtype=0) == E_UNSUP
    assert call(layout=3) == E_VALUE
    assert call(B=0, q=None) == OK


def test_prefill_empty_is_noop(lib):
    assert _prefill(lib, B=0, q=None) == OK
    assert _prefill(lib, mq=0, q=None) == OK


def test_prefill_paged_rejects(lib):
    def call(**kw):
        a = dict(dtype=1, q=16, cq=16, k=16, v=16, t=16, lens=16, B=2, Hq=4, Hkv=4, D=256, Tq=10,
                 P=16, num_pages=10, max_pages=4, mq=5, mkv=64, causal=1, scale=0.1, out=16, lse=16)
        a.update(kw)
        return lib.attn_prefill_paged(a["dtype"], a["q"], a["cq"], a["k"], a["v"], a["t"], a["lens"],
                                      a["B"], a["Hq"], a["Hkv"], a["D"], a["Tq"], a["P"],
                                      a["num_pages"], a["max_pages"], a["mq"], a["mkv"], a["causal"],
                                      a["scale"], a["out"], a["lse"], None)
    assert call(P=8) == E_UNSUP
    assert call(P=48, max_pages=2) == E_UNSUP       # not 16 << k
    assert call(P=512, max_pages=1) == E_UNSUP      # above 256
    for P in (32, 64, 128, 256):                    # B = 0: every check runs, no launch
        assert call(P=P, max_pages=max(1, 64 // P), B=0, q=None) == OK
    assert call(mkv=65) == E_SHAPE
    assert call(t=None) == E_NULL
    assert call(D=100) == E_UNSUP
    assert call(B=0, q=None) == OK


def _cascade(lib, **kw):
    a = dict(dtype=1, q=16, cq=16, k=16, v=16, t=16, lens=16, B=2, Hq=4, Hkv=4, D=256, Tq=10,
             P=16, num_pages=10, max_pages=4, mq=5, mkv=64, prefix=32, causal=1, scale=0.1,
             out=16, lse=16, ws=256, ws_bytes=1 << 20)
    a.update(kw)
    return lib.attn_prefill_paged_cascade(
        a["dtype"], a["q"], a["cq"], a["k"], a["v"], a["t"], a["lens"], a["B"], a["Hq"], a["Hkv"],
        a["D"], a["Tq"], a["P"], a["num_pages"], a["max_pages"], a["mq"], a["mkv"], a["prefix"],
        a["causal"], a["scale"], a["out"], a["lse"], a["ws"], a["ws_bytes"], None)


def test_cascade_rejects(lib):
    assert _cascade(lib, prefix=8) == E_SHAPE           # not a whole number of pages
    assert _cascade(lib, prefix=-16) == E_SHAPE
    assert _cascade(lib, prefix=80) == E_SHAPE          # beyond max_kv_len
    assert _cascade(lib, ws=None) == E_WS
    need = lib.attn_prefill_paged_cascade_workspace_size(1, 10, 4, 256)
    assert _cascade(lib, ws_bytes=need - 1) == E_WS
    assert _cascade(lib, ws=512 + 16) == E_UNSUP        # workspace not 256-byte aligned
    assert _cascade(lib, P=8) == E_UNSUP                # checks of attn_prefill_paged apply
    assert _cascade(lib, t=None) == E_NULL
    assert _cascade(lib, D=64) == E_UNSUP
    # the prefix pass runs Hq x ceil(total_q / 128) work items: 2^14 x 2^17 overflows
    assert _cascade(lib, B=1, Hq=1 << 14, Hkv=1 << 14, Tq=1 << 24, mq=16) == E_SHAPE
    assert _cascade(lib, B=0, q=None, ws=None) == OK


def test_cascade_workspace_size(lib):
    # [total_q, Hq, D] of the input type + [total_q, Hq] float, each rounded up to 256 bytes
    assert lib.attn_prefill_paged_cascade_workspace_size(1, 10, 4, 256) == 20480 + 256
    assert lib.attn_prefill_paged_cascade_workspace_size(2, 8192, 16, 256) == (64 << 20) + (512 << 10)
    assert lib.attn_prefill_paged_cascade_workspace_size(0, 3, 1, 64) == 768 + 256
    assert lib.attn_prefill_paged_cascade_workspace_size(9, 3, 1, 64) == 0
    assert lib.attn_prefill_paged_cascade_workspace_size(1, -1, 1, 64) == 0


def test_merge_rejects(lib):
    def call(**kw):
        a = dict(dtype=1, oa=16, la=16, ob=16, lb=16, rows=10, D=128, out=16, lo=16)
        a.update(kw)
        return lib.attn_merge_states(a["dtype"], a["oa"], a["la"], a["ob"], a["lb"], a["rows"],
                                     a["D"], a["out"], a["lo"], None)
    assert call(dtype=3) == E_DTYPE
    assert call(D=100) == E_UNSUP
    assert call(D=0) == E_SHAPE
    assert call(rows=-1) == E_SHAPE
    assert call(lb=None) == E_NULL
    assert call(out=24) == E_UNSUP
    assert call(rows=0, oa=None) == OK


def test_binding_checks_layout_name():
    import attention_qk_online_amd as A
    assert A._layout("NHD") == "" and A._layout("HND") == "_hnd"
    with pytest.raises(ValueError):
        A._layout("nhd")


def test_binding_rejects_host_tensors():
    import attention_qk_online_amd as A
    q = torch.zeros(2, 4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        A.decode_paged(q, q, q, torch.zeros(2, 1, dtype=torch.int32), torch.zeros(2, dtype=torch.int32))


def test_binding_fails_loudly_without_library(tmp_path):
    import attention_qk_online_amd as A
    with pytest.raises(RuntimeError):
        A.load_library(str(tmp_path / "missing.so"))


def test_timing_api_without_gpu(lib):
    assert lib.attn_timing_begin(0) == E_SHAPE


def test_last_hip_error_is_empty_after_argument_errors(lib):
    assert _decode(lib, B=-1) == E_SHAPE
    assert lib.attn_last_error() and lib.attn_last_hip_error() == b""


def test_hip_failure_is_reported_with_the_runtime_text(lib):
    """Without a GPU, a launch the argument checks accept fails in the HIP
    runtime: ATTN_E_HIP, and attn_last_hip_error() carries the runtime's
    text.  (Skipped where a GPU is visible: the pointers here are not real.)"""
    if torch.cuda.is_available():
        pytest.skip("needs a host without a GPU (the call would launch)")
    assert _decode(lib) == E_HIP
    assert b"decode" in lib.attn_last_error()
    assert lib.attn_last_hip_error() != b""
    assert _decode(lib, B=-1) == E_SHAPE       # cleared by the next call
    assert lib.attn_last_hip_error() == b""


def test_binding_maps_statuses_to_exceptions(lib):
    import attention_qk_online_amd as A
    for status in (E_NULL, E_SHAPE, E_DTYPE, E_UNSUP, E_VALUE, E_WS):
        with pytest.raises(ValueError):
            A._check(status)
    with pytest.raises(A.AttnError) as ei:
        A._check(E_HIP)
    assert not isinstance(ei.value, ValueError)


def test_timing_capacity_limit(lib):
    text = open(HEADER).read()
    m = re.search(r"#define ATTN_TIMING_MAX_LAUNCHES \(1 << (\d+)\)", text)
    assert m
    assert lib.attn_timing_begin((1 << int(m.group(1))) + 1) == E_SHAPE
    assert lib.attn_last_error()
