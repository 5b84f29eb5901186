"""The plain C client of the C ABI (tests/c_client/attn_client.c): device memory
from hipMalloc, no Python in the loop.  The GPU tests write seeded inputs as raw
files, run the client and compare what it writes with the oracle."""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import assert_parity

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c_client", "attn_client")


def _client():
    # The client is test infrastructure built by __graft_entry__.build(); the
    # library it drives is checked by every other test, so a missing client
    # skips these tests rather than stopping the run.
    if not os.path.exists(CLIENT):
        pytest.skip("tests/c_client/attn_client is not built (run __graft_entry__.build())")
    return CLIENT


def test_client_built_and_prints_usage():
    """Built with the library; without arguments it prints its usage and exits 1
    before any HIP call."""
    r = subprocess.run([_client()], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage: attn_client decode" in r.stderr


def _write(d, name, t):
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    t.numpy().tofile(os.path.join(d, name))


def _read_bf16(d, name, shape):
    a = np.fromfile(os.path.join(d, name), dtype=np.int16)
    return torch.from_numpy(a).view(torch.bfloat16).reshape(shape)


def _read_f32(d, name, shape):
    return torch.from_numpy(np.fromfile(os.path.join(d, name), dtype=np.float32)).reshape(shape)


@pytest.mark.gpu
def test_client_decode(tmp_path):
    case = workloads.make_decode(B=5, Hq=16, Hkv=4, D=128, page_size=16,
                                 kv_lens=[1, 300, 0, 1000, 64], dtype=torch.bfloat16, seed=1400,
                                 extra_pages=3)
    kp, vp = case.pools()
    d = str(tmp_path)
    for name, t in (("q.bin", case.q), ("k.bin", kp), ("v.bin", vp), ("table.bin", case.page_table),
                    ("lens.bin", case.kv_lens)):
        _write(d, name, t)
    args = [case.B, case.Hq, case.Hkv, case.D, case.page_size, case.num_pages,
            case.page_table.shape[1], case.max_kv_len, repr(case.scale)]
    print("client decode", args, flush=True)
    r = subprocess.run([_client(), "decode", d] + [str(a) for a in args], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    out = _read_bf16(d, "out.bin", (case.B, case.Hq, case.D))
    lse = _read_f32(d, "lse.bin", (case.B, case.Hq))
    ro, rl = oracle.ref_decode_paged(case.q, kp, vp, case.page_table, case.kv_lens, case.scale)
    assert_parity(out, lse, ro, rl, torch.bfloat16, "C client decode")


@pytest.mark.gpu
def test_client_prefill(tmp_path):
    case = workloads.make_prefill(B=3, Hq=8, Hkv=2, D=128, lens_q=[200, 1, 257], dtype=torch.bfloat16,
                                  seed=1401, causal=True)
    d = str(tmp_path)
    for name, t in (("q.bin", case.q), ("k.bin", case.k), ("v.bin", case.v),
                    ("cuq.bin", case.cu_seqlens_q), ("cuk.bin", case.cu_seqlens_k)):
        _write(d, name, t)
    Tq, Tk = case.q.shape[0], case.k.shape[0]
    args = [case.B, case.Hq, case.Hkv, case.D, Tq, Tk, case.max_seqlen_q, case.max_seqlen_k, 1,
            repr(case.scale)]
    print("client prefill", args, flush=True)
    r = subprocess.run([_client(), "prefill", d] + [str(a) for a in args], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    out = _read_bf16(d, "out.bin", (Tq, case.Hq, case.D))
    lse = _read_f32(d, "lse.bin", (Tq, case.Hq))
    ro, rl = oracle.ref_prefill_varlen(case.q, case.k, case.v, case.cu_seqlens_q, case.cu_seqlens_k,
                                       True, case.scale)
    assert_parity(out, lse, ro, rl, torch.bfloat16, "C client prefill")


@pytest.mark.gpu
def test_client_reports_library_errors(tmp_path):
    """A status other than ATTN_OK reaches the C caller with its text (here an
    unsupported head_dim); nothing is launched."""
    d = str(tmp_path)
    for name, n in (("q.bin", 2 * 4 * 96), ("k.bin", 4 * 16 * 2 * 96), ("v.bin", 4 * 16 * 2 * 96)):
        _write(d, name, torch.zeros(n, dtype=torch.bfloat16))
    _write(d, "table.bin", torch.zeros(2, 2, dtype=torch.int32))
    _write(d, "lens.bin", torch.tensor([3, 4], dtype=torch.int32))
    r = subprocess.run([_client(), "decode", d, "2", "4", "2", "96", "16", "4", "2", "32", "0.1"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "not built" in r.stderr, r.stderr
