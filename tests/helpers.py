"""Shared helpers for the GPU parity tests: tolerance checks against the oracle."""
import math

import torch

import oracle

# Tolerances of the parity gate: bf16 inputs 2e-2, fp32 inputs 1e-5, applied
# to max|d| and to the normwise relative error max|d| / max|ref|, separately
# for out and lse.  fp16 inputs: 5e-3.  The fp16 paths round the softmax
# weights and the output to half (relative step 2^-11 = 4.9e-4 each, against
# 2^-8 = 3.9e-3 for bf16) and accumulate in fp32, so their error is about
# 8x below the bf16 paths'; 5e-3 keeps the bf16 gate's margin at that scale.
TOL = {torch.bfloat16: 2e-2, torch.float16: 5e-3, torch.float32: 1e-5}


def assert_parity(got_out, got_lse, ref_out, ref_lse, dtype, what="", rows=None):
    """Compare GPU (out, lse) with the oracle's; ``rows`` restricts to a subset
    of leading-dimension indices (sampled parity at full size)."""
    assert tuple(got_out.shape) == tuple(ref_out.shape), (got_out.shape, ref_out.shape)
    assert tuple(got_lse.shape) == tuple(ref_lse.shape), (got_lse.shape, ref_lse.shape)
    assert got_lse.dtype == torch.float32 and got_out.dtype == dtype
    go, gl = got_out.detach().cpu(), got_lse.detach().cpu()
    if rows is not None:
        go, gl, ref_out, ref_lse = go[rows], gl[rows], ref_out[rows], ref_lse[rows]
    tol = TOL[dtype]
    so = oracle.error_stats(go, ref_out)
    sl = oracle.error_stats(gl, ref_lse)
    msg = f"{what}: out {so}, lse {sl}, tol {tol}"
    print(msg, flush=True)
    for st in (so, sl):
        assert st["inf_match"], msg
        assert not math.isnan(st["max_abs"]), msg
        assert st["max_abs"] <= tol and st["max_rel"] <= tol, msg
    return so, sl
