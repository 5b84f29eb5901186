"""Fused attention forward for AMD MI355X (gfx950): Python binding of libattn.so.

Every function here only checks arguments, allocates outputs with torch and
passes raw device pointers plus the current HIP stream to the C ABI declared
in ``include/attn.h``; all arithmetic runs in the library's HIP kernels.  If
the library has not been built the import still succeeds, but every call
raises ``RuntimeError`` -- there is no fallback path.

Entry points (names follow the C ABI):

* :func:`decode_paged` -- batched decode over a paged KV cache (split-KV +
  log-sum-exp merge), the analogue of FlashInfer's single/batch decode calls
  described in "FlashInfer内核库深度解析".
* :func:`decode_paged_fp8` -- the same over a cache of 8-bit E4M3 floats with
  one scale per K / V tensor (half the bytes streamed).
* :func:`prefill_varlen` -- ragged (causal) prefill addressed by cu_seqlens,
  with the argument list of ``varlen_fwd`` in "FlashAttention-3 内核在最新大模型
  推理中的集成实践" section 二.
* :func:`prefill_paged` -- chunked prefill over a paged KV cache (same page).
* :func:`prefill_paged_cascade` -- the same result when every request starts
  with the same pages: the shared prefix is attended once for the whole batch
  and merged into each request's own part (shared-prefix reuse in
  "FlashInfer内核库深度解析").
* :func:`merge_states` -- log-sum-exp merge of two partial attention states.

The paged calls take ``kv_layout="NHD"`` (pools [pages, page_size, Hkv, D])
or ``"HND"`` ([pages, Hkv, page_size, D]), the two KV-cache layouts of
"FlashInfer内核库深度解析".

The softmax scale defaults to 1/sqrt(head_dim) (same page, section 二).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

__all__ = ["decode_paged", "decode_paged_noalloc", "DECODE_NOALLOC_SCRATCH_BYTES", "decode_paged_fp8",
           "decode_paged_workspace_size", "prefill_varlen", "prefill_paged",
           "prefill_paged_cascade", "prefill_paged_cascade_workspace_size", "merge_states",
           "timing_begin", "timing_end", "library_path", "load_library", "AttnError", "AttnValueError",
           "KERNEL_KINDS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libattn.so")
_lib = None

ATTN_F32, ATTN_BF16, ATTN_F16 = 0, 1, 2
KERNEL_KINDS = ("decode_split", "decode_combine", "prefill", "prefill_paged", "merge",
                "cascade_prefix", "cascade_suffix")
_STATUS = {0: "ok", 1: "null", 2: "shape", 3: "dtype", 4: "unsupported", 5: "value",
           6: "workspace", 7: "hip"}


class AttnError(RuntimeError):
    """A call into libattn.so returned a non-zero status."""

    def __init__(self, status: int, detail: str):
        super().__init__(f"libattn: {_STATUS.get(status, status)} error: {detail}")
        self.status = status


class AttnValueError(AttnError, ValueError):
    """A call into libattn.so rejected its arguments (nothing was launched)."""


def library_path() -> str:
    return _LIB_PATH


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libattn.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m attention_qk_online_amd.build` "
                           "(hipcc, gfx950); there is no fallback implementation")
    lib = ctypes.CDLL(p)
    c_int, c_float, c_size, vp = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
    lib.attn_decode_paged_workspace_size.restype = c_size
    lib.attn_decode_paged_workspace_size.argtypes = [c_int] * 8
    lib.attn_decode_paged.restype = c_int
    lib.attn_decode_paged.argtypes = [c_int, vp, vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int,
                                      c_int, c_int, c_int, c_int, c_float, vp, vp, vp, c_size, vp]
    lib.attn_decode_paged_noalloc.restype = c_int
    lib.attn_decode_paged_noalloc.argtypes = [c_int, vp, vp, vp, vp, vp] + [c_int] * 9 + [
        c_float, vp, vp, vp]
    lib.attn_decode_paged_fp8.restype = c_int
    lib.attn_decode_paged_fp8.argtypes = [c_int, vp, vp, vp, vp, vp] + [c_int] * 9 + [
        c_float, c_float, c_float, vp, vp, vp, c_size, vp]
    lib.attn_prefill_varlen.restype = c_int
    lib.attn_prefill_varlen.argtypes = [c_int, vp, vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int,
                                        c_int, c_int, c_int, c_int, c_float, vp, vp, vp]
    lib.attn_prefill_paged.restype = c_int
    lib.attn_prefill_paged.argtypes = [c_int, vp, vp, vp, vp, vp, vp, c_int, c_int, c_int, c_int,
                                       c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_float,
                                       vp, vp, vp]
    lib.attn_prefill_paged_cascade_workspace_size.restype = c_size
    lib.attn_prefill_paged_cascade_workspace_size.argtypes = [c_int] * 4
    lib.attn_prefill_paged_cascade.restype = c_int
    lib.attn_prefill_paged_cascade.argtypes = [c_int, vp, vp, vp, vp, vp, vp] + [c_int] * 12 + [
        c_float, vp, vp, vp, c_size, vp]
    lib.attn_merge_states.restype = c_int
    lib.attn_merge_states.argtypes = [c_int, vp, vp, vp, vp, c_int, c_int, vp, vp, vp]
    lib.attn_decode_paged_window.restype = c_int
    lib.attn_decode_paged_window.argtypes = [c_int, c_int, c_int, vp, vp, vp, vp, vp] + [c_int] * 9 + [
        c_float, vp, vp, vp, c_size, vp]
    lib.attn_decode_paged_rope.restype = c_int
    lib.attn_decode_paged_rope.argtypes = [c_int, c_int, c_int, c_float, c_float, vp, vp, vp, vp,
                                           vp] + [c_int] * 9 + [c_float, vp, vp, vp, c_size, vp]
    lib.attn_decode_paged_fp8_window.restype = c_int
    lib.attn_decode_paged_fp8_window.argtypes = [c_int, c_int, c_int, vp, vp, vp, vp, vp] + [c_int] * 9 + [
        c_float, c_float, c_float, vp, vp, vp, c_size, vp]
    lib.attn_prefill_varlen_window.restype = c_int
    lib.attn_prefill_varlen_window.argtypes = [c_int, vp, vp, vp, vp, vp] + [c_int] * 11 + [
        c_float, vp, vp, vp]
    lib.attn_prefill_paged_window.restype = c_int
    lib.attn_prefill_paged_window.argtypes = [c_int, c_int, vp, vp, vp, vp, vp, vp] + [c_int] * 13 + [
        c_float, vp, vp, vp]
    # HND twins: same argument lists
    for name in ("attn_decode_paged", "attn_decode_paged_fp8", "attn_prefill_paged",
                 "attn_prefill_paged_cascade"):
        f, g = getattr(lib, name), getattr(lib, name + "_hnd")
        g.restype, g.argtypes = c_int, f.argtypes
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [c_int]
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    lib.attn_last_hip_error.restype = ctypes.c_char_p
    lib.attn_last_hip_error.argtypes = []
    lib.attn_timing_begin.restype = c_int
    lib.attn_timing_begin.argtypes = [c_int]
    lib.attn_timing_end.restype = c_int
    lib.attn_timing_end.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(c_int)]
    lib.attn_kernel_name.restype = ctypes.c_char_p
    lib.attn_kernel_name.argtypes = [c_int]
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    """Raise for a non-zero status: ValueError for argument errors (null,
    shape, dtype, unsupported, value, workspace), AttnError (a RuntimeError)
    for a failure of the HIP runtime."""
    if status != 0:
        lib = load_library()
        detail = lib.attn_last_error().decode() or lib.attn_status_string(status).decode()
        if status == 7:
            raise AttnError(status, detail + f" [{lib.attn_last_hip_error().decode()}]")
        raise AttnValueError(status, detail)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return ATTN_F32
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float16:
        return ATTN_F16
    raise ValueError(f"unsupported dtype {t.dtype} (float32, bfloat16 or float16)")


def _dev(t: torch.Tensor, name: str, dtype=None, dim=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (no silent copies are made)")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got shape {tuple(t.shape)}")
    return t.data_ptr()


def _layout(kv_layout: str) -> str:
    """C-function suffix for a page layout: NHD pools are [pages, page_size,
    Hkv, D], HND pools [pages, Hkv, page_size, D]."""
    if kv_layout == "NHD":
        return ""
    if kv_layout == "HND":
        return "_hnd"
    raise ValueError(f"kv_layout must be 'NHD' or 'HND', got {kv_layout!r}")


def _pool_dims(pages: torch.Tensor, kv_layout: str):
    """(num_pages, page_size, Hkv, D) of a pool in either layout."""
    if kv_layout == "HND":
        n, h, ps, d = pages.shape
        return n, ps, h, d
    return tuple(pages.shape)


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _scale(scale: Optional[float], D: int) -> float:
    s = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if not math.isfinite(s):
        raise ValueError("scale must be finite")
    return s


def decode_paged_workspace_size(dtype: torch.dtype, B: int, Hq: int, Hkv: int, D: int,
                                page_size: int, max_kv_len: int, split_pages: int = 0) -> int:
    code = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16, torch.float16: ATTN_F16}.get(dtype)
    if code is None:
        raise ValueError(f"unsupported dtype {dtype} (float32, bfloat16 or float16)")
    return int(load_library().attn_decode_paged_workspace_size(code, B, Hq, Hkv, D, page_size,
                                                               max_kv_len, split_pages))


def _decode(q, k_pages, v_pages, page_table, kv_lens, scale, max_kv_len, split_pages, out, lse,
            workspace, fp8_scales=None, kv_layout="NHD", window_left=-1, rope=None):
    lib = load_library()
    suffix = _layout(kv_layout)
    dt = _dtype_code(q)
    kv_dtype = q.dtype if fp8_scales is None else torch.uint8
    pq = _dev(q, "q", dim=3)
    pk = _dev(k_pages, "k_pages", kv_dtype, 4)
    pv = _dev(v_pages, "v_pages", kv_dtype, 4)
    pt = _dev(page_table, "page_table", torch.int32, 2)
    pl = _dev(kv_lens, "kv_lens", torch.int32, 1)
    B, Hq, D = q.shape
    num_pages, page_size, Hkv, Dk = _pool_dims(k_pages, kv_layout)
    if tuple(v_pages.shape) != tuple(k_pages.shape) or Dk != D:
        raise ValueError(f"k_pages {tuple(k_pages.shape)} / v_pages {tuple(v_pages.shape)} do not "
                         f"match q {tuple(q.shape)}")
    if page_table.shape[0] != B or kv_lens.shape[0] != B:
        raise ValueError("page_table and kv_lens need one row per request")
    if max_kv_len is None:
        max_kv_len = int(kv_lens.max().item()) if B > 0 else 0
    s = _scale(scale, D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _dev(out, "out", q.dtype, 3)
    _dev(lse, "lse", torch.float32, 2)
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq):
        raise ValueError("out/lse have the wrong shape")
    ws_bytes = int(lib.attn_decode_paged_workspace_size(dt, B, Hq, Hkv, D, page_size, max_kv_len,
                                                        split_pages))
    if workspace is None:
        # A call that keeps no partial states (one fp32 split) passes no workspace.
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    elif workspace.numel() * workspace.element_size() < ws_bytes:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, "
                         f"this call needs {ws_bytes} (decode_paged_workspace_size)")
    pw = 0 if workspace is None else _dev(workspace, "workspace")
    ws_size = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (pq, pk, pv, pt, pl, B, Hq, Hkv, D, page_size, num_pages, page_table.shape[1],
            max_kv_len, split_pages, s)
    tail = (out.data_ptr(), lse.data_ptr(), pw, ws_size, _stream(q.device))
    if rope is not None:
        if fp8_scales is not None:
            raise ValueError("the rotary embedding is not built for the E4M3 cache")
        _check(lib.attn_decode_paged_rope(dt, 1 if suffix else 0, int(window_left),
                                          float(rope[0]), float(rope[1]), *args, *tail))
    elif window_left != -1 and fp8_scales is not None:
        _check(lib.attn_decode_paged_fp8_window(dt, 1 if suffix else 0, int(window_left), *args,
                                                float(fp8_scales[0]), float(fp8_scales[1]),
                                                *tail))
    elif window_left != -1:
        _check(lib.attn_decode_paged_window(dt, 1 if suffix else 0, int(window_left), *args,
                                            *tail))
    elif fp8_scales is None:
        _check(getattr(lib, "attn_decode_paged" + suffix)(dt, *args, *tail))
    else:
        _check(getattr(lib, "attn_decode_paged_fp8" + suffix)(
            dt, *args, float(fp8_scales[0]), float(fp8_scales[1]), *tail))
    return out, lse


def decode_paged(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                 page_table: torch.Tensor, kv_lens: torch.Tensor, scale: Optional[float] = None,
                 max_kv_len: Optional[int] = None, split_pages: int = 0,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, kv_layout: str = "NHD",
                 window_left: int = -1, rope_theta: Optional[float] = None,
                 rope_scale: float = 1.0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Batched decode over a paged KV cache (``window_left`` >= 0: the query sees
    only the last window_left + 1 keys; ``rope_theta``: rotate q (position
    kv_len - 1) and the keys (their token index) in the kernel, rotate-half
    convention, angle position / rope_scale * rope_theta^(-2d/D)).

    q [B, Hq, D]; k_pages, v_pages [num_pages, page_size, Hkv, D] (NHD) or
    [num_pages, Hkv, page_size, D] (``kv_layout="HND"``); page_table
    [B, max_pages] int32; kv_lens [B] int32.  ``max_kv_len`` is a host bound
    on every kv_len; when omitted it is read from ``kv_lens`` with one
    device-to-host copy.  Returns (out [B, Hq, D], lse [B, Hq] float32).
    """
    return _decode(q, k_pages, v_pages, page_table, kv_lens, scale, max_kv_len, split_pages, out,
                   lse, workspace, kv_layout=kv_layout, window_left=window_left,
                   rope=None if rope_theta is None else (rope_theta, rope_scale))


DECODE_NOALLOC_SCRATCH_BYTES = 64 << 20   # ATTN_DECODE_NOALLOC_SCRATCH_BYTES in attn.h


def decode_paged_noalloc(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                         page_table: torch.Tensor, kv_lens: torch.Tensor, out: torch.Tensor,
                         lse: torch.Tensor, max_kv_len: int, scale: Optional[float] = None,
                         split_pages: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """:func:`decode_paged` (NHD pages) that allocates nothing: the caller
    passes ``out`` [B, Hq, D] and ``lse`` [B, Hq] and the host bound
    ``max_kv_len``; the partial states live in the library's static per-GPU
    scratch array (``DECODE_NOALLOC_SCRATCH_BYTES``), so calls that overlap
    on one GPU race.  For code under graph capture or loops that must not
    allocate."""
    lib = load_library()
    dt = _dtype_code(q)
    pq = _dev(q, "q", dim=3)
    pk = _dev(k_pages, "k_pages", q.dtype, 4)
    pv = _dev(v_pages, "v_pages", q.dtype, 4)
    pt = _dev(page_table, "page_table", torch.int32, 2)
    pl = _dev(kv_lens, "kv_lens", torch.int32, 1)
    B, Hq, D = q.shape
    num_pages, page_size, Hkv, Dk = k_pages.shape
    if tuple(v_pages.shape) != tuple(k_pages.shape) or Dk != D:
        raise ValueError(f"k_pages {tuple(k_pages.shape)} / v_pages {tuple(v_pages.shape)} do not "
                         f"match q {tuple(q.shape)}")
    if page_table.shape[0] != B or kv_lens.shape[0] != B:
        raise ValueError("page_table and kv_lens need one row per request")
    _dev(out, "out", q.dtype, 3)
    _dev(lse, "lse", torch.float32, 2)
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq):
        raise ValueError("out/lse have the wrong shape")
    _check(lib.attn_decode_paged_noalloc(dt, pq, pk, pv, pt, pl, B, Hq, Hkv, D, page_size,
                                         num_pages, page_table.shape[1], int(max_kv_len),
                                         int(split_pages), _scale(scale, D), out.data_ptr(),
                                         lse.data_ptr(), _stream(q.device)))
    return out, lse


def decode_paged_fp8(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                     page_table: torch.Tensor, kv_lens: torch.Tensor, k_scale: float,
                     v_scale: float, scale: Optional[float] = None,
                     max_kv_len: Optional[int] = None, split_pages: int = 0,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, kv_layout: str = "NHD",
                     window_left: int = -1) -> Tuple[torch.Tensor, torch.Tensor]:
    """:func:`decode_paged` over a cache of E4M3 bytes (uint8 pools): token t's
    key is ``k_scale * E4M3(k_pages[...])`` and its value ``v_scale * E4M3(...)``.
    q and out are bf16 or fp16; ``window_left`` as in :func:`decode_paged`."""
    return _decode(q, k_pages, v_pages, page_table, kv_lens, scale, max_kv_len, split_pages, out,
                   lse, workspace, fp8_scales=(k_scale, v_scale), kv_layout=kv_layout,
                   window_left=window_left)


def prefill_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                   cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                   causal: bool = True, scale: Optional[float] = None,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   window_left: int = -1, window_right: int = -1) -> Tuple[torch.Tensor, torch.Tensor]:
    """Ragged prefill: q [Tq, Hq, D], k/v [Tk, Hkv, D] packed by cu_seqlens [B+1].
    ``window_left`` >= 0 restricts query i to keys >= i + (Lk - Lq) - window_left,
    ``window_right`` >= 0 to keys <= i + (Lk - Lq) + window_right (``causal``
    is the right window 0 and takes precedence).

    Returns (out [Tq, Hq, D], lse [Tq, Hq] float32).
    """
    lib = load_library()
    dt = _dtype_code(q)
    pq = _dev(q, "q", dim=3)
    pk = _dev(k, "k", q.dtype, 3)
    pv = _dev(v, "v", q.dtype, 3)
    pcq = _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    pck = _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    Tq, Hq, D = q.shape
    Tk, Hkv, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Dk != D:
        raise ValueError(f"k {tuple(k.shape)} / v {tuple(v.shape)} do not match q {tuple(q.shape)}")
    B = cu_seqlens_q.shape[0] - 1
    if B < 0 or cu_seqlens_k.shape[0] != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have B+1 entries")
    s = _scale(scale, D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((Tq, Hq), dtype=torch.float32, device=q.device)
    _dev(out, "out", q.dtype, 3)
    _dev(lse, "lse", torch.float32, 2)
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (Tq, Hq):
        raise ValueError("out/lse have the wrong shape")
    if window_left == -1 and window_right == -1:
        _check(lib.attn_prefill_varlen(dt, pq, pk, pv, pcq, pck, B, Hq, Hkv, D, Tq, Tk,
                                       int(max_seqlen_q), int(max_seqlen_k), int(bool(causal)),
                                       s, out.data_ptr(), lse.data_ptr(), _stream(q.device)))
    else:
        _check(lib.attn_prefill_varlen_window(dt, pq, pk, pv, pcq, pck, B, Hq, Hkv, D, Tq, Tk,
                                              int(max_seqlen_q), int(max_seqlen_k),
                                              int(bool(causal)), int(window_left),
                                              int(window_right), s,
                                              out.data_ptr(), lse.data_ptr(), _stream(q.device)))
    return out, lse


def prefill_paged(q: torch.Tensor, cu_seqlens_q: torch.Tensor, k_pages: torch.Tensor,
                  v_pages: torch.Tensor, page_table: torch.Tensor, kv_lens: torch.Tensor,
                  max_seqlen_q: int, max_kv_len: int, causal: bool = True,
                  scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None, kv_layout: str = "NHD",
                  window_left: int = -1, window_right: int = -1) -> Tuple[torch.Tensor, torch.Tensor]:
    """Chunked prefill over a paged KV cache: request b's queries are the last
    Lq_b of its kv_lens[b] cached tokens.  Pools are NHD or, with
    ``kv_layout="HND"``, [num_pages, Hkv, page_size, D].  ``window_left`` and
    ``window_right`` as in :func:`prefill_varlen`.  Returns (out, lse)."""
    lib = load_library()
    suffix = _layout(kv_layout)
    dt = _dtype_code(q)
    pq = _dev(q, "q", dim=3)
    pcq = _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    pk = _dev(k_pages, "k_pages", q.dtype, 4)
    pv = _dev(v_pages, "v_pages", q.dtype, 4)
    pt = _dev(page_table, "page_table", torch.int32, 2)
    pl = _dev(kv_lens, "kv_lens", torch.int32, 1)
    Tq, Hq, D = q.shape
    num_pages, page_size, Hkv, Dk = _pool_dims(k_pages, kv_layout)
    if tuple(v_pages.shape) != tuple(k_pages.shape) or Dk != D:
        raise ValueError("k_pages / v_pages do not match q")
    B = cu_seqlens_q.shape[0] - 1
    if page_table.shape[0] != B or kv_lens.shape[0] != B:
        raise ValueError("page_table and kv_lens need one row per request")
    s = _scale(scale, D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((Tq, Hq), dtype=torch.float32, device=q.device)
    _dev(out, "out", q.dtype, 3)
    _dev(lse, "lse", torch.float32, 2)
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (Tq, Hq):
        raise ValueError("out/lse have the wrong shape")
    if window_left != -1 or window_right != -1:
        _check(lib.attn_prefill_paged_window(
            dt, 1 if suffix else 0, pq, pcq, pk, pv, pt, pl, B, Hq, Hkv, D, Tq, page_size,
            num_pages, page_table.shape[1], int(max_seqlen_q), int(max_kv_len), int(bool(causal)),
            int(window_left), int(window_right), s, out.data_ptr(), lse.data_ptr(),
            _stream(q.device)))
        return out, lse
    _check(getattr(lib, "attn_prefill_paged" + suffix)(
        dt, pq, pcq, pk, pv, pt, pl, B, Hq, Hkv, D, Tq, page_size,
                                  num_pages, page_table.shape[1], int(max_seqlen_q),
                                  int(max_kv_len), int(bool(causal)), s, out.data_ptr(),
                                  lse.data_ptr(), _stream(q.device)))
    return out, lse


def prefill_paged_cascade_workspace_size(dtype: torch.dtype, total_q: int, Hq: int, D: int) -> int:
    code = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16, torch.float16: ATTN_F16}.get(dtype)
    if code is None:
        raise ValueError(f"unsupported dtype {dtype} (float32, bfloat16 or float16)")
    return int(load_library().attn_prefill_paged_cascade_workspace_size(code, int(total_q), int(Hq),
                                                                        int(D)))


def prefill_paged_cascade(q: torch.Tensor, cu_seqlens_q: torch.Tensor, k_pages: torch.Tensor,
                          v_pages: torch.Tensor, page_table: torch.Tensor, kv_lens: torch.Tensor,
                          max_seqlen_q: int, max_kv_len: int, shared_prefix_len: int,
                          causal: bool = True, scale: Optional[float] = None,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, kv_layout: str = "NHD"
                          ) -> Tuple[torch.Tensor, torch.Tensor]:
    """:func:`prefill_paged` for a batch whose page-table rows all begin with the
    same ``shared_prefix_len / page_size`` pages: the prefix is attended once
    for every query row, then merged into each request's pass over its own
    keys.  ``workspace`` (uint8, on the device) is allocated when not given."""
    lib = load_library()
    suffix = _layout(kv_layout)
    dt = _dtype_code(q)
    pq = _dev(q, "q", dim=3)
    pcq = _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    pk = _dev(k_pages, "k_pages", q.dtype, 4)
    pv = _dev(v_pages, "v_pages", q.dtype, 4)
    pt = _dev(page_table, "page_table", torch.int32, 2)
    pl = _dev(kv_lens, "kv_lens", torch.int32, 1)
    Tq, Hq, D = q.shape
    num_pages, page_size, Hkv, Dk = _pool_dims(k_pages, kv_layout)
    if tuple(v_pages.shape) != tuple(k_pages.shape) or Dk != D:
        raise ValueError("k_pages / v_pages do not match q")
    B = cu_seqlens_q.shape[0] - 1
    if page_table.shape[0] != B or kv_lens.shape[0] != B:
        raise ValueError("page_table and kv_lens need one row per request")
    s = _scale(scale, D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((Tq, Hq), dtype=torch.float32, device=q.device)
    _dev(out, "out", q.dtype, 3)
    _dev(lse, "lse", torch.float32, 2)
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (Tq, Hq):
        raise ValueError("out/lse have the wrong shape")
    need = lib.attn_prefill_paged_cascade_workspace_size(dt, Tq, Hq, D)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    pw = _dev(workspace, "workspace", torch.uint8, 1)
    if workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, this call needs {need} "
                         "(prefill_paged_cascade_workspace_size)")
    _check(getattr(lib, "attn_prefill_paged_cascade" + suffix)(
        dt, pq, pcq, pk, pv, pt, pl, B, Hq, Hkv, D, Tq,
                                          page_size, num_pages, page_table.shape[1],
                                          int(max_seqlen_q), int(max_kv_len),
                                          int(shared_prefix_len), int(bool(causal)), s,
                                          out.data_ptr(), lse.data_ptr(), pw, workspace.numel(),
                                          _stream(q.device)))
    return out, lse


def merge_states(o_a: torch.Tensor, lse_a: torch.Tensor, o_b: torch.Tensor, lse_b: torch.Tensor,
                 out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None
                 ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Merge two attention states (o [..., D], lse [...]) over disjoint keys.
    ``out`` / ``lse_out`` may be the a or b inputs (in place)."""
    lib = load_library()
    dt = _dtype_code(o_a)
    D = o_a.shape[-1]
    if tuple(o_b.shape) != tuple(o_a.shape) or o_b.dtype != o_a.dtype:
        raise ValueError("o_a and o_b differ in shape or dtype")
    if tuple(lse_a.shape) != tuple(o_a.shape[:-1]) or tuple(lse_b.shape) != tuple(lse_a.shape):
        raise ValueError("lse_a / lse_b must have the shape of o without its last dim")
    pa, pb = _dev(o_a, "o_a"), _dev(o_b, "o_b")
    pla = _dev(lse_a, "lse_a", torch.float32)
    plb = _dev(lse_b, "lse_b", torch.float32)
    if out is None:
        out = torch.empty_like(o_a)
    if lse_out is None:
        lse_out = torch.empty_like(lse_a)
    _dev(out, "out", o_a.dtype)
    _dev(lse_out, "lse_out", torch.float32)
    if tuple(out.shape) != tuple(o_a.shape) or tuple(lse_out.shape) != tuple(lse_a.shape):
        raise ValueError("out/lse_out have the wrong shape")
    rows = lse_a.numel()
    _check(lib.attn_merge_states(dt, pa, pla, pb, plb, rows, D, out.data_ptr(),
                                 lse_out.data_ptr(), _stream(o_a.device)))
    return out, lse_out


def timing_begin(capacity: int = 4096) -> None:
    """Start recording per-kernel HIP-event timings inside the library."""
    _check(load_library().attn_timing_begin(int(capacity)))


def timing_end() -> dict:
    """Stop recording; returns {kernel_kind: (total_ms, launches)}."""
    n = len(KERNEL_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int * n)()
    _check(load_library().attn_timing_end(ms, cnt))
    return {KERNEL_KINDS[i]: (ms[i], cnt[i]) for i in range(n)}
