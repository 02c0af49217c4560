"""NVFP4 post-training quantization on MI355X (gfx950): Python binding.

A thin ctypes layer over libnvfp4mi.so (include/nvfp4mi.h).  Every step runs
in the HIP kernels of that library; this module only checks tensor dtypes,
devices and layouts, allocates outputs with torch, and passes pointers and
the current HIP stream.  It fails loudly when the library is missing.

Functions (names as in the C ABI):
  compute_scale2(x)                         -> (scale2[1] f32, amax[1] f32)
  hessian_accum(x, H, amax=None, workspace=None)   H += block-diag X^T X (in place)
  scale_sweep(w, H, scale2, want_cost=False) -> (packed u8, codes u8, cost f32 | None)
  quantize_dynamic(x, scale2)               -> (packed u8, codes u8)
  dequant(packed, codes, scale2)            -> bf16
  mxfp4_to_nvfp4_cast(packed, e8m0, want_fallback=True) -> (codes, scale2, fallback)
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "LIB_PATH", "load", "NvFp4Error", "compute_scale2", "compute_scale2_batch", "hessian_workspace_bytes",
    "hessian_accum", "hessian_accum_chunks", "hessian_chunks_workspace_bytes", "hessian_accum_noalloc", "hessian_accum_fq",
    "hessian_accum_fq_chunks", "scale_sweep", "quantize_dynamic", "dequant", "mxfp4_to_nvfp4_cast",
    "fp8_compute_scale", "fp8_quantize", "fp8_dequant", "block_hadamard", "hessian_hadamard",
    "fakequant", "quantlinear_workspace_bytes", "quantlinear_forward", "scale_sweep_stats",
]

# NVFP4MI_LIB names another build of the same library (the host-sanitizer
# build of tests/test_abi_sanitized.py); by default the in-tree build.
LIB_PATH = os.environ.get("NVFP4MI_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4mi.so")

_c_void_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_SIGS = {
    "nvfp4_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "nvfp4_compute_scale2": (ctypes.c_int, [_c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p]),
    "nvfp4_compute_scale2_batch": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(_i64), ctypes.c_int,
                                                  _c_void_p, _c_void_p, _c_void_p]),
    "nvfp4_hessian_workspace_bytes": (ctypes.c_size_t, [_i64, _i64]),
    "nvfp4_hessian_accum": (ctypes.c_int, [_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p,
                                           ctypes.c_size_t, _c_void_p]),
    "nvfp4_hessian_accum_noalloc": (ctypes.c_int, [_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p]),
    "nvfp4_hessian_chunks_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, ctypes.c_int]),
    "nvfp4_hessian_accum_chunks": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, _i64, _i64, _i64,
                                                  _c_void_p, _c_void_p, _c_void_p, ctypes.c_size_t, _c_void_p]),
    "nvfp4_hessian_accum_fq": (ctypes.c_int, [_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p,
                                              _c_void_p, ctypes.c_size_t, _c_void_p]),
    "nvfp4_hessian_accum_fq_chunks": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, _i64, _i64, _i64,
                                                     _c_void_p, _c_void_p, _c_void_p, _c_void_p, ctypes.c_size_t,
                                                     _c_void_p]),
    "nvfp4_scale_sweep": (ctypes.c_int, [_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p,
                                         _c_void_p, _c_void_p, _c_void_p]),
    "nvfp4_scale_sweep_ex": (ctypes.c_int, [_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p,
                                            _c_void_p, _c_void_p, ctypes.c_int, _c_void_p]),
    "nvfp4_quantize_dynamic": (ctypes.c_int, [_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p,
                                              _c_void_p]),
    "nvfp4_dequant": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _i64, _i64, _c_void_p, _c_void_p]),
    "mxfp4_to_nvfp4_cast": (ctypes.c_int, [_c_void_p, _c_void_p, _i64, _i64, _i64, _i64, _c_void_p, _c_void_p,
                                           _c_void_p, _c_void_p]),
    "fp8e4m3_compute_scale": (ctypes.c_int, [_c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p]),
    "fp8e4m3_quantize": (ctypes.c_int, [_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p]),
    "fp8e4m3_dequant": (ctypes.c_int, [_c_void_p, _c_void_p, _i64, _i64, _c_void_p, _c_void_p]),
    "nvfp4_block_hadamard": (ctypes.c_int, [_c_void_p, _i64, _i64, _i64, _c_void_p, _i64, _c_void_p]),
    "nvfp4_hessian_hadamard": (ctypes.c_int, [_c_void_p, _i64, _c_void_p, _c_void_p]),
    "nvfp4_fakequant": (ctypes.c_int, [_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _i64, _c_void_p]),
    "nvfp4_scale_sweep_stats": (ctypes.c_int, [_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p,
                                               _c_void_p, _c_void_p, _c_void_p]),
    "nvfp4_probe_read": (ctypes.c_int, [_c_void_p, ctypes.c_size_t, _c_void_p, ctypes.c_int, _c_void_p]),
    "nvfp4_probe_write": (ctypes.c_int, [_c_void_p, ctypes.c_size_t, ctypes.c_uint32, ctypes.c_int, _c_void_p]),
    "nvfp4_probe_copy": (ctypes.c_int, [_c_void_p, _c_void_p, ctypes.c_size_t, ctypes.c_int, _c_void_p]),
    "nvfp4_quantlinear_workspace_bytes": (ctypes.c_size_t, [_i64, _i64]),
    "nvfp4_quantlinear_forward": (ctypes.c_int, [_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _i64, _i64,
                                                 _c_void_p, _i64, _c_void_p, ctypes.c_size_t, _c_void_p]),
}

_lib = None


class NvFp4Error(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libnvfp4mi.so (built by nvfp4_post_quantization_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m nvfp4_post_quantization_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        text = load().nvfp4_status_string(status).decode(errors="replace")
        raise NvFp4Error(fn, status, text)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, dtype, name: str, dims: int | None = None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dimensions (got {t.dim()})")
    return t


def _row_major(t: torch.Tensor, name: str) -> int:
    """Row stride of a 2-D tensor whose rows are contiguous."""
    if t.stride(1) != 1:
        raise ValueError(f"{name} rows must be contiguous")
    return t.stride(0) if t.size(0) > 1 else t.size(1)


def compute_scale2(x: torch.Tensor, out=None):
    """Tensor amax and scale_2 = amax / (6 * 448) of a contiguous bf16 tensor.

    Returns (scale2, amax), each f32[1]; out=(scale2, amax) reuses buffers."""
    _dev(x, torch.bfloat16, "x")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if out is None:
        s2 = torch.empty(1, dtype=torch.float32, device=x.device)
        am = torch.empty(1, dtype=torch.float32, device=x.device)
    else:
        s2, am = out
        _dev(s2, torch.float32, "scale2")
        _dev(am, torch.float32, "amax")
    _check("nvfp4_compute_scale2",
           load().nvfp4_compute_scale2(x.data_ptr(), x.numel(), s2.data_ptr(), am.data_ptr(), _stream(x)))
    return s2, am


def compute_scale2_batch(xs, out=None):
    """compute_scale2 for up to 16 contiguous bf16 tensors in one call (three
    launches in all).  Returns (scale2, amax), each f32[len(xs)], on the first
    tensor's device and stream; out=(scale2, amax) reuses buffers."""
    xs = list(xs)
    if not xs or len(xs) > 16:
        raise ValueError("compute_scale2_batch takes 1 to 16 tensors")
    for i, x in enumerate(xs):
        _dev(x, torch.bfloat16, f"xs[{i}]")
        if not x.is_contiguous():
            raise ValueError(f"xs[{i}] must be contiguous")
        if x.device != xs[0].device:
            raise ValueError("all tensors must be on one device")
    n = len(xs)
    if out is None:
        s2 = torch.empty(n, dtype=torch.float32, device=xs[0].device)
        am = torch.empty(n, dtype=torch.float32, device=xs[0].device)
    else:
        s2, am = out
        _dev(s2, torch.float32, "scale2")
        _dev(am, torch.float32, "amax")
        if s2.numel() < n or am.numel() < n:
            raise ValueError("out buffers too small")
    ptrs = (ctypes.c_void_p * n)(*[x.data_ptr() for x in xs])
    counts = (_i64 * n)(*[x.numel() for x in xs])
    _check("nvfp4_compute_scale2_batch", load().nvfp4_compute_scale2_batch(
        ptrs, counts, n, s2.data_ptr(), am.data_ptr(), _stream(xs[0])))
    return s2, am


def hessian_workspace_bytes(tokens: int, k: int) -> int:
    return int(load().nvfp4_hessian_workspace_bytes(tokens, k))


def hessian_accum(x: torch.Tensor, H: torch.Tensor, amax: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None) -> torch.Tensor:
    """H[k/16,16,16] (f32) += block-diagonal X^T X of bf16 x[tokens, k]; in place.

    amax (f32[1]) is raised to max(amax, max|x|) when given.  workspace is a
    uint8 tensor of at least hessian_workspace_bytes(tokens, k) bytes
    (allocated here when omitted).
    """
    _dev(x, torch.bfloat16, "x", 2)
    _dev(H, torch.float32, "H")
    tokens, k = x.shape
    if H.numel() != (k // 16) * 256 or not H.is_contiguous():
        raise ValueError("H must be a contiguous float32 [k/16, 16, 16] tensor")
    ldx = _row_major(x, "x")
    need = hessian_workspace_bytes(tokens, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _dev(workspace, torch.uint8, "workspace")
    if amax is not None:
        _dev(amax, torch.float32, "amax")
    _check("nvfp4_hessian_accum", load().nvfp4_hessian_accum(
        x.data_ptr(), tokens, k, ldx, H.data_ptr(), amax.data_ptr() if amax is not None else None,
        workspace.data_ptr(), workspace.numel(), _stream(x)))
    return H


def hessian_chunks_workspace_bytes(tokens: int, k: int, nchunks: int) -> int:
    return int(load().nvfp4_hessian_chunks_workspace_bytes(tokens, k, nchunks))


def hessian_accum_chunks(xs, H: torch.Tensor, amax: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None) -> torch.Tensor:
    """H += block-diagonal sum over chunks of X_c^T X_c for up to 64 bf16
    chunks of one shape [tokens, k] (row-major, same row stride): one
    accumulate launch per chunk and one reduce over all of them; in place.
    amax is raised to the max |x| over all chunks when given."""
    xs = list(xs)
    if not xs or len(xs) > 64:
        raise ValueError("hessian_accum_chunks takes 1 to 64 chunks")
    for i, x in enumerate(xs):
        _dev(x, torch.bfloat16, f"xs[{i}]", 2)
        if x.shape != xs[0].shape or x.stride() != xs[0].stride():
            raise ValueError("all chunks must have one shape and row stride")
    _dev(H, torch.float32, "H")
    tokens, k = xs[0].shape
    if H.numel() != (k // 16) * 256 or not H.is_contiguous():
        raise ValueError("H must be a contiguous float32 [k/16, 16, 16] tensor")
    ldx = _row_major(xs[0], "xs[0]")
    n = len(xs)
    need = hessian_chunks_workspace_bytes(tokens, k, n)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=xs[0].device)
    _dev(workspace, torch.uint8, "workspace")
    if amax is not None:
        _dev(amax, torch.float32, "amax")
    ptrs = (ctypes.c_void_p * n)(*[x.data_ptr() for x in xs])
    _check("nvfp4_hessian_accum_chunks", load().nvfp4_hessian_accum_chunks(
        ptrs, n, tokens, k, ldx, H.data_ptr(), amax.data_ptr() if amax is not None else None,
        workspace.data_ptr(), workspace.numel(), _stream(xs[0])))
    return H


def hessian_accum_noalloc(x: torch.Tensor, H: torch.Tensor, amax: torch.Tensor | None = None) -> torch.Tensor:
    """hessian_accum without a workspace: the library's static per-device
    buffer holds the partial slots (k <= 131072).  Calls that overlap in time
    on one GPU race on that buffer."""
    _dev(x, torch.bfloat16, "x", 2)
    _dev(H, torch.float32, "H")
    tokens, k = x.shape
    if H.numel() != (k // 16) * 256 or not H.is_contiguous():
        raise ValueError("H must be a contiguous float32 [k/16, 16, 16] tensor")
    ldx = _row_major(x, "x")
    if amax is not None:
        _dev(amax, torch.float32, "amax")
    _check("nvfp4_hessian_accum_noalloc", load().nvfp4_hessian_accum_noalloc(
        x.data_ptr(), tokens, k, ldx, H.data_ptr(), amax.data_ptr() if amax is not None else None, _stream(x)))
    return H


def hessian_accum_fq(x: torch.Tensor, scale2: torch.Tensor, H: torch.Tensor, amax: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None) -> torch.Tensor:
    """W4A4 form of hessian_accum: H += block-diagonal Xh^T Xh, where Xh is x
    after the dynamic NVFP4 quantizer at tensor scale scale2 (f32[1]) and the
    two-level dequantization, computed in one pass over x.  amax, if given, is
    raised to the raw max|x|."""
    _dev(x, torch.bfloat16, "x", 2)
    _dev(H, torch.float32, "H")
    _dev(scale2, torch.float32, "scale2")
    tokens, k = x.shape
    if H.numel() != (k // 16) * 256 or not H.is_contiguous():
        raise ValueError("H must be a contiguous float32 [k/16, 16, 16] tensor")
    ldx = _row_major(x, "x")
    need = hessian_workspace_bytes(tokens, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _dev(workspace, torch.uint8, "workspace")
    if amax is not None:
        _dev(amax, torch.float32, "amax")
    _check("nvfp4_hessian_accum_fq", load().nvfp4_hessian_accum_fq(
        x.data_ptr(), tokens, k, ldx, scale2.data_ptr(), H.data_ptr(),
        amax.data_ptr() if amax is not None else None, workspace.data_ptr(), workspace.numel(), _stream(x)))
    return H


def hessian_accum_fq_chunks(xs, scale2: torch.Tensor, H: torch.Tensor, amax: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None) -> torch.Tensor:
    """hessian_accum_fq over up to 64 bf16 chunks of one shape [tokens, k]
    (row-major, same row stride): one accumulate launch per chunk and one
    reduce over all of them; in place.  amax is raised to the raw max |x|
    over all chunks when given."""
    xs = list(xs)
    if not xs or len(xs) > 64:
        raise ValueError("hessian_accum_fq_chunks takes 1 to 64 chunks")
    for i, x in enumerate(xs):
        _dev(x, torch.bfloat16, f"xs[{i}]", 2)
        if x.shape != xs[0].shape or x.stride() != xs[0].stride():
            raise ValueError("all chunks must have one shape and row stride")
    _dev(H, torch.float32, "H")
    _dev(scale2, torch.float32, "scale2")
    tokens, k = xs[0].shape
    if H.numel() != (k // 16) * 256 or not H.is_contiguous():
        raise ValueError("H must be a contiguous float32 [k/16, 16, 16] tensor")
    ldx = _row_major(xs[0], "xs[0]")
    n = len(xs)
    need = hessian_chunks_workspace_bytes(tokens, k, n)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=xs[0].device)
    _dev(workspace, torch.uint8, "workspace")
    if amax is not None:
        _dev(amax, torch.float32, "amax")
    ptrs = (ctypes.c_void_p * n)(*[x.data_ptr() for x in xs])
    _check("nvfp4_hessian_accum_fq_chunks", load().nvfp4_hessian_accum_fq_chunks(
        ptrs, n, tokens, k, ldx, scale2.data_ptr(), H.data_ptr(), amax.data_ptr() if amax is not None else None,
        workspace.data_ptr(), workspace.numel(), _stream(xs[0])))
    return H


def scale_sweep(w: torch.Tensor, H: torch.Tensor, scale2: torch.Tensor, want_cost: bool = False,
                out=None, wgs_per_cu: int = 0, stream: torch.cuda.Stream | None = None):
    """Hessian-weighted sweep of the E4M3 block scale of bf16 w[rows, k].

    wgs_per_cu = 1 caps the sweep at one workgroup per CU (to run beside an
    HBM-bound kernel on another stream); stream defaults to the current one."""
    _dev(w, torch.bfloat16, "w", 2)
    _dev(H, torch.float32, "H")
    _dev(scale2, torch.float32, "scale2")
    rows, k = w.shape
    if H.numel() != (k // 16) * 256 or not H.is_contiguous():
        raise ValueError("H must be a contiguous float32 [k/16, 16, 16] tensor")
    ldw = _row_major(w, "w")
    if out is None:
        packed = torch.empty((rows, k // 2), dtype=torch.uint8, device=w.device)
        codes = torch.empty((rows, k // 16), dtype=torch.uint8, device=w.device)
        cost = torch.empty((rows, k // 16), dtype=torch.float32, device=w.device) if want_cost else None
    else:
        packed, codes, cost = out
    sp = stream.cuda_stream if stream is not None else _stream(w)
    _check("nvfp4_scale_sweep_ex", load().nvfp4_scale_sweep_ex(
        w.data_ptr(), rows, k, ldw, H.data_ptr(), scale2.data_ptr(), packed.data_ptr(), codes.data_ptr(),
        cost.data_ptr() if cost is not None else None, int(wgs_per_cu), sp))
    return packed, codes, cost


def quantize_dynamic(x: torch.Tensor, scale2: torch.Tensor, out=None):
    """Dynamic per-16 NVFP4 quantization of bf16 x[rows, k]."""
    _dev(x, torch.bfloat16, "x", 2)
    _dev(scale2, torch.float32, "scale2")
    rows, k = x.shape
    ldx = _row_major(x, "x")
    if out is None:
        packed = torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device)
        codes = torch.empty((rows, k // 16), dtype=torch.uint8, device=x.device)
    else:
        packed, codes = out
    _check("nvfp4_quantize_dynamic", load().nvfp4_quantize_dynamic(
        x.data_ptr(), rows, k, ldx, scale2.data_ptr(), packed.data_ptr(), codes.data_ptr(), _stream(x)))
    return packed, codes


def dequant(packed: torch.Tensor, codes: torch.Tensor, scale2: torch.Tensor, out=None) -> torch.Tensor:
    """bf16[rows, k] from NVFP4 (packed u8 [rows, k/2], codes u8 [rows, k/16])."""
    _dev(packed, torch.uint8, "packed", 2)
    _dev(codes, torch.uint8, "codes", 2)
    _dev(scale2, torch.float32, "scale2")
    rows, kh = packed.shape
    k = kh * 2
    if not (packed.is_contiguous() and codes.is_contiguous()) or codes.shape != (rows, k // 16):
        raise ValueError("packed/codes must be contiguous [rows, k/2] / [rows, k/16]")
    if out is None:
        out = torch.empty((rows, k), dtype=torch.bfloat16, device=packed.device)
    _check("nvfp4_dequant", load().nvfp4_dequant(
        packed.data_ptr(), codes.data_ptr(), scale2.data_ptr(), rows, k, out.data_ptr(), _stream(packed)))
    return out


def mxfp4_to_nvfp4_cast(packed: torch.Tensor, e8m0: torch.Tensor, want_fallback: bool = True, out=None):
    """Cast MXFP4 [groups, mats, rows, k/2] (+ E8M0 [.., k/32]) to NVFP4 in place.

    Returns (codes u8 [groups, mats, rows, k/16], scale2 f32 [groups],
    fallback int64 [groups] | None); packed is rewritten only where a block
    falls outside the exact window.
    """
    _dev(packed, torch.uint8, "packed", 4)
    _dev(e8m0, torch.uint8, "e8m0", 4)
    g, m, r, kh = packed.shape
    k = kh * 2
    if e8m0.shape != (g, m, r, k // 32) or not (packed.is_contiguous() and e8m0.is_contiguous()):
        raise ValueError("e8m0 must be contiguous [groups, mats, rows, k/32] matching packed")
    if out is None:
        codes = torch.empty((g, m, r, k // 16), dtype=torch.uint8, device=packed.device)
        s2 = torch.empty(g, dtype=torch.float32, device=packed.device)
        fb = torch.empty(g, dtype=torch.int64, device=packed.device) if want_fallback else None
    else:
        codes, s2, fb = out
    _check("mxfp4_to_nvfp4_cast", load().mxfp4_to_nvfp4_cast(
        packed.data_ptr(), e8m0.data_ptr(), g, m, r, k, codes.data_ptr(), s2.data_ptr(),
        fb.data_ptr() if fb is not None else None, _stream(packed)))
    return codes, s2, fb


def fp8_compute_scale(x: torch.Tensor, out=None):
    """(s, amax) as float32[1] device tensors: s = RN_f32(amax/448) of bf16 x."""
    _dev(x, torch.bfloat16, "x")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if out is None:
        s = torch.empty(1, dtype=torch.float32, device=x.device)
        am = torch.empty(1, dtype=torch.float32, device=x.device)
    else:
        s, am = out
    _check("fp8e4m3_compute_scale", load().fp8e4m3_compute_scale(x.data_ptr(), x.numel(), s.data_ptr(),
                                                                  am.data_ptr(), _stream(x)))
    return s, am


def fp8_quantize(x: torch.Tensor, scale: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """E4M3FN codes uint8 [rows, k] of bf16 x [rows, k] / scale (per-tensor, static)."""
    _dev(x, torch.bfloat16, "x", 2)
    _dev(scale, torch.float32, "scale")
    rows, k = x.shape
    ldx = _row_major(x, "x")
    q = torch.empty((rows, k), dtype=torch.uint8, device=x.device) if out is None else out
    _check("fp8e4m3_quantize", load().fp8e4m3_quantize(x.data_ptr(), rows, k, ldx, scale.data_ptr(),
                                                        q.data_ptr(), _stream(x)))
    return q


def fp8_dequant(q: torch.Tensor, scale: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 [rows, k] = RN_bf16(RN_f32(e4m3(q) * scale))."""
    _dev(q, torch.uint8, "q", 2)
    _dev(scale, torch.float32, "scale")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    rows, k = q.shape
    o = torch.empty((rows, k), dtype=torch.bfloat16, device=q.device) if out is None else out
    _check("fp8e4m3_dequant", load().fp8e4m3_dequant(q.data_ptr(), scale.data_ptr(), rows, k, o.data_ptr(),
                                                      _stream(q)))
    return o


def block_hadamard(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 X R: each 16-element row block times H16 / 4 (fp64 butterfly, one
    rounding).  out may be x itself (in place)."""
    _dev(x, torch.bfloat16, "x", 2)
    rows, k = x.shape
    ldx = _row_major(x, "x")
    if out is None:
        out = torch.empty((rows, k), dtype=torch.bfloat16, device=x.device)
    _dev(out, torch.bfloat16, "out", 2)
    ldo = _row_major(out, "out")
    _check("nvfp4_block_hadamard", load().nvfp4_block_hadamard(x.data_ptr(), rows, k, ldx, out.data_ptr(), ldo,
                                                                _stream(x)))
    return out


def hessian_hadamard(H: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """R^T H R per group of a float32 [groups, 16, 16] Hessian (out may be H)."""
    _dev(H, torch.float32, "H")
    if not H.is_contiguous() or H.numel() % 256:
        raise ValueError("H must be a contiguous float32 [groups, 16, 16] tensor")
    if out is None:
        out = torch.empty_like(H)
    _check("nvfp4_hessian_hadamard", load().nvfp4_hessian_hadamard(H.data_ptr(), H.numel() // 256,
                                                                    out.data_ptr(), _stream(H)))
    return out


def fakequant(x: torch.Tensor, scale2: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 NVFP4 block fake QDQ of x [rows, k] at tensor scale scale2 (f32[1])."""
    _dev(x, torch.bfloat16, "x", 2)
    _dev(scale2, torch.float32, "scale2")
    rows, k = x.shape
    ldx = _row_major(x, "x")
    if out is None:
        out = torch.empty((rows, k), dtype=torch.bfloat16, device=x.device)
    ldo = _row_major(out, "out")
    _check("nvfp4_fakequant", load().nvfp4_fakequant(x.data_ptr(), rows, k, ldx, scale2.data_ptr(), out.data_ptr(),
                                                      ldo, _stream(x)))
    return out


def quantlinear_workspace_bytes(tokens: int, k: int) -> int:
    return int(load().nvfp4_quantlinear_workspace_bytes(tokens, k))


def quantlinear_forward(x: torch.Tensor, x_scale2: torch.Tensor, w_hat: torch.Tensor,
                        out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y [tokens, out] = fakequant(x) @ w_hat^T (bf16 GEMM, fp32 accumulate);
    w_hat is the fake-quantized weight [out, k] (nvfp4 dequant of the swept weight)."""
    _dev(x, torch.bfloat16, "x", 2)
    _dev(w_hat, torch.bfloat16, "w_hat", 2)
    _dev(x_scale2, torch.float32, "x_scale2")
    tokens, k = x.shape
    o = w_hat.shape[0]
    if w_hat.shape[1] != k:
        raise ValueError("w_hat must be [out_features, k]")
    ldx, ldw = _row_major(x, "x"), _row_major(w_hat, "w_hat")
    if out is None:
        out = torch.empty((tokens, o), dtype=torch.bfloat16, device=x.device)
    ldy = _row_major(out, "out")
    need = quantlinear_workspace_bytes(tokens, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check("nvfp4_quantlinear_forward", load().nvfp4_quantlinear_forward(
        x.data_ptr(), tokens, k, ldx, x_scale2.data_ptr(), w_hat.data_ptr(), o, ldw, out.data_ptr(), ldy,
        workspace.data_ptr(), workspace.numel(), _stream(x)))
    return out


def scale_sweep_stats(w: torch.Tensor, H: torch.Tensor, scale2: torch.Tensor, stats: torch.Tensor | None = None,
                      out=None):
    """The sweep's counting build (measurement): scale_sweep's outputs bit for
    bit, plus its search counters added to stats (int64[6] on the device:
    evaluated codes, wave steps, full-form steps, screen steps, blocks,
    waves).  Returns (packed, codes, stats)."""
    _dev(w, torch.bfloat16, "w", 2)
    _dev(H, torch.float32, "H")
    _dev(scale2, torch.float32, "scale2")
    rows, k = w.shape
    if H.numel() != (k // 16) * 256 or not H.is_contiguous():
        raise ValueError("H must be a contiguous float32 [k/16, 16, 16] tensor")
    ldw = _row_major(w, "w")
    if stats is None:
        stats = torch.zeros(6, dtype=torch.int64, device=w.device)
    _dev(stats, torch.int64, "stats")
    if out is None:
        packed = torch.empty((rows, k // 2), dtype=torch.uint8, device=w.device)
        codes = torch.empty((rows, k // 16), dtype=torch.uint8, device=w.device)
    else:
        packed, codes = out
    _check("nvfp4_scale_sweep_stats", load().nvfp4_scale_sweep_stats(
        w.data_ptr(), rows, k, ldw, H.data_ptr(), scale2.data_ptr(), packed.data_ptr(), codes.data_ptr(),
        stats.data_ptr(), _stream(w)))
    return packed, codes, stats
