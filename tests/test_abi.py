"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments before any HIP call.

Pointers used here are never dereferenced: every call is built to fail
validation (a call that passed it would launch kernels).
"""
import ctypes
import os
import re

import pytest

import nvfp4_post_quantization_amd as nq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("nvfp4mi.h", "nvfp4mi_probe.h")]

OK, NULL, SHAPE, ALIGN, WS, BADIN, HIP, SCRATCH = 0, 1, 2, 3, 4, 5, 6, 7
P = 0x10000          # a 16-byte-aligned fake address (never dereferenced)


def _declared():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z0-9_]+)\s*\(", text, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(nq.LIB_PATH):
        pytest.skip("libnvfp4mi.so not built")
    return nq.load()


def test_header_symbols_exported(lib):
    names = _declared()
    assert set(names) == {
        "nvfp4_status_string", "nvfp4_compute_scale2", "nvfp4_compute_scale2_batch", "nvfp4_hessian_workspace_bytes",
        "nvfp4_hessian_accum", "nvfp4_hessian_accum_noalloc", "nvfp4_hessian_accum_fq",
        "nvfp4_hessian_chunks_workspace_bytes", "nvfp4_hessian_accum_chunks", "nvfp4_hessian_accum_fq_chunks",
        "nvfp4_scale_sweep", "nvfp4_quantize_dynamic", "nvfp4_dequant",
        "mxfp4_to_nvfp4_cast", "fp8e4m3_compute_scale", "fp8e4m3_quantize", "fp8e4m3_dequant",
        "nvfp4_block_hadamard", "nvfp4_hessian_hadamard", "nvfp4_fakequant", "nvfp4_scale_sweep_ex",
        "nvfp4_quantlinear_workspace_bytes", "nvfp4_quantlinear_forward",
        "nvfp4_probe_read", "nvfp4_probe_write", "nvfp4_probe_copy", "nvfp4_scale_sweep_stats",
    }
    assert {os.path.basename(h) for h in HEADERS} == set(os.listdir(os.path.join(ROOT, "include")))
    for n in names:
        assert hasattr(lib, n), n
    raw = ctypes.CDLL(nq.LIB_PATH)
    for n in names:
        getattr(raw, n)


def test_status_strings(lib):
    for s in range(0, 8):
        assert lib.nvfp4_status_string(s)
    assert b"static buffer" in lib.nvfp4_status_string(SCRATCH)
    assert lib.nvfp4_status_string(0) == b"ok"
    assert b"unknown" in lib.nvfp4_status_string(99)


def test_compute_scale2_validation(lib):
    assert lib.nvfp4_compute_scale2(P, -1, P, None, None) == SHAPE
    assert lib.nvfp4_compute_scale2(None, 16, P, None, None) == NULL
    assert lib.nvfp4_compute_scale2(P, 16, None, None, None) == NULL
    assert lib.nvfp4_compute_scale2(P + 2, 16, P, None, None) == ALIGN
    assert lib.nvfp4_compute_scale2(P, 16, P + 2, None, None) == ALIGN      # scale2_out: an atomic target
    assert lib.nvfp4_compute_scale2(P, 16, P, P + 1, None) == ALIGN         # amax_out


def test_compute_scale2_batch_validation(lib):
    f = lib.nvfp4_compute_scale2_batch
    def arrs(ptrs, ns):
        return (ctypes.c_void_p * len(ptrs))(*ptrs), (ctypes.c_int64 * len(ns))(*ns)
    xs, ns = arrs([P, P + 16], [16, 32])
    assert f(xs, ns, 0, P, None, None) == SHAPE                           # count < 1
    assert f(xs, ns, 17, P, None, None) == SHAPE                          # count > 16
    assert f(None, ns, 2, P, None, None) == NULL
    assert f(xs, None, 2, P, None, None) == NULL
    assert f(xs, ns, 2, None, None, None) == NULL
    xs2, ns2 = arrs([P, None], [16, 8])
    assert f(xs2, ns2, 2, P, None, None) == NULL                          # null tensor with n > 0
    xs3, ns3 = arrs([P, P + 2], [16, 8])
    assert f(xs3, ns3, 2, P, None, None) == ALIGN                         # tensor not 16-byte aligned
    xs4, ns4 = arrs([P, P], [16, -1])
    assert f(xs4, ns4, 2, P, None, None) == SHAPE                         # n < 0
    assert f(xs, ns, 2, P + 2, None, None) == ALIGN                       # scale2_out not 4-byte aligned
    assert f(xs, ns, 2, P, P + 1, None) == ALIGN                          # amax_out


def test_hessian_validation(lib):
    ws = lib.nvfp4_hessian_workspace_bytes(65536, 4096)
    assert ws > 0 and ws % 1024 == 0
    assert lib.nvfp4_hessian_workspace_bytes(0, 4096) == 0
    assert lib.nvfp4_hessian_workspace_bytes(16, 24) == 0
    f = lib.nvfp4_hessian_accum
    assert f(P, 16, 24, 24, P, None, P, 1 << 20, None) == SHAPE           # k % 16
    assert f(P, 16, 32, 16, P, None, P, 1 << 20, None) == SHAPE           # ld < k
    assert f(P, -1, 32, 32, P, None, P, 1 << 20, None) == SHAPE
    assert f(P, 16, 0, 0, P, None, P, 1 << 20, None) == SHAPE
    assert f(P, 16, 32, 32, None, None, P, 1 << 20, None) == NULL
    assert f(None, 16, 32, 32, P, None, P, 1 << 20, None) == NULL
    assert f(P + 2, 16, 32, 32, P, None, P, 1 << 20, None) == ALIGN
    assert f(P, 16, 32, 36, P, None, P, 1 << 20, None) == ALIGN           # row stride not 16 B
    assert f(P, 16, 32, 32, P + 4, None, P, 1 << 20, None) == ALIGN       # H
    assert f(P, 16, 32, 32, P, None, P + 8, 1 << 20, None) == ALIGN       # workspace
    assert f(P, 16, 32, 32, P, P + 2, P, 1 << 20, None) == ALIGN          # amax: an atomic target
    need = lib.nvfp4_hessian_workspace_bytes(16, 32)
    assert f(P, 16, 32, 32, P, None, P, need - 1, None) == WS
    assert f(P, 16, 32, 32, P, None, None, need, None) == NULL
    assert f(P, 0, 32, 32, P, None, None, 0, None) == OK                  # nothing to do
    assert f(P, 1 << 62, 32, 1 << 40, P, None, P, 1 << 20, None) == SHAPE   # overflow


def test_hessian_chunks_validation(lib):
    q = lib.nvfp4_hessian_chunks_workspace_bytes
    one = lib.nvfp4_hessian_workspace_bytes(65536, 4096)
    assert q(65536, 4096, 16) >= 16 * 8 * 1024 and q(65536, 4096, 16) == 16 * q(65536, 4096, 1)
    assert q(65536, 4096, 0) == 0 and q(65536, 4096, 65) == 0 and q(0, 4096, 2) == 0 and q(16, 24, 2) == 0
    assert q(65536, 4096, 1) <= one
    f = lib.nvfp4_hessian_accum_chunks
    xs = (ctypes.c_void_p * 2)(P, P + 4096)
    need = q(16, 32, 2)
    assert f(xs, 0, 16, 32, 32, P, None, P, need, None) == SHAPE            # nchunks < 1
    assert f(xs, 65, 16, 32, 32, P, None, P, need, None) == SHAPE           # nchunks > 64
    assert f(xs, 2, 16, 24, 24, P, None, P, need, None) == SHAPE            # k % 16
    assert f(xs, 2, 16, 32, 16, P, None, P, need, None) == SHAPE            # ld < k
    assert f(None, 2, 16, 32, 32, P, None, P, need, None) == NULL
    assert f(xs, 2, 16, 32, 32, None, None, P, need, None) == NULL
    bad = (ctypes.c_void_p * 2)(P, None)
    assert f(bad, 2, 16, 32, 32, P, None, P, need, None) == NULL            # a NULL chunk
    mis = (ctypes.c_void_p * 2)(P, P + 2)
    assert f(mis, 2, 16, 32, 32, P, None, P, need, None) == ALIGN           # a misaligned chunk
    assert f(xs, 2, 16, 32, 32, P, None, P, need - 1, None) == WS
    assert f(xs, 2, 16, 32, 32, P, None, None, need, None) == NULL
    assert f(xs, 2, 16, 32, 32, P + 4, None, P, need, None) == ALIGN        # H
    assert f(xs, 2, 16, 32, 32, P, None, P + 8, need, None) == ALIGN        # workspace
    assert f(xs, 2, 16, 32, 32, P, P + 2, P, need, None) == ALIGN           # amax
    assert f(xs, 2, 0, 32, 32, P, None, None, 0, None) == OK                # nothing to do
    fq = lib.nvfp4_hessian_accum_fq_chunks
    assert fq(xs, 0, 16, 32, 32, P, P, None, P, need, None) == SHAPE          # nchunks < 1
    assert fq(xs, 2, 16, 24, 24, P, P, None, P, need, None) == SHAPE          # k % 16
    assert fq(xs, 2, 16, 32, 32, None, P, None, P, need, None) == NULL        # scale2
    assert fq(xs, 2, 16, 32, 32, P, None, None, P, need, None) == NULL        # H
    assert fq(bad, 2, 16, 32, 32, P, P, None, P, need, None) == NULL          # a NULL chunk
    assert fq(mis, 2, 16, 32, 32, P, P, None, P, need, None) == ALIGN
    assert fq(xs, 2, 16, 32, 32, P, P, None, P, need - 1, None) == WS
    assert fq(xs, 2, 16, 32, 32, P, P, P + 2, P, need, None) == ALIGN         # amax
    assert fq(xs, 2, 0, 32, 32, P, P, None, None, 0, None) == OK              # nothing to do
    assert fq(xs, 2, 0, 32, 32, None, P, None, None, 0, None) == NULL         # scale2 even when empty


def test_hessian_noalloc_validation(lib):
    f = lib.nvfp4_hessian_accum_noalloc
    assert f(P, 16, 24, 24, P, None, None) == SHAPE                       # k % 16
    assert f(P, 16, 32, 16, P, None, None) == SHAPE                       # ld < k
    assert f(P, -1, 32, 32, P, None, None) == SHAPE
    assert f(P, 16, 32, 32, None, None, None) == NULL
    assert f(None, 16, 32, 32, P, None, None) == NULL
    assert f(P + 2, 16, 32, 32, P, None, None) == ALIGN
    assert f(P, 16, 32, 36, P, None, None) == ALIGN                       # row stride not 16 B
    assert f(P, 16, 32, 32, P + 4, None, None) == ALIGN                   # H
    assert f(P, 16, 32, 32, P, P + 2, None) == ALIGN                      # amax
    assert f(P, 0, 32, 32, P, None, None) == OK                           # nothing to do
    assert f(P, 1 << 62, 32, 1 << 40, P, None, None) == SHAPE             # overflow
    # beyond the static buffer: 513 slabs of 16 groups need three partial
    # slots for each of 512 workgroups (24 MiB); rejected before any HIP call
    assert f(P, 65536, 131088, 131088, P, None, None) == SCRATCH
    assert f(P, 64, 131088, 131088, P, None, None) == SCRATCH


def test_hessian_fq_validation(lib):
    f = lib.nvfp4_hessian_accum_fq
    need = lib.nvfp4_hessian_workspace_bytes(16, 32)
    assert f(P, 16, 24, 24, P, P, None, P, 1 << 20, None) == SHAPE         # k % 16
    assert f(P, 16, 32, 16, P, P, None, P, 1 << 20, None) == SHAPE         # ld < k
    assert f(P, 16, 32, 32, None, P, None, P, need, None) == NULL          # scale2
    assert f(P, 16, 32, 32, P, None, None, P, need, None) == NULL          # H
    assert f(None, 16, 32, 32, P, P, None, P, need, None) == NULL
    assert f(P + 2, 16, 32, 32, P, P, None, P, need, None) == ALIGN
    assert f(P, 16, 32, 32, P, P + 4, None, P, need, None) == ALIGN        # H
    assert f(P, 16, 32, 32, P, P, None, P + 8, need, None) == ALIGN        # workspace
    assert f(P, 16, 32, 32, P, P, P + 2, P, need, None) == ALIGN           # amax
    assert f(P, 16, 32, 32, P, P, None, P, need - 1, None) == WS
    assert f(P, 0, 32, 32, P, P, None, None, 0, None) == OK                # nothing to do
    assert f(P, 0, 32, 32, None, P, None, None, 0, None) == NULL           # scale2 even when empty


def test_sweep_quant_dequant_validation(lib):
    s = lib.nvfp4_scale_sweep
    assert s(P, 4, 24, 24, P, P, P, P, None, None) == SHAPE
    assert s(P, 4, 32, 32, None, P, P, P, None, None) == NULL
    assert s(P, 4, 32, 32, P, None, P, P, None, None) == NULL
    assert s(P, 4, 32, 32, P, P, None, P, None, None) == NULL
    assert s(P + 8, 4, 32, 32, P, P, P, P, None, None) == ALIGN
    assert s(P, 4, 32, 32, P, P, P + 4, P, None, None) == ALIGN          # packed: 8-byte stores
    assert s(P, 4, 32, 32, P, P, P, P, P + 2, None) == ALIGN             # cost: float stores
    assert s(P, 0, 32, 32, P, P, P, P, None, None) == OK
    qd = lib.nvfp4_quantize_dynamic
    assert qd(P, 4, 40, 40, P, P, P, None) == SHAPE
    assert qd(P, 4, 32, 32, None, P, P, None) == NULL
    assert qd(P + 4, 4, 32, 32, P, P, P, None) == ALIGN
    assert qd(P, 4, 32, 32, P, P + 1, P, None) == ALIGN
    dq = lib.nvfp4_dequant
    assert dq(P, P, P, 4, 8, P, None) == SHAPE
    assert dq(P, None, P, 4, 32, P, None) == NULL
    assert dq(P, P, P, 4, 32, P + 2, None) == ALIGN
    assert dq(P, P, P, 0, 32, P, None) == OK


def test_cast_validation(lib):
    c = lib.mxfp4_to_nvfp4_cast
    assert c(P, P, 2, 2, 4, 48, P, P, None, None) == SHAPE        # k % 32
    assert c(P, P, -1, 2, 4, 64, P, P, None, None) == SHAPE
    assert c(P, P, 2, 0, 4, 64, P, P, None, None) == BADIN
    assert c(P, P, 2, 2, 4, 64, P, None, None, None) == NULL
    assert c(None, P, 2, 2, 4, 64, P, P, None, None) == NULL
    assert c(P, P + 1, 2, 2, 4, 64, P, P, None, None) == ALIGN
    assert c(P, P, 2, 2, 4, 64, P, P + 2, None, None) == ALIGN     # scale2_out
    assert c(P, P, 2, 2, 4, 64, P, P, P + 4, None) == ALIGN        # fallback counts: 8-byte atomics
    assert c(P, P, 0, 2, 4, 64, P, P, None, None) == OK


def test_python_layer_rejects_cpu_tensors():
    import torch
    x = torch.zeros(4, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        nq.quantize_dynamic(x, torch.zeros(1))


def test_fp8_validation(lib):
    cs = lib.fp8e4m3_compute_scale
    assert cs(P, -1, P, None, None) == SHAPE
    assert cs(None, 8, P, None, None) == NULL
    assert cs(P, 8, None, None, None) == NULL
    assert cs(P + 2, 8, P, None, None) == ALIGN
    assert cs(P, 8, P + 2, None, None) == ALIGN            # scale_out: an atomic target
    assert cs(P, 8, P, P + 1, None) == ALIGN               # amax_out
    q = lib.fp8e4m3_quantize
    assert q(P, 4, 12, 16, P, P, None) == SHAPE            # k % 8
    assert q(P, 4, 16, 8, P, P, None) == SHAPE             # ld < k
    assert q(P, -1, 16, 16, P, P, None) == SHAPE
    assert q(P, 4, 16, 16, None, P, None) == NULL          # scale
    assert q(None, 4, 16, 16, P, P, None) == NULL
    assert q(P, 4, 16, 16, P, None, None) == NULL
    assert q(P + 2, 4, 16, 16, P, P, None) == ALIGN
    assert q(P, 4, 16, 20, P, P, None) == ALIGN            # row stride not 16 B
    assert q(P, 4, 16, 16, P, P + 4, None) == ALIGN        # q not 8-byte aligned
    assert q(P, 0, 16, 16, P, None, None) == OK
    assert q(P, 1 << 62, 16, 1 << 40, P, P, None) == SHAPE
    d = lib.fp8e4m3_dequant
    assert d(P, P, 4, 12, P, None) == SHAPE
    assert d(P, None, 4, 16, P, None) == NULL
    assert d(None, P, 4, 16, P, None) == NULL
    assert d(P + 4, P, 4, 16, P, None) == ALIGN
    assert d(P, P, 4, 16, P + 8, None) == ALIGN
    assert d(None, P, 0, 16, None, None) == OK


def test_hadamard_validation(lib):
    b = lib.nvfp4_block_hadamard
    assert b(P, 4, 24, 24, P, 24, None) == SHAPE            # k % 16
    assert b(P, 4, 32, 16, P, 32, None) == SHAPE            # ldx < k
    assert b(P, 4, 32, 32, P, 16, None) == SHAPE            # ldo < k
    assert b(None, 4, 32, 32, P, 32, None) == NULL
    assert b(P, 4, 32, 32, None, 32, None) == NULL
    assert b(P + 2, 4, 32, 32, P, 32, None) == ALIGN
    assert b(P, 4, 32, 32, P + 2, 32, None) == ALIGN
    assert b(P, 4, 32, 36, P, 32, None) == ALIGN
    assert b(P, 0, 32, 32, None, 32, None) == OK
    h = lib.nvfp4_hessian_hadamard
    assert h(P, -1, P, None) == SHAPE
    assert h(None, 4, P, None) == NULL
    assert h(P, 4, None, None) == NULL
    assert h(P + 2, 4, P, None) == ALIGN
    assert h(P, 4, P + 1, None) == ALIGN
    assert h(None, 0, None, None) == OK


def test_fakequant_and_forward_validation(lib):
    f = lib.nvfp4_fakequant
    assert f(P, 4, 24, 24, P, P, 24, None) == SHAPE             # k % 16
    assert f(P, 4, 32, 32, None, P, 32, None) == NULL           # scale2
    assert f(P, 4, 32, 32, P, P, 16, None) == SHAPE             # ldo < k
    assert f(P + 2, 4, 32, 32, P, P, 32, None) == ALIGN
    assert f(P, 4, 32, 32, P, P + 2, 32, None) == ALIGN
    assert f(P, 0, 32, 32, P, None, 32, None) == OK
    assert lib.nvfp4_quantlinear_workspace_bytes(0, 32) > 0
    assert lib.nvfp4_quantlinear_workspace_bytes(8, 24) == 0
    need = lib.nvfp4_quantlinear_workspace_bytes(8, 32)
    assert need >= 8 * 32 * 2
    q = lib.nvfp4_quantlinear_forward
    assert q(P, 8, 24, 24, P, P, 16, 24, P, 16, P, need, None) == SHAPE       # k % 16
    assert q(P, 8, 32, 32, P, P, 0, 32, P, 16, P, need, None) == SHAPE        # out_features = 0
    assert q(P, 8, 32, 32, P, P, 16, 32, P, 8, P, need, None) == SHAPE        # ldy < out
    assert q(P, 8, 32, 32, None, P, 16, 32, P, 16, P, need, None) == NULL     # x_scale2
    assert q(P, 8, 32, 32, P, None, 16, 32, P, 16, P, need, None) == NULL     # w
    assert q(P, 8, 32, 32, P, P, 16, 32, P, 16, P, need - 1, None) == WS
    assert q(P, 8, 32, 32, P, P, 16, 32, P, 16, None, need, None) == NULL     # workspace
    assert q(P, 8, 32, 32, P, P, 16, 32, P, 16, P + 16, need, None) == ALIGN  # workspace not 256-aligned
    assert q(P, 8, 32, 32, P, P + 2, 16, 32, P, 16, P, need, None) == ALIGN
    assert q(P, 0, 32, 32, P, P, 16, 32, None, 16, None, 0, None) == OK       # nothing to do


def test_sweep_ex_validation(lib):
    s = lib.nvfp4_scale_sweep_ex
    assert s(P, 4, 32, 32, P, P, P, P, None, 2, None) == BADIN     # wgs_per_cu
    assert s(P, 4, 32, 32, P, P, P, P, None, -1, None) == BADIN
    assert s(P, 4, 24, 24, P, P, P, P, None, 1, None) == SHAPE
    assert s(P, 4, 32, 32, None, P, P, P, None, 1, None) == NULL
    assert s(P, 0, 32, 32, P, P, None, None, None, 1, None) == OK


def test_probe_and_stats_validation(lib):
    r, w, c = lib.nvfp4_probe_read, lib.nvfp4_probe_write, lib.nvfp4_probe_copy
    assert r(P, 24, P, 0, None) == SHAPE                     # bytes % 16
    assert r(None, 32, P, 0, None) == NULL
    assert r(P, 32, None, 0, None) == NULL                   # sink
    assert r(P + 8, 32, P, 0, None) == ALIGN
    assert r(P, 32, P + 2, 0, None) == ALIGN
    assert r(P, 32, P, -1, None) == BADIN                    # workgroups
    assert r(P, 32, P, 65536, None) == BADIN
    assert r(P, 0, P, 0, None) == OK
    assert w(P, 20, 0, 0, None) == SHAPE
    assert w(None, 32, 0, 0, None) == NULL
    assert w(P + 4, 32, 0, 0, None) == ALIGN
    assert w(P, 32, 0, -2, None) == BADIN
    assert w(P, 0, 0, 0, None) == OK
    assert c(P, P + 4096, 24, 0, None) == SHAPE
    assert c(None, P, 32, 0, None) == NULL
    assert c(P, None, 32, 0, None) == NULL
    assert c(P, P + 8, 32, 0, None) == ALIGN
    assert c(P, P + 16, 32, 0, None) == BADIN                # overlapping
    assert c(P, P + 4096, 32, 70000, None) == BADIN
    assert c(P, P + 4096, 0, 0, None) == OK
    st = lib.nvfp4_scale_sweep_stats
    assert st(P, 4, 32, 32, P, P, P, P, None, None) == NULL           # stats
    assert st(P, 4, 24, 24, P, P, P, P, P, None) == SHAPE
    assert st(P, 4, 32, 32, P, P, P, P, P + 4, None) == ALIGN          # stats: uint64
    assert st(P, 0, 32, 32, P, P, P, P, P, None) == OK
