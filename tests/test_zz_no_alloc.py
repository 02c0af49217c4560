"""nvfp4_hessian_accum_noalloc (partial slots in the library's static device
buffer) against nvfp4_hessian_accum (caller workspace), through the C ABI:
the same kernels, so H and the fused amax must agree bit for bit.  Two
calls in a row share the buffer, the second on a smaller input, so a slot
left over from the first call would show up in the second."""
import numpy as np
import pytest
import torch

import datagen
import nvfp4_post_quantization_amd as nq

from _gpu import DEV, need_gpu, note, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _both(lib, x, ldx, k, h0, a0):
    """H and amax after one call of each entry point from the same start."""
    tokens = x.shape[0]
    sp = torch.cuda.current_stream(DEV).cuda_stream
    h_ws, h_na = h0.clone(), h0.clone()
    a_ws, a_na = a0.clone(), a0.clone()
    need = lib.nvfp4_hessian_workspace_bytes(tokens, k)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    st = lib.nvfp4_hessian_accum(x.data_ptr(), tokens, k, ldx, h_ws.data_ptr(), a_ws.data_ptr(), ws.data_ptr(),
                                 ws.numel(), sp)
    assert st == 0, lib.nvfp4_status_string(st)
    st = lib.nvfp4_hessian_accum_noalloc(x.data_ptr(), tokens, k, ldx, h_na.data_ptr(), a_na.data_ptr(), sp)
    assert st == 0, lib.nvfp4_status_string(st)
    torch.cuda.synchronize()
    return h_ws, h_na, a_ws, a_na


def test_noalloc_matches_workspace_entry_two_calls():
    lib = nq.load()
    # call 1: a whole 65536-token calibration chunk of the K = 12288 stream
    note("noalloc hessian call 1: [65536, 12288]")
    x = datagen.config4_chunk_torch(1, 0, DEV)
    k = x.shape[1]
    h0 = torch.zeros((k // 16, 16, 16), dtype=torch.float32, device=DEV)
    a0 = torch.zeros(1, dtype=torch.float32, device=DEV)
    h_ws, h_na, a_ws, a_na = _both(lib, x, k, k, h0, a0)
    assert torch.equal(h_ws, h_na) and torch.equal(a_ws, a_na)
    assert float(h_na.abs().max()) > 0
    del x, h_ws, h_na
    # call 2: smaller, ragged and strided (300 tokens, k = 272 of a 280-wide
    # row), accumulating into a nonzero H and amax
    note("noalloc hessian call 2: [300, 272] ldx 280")
    rng = np.random.default_rng(5)
    xb = datagen.laplace_bf16(rng, (300, 280), 1.0)
    xs = to_dev_bf16(xb)
    k = 272
    h0 = torch.from_numpy(rng.standard_normal((k // 16, 16, 16)).astype(np.float32)).to(DEV)
    a0 = torch.tensor([0.5], dtype=torch.float32, device=DEV)
    h_ws, h_na, a_ws, a_na = _both(lib, xs, 280, k, h0, a0)
    assert torch.equal(h_ws, h_na) and torch.equal(a_ws, a_na)
    assert not torch.equal(h_na, h0)


def test_noalloc_python_binding_small():
    note("noalloc hessian via the binding: C1 X [512, 256]")
    _, xb = datagen.config1()
    x = to_dev_bf16(xb)
    h1 = torch.zeros((16, 16, 16), dtype=torch.float32, device=DEV)
    h2 = torch.zeros_like(h1)
    nq.hessian_accum(x, h1)
    nq.hessian_accum_noalloc(x, h2)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2)
