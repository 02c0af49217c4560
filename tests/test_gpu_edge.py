"""GPU edge cases through the C ABI: empty inputs leave every output as it
was (nothing is enqueued), and the smallest non-empty shapes match the
oracle.  Inputs from datagen or built here; expected values from the
oracle only."""
import numpy as np
import pytest
import torch

import datagen
from oracle import nvfp4 as N
from oracle import formats as F
import nvfp4_post_quantization_amd as nq

from _gpu import DEV, need_gpu, note, to_dev_bf16, to_dev_f32, host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def test_empty_hessian_keeps_h_and_amax():
    note("hessian with zero tokens")
    H = torch.full((4, 16, 16), 3.5, dtype=torch.float32, device=DEV)
    amax = torch.full((1,), 2.25, dtype=torch.float32, device=DEV)
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    nq.hessian_accum(x, H, amax=amax)
    assert (host(H) == 3.5).all() and float(host(amax)[0]) == 2.25


def test_empty_sweep_quant_dequant():
    note("sweep / quantize / dequant with zero rows")
    s2 = to_dev_f32([2.0 ** -10])
    w = torch.empty((0, 32), dtype=torch.bfloat16, device=DEV)
    H = torch.eye(16, device=DEV).repeat(2, 1, 1).contiguous()
    packed, codes, cost = nq.scale_sweep(w, H, s2, want_cost=True)
    assert packed.shape == (0, 16) and codes.shape == (0, 2) and cost.shape == (0, 2)
    packed, codes = nq.quantize_dynamic(w, s2)
    assert packed.shape == (0, 16) and codes.shape == (0, 2)
    out = nq.dequant(packed, codes, s2)
    assert out.shape == (0, 32)


def test_smallest_shapes():
    """One 16-element block everywhere: tokens = 1, rows = 1, k = 16."""
    note("one block: hessian, sweep, quantize, dequant")
    rng = np.random.default_rng(21)
    x = datagen.f32_to_bf16_bits(rng.standard_normal((1, 16)).astype(np.float32))
    H = torch.zeros((1, 16, 16), dtype=torch.float32, device=DEV)
    nq.hessian_accum(to_dev_bf16(x), H)
    h_ref = N.hessian(x)
    assert np.allclose(host(H), h_ref, rtol=1e-6, atol=0)            # products of bf16 are exact in fp32
    w = datagen.f32_to_bf16_bits((rng.standard_normal((1, 16)) * 0.02).astype(np.float32))
    _, s2 = N.tensor_scale(w)
    h32 = (h_ref + np.eye(16)).astype(np.float32)                     # rank-1 plus identity: PD
    packed, codes, _ = nq.scale_sweep(to_dev_bf16(w), torch.from_numpy(h32).to(DEV), to_dev_f32([s2]))
    c_ref, p_ref, _ = N.scale_sweep(w, h32.astype(np.float64), s2)
    assert host(codes)[0, 0] == c_ref[0, 0] and np.array_equal(host(packed), p_ref)
    pq, cq = nq.quantize_dynamic(to_dev_bf16(w), to_dev_f32([s2]))
    pr, cr = N.quantize_dynamic(w, s2)
    assert np.array_equal(host(pq), pr) and np.array_equal(host(cq), cr)
    out = nq.dequant(pq, cq, to_dev_f32([s2]))
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), N.dequant(pr, cr, s2))
