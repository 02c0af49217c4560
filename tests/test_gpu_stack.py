"""GPU: a synthetic two-layer stack calibrated end to end through the library.

Layer l takes its input X_l (layer 1: synthetic calibration tokens; layer 2:
the fake-quant forward output of layer 1, as the calibration pass produces
it) and runs, all on the GPU:
  scale_2 of W_l and of X_l (a1), H_l from X_l in two chunks (a2) and from
  the fake-quantized X_l (the W4A4 form), the sweep of W_l under H_l (a3),
  the two-DQ weight w_hat_l (a5), then y_l = fakequant(X_l) w_hat_l^T.
Every stage is compared with the oracle on the very inputs the GPU stage
saw, to that stage's own bar (exact for scales, codes, nibbles and the
dequant; relative Frobenius 1e-5 for H; the forward's rounding bound for y).
Inputs come from seeded generators; expected values from the oracle only."""
import numpy as np
import pytest
import torch

import datagen
from oracle import formats as F
from oracle import nvfp4 as N
import nvfp4_post_quantization_amd as nq

from _gpu import DEV, need_gpu, note, to_dev_bf16, host, to_host_bits, rel_frobenius, compare_sweep

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _forward_bound_ok(x_bits, w_hat_bits, s2x, y_bits):
    """y within bf16 rounding (2^-8 relative) plus k 2^-24 sum |x_hat||w_hat|
    of the oracle's exact product, element by element."""
    y = F.bf16_bits_to_f64(y_bits)
    ref = N.quantlinear_forward(x_bits, s2x, w_hat_bits)
    xh = F.bf16_bits_to_f64(N.fakequant(x_bits, s2x))
    mag = np.abs(xh) @ np.abs(F.bf16_bits_to_f64(w_hat_bits)).T
    bound = 2.0 ** -8 * np.abs(ref) + x_bits.shape[1] * 2.0 ** -24 * mag + 1e-38
    return np.all(np.abs(y - ref) <= bound) and np.linalg.norm(y - ref) <= 2.0 ** -8 * np.linalg.norm(ref)


def _layer(x_dev, w_bits):
    """One layer's calibration on the GPU, each stage checked; returns y."""
    x_bits = to_host_bits(x_dev)
    t, k = x_bits.shape
    w_dev = to_dev_bf16(w_bits)
    # a1: tensor scales of the weight and of the layer input
    s2w, amw = nq.compute_scale2(w_dev)
    s2x, amx = nq.compute_scale2(x_dev)
    for (s2, am), bits in (((s2w, amw), w_bits), ((s2x, amx), x_bits)):
        am_ref, s2_ref = N.tensor_scale(bits)
        assert float(host(am)[0]) == am_ref and float(host(s2)[0]) == s2_ref
    # a2: H in two chunks, amax fused; and the W4A4 form
    H = torch.zeros((k // 16, 16, 16), dtype=torch.float32, device=DEV)
    am_run = torch.zeros(1, dtype=torch.float32, device=DEV)
    for a, b in ((0, t // 2), (t // 2, t)):
        nq.hessian_accum(x_dev[a:b], H, am_run)
    h = host(H)
    assert rel_frobenius(h, N.hessian(x_bits)).max() <= 1e-5
    assert float(host(am_run)[0]) == N.tensor_scale(x_bits)[0]
    Hq = torch.zeros_like(H)
    nq.hessian_accum_fq(x_dev, s2x, Hq)
    assert rel_frobenius(host(Hq), N.hessian_fakequant(x_bits, float(host(s2x)[0]))).max() <= 1e-5
    # a3: the sweep under the GPU's H (the oracle sweeps with the same fp32 H)
    packed, codes, cost = nq.scale_sweep(w_dev, H, s2w, want_cost=True)
    s2w_f = float(host(s2w)[0])
    compare_sweep(w_bits, h, s2w_f, host(packed), host(codes), host(cost))
    # a5: w_hat, bit-exact
    w_hat = nq.dequant(packed, codes, s2w)
    w_hat_bits = to_host_bits(w_hat)
    assert np.array_equal(w_hat_bits, N.dequant(host(packed), host(codes), s2w_f))
    # the fake-quant forward gives the next layer's input
    y = nq.quantlinear_forward(x_dev, s2x, w_hat)
    assert _forward_bound_ok(x_bits, w_hat_bits, float(host(s2x)[0]), to_host_bits(y))
    return y


def test_two_layer_stack_calibration():
    note("two-layer stack calibration")
    rng = np.random.default_rng(2024)
    x = rng.laplace(0.0, 1.0, (4096, 1024))
    x[:, rng.choice(1024, 8, replace=False)] *= 40.0
    w1 = rng.normal(0.0, 0.02, (512, 1024)) + rng.laplace(0.0, 0.01, (512, 1024))
    w2 = rng.normal(0.0, 0.02, (256, 512)) + rng.laplace(0.0, 0.01, (256, 512))
    to_bits = lambda a: datagen.f32_to_bf16_bits(a.astype(np.float32))
    x1 = to_dev_bf16(to_bits(x))
    y1 = _layer(x1, to_bits(w1))
    assert y1.shape == (4096, 512)
    y2 = _layer(y1, to_bits(w2))
    assert y2.shape == (4096, 256)
    assert torch.isfinite(y2.float()).all()
