"""GPU parity: NVFP4 block fake QDQ (bit-exact) and the fake-quant
QuantLinear forward y = fakequant(x) w_hat^T (bf16 GEMM, fp32 accumulation)
against the oracle.

The forward's bar comes from its arithmetic: the output is rounded once to
bf16 (at most 2^-9 relative, 2^-8 allowed) and the fp32 accumulation of k
exact bf16 products in any order is off by at most k 2^-24 sum |x_hat||w_hat|;
every element must lie within the sum of the two, and the whole output
within 2^-8 relative Frobenius.
Inputs come from datagen; expected values from the oracle only."""
import numpy as np
import pytest
import torch

import datagen
from oracle import formats as F
from oracle import nvfp4 as N
import nvfp4_post_quantization_amd as nq

from _gpu import DEV, need_gpu, note, to_dev_bf16, to_dev_f32, host, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.fixture(params=["fast", "twofloat", "nudged", "exact"])
def path(request, monkeypatch):
    flag = {"fast": None, "twofloat": "2", "nudged": "3", "exact": "1"}[request.param]
    if flag is None:
        monkeypatch.delenv("NVFP4MI_FORCE_EXACT", raising=False)
    else:
        monkeypatch.setenv("NVFP4MI_FORCE_EXACT", flag)
    return request.param


def _dev(bits, ld=None):
    if ld is None:
        return to_dev_bf16(bits)
    full = np.zeros((bits.shape[0], ld), np.uint16)
    full[:, :bits.shape[1]] = bits
    return to_dev_bf16(full)[:, :bits.shape[1]]


@pytest.mark.parametrize("which", ["c1x", "c2x", "c3x", "c2w"])
def test_fakequant_tensors(path, which):
    note(f"fakequant {which} path={path}")
    w2, x2 = datagen.config2()
    bits = {"c1x": datagen.config1()[1], "c2x": x2, "c3x": datagen.config3()[:1024], "c2w": w2}[which]
    _, s2 = N.tensor_scale(bits)
    got = to_host_bits(nq.fakequant(to_dev_bf16(bits), to_dev_f32([s2])))
    assert np.array_equal(got, N.fakequant(bits, s2))


@pytest.mark.parametrize("rows,k,ld,ldo,factor", [(1, 16, None, None, 1.0), (333, 48, 56, 64, 1.0),
                                                  (65, 272, None, 280, 1 / 64), (100, 64, None, None, 4096.0),
                                                  (9, 1024, 1040, 1048, 1.0), (130, 3072, None, 3080, 1 / 64)])
def test_fakequant_ragged_strided_scales(rows, k, ld, ldo, factor):
    note(f"fakequant rows={rows} k={k} ld={ld} ldo={ldo} x{factor}")
    rng = np.random.default_rng(rows + k)
    bits = datagen.f32_to_bf16_bits(rng.laplace(0, 1, (rows, k)).astype(np.float32))
    s2 = float(np.float32(N.tensor_scale(bits)[1] * factor))
    out = None if ldo is None else torch.zeros((rows, ldo), dtype=torch.bfloat16, device=DEV)[:, :k]
    got = to_host_bits(nq.fakequant(_dev(bits, ld), to_dev_f32([s2]), out=out))
    assert np.array_equal(got, N.fakequant(bits, s2))


def _check_forward(x_bits, w_hat_bits, s2x, y_dev, rows=None):
    y = F.bf16_bits_to_f64(to_host_bits(y_dev))
    if rows is not None:
        y = y[rows]
        x_bits = x_bits[rows]
    ref = N.quantlinear_forward(x_bits, s2x, w_hat_bits)
    xh = F.bf16_bits_to_f64(N.fakequant(x_bits, s2x))
    mag = np.abs(xh) @ np.abs(F.bf16_bits_to_f64(w_hat_bits)).T
    k = x_bits.shape[1]
    bound = 2.0 ** -8 * np.abs(ref) + k * 2.0 ** -24 * mag + 1e-38
    assert np.all(np.abs(y - ref) <= bound), f"max excess {np.max(np.abs(y - ref) / bound):.3f}"
    assert np.linalg.norm(y - ref) <= 2.0 ** -8 * np.linalg.norm(ref)


@pytest.mark.parametrize("cfg", [1, 2])
def test_quantlinear_forward_configs(cfg):
    note(f"quantlinear forward config{cfg}")
    w, x = datagen.config1() if cfg == 1 else datagen.config2()
    _, s2w = N.tensor_scale(w)
    w_hat = N.fakequant(w, s2w)                      # a fake-quantized weight (max-based codes)
    _, s2x = N.tensor_scale(x)
    y = nq.quantlinear_forward(to_dev_bf16(x), to_dev_f32([s2x]), to_dev_bf16(w_hat))
    _check_forward(x, w_hat, s2x, y)


@pytest.mark.parametrize("t,k,o,ld,ldw,ldy", [(1, 16, 16, None, None, None), (37, 272, 48, 280, None, 56),
                                              (1000, 64, 264, None, 72, None), (5, 4096, 24, None, None, 32)])
def test_quantlinear_forward_ragged(t, k, o, ld, ldw, ldy):
    note(f"quantlinear t={t} k={k} o={o}")
    rng = np.random.default_rng(t * 3 + k + o)
    x = datagen.f32_to_bf16_bits(rng.laplace(0, 1, (t, k)).astype(np.float32))
    w = datagen.f32_to_bf16_bits(rng.normal(0, 0.02, (o, k)).astype(np.float32))
    w_hat = N.fakequant(w, N.tensor_scale(w)[1])
    _, s2x = N.tensor_scale(x)
    out = None if ldy is None else torch.zeros((t, ldy), dtype=torch.bfloat16, device=DEV)[:, :o]
    y = nq.quantlinear_forward(_dev(x, ld), to_dev_f32([s2x]), _dev(w_hat, ldw), out=out)
    _check_forward(x, w_hat, s2x, y)


def test_quantlinear_forward_full_chunk():
    """A 65536-token calibration chunk [65536, 4096] through the gate weight
    [12288, 4096], as the benchmark runs it: sampled rows against the oracle."""
    note("quantlinear forward full chunk x gate")
    w = datagen.config4_weights("gate")
    w_hat = N.fakequant(w, N.tensor_scale(w)[1])
    x = datagen.config4_chunk_torch(0, 0, DEV)
    xb = x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    s2x = max((N.tensor_scale(xb[r:r + 8192]) for r in range(0, xb.shape[0], 8192)), key=lambda t: t[0])[1]
    y = nq.quantlinear_forward(x, to_dev_f32([s2x]), to_dev_bf16(w_hat))
    rows = np.sort(np.random.default_rng(5).choice(xb.shape[0], 12, replace=False))
    _check_forward(xb, w_hat, s2x, y, rows=rows)
