"""GPU parity: Hessian-weighted E4M3 scale sweep against the float64 oracle.

Bar (per block): the chosen code equals the oracle's on >= 99.99% of blocks;
where it differs, the oracle's cost of the GPU's code is within 1e-5 relative
of the oracle minimum; the nibbles always equal the oracle's quantization at
the GPU's code, bit for bit; the fp32 cost output is within 1e-4 relative of
the oracle's cost of that code.  H and scale_2 are the same float32 values on
both sides (the oracle's H rounded to float32)."""
import numpy as np
import pytest
import torch

import datagen
from oracle import nvfp4 as N
from oracle import formats as F
import nvfp4_post_quantization_amd as nq

from _gpu import DEV, need_gpu, note, to_dev_bf16, to_dev_f32, host, compare_sweep

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


# The E2M1 decisions run on the certified fast quotients by default; the test
# hook forces the two-float quotient (2), the corrected two-float quotient (3)
# or the exact thresholds (1), so that every path meets the same parity bar.
@pytest.fixture(params=["fast", "twofloat", "nudged", "exact"])
def path(request, monkeypatch):
    flag = {"fast": None, "twofloat": "2", "nudged": "3", "exact": "1"}[request.param]
    if flag is None:
        monkeypatch.delenv("NVFP4MI_FORCE_EXACT", raising=False)
    else:
        monkeypatch.setenv("NVFP4MI_FORCE_EXACT", flag)
    return request.param


def gpu_sweep(w_bits, h32, s2, ld=None):
    rows, k = w_bits.shape
    if ld is None:
        w = to_dev_bf16(w_bits)
    else:
        full = np.zeros((rows, ld), np.uint16)
        full[:, :k] = w_bits
        w = to_dev_bf16(full)[:, :k]
    H = torch.from_numpy(np.ascontiguousarray(h32, dtype=np.float32)).to(DEV)
    packed, codes, cost = nq.scale_sweep(w, H, to_dev_f32([s2]), want_cost=True)
    return host(packed), host(codes), host(cost)


def check_sweep(w_bits, h32, s2, ld=None, max_mismatch_frac=1e-4):
    packed, codes, cost = gpu_sweep(w_bits, h32, s2, ld)
    n_mism = compare_sweep(w_bits, h32, s2, packed, codes, cost, max_mismatch_frac)
    return codes, n_mism


def _inputs_c1():
    w, x = datagen.config1()
    h = N.hessian(x).astype(np.float32)
    _, s2 = N.tensor_scale(w)
    return w, h, s2


def test_sweep_config1_full(path):
    note(f"sweep config1 ({path})")
    w, h, s2 = _inputs_c1()
    check_sweep(w, h, s2)


def test_sweep_config2_rows(path):
    note(f"sweep config2 sampled rows ({path})")
    w, x = datagen.config2()
    h = N.hessian(x).astype(np.float32)
    _, s2 = N.tensor_scale(w)                     # the tensor scale of the whole matrix
    rows = np.sort(np.random.default_rng(2).choice(w.shape[0], 192, replace=False))
    check_sweep(w[rows], h, s2)


@pytest.mark.parametrize("rows,k,ld", [(1, 16, None), (5, 48, None), (13, 32, 40), (4, 2048, 2056)])
def test_sweep_ragged(rows, k, ld, path):
    note(f"sweep rows={rows} k={k} ld={ld} ({path})")
    rng = np.random.default_rng(rows * 7 + k)
    w = datagen.f32_to_bf16_bits((rng.standard_normal((rows, k)) * 0.02).astype(np.float32))
    x = datagen.f32_to_bf16_bits(rng.laplace(0, 1, (300, k)).astype(np.float32))
    h = N.hessian(x).astype(np.float32)
    _, s2 = N.tensor_scale(w)
    check_sweep(w, h, s2, ld)


def test_sweep_special_hessians():
    note("sweep special Hessians")
    rng = np.random.default_rng(3)
    w = datagen.f32_to_bf16_bits((rng.laplace(0, 0.02, (24, 64))).astype(np.float32))
    _, s2 = N.tensor_scale(w)
    eye = np.broadcast_to(np.eye(16, dtype=np.float32), (4, 16, 16)).copy()
    check_sweep(w, eye, s2)
    zero = np.zeros((4, 16, 16), np.float32)
    codes, _ = check_sweep(w, zero, s2)
    assert (codes == 0).all()                      # every cost is 0: lowest code wins
    # singular H: channel 5 never active
    x = rng.laplace(0, 1, (64, 64))
    x[:, 5] = 0.0
    hs = N.hessian(datagen.f32_to_bf16_bits(x.astype(np.float32))).astype(np.float32)
    check_sweep(w, hs, s2)


def _scaled_correlation(c, rng, groups):
    """H_g = D C D with C unit-diagonal and D spanning 1 .. 40 (outlier channels)."""
    d = np.exp(rng.uniform(0.0, np.log(40.0), (groups, 16)))
    return (d[:, :, None] * c * d[:, None, :]).astype(np.float32)


@pytest.mark.parametrize("kind,rho", [("equi", 0.05), ("equi", 0.059), ("equi", 0.07), ("equi", 0.5),
                                      ("signed", 0.85), ("signed", 0.95)])
def test_sweep_correlated_hessians(kind, rho, path):
    """Row sums of |C_ij| (j != i) of 15 rho ("equi") or exactly rho with random
    signs ("signed"), below and above 0.9: the sweep's diagonal screen is on
    for the first and off for the others; every case meets the oracle bar on
    every E2M1 decision path (each mode has its own step loop)."""
    note(f"sweep correlated H {kind} {rho}")
    rng = np.random.default_rng(int(rho * 1000) + (7 if kind == "signed" else 0))
    groups = 8
    if kind == "equi":
        c = np.broadcast_to((1.0 - rho) * np.eye(16) + rho * np.ones((16, 16)), (groups, 16, 16))
    else:
        a = rng.uniform(0.1, 1.0, (groups, 16, 16)) * rng.choice([-1.0, 1.0], (groups, 16, 16))
        a = np.triu(a, 1)
        a = a + np.swapaxes(a, 1, 2)
        a *= rho / np.abs(a).sum(axis=2).max(axis=1)[:, None, None]
        c = np.eye(16) + a
    h = _scaled_correlation(c, rng, groups)
    w = datagen.f32_to_bf16_bits(rng.laplace(0.0, 0.02, (320, groups * 16)).astype(np.float32))
    _, s2 = N.tensor_scale(w)
    check_sweep(w, h, s2)


def test_sweep_exact_and_zero_blocks(path):
    note(f"sweep exact/zero blocks ({path})")
    s2 = 2.0 ** -10
    rng = np.random.default_rng(4)
    x = datagen.f32_to_bf16_bits(rng.standard_normal((128, 32)).astype(np.float32))
    h = N.hessian(x).astype(np.float32)
    qv = np.array([6, -4, 3, 0.5, -1.5, 2, 1, 0, -6, 4, -3, 0.5, 1.5, -2, -1, 6.0])
    w = np.zeros((4, 32))
    w[0, :16] = qv * float(F.E4M3_VALUES[0x3B]) * s2
    w[1, 16:] = qv * float(F.E4M3_VALUES[0x01]) * s2
    w[2, :] = -0.0
    w[3, :16] = 1e6
    wb = datagen.f32_to_bf16_bits(w.astype(np.float32))
    codes, _ = check_sweep(wb, h, s2)
    assert codes[2, 0] == 0 and codes[2, 1] == 0


def test_sweep_short_mantissa_scale_ties(path):
    """A power-of-two scale_2 with blocks built on E2M1 midpoints: the sweep's
    quantization must break every tie exactly as the oracle does."""
    note(f"sweep dyadic scale_2 with ties ({path})")
    s2 = 2.0 ** -15
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    rng = np.random.default_rng(8)
    rows = []
    for r in range(32):
        code = int(rng.integers(8, 120))
        d = float(F.E4M3_VALUES[code]) * s2
        rows.append(np.concatenate([mids, -mids[::-1]]) * d * rng.choice([1.0, 2.0, 0.5], 16))
    w = datagen.f32_to_bf16_bits(np.array(rows).astype(np.float32))
    x = datagen.f32_to_bf16_bits(rng.laplace(0, 1, (256, 16)).astype(np.float32))
    h = N.hessian(x).astype(np.float32)
    check_sweep(w, h, s2)


@pytest.mark.parametrize("s2", [2.0 ** -128, 1e-30])
def test_sweep_extreme_scales(s2, path):
    """Tiny tensor scales with weights up to 1e12: quotients w/d overflow FP32
    for the large codes.  Costs of most codes then agree to far below FP32
    resolution, so codes may differ from the float64 argmin, but every
    difference must be a near-tie and every nibble exact at the GPU's code."""
    note(f"sweep extreme scale_2={s2} ({path})")
    rng = np.random.default_rng(12)
    mag = np.exp(rng.uniform(np.log(1e-38), np.log(1e12), (24, 64)))
    w = datagen.f32_to_bf16_bits((mag * rng.choice([-1.0, 1.0], (24, 64))).astype(np.float32))
    x = datagen.f32_to_bf16_bits(rng.standard_normal((300, 64)).astype(np.float32))
    h = N.hessian(x).astype(np.float32)
    check_sweep(w, h, float(np.float32(s2)), max_mismatch_frac=1.0)
