"""Pins of the oracle's NVFP4 steps (CPU only).

Tensor scale: the closed form RN_f32(amax/2688) checked exhaustively with
exact rationals.  Hessian: per-token brute force, symmetry, PSD, trace,
additivity, rank 1.  Sweep: exact-rational brute force over all 127 codes,
an independent MSE minimiser for H = I, exactly representable blocks, zero
blocks, and the max-based code as an upper bound.  Quantizer/dequant:
closed-form properties and torch's float8_e4m3fn decode.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import datagen
import oracle
from oracle import formats as F
from oracle import nvfp4 as N

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def _nearest_f32(q: Fraction) -> float:
    """Round a positive rational to float32, nearest with ties to even, by brute force."""
    f = np.float32(float(q))
    cands = [np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(np.inf))]
    best = None
    for c in cands:
        dist = abs(Fraction(float(c)) - q)
        even = (np.array(c, dtype=np.float32).view(np.uint32) & 1) == 0
        if best is None or dist < best[0] or (dist == best[0] and even):
            best = (dist, float(c))
    return best[1]


def _exact_quant(w: Fraction, d: Fraction):
    """Brute force E2M1 quantization of one element at block scale d: (nibble, wq)."""
    if d == 0:
        return (8 if w < 0 else 0), Fraction(0)
    y = abs(w) / d
    best, bd = None, None
    for i, g in enumerate(GRID):
        dist = abs(y - g)
        if best is None or dist < bd or (dist == bd and i % 2 == 0):
            best, bd = i, dist
    sgn = -1 if w < 0 else 1
    return ((8 if w < 0 else 0) | best), sgn * GRID[best] * d


def test_tensor_scale_is_correctly_rounded_quotient(page_constants):
    """The page's double-precision amax/6/448 stored as FP32 equals the correctly
    rounded FP32 value of amax/2688 for every positive finite bf16 amax."""
    k = page_constants["e2m1_max"][0] * page_constants["e4m3_max"][0]
    assert k == 2688.0
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    amax = F.bf16_bits_to_f64(bits)
    s2 = (amax / 6.0 / 448.0).astype(np.float32)
    step = 37          # every 37th value exactly (all 32639 take ~10 s)
    for a, s in zip(amax[::step], s2[::step]):
        assert float(s) == _nearest_f32(Fraction(float(a)) / 2688)
    # the oracle entry point uses that formula
    x = np.array([[0x4000, 0xC2C8, 0x0001]], dtype=np.uint16)      # 2, -100, tiny
    am, sc = N.tensor_scale(x)
    assert am == 100.0 and sc == float(np.float32(100.0 / 2688.0))
    assert N.tensor_scale(np.zeros((2, 16), np.uint16)) == (0.0, 0.0)


def test_tensor_scale_order_matters():
    """A sequential float32 amax/6/448 is NOT the same rounding: the oracle must
    not be that (guards against a plausible mistake)."""
    amax = F.bf16_bits_to_f64(np.arange(0x3F80, 0x4080, dtype=np.uint16)).astype(np.float32)
    seq = (amax / np.float32(6.0)) / np.float32(448.0)
    ref = (amax.astype(np.float64) / 2688.0).astype(np.float32)
    assert (seq != ref).any()


def test_hessian_brute_force_and_invariants():
    rng = np.random.default_rng(7)
    x = datagen.f32_to_bf16_bits(rng.standard_normal((5, 32)).astype(np.float32))
    h = N.hessian(x)
    xv = F.bf16_bits_to_f64(x)
    for g in range(2):
        for i in range(16):
            for j in range(16):
                s = sum(Fraction(float(xv[t, 16 * g + i])) * Fraction(float(xv[t, 16 * g + j])) for t in range(5))
                assert h[g, i, j] == float(s)
    assert np.array_equal(h, np.transpose(h, (0, 2, 1)))
    for g in range(2):
        assert np.linalg.eigvalsh(h[g]).min() >= -1e-12 * np.trace(h[g])
        assert np.isclose(np.trace(h[g]), np.sum(xv[:, 16 * g:16 * g + 16] ** 2), rtol=1e-14)
    # additivity over token chunks and rank 1 for a single token
    x2 = datagen.f32_to_bf16_bits(rng.standard_normal((7, 32)).astype(np.float32))
    assert np.allclose(N.hessian(np.concatenate([x, x2])), N.hessian(x) + N.hessian(x2), rtol=1e-14, atol=0)
    assert np.allclose(N.hessian(x2, h_init=h), h + N.hessian(x2), rtol=1e-14, atol=0)
    h1 = N.hessian(x[:1])
    assert np.linalg.matrix_rank(h1[0]) == 1


def _exact_sweep_block(w, hg, s2):
    """Exact-rational brute force of one block: (best code, exact costs)."""
    wf = [Fraction(float(v)) for v in w]
    hf = [[Fraction(float(hg[i, j])) for j in range(16)] for i in range(16)]
    costs = []
    for c in range(127):
        d = Fraction(float(np.float32(float(F.E4M3_VALUES[c]) * s2)))
        e = []
        for v in wf:
            _, q = _exact_quant(v, d)
            e.append(v - q)
        cost = sum(e[i] * hf[i][j] * e[j] for i in range(16) for j in range(16))
        costs.append(cost)
    m = min(costs)
    return costs.index(m), costs


def test_sweep_matches_exact_rational_brute_force():
    w_bits, x_bits = datagen.config1()
    h = N.hessian(x_bits)
    _, s2 = N.tensor_scale(w_bits)
    rows = [0, 5, 17, 40]
    sub = w_bits[rows, :64]                       # 4 rows x 4 groups = 16 blocks
    codes, packed, best = N.scale_sweep(sub, h[:4], s2)
    costs_all = N.sweep_costs(sub, h[:4], s2)
    wv = F.bf16_bits_to_f64(sub)
    for r in range(len(rows)):
        for g in range(4):
            blk = wv[r, 16 * g:16 * g + 16]
            c_exact, costs = _exact_sweep_block(blk, h[g], s2)
            assert codes[r, g] == c_exact
            for c in range(0, 127, 9):
                ex = float(costs[c])
                assert abs(costs_all[r, g, c] - ex) <= 1e-12 * max(ex, 1e-300)
            d = Fraction(float(np.float32(float(F.E4M3_VALUES[c_exact]) * s2)))
            nib = [_exact_quant(Fraction(float(v)), d)[0] for v in blk]
            assert F.unpack_nibbles(packed[r, 8 * g:8 * g + 8]).tolist() == nib


def test_sweep_identity_hessian_is_mse_minimiser():
    """With H = I the sweep must pick the code with the least squared error; the
    squared errors here come from an independent nearest-value search."""
    rng = np.random.default_rng(11)
    w_bits = datagen.f32_to_bf16_bits((rng.laplace(0, 0.02, (6, 32))).astype(np.float32))
    _, s2 = N.tensor_scale(w_bits)
    h = np.broadcast_to(np.eye(16), (2, 16, 16))
    codes, _, _ = N.scale_sweep(w_bits, h, s2)
    wv = F.bf16_bits_to_f64(w_bits)
    for r in range(6):
        for g in range(2):
            blk = wv[r, 16 * g:16 * g + 16]
            errs = []
            for c in range(127):
                d = float(np.float32(float(F.E4M3_VALUES[c]) * s2))
                cand = np.array([0, .5, 1, 1.5, 2, 3, 4, 6]) * d
                err = 0.0
                for v in blk:
                    dist = np.abs(abs(v) - cand)
                    err += float(dist.min()) ** 2
                errs.append(err)
            errs = np.array(errs)
            # the oracle's choice attains the minimum squared error (up to fp64 noise)
            assert errs[codes[r, g]] <= errs.min() * (1 + 1e-12) + 1e-300


def test_sweep_special_blocks():
    s2 = 2.0 ** -10                     # dyadic, so e2m1 * d is bf16-exact
    rng = np.random.default_rng(12)
    xb = datagen.f32_to_bf16_bits(rng.standard_normal((64, 32)).astype(np.float32))
    h = N.hessian(xb)
    # an exactly representable block costs 0 at its code; a zero block picks code 0
    c0 = 0x3B
    d = float(np.float32(float(F.E4M3_VALUES[c0]) * s2))
    q = np.array([6, -4, 3, 0.5, -1.5, 2, 1, 0, -6, 4, -3, 0.5, 1.5, -2, -1, 6]) * d
    w = np.zeros((2, 32))
    w[0, :16] = q
    w_bits = datagen.f32_to_bf16_bits(w.astype(np.float32))
    assert np.array_equal(F.bf16_bits_to_f64(w_bits)[0, :16], q), "test block must be bf16-exact"
    codes, packed, best = N.scale_sweep(w_bits, h, s2)
    assert best[0, 0] == 0.0
    assert codes[1, 0] == 0 and codes[1, 1] == 0 and codes[0, 1] == 0
    assert (packed[1] == 0).all()
    # the max-based code is one of the candidates, so the sweep can only do better
    wb, _ = datagen.config1()
    hx = N.hessian(datagen.config1()[1])
    _, s2w = N.tensor_scale(wb)
    codes, _, best = N.scale_sweep(wb[:8], hx, s2w)
    wv = F.bf16_bits_to_f64(wb[:8]).reshape(8, 16, 16)
    mc = N.max_code(np.abs(wv).max(axis=2), s2w)
    _, wq = N.quantize_at_code(wv, mc, s2w)
    cmax = N.block_cost(wv, wq, hx[None])
    assert (best <= cmax * (1 + 1e-12)).all()
    assert (codes != mc).any()     # the Hessian weighting actually changes some choices


def test_dynamic_quantizer_properties(page_constants):
    x = datagen.config3(tokens=64, k=256)
    _, s2 = N.tensor_scale(x)
    packed, codes = N.quantize_dynamic(x, s2)
    assert packed.shape == (64, 128) and codes.shape == (64, 16)
    bits = (packed.size * 8 + codes.size * 8) / x.size + 32 / x.size
    assert abs(bits - page_constants["bits_per_element_nvfp4"][0]) < 0.01
    xv = F.bf16_bits_to_f64(x).reshape(64, 16, 16)
    nib = F.unpack_nibbles(packed).reshape(64, 16, 16)
    d = N.block_scale(codes, s2)
    # the block max always lands on magnitude 6 for normal E4M3 codes
    imax = np.argmax(np.abs(xv), axis=2)
    top = np.take_along_axis(nib, imax[..., None], axis=2)[..., 0] & 7
    normal = codes >= 8
    assert (top[normal] == 7).all()
    # every unsaturated element is within half a grid step of its value
    q = np.abs(F.e2m1_decode(nib)) * d[..., None]
    a = np.abs(xv)
    step = np.where(a < 2 * d[..., None], 0.5, np.where(a < 4 * d[..., None], 1.0, 2.0)) * d[..., None]
    assert (np.abs(a - q) <= step / 2 + 1e-300).all()
    # exactly representable blocks round-trip (dyadic scale_2 keeps them bf16-exact)
    s2d = 2.0 ** -8
    qv = np.array([6, -4, 3, 0.5, -1.5, 2, 1, 0, -6, 4, -3, 0.5, 1.5, -2, -1, 6.0])
    for code in (0x01, 0x07, 0x08, 0x40, 0x5D, 0x7E):
        d0 = float(F.E4M3_VALUES[code]) * s2d
        xb = datagen.f32_to_bf16_bits((qv * d0).astype(np.float32))[None]
        assert np.array_equal(F.bf16_bits_to_f64(xb)[0], qv * d0)
        p2, c2 = N.quantize_dynamic(xb, s2d)
        assert c2[0, 0] == code
        assert np.array_equal(F.e2m1_decode(F.unpack_nibbles(p2)[0]) * d0, qv * d0)


def test_dynamic_quantizer_small_block_raised_to_code_one():
    s2 = float(np.float32(1000.0 / 2688))
    x = np.zeros((1, 32))
    x[0, 0] = 1000.0
    x[0, 16] = 1e-6
    xb = datagen.f32_to_bf16_bits(x.astype(np.float32))
    _, codes = N.quantize_dynamic(xb, s2)
    assert codes.tolist() == [[0x7E, 0x01]]
    _, codes0 = N.quantize_dynamic(np.zeros((1, 16), np.uint16), 0.0)
    assert codes0.tolist() == [[0]]


def test_dequant_chain_against_torch_decode():
    x = datagen.config3(tokens=32, k=128)
    _, s2 = N.tensor_scale(x)
    packed, codes = N.quantize_dynamic(x, s2)
    out = N.dequant(packed, codes, s2)
    sc = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32)
    d = sc * torch.tensor(s2, dtype=torch.float32)                     # DQ1 in FP32
    nib = F.unpack_nibbles(packed).astype(np.int64)
    mag = torch.tensor([0, .5, 1, 1.5, 2, 3, 4, 6], dtype=torch.float32)[torch.from_numpy(nib & 7)]
    val = torch.where(torch.from_numpy((nib >> 3) == 1), -mag, mag)
    y = (val.view(32, 8, 16) * d[..., None]).reshape(32, 128)          # DQ2 in FP32
    ref = y.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, ref)


def test_hessian_fakequant_identity_and_zero():
    """W4A4 Hessian variant: an input that the dynamic quantizer reproduces
    exactly (every element e2m1 * d at its block's own max-based code) gives
    the plain Hessian; a zero tensor scale quantizes everything to zero."""
    rng = np.random.default_rng(31)
    s2 = 2.0 ** -8
    rows = []
    for t in range(40):
        code = int(rng.integers(8, 120))
        d = float(F.E4M3_VALUES[code]) * s2
        q = rng.choice(F.E2M1_MAGNITUDES, 32) * rng.choice([-1.0, 1.0], 32)
        q[0], q[16] = 6.0, -6.0                       # each block's max is 6 d: the block keeps this code
        rows.append(q * d)
    x = datagen.f32_to_bf16_bits(np.array(rows).astype(np.float32))
    assert np.array_equal(F.bf16_bits_to_f64(x), np.array(rows)), "test inputs must be bf16-exact"
    assert np.array_equal(N.hessian_fakequant(x, s2), N.hessian(x))
    y = datagen.f32_to_bf16_bits(rng.standard_normal((40, 32)).astype(np.float32))
    assert np.array_equal(N.hessian_fakequant(y, 0.0), np.zeros((2, 16, 16)))
    # a generic input differs from the plain Hessian, and stays PSD and symmetric
    _, s2y = N.tensor_scale(y)
    hf = N.hessian_fakequant(y, s2y)
    assert not np.array_equal(hf, N.hessian(y))
    assert np.array_equal(hf, hf.transpose(0, 2, 1))
    assert np.min(np.linalg.eigvalsh(hf)) >= -1e-9 * np.max(np.abs(hf))


def test_fakequant_identity_bound_and_zero_scale():
    """Fake QDQ of an activation: identity on values the quantizer reproduces,
    error at most half a step d/2 per element below saturation, all zero at
    scale_2 = 0."""
    rng = np.random.default_rng(41)
    s2 = 2.0 ** -9
    rows = []
    for _ in range(24):
        code = int(rng.integers(16, 110))
        d = float(F.E4M3_VALUES[code]) * s2
        q = rng.choice(F.E2M1_MAGNITUDES, 32) * rng.choice([-1.0, 1.0], 32)
        q[3], q[20] = -6.0, 6.0
        rows.append(q * d)
    x = datagen.f32_to_bf16_bits(np.array(rows).astype(np.float32))
    assert np.array_equal(N.fakequant(x, s2), x)
    y = datagen.config1()[1]
    _, s2y = N.tensor_scale(y)
    yv = F.bf16_bits_to_f64(y).reshape(-1, 16)
    fq = F.bf16_bits_to_f64(N.fakequant(y, s2y)).reshape(-1, 16)
    d = N.block_scale(N.max_code(np.max(np.abs(yv), axis=1), s2y), s2y)[:, None]
    # E2M1 spacing is at most 2 d below 6 d: the error is at most d, plus the bf16 rounding
    assert np.all(np.abs(fq - yv) <= d * (1 + 2.0 ** -7) + 2.0 ** -8 * np.abs(yv))
    assert not np.any(F.bf16_bits_to_f64(N.fakequant(y, 0.0)))


def test_quantlinear_forward_equals_integer_matmul():
    """With inputs the quantizers reproduce exactly (small integers times a
    power of two, block max 6 d), the forward is an exact integer matmul."""
    rng = np.random.default_rng(42)
    s2 = 2.0 ** -10
    code = 0x48                          # e4m3 value 16 -> d = 2^-6; every block holds E2M1 levels times d
    d = float(F.E4M3_VALUES[code]) * s2
    lv = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    xi = rng.integers(0, 8, (40, 64)); xs = rng.choice([-1, 1], (40, 64))
    xi[:, ::16] = 7                      # block max 6 d: the block keeps code 0x48
    x_val = xs * lv[xi] * d
    x = datagen.f32_to_bf16_bits(x_val.astype(np.float32))
    w_int = rng.integers(-8, 9, (24, 64))
    w = datagen.f32_to_bf16_bits((w_int * 2.0 ** -5).astype(np.float32))
    y = N.quantlinear_forward(x, s2, w)
    # exact: x = (2 * xs * lv) * d / 2 with 2*lv integer; y = sum x w
    xi2 = (xs * (2 * lv[xi])).astype(np.int64)
    y_int = xi2 @ w_int.T                # in units of d/2 * 2^-5
    assert np.array_equal(y, y_int * (d / 2) * 2.0 ** -5)
