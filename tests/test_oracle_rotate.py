"""Pins of the oracle's block-Hadamard rotation (CPU only).

The rotation of "FP4量化技术概述" §3.1 is checked against exact rational
arithmetic, scipy's Hadamard matrix, and the algebraic identities the rotated
sweep relies on (R R = I, H' = R^T H R is the Hessian of X R, and the
Hessian-weighted cost is the same in both bases)."""
from fractions import Fraction

import numpy as np
import scipy.linalg

import datagen
from oracle import formats as F
from oracle import nvfp4 as N
from oracle import rotate as RT


def _bf16_value(p: int) -> Fraction:
    return Fraction(float(np.array(np.uint32(p) << 16, np.uint32).view(np.float32)))


def _nearest_bf16(v: Fraction) -> int:
    """bf16 pattern nearest to v (ties to the even pattern; at or beyond the
    midpoint above the largest finite value, infinity), found by walking the
    patterns around a float32 guess with exact comparisons."""
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    p = int(np.array(np.float32(float(a))).view(np.uint32) >> 16)
    p = min(p, 0x7F7F)
    while p > 0 and _bf16_value(p) > a:
        p -= 1
    while p < 0x7F7F and _bf16_value(p + 1) <= a:
        p += 1
    if p == 0x7F7F:
        top = _bf16_value(0x7F7F)
        mid = top + (top - _bf16_value(0x7F7E)) / 2
        return sign | (0x7F80 if a >= mid else 0x7F7F)
    dl, dh = a - _bf16_value(p), _bf16_value(p + 1) - a
    return sign | (p if (dl < dh or (dl == dh and p % 2 == 0)) else p + 1)


def test_f64_to_bf16_rne_against_brute_force():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        np.exp(rng.uniform(-90, 88, 400)) * rng.choice([-1.0, 1.0], 400),
        (1.0 + (2 * rng.integers(0, 128, 50) + 1) * 2.0 ** -8) * 2.0 ** rng.integers(-120, 120, 50),  # ties
        np.array([2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 2.0 ** -126 * (1 - 2.0 ** -9), 0.0, -0.0]),
    ])
    got = F.f64_to_bf16_rne(x)
    want = [_nearest_bf16(Fraction(float(v))) | (0x8000 if np.signbit(v) else 0) for v in x]
    assert list(got) == want


def test_hadamard16_is_sylvester():
    h = RT.hadamard16()
    assert np.array_equal(h, scipy.linalg.hadamard(16).astype(np.float64))
    assert np.array_equal(h, h.T)
    assert np.array_equal(h @ h, 16.0 * np.eye(16))


def test_rotate_blocks_equals_exact_product():
    """Values spanning a moderate range: the butterfly is exact, so the result
    is the exact (x H16)/4 rounded once."""
    rng = np.random.default_rng(4)
    x = datagen.f32_to_bf16_bits((rng.laplace(0, 1, (12, 64)) * np.exp(rng.uniform(-6, 6, (12, 64)))).astype(np.float32))
    got = RT.rotate_blocks(x)
    xv = F.bf16_bits_to_f64(x)
    h = RT.hadamard16().astype(np.int64)
    for r in range(x.shape[0]):
        for g in range(4):
            blk = [Fraction(float(v)) for v in xv[r, 16 * g:16 * g + 16]]
            for i in range(16):
                exact = sum(blk[j] * int(h[j, i]) for j in range(16)) / 4
                g_bits = int(got[r, 16 * g + i])
                if exact == 0:
                    assert g_bits in (0, 0x8000)                  # the sign of an exact zero is free
                else:
                    assert g_bits == _nearest_bf16(exact), (r, g, i)


def test_rotate_twice_is_identity_up_to_rounding():
    w = datagen.config1()[0]
    rr = F.bf16_bits_to_f64(RT.rotate_blocks(RT.rotate_blocks(w)))
    x = F.bf16_bits_to_f64(w)
    err = np.linalg.norm((rr - x).reshape(-1, 16), axis=1)
    nrm = np.linalg.norm(x.reshape(-1, 16), axis=1)
    assert np.all(err <= 2.0 ** -7 * nrm)


def test_rotated_hessian_is_hessian_of_rotated_input():
    x = datagen.config1()[1]
    h = N.hessian(x)
    hp = RT.rotate_hessian(h)
    xv = F.bf16_bits_to_f64(x)
    r = RT.hadamard16() / 4.0
    xr = (xv.reshape(xv.shape[0], -1, 16) @ r).reshape(xv.shape)     # exact-ish X R, no bf16 rounding
    g = xr.shape[1] // 16
    h_direct = np.einsum("tgi,tgj->gij", xr.reshape(-1, g, 16), xr.reshape(-1, g, 16))
    assert np.allclose(hp, h_direct, rtol=1e-6, atol=1e-9 * np.abs(h_direct).max())
    assert np.allclose(np.trace(hp, axis1=1, axis2=2), np.trace(h, axis1=1, axis2=2), rtol=1e-6)
    assert np.array_equal(hp, hp.transpose(0, 2, 1))


def test_cost_is_the_same_in_both_bases():
    """(w' - q')^T R^T H R (w' - q') == (w - q)^T H (w - q) with w = w' R^T,
    q = q' R^T: the rotated sweep's cost is the error of the un-rotated
    dequantized weights."""
    w, x = datagen.config1()
    h = N.hessian(x)
    wr_bits = RT.rotate_blocks(w)
    wr = F.bf16_bits_to_f64(wr_bits)
    _, s2 = N.tensor_scale(wr_bits)
    rows, k = wr.shape
    codes = N.max_code(np.max(np.abs(wr.reshape(rows, -1, 16)), axis=2), s2)
    _, qr = N.quantize_at_code(wr.reshape(rows, -1, 16), codes, s2)
    r = RT.hadamard16() / 4.0
    hp = np.einsum("ai,gab,bj->gij", r, h, r)                         # unrounded H'
    e_rot = wr.reshape(rows, -1, 16) - qr
    c_rot = np.einsum("rgi,gij,rgj->rg", e_rot, hp, e_rot)
    e_orig = e_rot @ r.T                                                # (w - q) = (w' - q') R^T
    c_orig = np.einsum("rgi,gij,rgj->rg", e_orig, h, e_orig)
    assert np.allclose(c_rot, c_orig, rtol=1e-9, atol=1e-12 * np.abs(c_orig).max())
