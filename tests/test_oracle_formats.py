"""Pins of the oracle's number formats (CPU only).

Each check ties the oracle to something other than itself: the constants the
pages print (tests/golden/page_constants.txt), exact-rational brute force, or
torch's own float8_e4m3fn / bfloat16 casts.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F


def _nearest_grid_index(y: Fraction) -> int:
    """Brute force: index of the E2M1 magnitude nearest to y >= 0, ties to even index."""
    grid = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
            Fraction(3), Fraction(4), Fraction(6)]
    best, bestd = None, None
    for i, g in enumerate(grid):
        dd = abs(y - g)
        if best is None or dd < bestd or (dd == bestd and i % 2 == 0):
            best, bestd = i, dd
    return best


def test_e2m1_value_set_matches_page(page_constants):
    pos = page_constants["e2m1_positive"]
    assert list(F.E2M1_MAGNITUDES[1:]) == pos
    assert F.E2M1_MAGNITUDES[0] == 0.0
    assert F.E2M1_MAGNITUDES.max() == page_constants["e2m1_max"][0]
    dec = F.e2m1_decode(np.arange(16))
    assert list(dec[:8]) == [0.0] + pos
    assert list(-dec[8:]) == [0.0] + pos
    assert np.signbit(dec[8]) and not np.signbit(dec[0])


def test_e2m1_roundtrip_all_codes():
    rng = np.random.default_rng(1)
    ds = np.concatenate([[1.0, 2.0 ** -20, 3.0], F.f32(rng.uniform(1e-4, 10, 50))])
    for d in ds:
        for c in range(16):
            x = F.e2m1_decode(c) * d
            assert F.e2m1_encode(x, d) == c, (c, d)


def test_e2m1_encode_matches_exact_brute_force():
    rng = np.random.default_rng(2)
    xs = oracle.bf16_bits_to_f64(rng.integers(0, 0x7F00, 3000).astype(np.uint16))
    xs = xs * np.where(rng.random(xs.size) < 0.5, -1.0, 1.0)
    ds = F.f32(np.exp(rng.uniform(-12, 6, xs.size)))
    # make a third of the cases exact midpoints m*d (hard ties)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    sel = rng.random(xs.size) < 0.33
    pick = mids[rng.integers(0, 7, xs.size)]
    xs = np.where(sel, pick * ds * np.sign(xs + 0.5), xs)
    got = F.e2m1_encode(xs, ds)
    for x, d, g in zip(xs, ds, got):
        y = abs(Fraction(float(x))) / Fraction(float(d))
        want = (8 if np.signbit(x) else 0) | _nearest_grid_index(y)
        assert int(g) == want, (x, d, g, want)


def test_e2m1_ties_go_to_even_and_zero_scale():
    # the seven midpoints at d = 1 land on the even-index neighbour
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0, 2, 2, 4, 4, 6, 6]
    assert list(F.e2m1_encode(np.array(mids), 1.0)) == want
    assert list(F.e2m1_encode(-np.array(mids), 1.0)) == [8 | w for w in want]
    assert F.e2m1_encode(np.array([7.0, 1e9]), 1.0).tolist() == [7, 7]
    # zero block scale: sign only
    assert F.e2m1_encode(np.array([3.0, -3.0, 0.0, -0.0]), 0.0).tolist() == [0, 8, 0, 8]


def test_pack_order_low_nibble_first(page_constants):
    nib = np.array([[1, 2, 3, 4]], dtype=np.uint8)
    p = F.pack_nibbles(nib)
    assert p.tolist() == [[0x21, 0x43]]
    assert nib.shape[1] / p.shape[1] == page_constants["fp4_per_byte"][0]
    assert (F.unpack_nibbles(p) == nib).all()


def test_e4m3_table_against_torch_and_page(page_constants):
    vals = F.E4M3_VALUES
    assert np.isnan(vals[127]) and np.isnan(vals[255])
    assert np.nanmax(vals) == page_constants["e4m3_max"][0]
    nonneg = vals[:128]
    assert len(nonneg) == page_constants["e4m3_scale_codes"][0]
    tv = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    fin = ~np.isnan(tv)
    assert np.array_equal(np.isnan(vals), ~fin)
    assert np.array_equal(vals[fin], tv[fin])
    assert np.all(np.diff(vals[:127]) > 0)


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(3)
    v = np.concatenate([
        F.f32(np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 20000))),
        F.E4M3_VALUES[:127],
        0.5 * (F.E4M3_VALUES[:126] + F.E4M3_VALUES[1:127]),     # exact midpoints
    ])
    ours = F.e4m3_encode_ratio(v, 1.0)
    theirs = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_e4m3_encode_ratio_exact_brute_force():
    rng = np.random.default_rng(4)
    fin = [Fraction(float(v)) for v in F.E4M3_VALUES[:127]]
    nums = oracle.bf16_bits_to_f64(rng.integers(0, 0x7F00, 400).astype(np.uint16))
    dens = 6.0 * F.f32(np.exp(rng.uniform(-10, 2, 400)))
    got = F.e4m3_encode_ratio(nums, dens)
    for n, dd, g in zip(nums, dens, got):
        y = Fraction(float(n)) / Fraction(float(dd))
        best, bd = None, None
        for i, fv in enumerate(fin):
            dist = abs(y - fv)
            if best is None or dist < bd or (dist == bd and i % 2 == 0):
                best, bd = i, dist
        assert int(g) == best
    assert F.e4m3_encode_ratio(np.array([1e30, 0.0, 5.0]), np.array([1.0, 0.0, 0.0])).tolist() == [0x7E, 0, 0x7E]


def test_e8m0_and_bf16_helpers():
    assert F.e8m0_value(127) == 1.0 and F.e8m0_value(130) == 8.0 and F.e8m0_value(120) == 2.0 ** -7
    assert np.isnan(F.e8m0_value(255))
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(5000) * np.exp(rng.uniform(-30, 30, 5000))).astype(np.float32)
    ours = F.f64_to_bf16_bits(x.astype(np.float64))
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    back = F.bf16_bits_to_f64(theirs)
    assert np.array_equal(back, torch.from_numpy(theirs.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy())
