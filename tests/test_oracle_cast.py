"""Pins of the oracle's MXFP4 -> NVFP4 cast (CPU only).

The pages fix: the tensor scale 2^(k_max-8) (global_amax = 6*448*2^(k_max-8)),
exact dequantization of every in-window block (nibbles move unchanged), the
window k_max - k_j <= 17, the data-derived fallback outside it, one scale_2
per gate/up pair, and that the scale bytes double.
"""
from fractions import Fraction

import numpy as np

import datagen
from oracle import formats as F
from oracle import mxcast as M


def _small_case(seed=0):
    return datagen.config5(seed=seed, experts=3, rows=16, k=256, forced_frac=0.05)


def test_cast_lossless_in_window_and_scale(page_constants):
    packed, e8, forced = _small_case()
    out, codes, s2, fb = M.mxfp4_to_nvfp4(packed, e8)
    win = page_constants["cast_window"][0]
    off = page_constants["cast_exponent_offset"][0]
    for g in range(packed.shape[0]):
        kj = e8[g].astype(np.int64) - 127
        kmax = kj.max()
        assert s2[g] == 2.0 ** (kmax + off)
        # global_amax = 6 * 448 * scale_2 with the page's constants
        gamax = page_constants["e2m1_max"][0] * page_constants["e4m3_max"][0] * s2[g]
        assert gamax == 6 * 448 * 2.0 ** (kmax - 8)
        inwin = (kmax - kj) <= win
        assert fb[g] == int((~inwin).sum()) == int(forced[g].sum())
        src = M.mxfp4_dequant(packed[g], e8[g])
        dst = M.nvfp4_dequant_f32(out[g][None], codes[g][None], s2[g:g + 1])[0]
        m = np.repeat(inwin, 32, axis=-1)
        assert np.array_equal(src[m], dst[m])                 # bit-exact dequant
        nib_src = F.unpack_nibbles(packed[g])
        nib_dst = F.unpack_nibbles(out[g])
        assert np.array_equal(nib_src[m], nib_dst[m])         # nibbles unchanged
        # the block holding k_max gets scale 2^8 = 256, code 0x78
        at_max = np.repeat(kj == kmax, 2, axis=-1)
        assert (codes[g][at_max] == 0x78).all()
    # scale bytes double: one byte per 16 instead of one per 32
    assert codes.size == 2 * e8.size


def test_cast_in_window_codes_closed_form():
    """Code of 2^e for e in [-9, 8]: (e+7)<<3 for normal, 0x04/0x02/0x01 below."""
    for e in range(-9, 9):
        want = ((e + 7) << 3) if e >= -6 else {-7: 0x04, -8: 0x02, -9: 0x01}[e]
        assert int(F.e4m3_encode_ratio(2.0 ** e, 1.0)) == want
        assert F.E4M3_VALUES[want] == 2.0 ** e


def test_cast_fallback_closed_form():
    """Outside the window the max-based code is below 2^-9 of the grid, so it is
    raised to 0x01 (scale 2^(k_max-17)) and each nibble becomes the E2M1 value
    nearest to e2m1 * 2^(k_j - k_max + 17), sign kept (exact brute force)."""
    packed, e8, _ = _small_case(seed=3)
    out, codes, s2, fb = M.mxfp4_to_nvfp4(packed, e8)
    grid = [Fraction(v) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    checked = 0
    for g in range(packed.shape[0]):
        kj = e8[g].astype(np.int64) - 127
        kmax = kj.max()
        src = F.unpack_nibbles(packed[g]).reshape(kj.shape + (32,))
        dst = F.unpack_nibbles(out[g]).reshape(kj.shape + (32,))
        cg = codes[g].reshape(kj.shape + (2,))
        for idx in zip(*np.nonzero(kmax - kj > 17)):
            for h in range(2):
                s = src[idx][16 * h:16 * h + 16]
                if (s & 7).max() == 0:
                    assert cg[idx][h] == 0
                    continue
                assert cg[idx][h] == 0x01
                scale = Fraction(2) ** int(kj[idx] - kmax + 17)
                for a, b in zip(s, dst[idx][16 * h:16 * h + 16]):
                    y = grid[a & 7] * scale
                    best = min(range(8), key=lambda i: (abs(y - grid[i]), i % 2))
                    assert b == ((a & 8) | best)
                    checked += 1
    assert checked > 0


def test_cast_nan_exponent_is_isolated():
    packed, e8, _ = _small_case(seed=5)
    e8 = e8.copy()
    e8[0, 0, 0, 0] = 255
    out, codes, s2, fb = M.mxfp4_to_nvfp4(packed, e8)
    assert codes[0, 0, 0, 0] == 0x7F and codes[0, 0, 0, 1] == 0x7F
    assert np.array_equal(out[0, 0, 0, :16], packed[0, 0, 0, :16])
    kj = e8[0].astype(np.int64) - 127
    assert s2[0] == 2.0 ** (kj[e8[0] != 255].max() - 8)
