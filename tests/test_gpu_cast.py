"""GPU parity: closed-form MXFP4 -> NVFP4 cast against the oracle, bit for bit
(codes, rewritten nibbles, scale_2, fallback counts)."""
import numpy as np
import pytest
import torch

import datagen
from oracle import mxcast as M
import nvfp4_post_quantization_amd as nq

from _gpu import DEV, need_gpu, note, to_dev_u8, host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _check(packed, e8):
    p_dev = to_dev_u8(packed)
    codes, s2, fb = nq.mxfp4_to_nvfp4_cast(p_dev, to_dev_u8(e8))
    p_ref, c_ref, s2_ref, fb_ref = M.mxfp4_to_nvfp4(packed, e8)
    assert np.array_equal(host(codes), c_ref)
    assert np.array_equal(host(s2).astype(np.float64), s2_ref)
    assert np.array_equal(host(fb), fb_ref)
    assert np.array_equal(host(p_dev), p_ref)
    return fb_ref


@pytest.mark.parametrize("seed,experts,rows,k,frac", [(0, 4, 64, 512, 0.01), (1, 3, 16, 7168, 0.005),
                                                      (2, 2, 8, 256, 0.2),
                                                      (3, 3, 96, 4096, 0.01),    # 1.5 kmax steps per group
                                                      (7, 3, 256, 8192, 0.01)])  # four kmax partials per group
def test_cast_small(seed, experts, rows, k, frac):
    note(f"cast seed={seed} experts={experts} rows={rows} k={k}")
    packed, e8, forced = datagen.config5(seed=seed, experts=experts, rows=rows, k=k, forced_frac=frac)
    fb = _check(packed, e8)
    assert np.array_equal(fb, forced.reshape(experts, -1).sum(axis=1))


def test_cast_generic_path_and_nan():
    """Groups whose block count is not a multiple of 4 (scalar path) and a NaN exponent."""
    note("cast generic path + NaN exponent")
    rng = np.random.default_rng(3)
    g, m, r, k = 5, 1, 3, 32
    packed = rng.integers(0, 256, (g, m, r, k // 2)).astype(np.uint8)
    e8 = (127 + rng.integers(-30, 10, (g, m, r, k // 32))).astype(np.uint8)
    e8[1, 0, 1, 0] = 255
    e8[2, 0, :, 0] = 255                  # a group with no valid exponent at all
    _check(packed, e8)


def test_cast_zero_halves_and_extremes():
    note("cast zero halves and extreme exponents")
    rng = np.random.default_rng(4)
    g, m, r, k = 2, 2, 4, 64
    packed = rng.integers(0, 256, (g, m, r, k // 2)).astype(np.uint8)
    packed[0, 0, 0, :8] &= 0x88           # a half with zero magnitudes (signs kept)
    e8 = np.full((g, m, r, k // 32), 127, np.uint8)
    e8[0, 0, 0, 0] = 60                   # far below k_max: fallback
    e8[0, 1, 2, 1] = 254                  # k_max = 127
    e8[1] = rng.integers(0, 30, (m, r, k // 32)).astype(np.uint8)   # tiny exponents
    e8[1, 0, 0, 0] = 0
    _check(packed, e8)


def test_cast_subnormal_tensor_scale():
    """Groups whose largest exponent is tiny (E8M0 codes 0..8): scale_2 =
    2^(k_max - 8) is an FP32 subnormal."""
    note("cast subnormal scale_2")
    rng = np.random.default_rng(6)
    g, m, r, k = 9, 2, 4, 64
    packed = rng.integers(0, 256, (g, m, r, k // 2)).astype(np.uint8)
    e8 = np.zeros((g, m, r, k // 32), np.uint8)
    for i in range(g):
        e8[i] = rng.integers(0, i + 1, (m, r, k // 32))   # k_max code <= i
        e8[i, 0, 0, 0] = i
    _check(packed, e8)


def test_cast_empty_rows():
    """Groups with no rows: no exponent, so scale_2 = 2^-8 (k_max taken as 0),
    no fallback blocks, nothing else written."""
    note("cast rows == 0")
    g, m, k = 3, 2, 64
    packed = np.zeros((g, m, 0, k // 2), np.uint8)
    e8 = np.zeros((g, m, 0, k // 32), np.uint8)
    _check(packed, e8)


def test_cast_several_slices_ragged():
    """A group of 134,400 exponents: three workgroup slices of 44,800 bytes,
    ragged against the 4 KiB units of a workgroup's loads."""
    note("cast three slices per group")
    packed, e8, forced = datagen.config5(seed=5, experts=2, rows=300, k=7168, forced_frac=0.01)
    fb = _check(packed, e8)
    assert np.array_equal(fb, forced.reshape(2, -1).sum(axis=1))


def test_cast_many_fallbacks_per_lane():
    """Most blocks out of the window: lanes with more than four fallback
    blocks take the one-by-one path."""
    note("cast many fallbacks per lane")
    packed, e8, forced = datagen.config5(seed=6, experts=2, rows=64, k=2048, forced_frac=0.7)
    fb = _check(packed, e8)
    assert np.array_equal(fb, forced.reshape(2, -1).sum(axis=1))
    assert fb.min() > 0.5 * 64 * 2 * (2048 // 32)


def test_cast_whole_chunks_with_nan_groups():
    """Groups of whole code chunks (every codes workgroup starts on a full
    chunk): one group with scattered NaN exponents, one with no valid
    exponent at all."""
    note("cast whole chunks, NaN groups")
    rng = np.random.default_rng(8)
    g, m, r, k = 2, 2, 64, 8192
    packed = rng.integers(0, 256, (g, m, r, k // 2)).astype(np.uint8)
    e8 = (127 + rng.integers(-20, 4, (g, m, r, k // 32))).astype(np.uint8)
    e8[0, 0, 5, 7] = 255
    e8[0, 1, 60, 200] = 255
    e8[1] = 255
    _check(packed, e8)
