"""Closed-form MXFP4 -> NVFP4 cast, in float64 numpy.  Test infrastructure only.

Follows the ModelOpt MXFP4->NVFP4 guide §2-§3 and the DeepSeek-V4 NVFP4
pipeline article (export stage):
  * MXFP4 = E2M1 nibbles with one E8M0 exponent k_j per 32 elements; the
    NVFP4 target keeps the nibbles and needs one E4M3 scale per 16 plus one
    FP32 tensor scale;
  * tensor scale: global_amax = 6 * 448 * 2^(k_max - 8), i.e. scale_2 =
    global_amax / (6 * 448) = 2^(k_max - 8), a power of two;
  * block scale: each NVFP4 block of MX block j gets _amax = 6 * 2^k_j, i.e.
    block scale 2^(k_j - k_max + 8), which E4M3 holds exactly while
    k_max - k_j <= 17; those blocks dequantize exactly as before and their
    nibbles move unchanged;
  * blocks outside that window fall back to a block amax taken from the data
    (max |w_block|);
  * the two matrices of a gate/up pair (w1, w3) share one scale_2, so k_max is
    taken over both.

Readings: the fallback re-quantizes each 16-element NVFP4 block with the
dynamic max-based quantizer of nvfp4.max_code (including its raise of a
nonzero block's code 0x00 to 0x01); an E8M0 code 255 (NaN) is left out of
k_max and its two NVFP4 blocks get the E4M3 NaN code 0x7F with nibbles kept.
"""
from __future__ import annotations

import numpy as np

from .formats import e2m1_decode, e4m3_encode_ratio, unpack_nibbles, pack_nibbles, f32
from .nvfp4 import max_code, quantize_at_code


def mxfp4_dequant(packed, e8m0):
    """Real values of MXFP4 tensors: e2m1(nibble) * 2^(e8m0 - 127)."""
    nib = unpack_nibbles(packed)
    k = nib.shape[-1]
    v = e2m1_decode(nib).reshape(nib.shape[:-1] + (k // 32, 32))
    e = np.asarray(e8m0).astype(np.float64)
    scale = np.where(e == 255, np.nan, np.exp2(e - 127.0))
    return (v * scale[..., None]).reshape(nib.shape)


def mxfp4_to_nvfp4(packed, e8m0):
    """Cast MXFP4 expert pairs to NVFP4.

    packed : uint8 [G, M, R, K/2]  (M matrices per group sharing scale_2)
    e8m0   : uint8 [G, M, R, K/32]
    Returns (packed_out uint8 [G, M, R, K/2], codes uint8 [G, M, R, K/16],
             scale_2 float64 [G] (float32 values), fallback int64 [G] =
             number of 32-element MX blocks outside the window per group).
    """
    packed = np.asarray(packed, dtype=np.uint8)
    e8m0 = np.asarray(e8m0, dtype=np.uint8)
    g_, m_, r_, kh = packed.shape
    k = kh * 2
    nb = k // 32
    out_packed = packed.copy()
    codes = np.zeros((g_, m_, r_, k // 16), dtype=np.uint8)
    s2 = np.zeros(g_)
    fallback = np.zeros(g_, dtype=np.int64)
    for g in range(g_):
        e = e8m0[g].astype(np.int64)
        valid = e != 255
        kj = e - 127
        kmax = int(kj[valid].max()) if valid.any() else 0
        s2[g] = float(np.float32(2.0 ** (kmax - 8)))
        in_win = valid & (kmax - kj <= 17)
        # in-window: block scale 2^(k_j - k_max + 8) exactly on the E4M3 grid
        blk = e4m3_encode_ratio(np.exp2(np.where(in_win, kj - kmax + 8, 0).astype(np.float64)), 1.0)
        blk = np.where(in_win, blk, 0).astype(np.uint8)
        blk = np.where(valid, blk, 0x7F).astype(np.uint8)
        codes[g] = np.repeat(blk, 2, axis=-1)
        fb = valid & ~in_win
        fallback[g] = int(fb.sum())
        if fb.any():
            nib = unpack_nibbles(packed[g]).reshape(m_, r_, nb, 2, 16)
            x = e2m1_decode(nib) * np.exp2(kj.astype(np.float64))[..., None, None]
            idx = np.nonzero(fb)
            xs = x[idx]                                   # [n, 2, 16]
            c = max_code(np.max(np.abs(xs), axis=2), s2[g])   # [n, 2]
            new_nib, _ = quantize_at_code(xs, c, s2[g])
            nib[idx] = new_nib
            out_packed[g] = pack_nibbles(nib.reshape(m_, r_, k))
            cg = codes[g].reshape(m_, r_, nb, 2)
            cg[idx] = c
            codes[g] = cg.reshape(m_, r_, nb * 2)
    return out_packed, codes, s2, fallback


def nvfp4_dequant_f32(packed, codes, s2):
    """FP32 values of NVFP4 tensors (e2m1 * RN_f32(e4m3(code) * scale_2)), for
    comparing a cast against its MXFP4 source; scale_2 per leading group."""
    from .formats import E4M3_VALUES
    nib = unpack_nibbles(packed)
    sh = nib.shape
    s2 = np.asarray(s2, dtype=np.float64).reshape((-1,) + (1,) * (codes.ndim - 1))
    d = f32(E4M3_VALUES[codes.astype(np.int64)] * s2)
    v = e2m1_decode(nib).reshape(sh[:-1] + (sh[-1] // 16, 16)) * d[..., None]
    return f32(v).reshape(sh)
