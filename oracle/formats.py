"""Number formats of NVFP4 / MXFP4, restated in float64 numpy.  Test infrastructure only.

* E2M1 (FP4): sign bit 3, then a 3-bit magnitude index into
  {0, 0.5, 1, 1.5, 2, 3, 4, 6} (FP4 survey, §1.1 lists the positive values;
  pi05 NVFP4 flow note §2.2 gives the (2,1) exponent/mantissa split).
* E4M3FN (FP8 block scale): code = (e << 3) | m, value m*2^-9 for e = 0,
  (8+m)*2^(e-10) otherwise; 0x7E = 448 is the largest finite value (pi05 flow
  note §3.4 and ModelOpt MXFP4->NVFP4 guide §2 both divide by 448), 0x7F is
  NaN.  The block scale has 128 non-negative codes (Coder390 calibration
  note §2, step 3).
* E8M0 (MXFP4 block scale): exponent only, value 2^(c-127), c = 255 is NaN
  (ModelOpt MXFP4->NVFP4 guide §1).
* bf16: the top 16 bits of an IEEE float32.

Rounding reading (the pages name no rounding mode): every encode rounds the
EXACT real value once, to nearest with ties to even, and saturates at the
format's largest finite value.  A negative value keeps its sign bit even when
its magnitude rounds to zero.
"""
from __future__ import annotations

import numpy as np

# --- E2M1 -------------------------------------------------------------------

E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e2m1_decode(nib) -> np.ndarray:
    """Signed value of 4-bit E2M1 codes (bit 3 = sign); -0.0 for code 8."""
    nib = np.asarray(nib).astype(np.int64)
    mag = E2M1_MAGNITUDES[nib & 7]
    return np.where((nib >> 3) & 1, -mag, mag)


def e2m1_encode(x, d) -> np.ndarray:
    """4-bit code of x/d rounded to the E2M1 grid, computed exactly.

    The quotient |x|/d is never formed: it is compared with each midpoint m
    between neighbouring grid magnitudes through |x| vs m*d, which float64
    holds exactly (m has at most 3 significant bits, d is a float32 value, x
    a bf16 or other short dyadic).  At an exact midpoint the neighbour with an
    even magnitude index wins.  Quotients beyond 6 saturate to 6.  d = 0 gives
    magnitude 0 (reading: a zero block scale quantizes the block to zero).
    """
    x = np.asarray(x, dtype=np.float64)
    d = np.broadcast_to(np.asarray(d, dtype=np.float64), x.shape)
    a = np.abs(x)
    idx = np.zeros(x.shape, dtype=np.int64)
    for k in range(7):
        mid = 0.5 * (E2M1_MAGNITUDES[k] + E2M1_MAGNITUDES[k + 1])
        t = mid * d
        upper_even = (k + 1) % 2 == 0
        up = (a > t) | ((a == t) & upper_even)
        idx += up
    idx = np.where(d == 0.0, 0, idx)
    sign = np.signbit(x).astype(np.int64)
    return ((sign << 3) | idx).astype(np.uint8)


def pack_nibbles(nib) -> np.ndarray:
    """Two codes per byte along the last axis: element 2i in the low nibble,
    element 2i+1 in the high nibble (reading of "two FP4 values per byte",
    pi05 flow note §5.4)."""
    nib = np.asarray(nib, dtype=np.uint8)
    return (nib[..., 0::2] & 0xF) | ((nib[..., 1::2] & 0xF) << 4)


def unpack_nibbles(packed) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


# --- E4M3FN -------------------------------------------------------------------

def e4m3_value(code) -> np.ndarray:
    """Value of E4M3FN codes 0..255: bit 7 is the sign; 0x7F and 0xFF are NaN."""
    code = np.asarray(code).astype(np.int64)
    mag = code & 0x7F
    e = mag >> 3
    m = mag & 7
    sub = m * 2.0 ** -9
    nrm = (8 + m) * np.exp2(e.astype(np.float64) - 10.0)
    v = np.where(e == 0, sub, nrm)
    v = np.where(code & 0x80, -v, v)
    return np.where(mag == 0x7F, np.nan, v)


E4M3_VALUES = e4m3_value(np.arange(256))   # [127], [255] are NaN; [128:] negative


def e4m3_encode_ratio(num, den) -> np.ndarray:
    """E4M3FN code of num/den rounded to nearest-even and saturated at 448.

    num >= 0, den >= 0, both exact dyadics.  The quotient is not formed: it is
    compared with each midpoint v between neighbouring finite codes through
    num vs v*den (exact in float64: v has at most 5 significant bits).
    den = 0 gives code 0 for num = 0 and saturates otherwise.
    """
    num = np.asarray(num, dtype=np.float64)
    den = np.broadcast_to(np.asarray(den, dtype=np.float64), num.shape)
    finite = E4M3_VALUES[:127]
    mids = 0.5 * (finite[:-1] + finite[1:])          # 126 midpoints, code c | c+1
    code = np.zeros(num.shape, dtype=np.int64)
    flat_num = num.reshape(-1)
    flat_den = den.reshape(-1)
    out = code.reshape(-1)
    step = 1 << 16
    for s in range(0, flat_num.size, step):
        n = flat_num[s:s + step, None]
        t = mids[None, :] * flat_den[s:s + step, None]
        upper_even = ((np.arange(126) + 1) % 2 == 0)[None, :]
        up = (n > t) | ((n == t) & upper_even)
        out[s:s + step] = up.sum(axis=1)
    code = out.reshape(num.shape)
    code = np.where(den == 0.0, np.where(num > 0.0, 0x7E, 0), code)
    return code.astype(np.uint8)


# --- E8M0 ---------------------------------------------------------------------

def e8m0_value(code) -> np.ndarray:
    code = np.asarray(code).astype(np.int64)
    v = np.exp2(code.astype(np.float64) - 127.0)
    return np.where(code == 255, np.nan, v)


# --- bf16 / f32 ---------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f32(x) -> np.ndarray:
    """Round to float32 (nearest, ties to even) and return as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float32-representable values to bf16 (nearest, ties to even).

    The argument must already be a float32 value; this is the second rounding
    of the dequantization chain (FP32 product, then a cast to BF16).
    """
    a = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u.astype(np.uint64) + np.uint64(0x7FFF) + lsb.astype(np.uint64)) >> np.uint64(16)
    return r.astype(np.uint16)


def f64_to_bf16_rne(x) -> np.ndarray:
    """bf16 bit patterns of float64 values rounded ONCE to nearest, ties to
    even (subnormals on the 2^-133 grid, overflow to infinity).

    Unlike f64_to_bf16_bits this does not go through float32 first.  The grid
    step at |x| in [2^e, 2^(e+1)) is 2^(max(e, -126) - 7); |x| divided by it
    is exact, rint rounds half to even, and the product is exact again.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    m, ex = np.frexp(a)                              # a = m 2^ex, 0.5 <= m < 1
    e = np.where(a > 0, ex - 1, -126)
    q = np.ldexp(1.0, np.maximum(e, -126) - 7)
    v = np.rint(a / q) * q
    with np.errstate(over="ignore"):
        u = v.astype(np.float32).view(np.uint32) >> np.uint32(16)   # exact; 2^128 and above -> inf
    u = u | np.where(np.signbit(x), np.uint32(0x8000), np.uint32(0))
    return u.astype(np.uint16)
