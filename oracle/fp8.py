"""FP8 E4M3 W8A8 tier with per-tensor static scales, in float64 numpy.
Test infrastructure only.

Source: "Coder390 NVFP4 校正（校准）方式" §3, the layer table of the mixed
W4A4+W8A8 tier: the attention projections use FP8 E4M3 weights and
activations with one static scale per tensor, and the FP8 activation scales
are the ones gathered during calibration (unlike the NVFP4 activations,
which are quantized dynamically per 16 elements).

Readings (the page gives no formula for the FP8 scale or rounding):
* the static scale is max calibration with the E4M3 range, the FP8 analog of
  the NVFP4 tensor scale of the pi05 flow note §3.4 without the E2M1 factor 6:
  s = amax / 448, evaluated in double precision and stored as FP32;
* a code is the E4M3FN encode of the EXACT quotient x / s, to nearest with
  ties to even, saturated at 448, sign kept (a negative value that rounds to
  zero gives 0x80), as the formats module does for every encode;
* s = 0 (an all-zero calibration tensor): x = 0 gives code 0, any other
  value saturates (the encode of x / 0);
* dequant is the one-DQ form of the pi05 flow note §5.4: RN_bf16(RN_f32(e4m3
  * s)).
These are readings: no worked example on the pages confirms them.  The
functions are pinned by tests/test_oracle_fp8.py (rational brute force,
torch's float8_e4m3fn cast on exact quotients, invariants).
"""
from __future__ import annotations

import numpy as np

from .formats import E4M3_VALUES, e4m3_encode_ratio, bf16_bits_to_f64, f32, f64_to_bf16_bits

E4M3_MAX = 448.0


def fp8_tensor_scale(x_bits):
    """(amax, s): amax = max |x| (exact), s = RN_f32(amax / 448)."""
    x = bf16_bits_to_f64(x_bits)
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    return amax, float(np.float32(amax / E4M3_MAX))


def fp8_quantize(x_bits, s):
    """E4M3FN codes (uint8, same shape as x) of x / s, exact quotient, RNE,
    saturating, sign in bit 7."""
    bits = np.asarray(x_bits, dtype=np.uint16)
    mag = bf16_bits_to_f64(bits & np.uint16(0x7FFF))
    code = e4m3_encode_ratio(mag, float(s)).astype(np.uint8)
    sign = ((bits >> np.uint16(15)) & np.uint16(1)).astype(np.uint8) << np.uint8(7)
    return code | sign


def fp8_dequant(codes, s):
    """bf16 bit patterns of RN_bf16(RN_f32(e4m3(code) * s))."""
    v = E4M3_VALUES[np.asarray(codes, dtype=np.uint8).astype(np.int64)] * float(s)   # exact in float64
    return f64_to_bf16_bits(f32(v))
