"""NVFP4 steps of the hot path, in float64 numpy.  Test infrastructure only.

Steps, in the order of the Coder390 NVFP4 calibration note §2:
  1. max calibration: per-tensor amax -> FP32 tensor scale scale_2
     (formula from the pi05 NVFP4 flow note §3.4: amax / 6 / 448);
  2. local Hessian: H_g = sum_t x_{t,g} x_{t,g}^T per group g of 16 input
     channels, from unquantized activations;
  3. scale sweep: for each 16-element weight block, try every finite E4M3
     block-scale code, quantize the block to E2M1 under that scale and
     scale_2, and keep the code minimising (w - wq)^T H_g (w - wq).
Then the runtime pieces of the pi05 flow note: the dynamic per-16 activation
quantizer (§3.4-§3.5) and the two-DequantizeLinear chain (§5.4): the E4M3
code times scale_2 gives an FP32 block scale, E2M1 times that gives the
output, which is cast to BF16.

Readings (pages silent):
* the swept codes are 0x00..0x7E (0x7F is NaN and cannot be a scale; 0x00 is
  the zero scale, which quantizes the block to zero);
* the argmin keeps the first strict minimum in ascending code order;
* H is the plain sum (no 1/N, no damping) and feeds the cost as is;
* wq in the cost is the exact product e2m1 * d (no bf16 rounding);
* the max-based block code of the dynamic quantizer is RNE(amax_b / (6 *
  scale_2)) on the E4M3 grid, saturated at 448, and raised to 0x01 when the
  block is nonzero but that rounding gives 0x00;
* scale_2 = 0 (an all-zero tensor) makes every block scale zero.
"""
from __future__ import annotations

import numpy as np

from .formats import (
    E4M3_VALUES, e2m1_decode, e2m1_encode, e4m3_encode_ratio, bf16_bits_to_f64,
    f32, f64_to_bf16_bits, pack_nibbles, unpack_nibbles,
)

N_CODES = 127          # finite non-negative E4M3 codes 0x00..0x7E
BLOCK = 16


def tensor_scale(x_bits):
    """Step 1: (amax, scale_2) of a bf16 tensor.

    amax = max |x| (exact).  scale_2 = amax / 6 / 448 evaluated in double
    precision in that order and stored as FP32, as the pi05 flow note §3.4
    writes it for the per-tensor scale.
    """
    x = bf16_bits_to_f64(x_bits)
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    s2 = float(np.float32(float(amax) / 6.0 / 448.0))
    return amax, s2


def hessian(x_bits, h_init=None):
    """Step 2: block-diagonal Hessian [K/16, 16, 16] in float64.

    H_g += X_g^T X_g where X_g = X[:, 16g:16g+16] (Coder390 note §2, step 2).
    """
    x = bf16_bits_to_f64(x_bits)
    t, k = x.shape
    g = k // BLOCK
    h = np.zeros((g, BLOCK, BLOCK)) if h_init is None else np.array(h_init, dtype=np.float64)
    step = 8192
    for s in range(0, t, step):
        xg = x[s:s + step].reshape(-1, g, BLOCK).transpose(1, 0, 2)   # [g, t, 16]
        h += np.matmul(xg.transpose(0, 2, 1), xg)
    return h


def block_scale(code, s2):
    """DQ1 of the two-DQ chain: FP32 block scale d = RN_f32(e4m3(code) * scale_2)."""
    return f32(E4M3_VALUES[np.asarray(code, dtype=np.int64)] * float(s2))


def quantize_at_code(w, code, s2):
    """Quantize 16-element blocks w[..., 16] at a block-scale code.

    Returns (nibbles[..., 16] uint8, wq[..., 16] float64) with
    wq = e2m1(nibble) * d exactly, d = block_scale(code, s2).
    """
    d = block_scale(code, s2)[..., None]
    nib = e2m1_encode(w, d)
    wq = e2m1_decode(nib) * d
    return nib, wq


def block_cost(w, wq, h):
    """(w - wq)^T H (w - wq) per block; w, wq [..., 16], h [..., 16, 16] broadcastable."""
    e = w - wq
    return np.einsum("...i,...ij,...j->...", e, h, e)


def sweep_costs(w_bits, h, s2):
    """Cost of every code 0..126 for every block: float64 [rows, K/16, 127]."""
    w = bf16_bits_to_f64(w_bits)
    rows, k = w.shape
    g = k // BLOCK
    wb = w.reshape(rows, g, BLOCK)
    h = np.asarray(h, dtype=np.float64)
    out = np.empty((rows, g, N_CODES))
    for c in range(N_CODES):
        _, wq = quantize_at_code(wb, c, s2)
        e = (wb - wq).transpose(1, 0, 2)             # [g, rows, 16]
        he = np.matmul(e, h)                         # [g, rows, 16] (H symmetric)
        out[:, :, c] = np.sum(he * e, axis=2).T
    return out


def scale_sweep(w_bits, h, s2):
    """Step 3 (fp8_scale_sweep): per-block E4M3 code minimising the Hessian cost.

    Returns (codes [rows, K/16] uint8, packed [rows, K/2] uint8,
    cost [rows, K/16] float64).  Ties keep the lowest code.
    """
    costs = sweep_costs(w_bits, h, s2)
    codes = np.argmin(costs, axis=2)                 # first minimum = lowest code
    best = np.take_along_axis(costs, codes[..., None], axis=2)[..., 0]
    w = bf16_bits_to_f64(w_bits)
    rows, k = w.shape
    nib, _ = quantize_at_code(w.reshape(rows, k // BLOCK, BLOCK), codes, s2)
    return codes.astype(np.uint8), pack_nibbles(nib.reshape(rows, k)), best


def max_code(amax_b, s2):
    """E4M3 code of a block from its max: RNE(amax_b / (6 * scale_2)), saturated,
    and 0x01 for a nonzero block whose rounding gives 0x00."""
    amax_b = np.asarray(amax_b, dtype=np.float64)
    den = 6.0 * float(s2)                            # exact: s2 is float32
    code = e4m3_encode_ratio(amax_b, den).astype(np.int64)
    code = np.where((code == 0) & (amax_b > 0.0), 1, code)
    return code.astype(np.uint8)


def quantize_dynamic(x_bits, s2):
    """Dynamic per-16 NVFP4 quantizer (pi05 flow note §3.4-§3.5).

    Per block: block amax, E4M3 code from max_code, E2M1 at that code.
    Returns (packed [T, K/2] uint8, codes [T, K/16] uint8).
    """
    x = bf16_bits_to_f64(x_bits)
    t, k = x.shape
    xb = x.reshape(t, k // BLOCK, BLOCK)
    codes = max_code(np.max(np.abs(xb), axis=2), s2)
    nib, _ = quantize_at_code(xb, codes, s2)
    return pack_nibbles(nib.reshape(t, k)), codes


def dequant(packed, codes, s2):
    """Two-DQ chain (pi05 flow note §5.4): out = RN_bf16(RN_f32(e2m1 * d)).

    Returns bf16 bit patterns [rows, K].
    """
    nib = unpack_nibbles(packed)
    rows, k = nib.shape
    d = block_scale(codes, s2)                       # [rows, K/16]
    v = e2m1_decode(nib).reshape(rows, k // BLOCK, BLOCK) * d[..., None]
    return f64_to_bf16_bits(f32(v).reshape(rows, k))


def fakequant(x_bits, s2):
    """bf16 bits of the NVFP4 block fake QDQ of an activation tensor: the
    dynamic quantizer followed by the two-DQ chain (pi05 flow note §2.2: the
    input quantizer of a QuantLinear; §3.4-§3.5, §5.4)."""
    packed, codes = quantize_dynamic(x_bits, s2)
    return dequant(packed, codes, s2)


def quantlinear_forward(x_bits, s2x, w_hat_bits):
    """Fake-quant QuantLinear forward (pi05 flow note §2.2, §2.4): x goes
    through its input quantizer (fake QDQ at tensor scale s2x), the weight is
    already fake-quantized (w_hat = dequant of the swept NVFP4 weight), and
    y = x_hat w_hat^T is a floating-point matmul.  Returned in float64,
    unrounded (reading: the GEMM accumulates in fp32 and rounds y once to
    bf16; that rounding and the accumulation order are left to the tests'
    error bound)."""
    xh = bf16_bits_to_f64(fakequant(x_bits, s2x))
    return xh @ bf16_bits_to_f64(w_hat_bits).T


def hessian_fakequant(x_bits, s2, h_init=None):
    """Step 2 for a W4A4 calibration (reading: the layer input is seen after
    its dynamic NVFP4 quantizer): H_g += Xh_g^T Xh_g with Xh the bf16 output
    of the two-DQ chain applied to the dynamic per-16 quantization of X at
    tensor scale s2 (pi05 flow note §3.4-§3.5, §5.4; Coder390 note §2 step 2).
    """
    packed, codes = quantize_dynamic(x_bits, s2)
    return hessian(dequant(packed, codes, s2), h_init=h_init)
