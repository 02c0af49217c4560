"""Block-Hadamard rotation under the local-Hessian sweep, in float64 numpy.
Test infrastructure only.

Source: "FP4量化技术概述：从理论到硬件实现" §3.1 (MR-GPTQ): the weight matrix
is cut into 16x16 (or 32x32) blocks, each block gets the normalised discrete
Hadamard transform H_n / sqrt(n), and the transform is fused into the
weights, W' = W H, while the activations are rotated online, X H.

Readings (the page prints the idea, not a format):
* the rotation acts on the input channels in the NVFP4 groups of 16: R is
  block diagonal with R_g = H16 / 4, H16 the Sylvester Hadamard matrix
  (symmetric, H16 H16 = 16 I).  y = X W^T = (X R)(W R)^T, so the rotated
  weights W' = W R and activations X' = X R give the same layer output, and
  the local Hessian of the rotated input is H'_g = R_g^T H_g R_g;
* a rotated row block is computed as the Sylvester butterfly (four stages of
  pairwise sums and differences, pairs (i, i + h) for h = 1, 2, 4, 8) in
  float64, then scaled by 1/4 and rounded once to bf16 (nearest even).  The
  butterfly sums are exact whenever the block's values span less than 2^41,
  so the result is then the correctly rounded exact product;
* H' is rounded once to float32;
* the rotated sweep uses the rotated tensor's own scale_2, and its cost
  (w' - q')^T H' (w' - q') equals the Hessian-weighted error of the
  un-rotated dequantized weights q' R^T, so costs compare directly.
These are readings: no worked example on the pages confirms them.  The
functions are pinned by tests/test_oracle_rotate.py (scipy's Hadamard
matrix, exact rational products, invariants).
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64, f64_to_bf16_rne

BLOCK = 16


def hadamard16() -> np.ndarray:
    """Sylvester Hadamard matrix of order 16 (entries +-1), by doubling."""
    h = np.array([[1.0]])
    while h.shape[0] < BLOCK:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate_blocks(x_bits) -> np.ndarray:
    """bf16 bits of X R: every 16-element block x of every row becomes
    RN_bf16((x H16) / 4) via the fp64 butterfly."""
    x = bf16_bits_to_f64(x_bits)
    rows, k = x.shape
    v = x.reshape(rows, k // BLOCK, BLOCK).copy()
    h = 1
    while h < BLOCK:
        v = v.reshape(rows, k // BLOCK, BLOCK // (2 * h), 2, h)
        a = v[:, :, :, 0, :].copy()
        b = v[:, :, :, 1, :].copy()
        v[:, :, :, 0, :] = a + b
        v[:, :, :, 1, :] = a - b
        h *= 2
    v = v.reshape(rows, k) * 0.25
    return f64_to_bf16_rne(v)


def rotate_hessian(h) -> np.ndarray:
    """H'_g = R_g^T H_g R_g for every group, rounded to float32 (as float64)."""
    r = hadamard16() / 4.0
    hp = np.einsum("ai,gab,bj->gij", r, np.asarray(h, dtype=np.float64), r)
    return hp.astype(np.float32).astype(np.float64)
