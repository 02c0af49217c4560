"""Helpers shared by the GPU parity tests: host <-> device conversions and the
parity criteria.  Inputs always come from datagen; expected values always
come from the oracle."""
import os
import sys

import numpy as np
import pytest
import torch

import nvfp4_post_quantization_amd as nq

DEV = torch.device("cuda:0")


def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    nq.load()          # raises if the HIP library is missing


def note(msg: str) -> None:
    """Name the case before any GPU work, so a fault points at it."""
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_dev_f32(a) -> torch.Tensor:
    return torch.as_tensor(np.asarray(a, dtype=np.float32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def rel_frobenius(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Per-group ||a - b||_F / ||b||_F over the last two axes."""
    num = np.sqrt(((a - b) ** 2).sum(axis=(-1, -2)))
    den = np.sqrt((b ** 2).sum(axis=(-1, -2)))
    return np.where(den > 0, num / np.maximum(den, 1e-300), num)


def compare_sweep(w_bits, h32, s2, packed, codes, cost, max_mismatch_frac=1e-4, costs=None):
    """Sweep parity of GPU outputs (packed, codes, cost) for the rows w_bits.

    Per block: the code equals the oracle's argmin on >= 1 - max_mismatch_frac
    of the blocks; where it differs, the oracle's cost of the GPU code is within
    1e-5 relative of the oracle minimum; the nibbles always equal the oracle's
    quantization at the GPU code, bit for bit; the fp32 cost is within 1e-4
    relative of the oracle's cost of that code.  costs, when given, are the
    oracle's sweep_costs of the same rows (computed elsewhere, e.g. in a
    process pool).  Returns the mismatch count."""
    from oracle import nvfp4 as N
    from oracle import formats as F
    h = np.asarray(h32, dtype=np.float32).astype(np.float64)
    if costs is None:
        costs = N.sweep_costs(w_bits, h, s2)                    # [rows, G, 127]
    ref = np.argmin(costs, axis=2)
    ref_min = np.min(costs, axis=2)
    rows, g = codes.shape
    cg = np.take_along_axis(costs, codes.astype(np.int64)[..., None], axis=2)[..., 0]
    w0 = costs[:, :, 0]                                         # cost of the zero scale = w^T H w
    mism = codes != ref
    n_mism = int(mism.sum())
    assert n_mism <= max_mismatch_frac * codes.size, f"{n_mism} of {codes.size} codes differ"
    if n_mism:
        tol = np.where(ref_min > 0, 1e-5 * ref_min, 1e-5 * w0)
        assert np.all(cg[mism] - ref_min[mism] <= tol[mism]), "a differing code is not a near-tie"
    w = F.bf16_bits_to_f64(w_bits).reshape(rows, g, 16)
    nib, _ = N.quantize_at_code(w, codes, s2)
    assert np.array_equal(packed, F.pack_nibbles(nib.reshape(rows, g * 16))), "nibbles differ"
    if cost is not None:
        scale = np.maximum(cg, 1e-6 * w0)
        assert np.all(np.abs(cost - cg) <= 1e-4 * scale + 1e-30), "cost output off"
    return n_mism
