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
