"""Seeded synthetic inputs for the NVFP4 post-training-quantization hot path.

This module draws random tensors and nothing else: it holds none of the
quantization arithmetic.  Both the CPU oracle (``oracle/``) and the HIP path
consume what it returns, so a parity test compares the two on the very same
bits.

Conventions
-----------
* Every tensor is drawn in float64 from a Philox stream keyed by
  ``SeedSequence([seed, config, tensor, chunk])``, scaled, rounded to float32
  and then to bfloat16 with round-to-nearest-even.  bf16 tensors are carried
  on the host as ``uint16`` bit patterns.
* "N(0, s)" means standard deviation ``s``; "Laplace(b)" has scale ``b``.
* Outlier entries/channels are picked without replacement from their own
  stream and multiplied by the stated factor before rounding.

The workloads mirror the calibration shapes on the pages: a tiny Linear, a
Gemma-2B q_proj (2048x2048 with 2048-wide inputs, pi05 NVFP4 flow note §2.4),
an activation tensor for the dynamic quantizer, a hybrid-model MLP set
calibrated on 2^20 tokens streamed in 65536-token chunks (Coder390 calibration
note §1-§2), and a 128-expert MXFP4 MoE whose gate/up pair shares one tensor
scale (ModelOpt MXFP4->NVFP4 guide §2-§3).  Laplace activations follow the
heavy-tail model of the FP4 survey page (§2.1).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "stream", "f32_to_bf16_bits", "normal_bf16", "laplace_bf16",
    "config1", "config2", "config3", "config4_weights", "config4_chunk_host",
    "config4_outlier_channels", "config4_chunk_torch", "config5", "torch_stream_seed",
    "C4_TOKENS", "C4_CHUNK", "C4_HIDDEN", "C4_INTER",
]

C4_TOKENS = 1 << 20      # 256 sequences x 4096 tokens
C4_CHUNK = 65536         # tokens per streamed chunk
C4_HIDDEN = 4096         # gate/up input width
C4_INTER = 12288         # down input width


def stream(config: int, tensor: int, chunk: int = 0, seed: int = 0) -> np.random.Generator:
    """Independent Philox stream for (seed, config, tensor, chunk)."""
    ss = np.random.SeedSequence([seed, config, tensor, chunk])
    return np.random.Generator(np.random.Philox(ss))


def torch_stream_seed(config: int, tensor: int, chunk: int = 0, seed: int = 0) -> int:
    """63-bit seed for a torch.Generator standing for the same key."""
    ss = np.random.SeedSequence([seed, config, tensor, chunk, 0x7F4A])
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64((1 << 63) - 1))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); finite inputs."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def _to_bf16(x64: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(x64.astype(np.float32))


def normal_bf16(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    return _to_bf16(rng.standard_normal(shape) * sigma)


def laplace_bf16(rng: np.random.Generator, shape, b: float) -> np.ndarray:
    return _to_bf16(rng.laplace(0.0, b, shape))


def config1(seed: int = 0):
    """Tiny single Linear.

    W [64, 256] ~ N(0, 0.02) with 1% of entries (164) multiplied by 20;
    X [512, 256] ~ N(0, 1) with channels 7 and 130 multiplied by 30.
    Returns (W_bits, X_bits) as uint16 arrays.
    """
    w = stream(1, 0, seed=seed).standard_normal((64, 256)) * 0.02
    n_out = int(round(0.01 * w.size))
    idx = stream(1, 1, seed=seed).choice(w.size, n_out, replace=False)
    w.reshape(-1)[idx] *= 20.0
    x = stream(1, 2, seed=seed).standard_normal((512, 256))
    x[:, [7, 130]] *= 30.0
    return _to_bf16(w), _to_bf16(x)


def config2(seed: int = 0):
    """Gemma-2B-like q_proj.

    W [2048, 2048] = N(0, 0.02) + Laplace(0.01) elementwise (heavier tails);
    X [4096, 2048] ~ Laplace(1) with 8 random channels multiplied by 40.
    """
    w = stream(2, 0, seed=seed).standard_normal((2048, 2048)) * 0.02
    w += stream(2, 1, seed=seed).laplace(0.0, 0.01, (2048, 2048))
    x = stream(2, 2, seed=seed).laplace(0.0, 1.0, (4096, 2048))
    ch = stream(2, 3, seed=seed).choice(2048, 8, replace=False)
    x[:, ch] *= 40.0
    return _to_bf16(w), _to_bf16(x)


def config3(seed: int = 0, tokens: int = 8192, k: int = 4096):
    """Activations for the dynamic quantizer: X [8192, 4096] ~ Laplace(1),
    16 random channels multiplied by 50."""
    x = stream(3, 0, seed=seed).laplace(0.0, 1.0, (tokens, k))
    ch = stream(3, 1, seed=seed).choice(k, 16, replace=False)
    x[:, ch] *= 50.0
    return _to_bf16(x)


def config4_weights(which: str, seed: int = 0, rows: int | None = None):
    """Hybrid-model MLP weights ~ N(0, 0.015): gate/up [12288, 4096], down [4096, 12288].

    ``rows`` draws only the first ``rows`` rows (same values as the full draw's
    leading rows), for bounded CPU work.
    """
    shapes = {"gate": (C4_INTER, C4_HIDDEN), "up": (C4_INTER, C4_HIDDEN), "down": (C4_HIDDEN, C4_INTER)}
    tensor = {"gate": 0, "up": 1, "down": 2}[which]
    r, k = shapes[which]
    n = r if rows is None else min(rows, r)
    g = stream(4, tensor, seed=seed)
    return normal_bf16(g, (n, k), 0.015)


def config4_outlier_channels(stream_id: int, seed: int = 0):
    """8 outlier channels (x40) of calibration stream 0 (K=4096) or 1 (K=12288)."""
    k = C4_HIDDEN if stream_id == 0 else C4_INTER
    return np.sort(stream(4, 10 + stream_id, seed=seed).choice(k, 8, replace=False))


def config4_chunk_host(stream_id: int, chunk: int, seed: int = 0, tokens: int = C4_CHUNK):
    """Host copy of one 65536-token calibration chunk (Laplace(1), 8 channels x40).

    ``tokens`` < C4_CHUNK draws a leading slice with different values (a
    smaller stand-in for CPU-only checks); the GPU benchmark draws chunks on
    the device with :func:`torch_stream_seed`.
    """
    k = C4_HIDDEN if stream_id == 0 else C4_INTER
    x = stream(4, 20 + stream_id, chunk, seed=seed).laplace(0.0, 1.0, (tokens, k))
    x[:, config4_outlier_channels(stream_id, seed)] *= 40.0
    return _to_bf16(x)


def config5(seed: int = 0, experts: int = 128, rows: int = 2048, k: int = 7168,
            forced_frac: float = 0.005):
    """MXFP4 MoE expert pairs (w1, w3) for the MXFP4->NVFP4 cast.

    Packed E2M1 nibbles are uniform over all 16 codes (two per byte).  Each
    32-element block has an E8M0 exponent k ~ round(N(-6, 3)); per expert the
    pair maximum k_max is taken, k is clipped to [k_max-17, k_max], and a seeded
    ``forced_frac`` of the blocks below k_max is pushed to k_max-17-U{1..4} so
    that the window test fails for exactly those blocks.  Returns (packed u8 [E,2,rows,k/2], e8m0 u8
    [E,2,rows,k/32], forced bool [E,2,rows,k/32]).
    """
    nb = k // 32
    rng_n = stream(5, 0, seed=seed)
    packed = rng_n.integers(0, 256, size=(experts, 2, rows, k // 2), dtype=np.uint8)
    rng_k = stream(5, 1, seed=seed)
    kk = np.rint(rng_k.standard_normal((experts, 2, rows, nb)) * 3.0 - 6.0).astype(np.int64)
    kmax = kk.reshape(experts, -1).max(axis=1)
    kk = np.maximum(kk, (kmax - 17)[:, None, None, None])
    rng_f = stream(5, 2, seed=seed)
    forced = rng_f.random((experts, 2, rows, nb)) < forced_frac
    # never force a block that holds its pair's k_max (that would move k_max)
    forced &= kk < kmax[:, None, None, None]
    drop = rng_f.integers(1, 5, size=(experts, 2, rows, nb))
    kk = np.where(forced, (kmax - 17)[:, None, None, None] - drop, kk)
    # keep every exponent inside the E8M0 finite range
    e8 = np.clip(kk + 127, 0, 254).astype(np.uint8)
    return packed, e8, forced


def config4_chunk_torch(stream_id: int, chunk: int, device, seed: int = 0, tokens: int = C4_CHUNK):
    """One calibration chunk drawn on the device (torch Philox, float64 draw).

    Same recipe as :func:`config4_chunk_host` (Laplace(1) by the inverse CDF,
    the same 8 outlier channels x40, float32 then bf16 rounding), but a
    different random stream: the device draw is what the benchmark and the
    full-size GPU checks use, and the oracle reads those very tensors back.
    """
    import torch
    k = C4_HIDDEN if stream_id == 0 else C4_INTER
    g = torch.Generator(device=device)
    g.manual_seed(torch_stream_seed(4, 20 + stream_id, chunk, seed))
    u = torch.rand((tokens, k), generator=g, device=device, dtype=torch.float64)
    u.sub_(0.5).clamp_(min=-0.5 + 2.0 ** -52)
    x = torch.sign(u).mul_(torch.log1p(u.abs().mul_(-2.0))).neg_()
    del u
    ch = torch.as_tensor(config4_outlier_channels(stream_id, seed), device=device)
    x[:, ch] *= 40.0
    return x.to(torch.float32).to(torch.bfloat16)
