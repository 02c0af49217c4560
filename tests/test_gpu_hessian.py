"""GPU parity: block-diagonal Hessian accumulation against the float64 oracle.

Bar: relative Frobenius error <= 1e-5 per 16x16 block H_g (fp32 on the GPU),
bitwise reproducible across runs, fused amax exact."""
import numpy as np
import pytest
import torch

import datagen
from oracle import nvfp4 as N
from oracle import formats as F
import nvfp4_post_quantization_amd as nq

from _gpu import DEV, need_gpu, note, to_dev_bf16, host, rel_frobenius

pytestmark = pytest.mark.gpu
TOL = 1e-5


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _run(bits: np.ndarray, chunks=1, ld=None, h0=None):
    t, k = bits.shape
    if ld is None:
        x = to_dev_bf16(bits)
    else:
        full = np.zeros((t, ld), np.uint16)
        full[:, :k] = bits
        x = to_dev_bf16(full)[:, :k]
    H = torch.zeros((k // 16, 16, 16), dtype=torch.float32, device=DEV)
    if h0 is not None:
        H.copy_(torch.from_numpy(h0.astype(np.float32)))
    amax = torch.zeros(1, dtype=torch.float32, device=DEV)
    bounds = np.linspace(0, t, chunks + 1).astype(int)
    for a, b in zip(bounds[:-1], bounds[1:]):
        nq.hessian_accum(x[a:b], H, amax)
    return host(H), float(host(amax)[0])


def _check(bits, **kw):
    h, am = _run(bits, **kw)
    h0 = kw.get("h0")
    ref = N.hessian(bits, h_init=h0)
    err = rel_frobenius(h, ref)
    assert err.max() <= TOL, f"max rel Frobenius error {err.max():.3e}"
    assert am == float(np.max(np.abs(F.bf16_bits_to_f64(bits))))
    return h


def test_hessian_config1():
    note("hessian config1")
    _, x = datagen.config1()
    _check(x)


def test_hessian_config2_chunked_and_reproducible():
    note("hessian config2 chunked")
    _, x = datagen.config2()
    h1 = _check(x, chunks=3)
    h2, _ = _run(x, chunks=3)
    assert np.array_equal(h1, h2), "accumulation must be bitwise reproducible"


@pytest.mark.parametrize("t,k,ld", [(1, 16, None), (63, 48, None), (65, 144, 152), (1000, 272, None),
                                    (3, 4096, None), (777, 2064, 2072)])
def test_hessian_ragged(t, k, ld):
    note(f"hessian t={t} k={k} ld={ld}")
    rng = np.random.default_rng(t + k)
    x = datagen.f32_to_bf16_bits(rng.laplace(0, 1, (t, k)).astype(np.float32))
    _check(x, ld=ld)


def test_hessian_accumulates_into_existing():
    note("hessian accumulate into existing H")
    rng = np.random.default_rng(5)
    x = datagen.f32_to_bf16_bits(rng.standard_normal((200, 64)).astype(np.float32))
    h0 = N.hessian(datagen.f32_to_bf16_bits(rng.standard_normal((50, 64)).astype(np.float32)))
    h0 = h0.astype(np.float32).astype(np.float64)
    _check(x, h0=h0)


def test_hessian_outlier_channels_precision():
    """x40 outlier channels and 65536 tokens (one calibration chunk, K=256)."""
    note("hessian 65536-token chunk with outliers")
    rng = np.random.default_rng(11)
    x = rng.laplace(0, 1, (65536, 256))
    x[:, [3, 77, 200]] *= 40.0
    _check(datagen.f32_to_bf16_bits(x.astype(np.float32)))


@pytest.mark.parametrize("t,k", [(130, 66048), (700, 65664), (65, 98304)])
def test_hessian_wide_k_ranges_cross_slabs(t, k):
    """At least as many slabs as workgroups: work ranges cross slab
    boundaries, so workgroups write up to three partial slots and the reduce
    combines several owners per group."""
    note(f"hessian wide k t={t} k={k}")
    rng = np.random.default_rng(t + k)
    x = datagen.f32_to_bf16_bits(rng.laplace(0, 1, (t, k)).astype(np.float32))
    _check(x)
