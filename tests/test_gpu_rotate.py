"""GPU parity: block-Hadamard rotation of the input channels and the sweep
under it, against the oracle.

* rotated rows bit for bit (C1-C3 tensors, ragged, strided, in place, blocks
  spanning 60 orders of magnitude, overflow, subnormals), and both full C4
  weights element by element;
* R^T H R per group: relative Frobenius <= 1e-6 (fp64 sums in a different
  order, one rounding to fp32); H = I stays I exactly;
* the sweep of (W R, R^T H R) at the rotated tensor's own scale_2 against
  the oracle's sweep of the oracle's rotated inputs, at the sweep's parity
  bar.
Inputs come from datagen; expected values from the oracle only."""
import numpy as np
import pytest
import torch

import datagen
from oracle import formats as F
from oracle import nvfp4 as N
from oracle import rotate as RT
import nvfp4_post_quantization_amd as nq

from _gpu import DEV, need_gpu, note, to_dev_bf16, to_dev_f32, host, to_host_bits, rel_frobenius, compare_sweep

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _rot(bits, ld=None, ldo=None):
    rows, k = bits.shape
    if ld is None:
        x = to_dev_bf16(bits)
    else:
        full = np.zeros((rows, ld), np.uint16)
        full[:, :k] = bits
        x = to_dev_bf16(full)[:, :k]
    out = None
    if ldo is not None:
        out = torch.zeros((rows, ldo), dtype=torch.bfloat16, device=DEV)[:, :k]
    return to_host_bits(nq.block_hadamard(x, out=out))


@pytest.mark.parametrize("which", ["c1w", "c1x", "c2w", "c3x"])
def test_rotate_tensors(which):
    note(f"block hadamard {which}")
    w1, x1 = datagen.config1()
    w2, _ = datagen.config2()
    bits = {"c1w": w1, "c1x": x1, "c2w": w2, "c3x": datagen.config3()[:512]}[which]
    assert np.array_equal(_rot(bits), RT.rotate_blocks(bits))


@pytest.mark.parametrize("rows,k,ld,ldo", [(1, 16, None, None), (333, 48, 56, None), (7, 4112, 4120, 4128),
                                           (65, 272, None, 280)])
def test_rotate_ragged_strided(rows, k, ld, ldo):
    note(f"block hadamard rows={rows} k={k} ld={ld} ldo={ldo}")
    rng = np.random.default_rng(rows + k)
    bits = datagen.f32_to_bf16_bits(rng.laplace(0, 1, (rows, k)).astype(np.float32))
    assert np.array_equal(_rot(bits, ld=ld, ldo=ldo), RT.rotate_blocks(bits))


def test_rotate_extremes_and_in_place():
    note("block hadamard extremes, in place")
    rng = np.random.default_rng(12)
    wide = rng.laplace(0, 1, (64, 64)) * np.exp(rng.uniform(-69, 69, (64, 64)))     # 1e-30 .. 1e30 in a block
    big = np.full((4, 64), 3.0e38) * rng.choice([-1.0, 1.0], (4, 64))                 # sums overflow
    tiny = rng.laplace(0, 1, (4, 64)) * 2.0 ** -128                                    # subnormal bf16
    zeros = np.zeros((2, 64)); zeros[1, ::2] = -0.0
    bits = np.concatenate([datagen.f32_to_bf16_bits(a.astype(np.float32)) for a in (wide, big, tiny, zeros)])
    want = RT.rotate_blocks(bits)
    assert np.array_equal(_rot(bits), want)
    x = to_dev_bf16(bits)
    nq.block_hadamard(x, out=x)                                                         # in place
    assert np.array_equal(to_host_bits(x), want)


def test_rotate_full_weights():
    """Both C4 weight shapes, every element."""
    for which in ("gate", "down"):
        note(f"block hadamard full {which}")
        w = datagen.config4_weights(which)
        assert np.array_equal(_rot(w), RT.rotate_blocks(w)), which


def test_hessian_hadamard():
    note("hessian hadamard")
    _, x = datagen.config2()
    h = N.hessian(x).astype(np.float32)
    ref = RT.rotate_hessian(h.astype(np.float64))
    H = torch.from_numpy(h).to(DEV)
    got = host(nq.hessian_hadamard(H))
    assert rel_frobenius(got, ref).max() <= 1e-6
    nq.hessian_hadamard(H, out=H)                                                      # in place
    assert np.array_equal(host(H), got)
    eye = torch.eye(16, dtype=torch.float32, device=DEV).repeat(5, 1, 1).contiguous()
    assert np.array_equal(host(nq.hessian_hadamard(eye)), np.tile(np.eye(16, dtype=np.float32), (5, 1, 1)))


@pytest.mark.parametrize("cfg", [1, 2])
def test_rotated_sweep(cfg):
    """Sweep of the rotated weights under the rotated Hessian, GPU end to end
    (rotate, rotate H, scale_2, sweep) against the oracle's."""
    note(f"rotated sweep config{cfg}")
    w, x = datagen.config1() if cfg == 1 else datagen.config2()
    h32 = N.hessian(x).astype(np.float32)
    wr_ref = RT.rotate_blocks(w)
    hr_ref = RT.rotate_hessian(h32.astype(np.float64)).astype(np.float32)
    _, s2_ref = N.tensor_scale(wr_ref)
    wr = nq.block_hadamard(to_dev_bf16(w))
    hr = nq.hessian_hadamard(torch.from_numpy(h32).to(DEV))
    s2, _ = nq.compute_scale2(wr)
    assert float(host(s2)[0]) == s2_ref
    packed, codes, cost = nq.scale_sweep(wr, hr, s2, want_cost=True)
    rows = w.shape[0] if cfg == 1 else 64
    compare_sweep(wr_ref[:rows], hr_ref, s2_ref, host(packed)[:rows], host(codes)[:rows], host(cost)[:rows])
