"""GPU parity at the benchmark's full sizes, in the launch configuration that
bench.py times (same shapes, strides and entry points):

* Hessian of whole 65536-token calibration chunks of both MLP input streams
  (K = 4096 and K = 12288), two chunks accumulated: sampled groups against the
  oracle, and the fused amax over every element;
* the scale sweep of the full gate [12288, 4096] and down [4096, 12288]
  weights: sampled rows against the oracle's full 127-code sweep, and for
  every block the nibbles at the GPU's code and the cost bound of the
  max-based code (a candidate of the sweep);
* the MXFP4 -> NVFP4 cast of all 128 expert pairs [2048, 7168]: sampled
  experts bit for bit, and for every expert the fallback count and scale_2.

Inputs come from datagen; expected values from the oracle only."""
import numpy as np
import pytest
import torch

import datagen
from oracle import nvfp4 as N
from oracle import formats as F
from oracle import mxcast as M
import nvfp4_post_quantization_amd as nq

from _gpu import DEV, need_gpu, note, to_dev_bf16, to_dev_u8, to_dev_f32, host, rel_frobenius, compare_sweep

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("stream_id", [0, 1])
def test_hessian_full_chunks(stream_id):
    k = datagen.C4_HIDDEN if stream_id == 0 else datagen.C4_INTER
    note(f"hessian full chunks stream={stream_id} k={k}")
    groups = k // 16
    rng = np.random.default_rng(100 + stream_id)
    gs = np.sort(rng.choice(groups, 24, replace=False))
    outl = datagen.config4_outlier_channels(stream_id) // 16
    gs = np.unique(np.concatenate([gs, outl]))               # include the outlier groups
    cols = (gs[:, None] * 16 + np.arange(16)).reshape(-1)
    H = torch.zeros((groups, 16, 16), dtype=torch.float32, device=DEV)
    amax = torch.zeros(1, dtype=torch.float32, device=DEV)
    ws = torch.empty(nq.hessian_workspace_bytes(datagen.C4_CHUNK, k), dtype=torch.uint8, device=DEV)
    ref = np.zeros((len(gs), 16, 16))
    amax_ref = 0.0
    cols_dev = torch.as_tensor(cols, device=DEV)
    for chunk in range(2):
        x = datagen.config4_chunk_torch(stream_id, chunk, DEV)
        nq.hessian_accum(x, H, amax=amax, workspace=ws)
        ref = N.hessian(_bits(x.index_select(1, cols_dev)), h_init=ref)
        for r0 in range(0, x.shape[0], 8192):                 # amax over every element, in slices
            amax_ref = max(amax_ref, N.tensor_scale(_bits(x[r0:r0 + 8192]))[0])
        del x
    h = host(H)[gs]
    err = rel_frobenius(h, ref)
    assert err.max() <= 1e-5, f"max rel Frobenius error {err.max():.3e}"
    assert float(host(amax)[0]) == amax_ref


@pytest.mark.parametrize("which", ["gate", "down"])
def test_sweep_full_weight(which):
    note(f"sweep full weight {which}")
    w_bits = datagen.config4_weights(which)
    rows, k = w_bits.shape
    stream_id = 0 if which == "gate" else 1
    h = N.hessian(datagen.config4_chunk_host(stream_id, 0, tokens=8192)).astype(np.float32)
    _, s2 = N.tensor_scale(w_bits)
    H = torch.from_numpy(h).to(DEV)
    packed, codes, cost = nq.scale_sweep(to_dev_bf16(w_bits), H, to_dev_f32([s2]), want_cost=True)
    packed, codes, cost = host(packed), host(codes), host(cost)

    # sampled rows: the oracle's full 127-code sweep
    sr = np.sort(np.random.default_rng(7).choice(rows, 32, replace=False))
    compare_sweep(w_bits[sr], h, s2, packed[sr], codes[sr], cost[sr])

    # every block: nibbles at the GPU's code, and its cost no worse than the
    # max-based code's (that code is one of the candidates)
    g = k // 16
    w = F.bf16_bits_to_f64(w_bits).reshape(rows, g, 16)
    nib, wq = N.quantize_at_code(w, codes, s2)
    assert np.array_equal(packed, F.pack_nibbles(nib.reshape(rows, k))), "nibbles differ"
    h64 = h.astype(np.float64)

    def costs_of(wq_):
        e = (w - wq_).transpose(1, 0, 2)                       # [g, rows, 16]
        return np.sum(np.matmul(e, h64) * e, axis=2).T         # [rows, g]

    c_gpu = costs_of(wq)
    del nib, wq
    _, wq_max = N.quantize_at_code(w, N.max_code(np.max(np.abs(w), axis=2), s2), s2)
    c_max = costs_of(wq_max)
    w0 = np.sum(np.matmul(w.transpose(1, 0, 2), h64) * w.transpose(1, 0, 2), axis=2).T
    assert np.all(c_gpu <= c_max + 1e-5 * np.maximum(c_max, 1e-6 * w0)), "worse than the max-based code"
    assert np.all(np.abs(cost - c_gpu) <= 1e-4 * np.maximum(c_gpu, 1e-6 * w0) + 1e-30), "cost output off"


def test_cast_all_experts():
    note("cast all 128 expert pairs [2048, 7168]")
    packed, e8, forced = datagen.config5()
    p_dev = to_dev_u8(packed)
    codes, s2, fb = nq.mxfp4_to_nvfp4_cast(p_dev, to_dev_u8(e8))
    codes, s2, fb = host(codes), host(s2), host(fb)
    experts = packed.shape[0]
    # every expert: fallback count = blocks the generator forced out of the
    # window; scale_2 = 2^(k_max - 8)
    assert np.array_equal(fb, forced.reshape(experts, -1).sum(axis=1))
    kmax = e8.reshape(experts, -1).astype(np.int64).max(axis=1) - 127
    assert np.array_equal(s2.astype(np.float64), np.ldexp(1.0, kmax - 8))
    # sampled experts, bit for bit (codes, rewritten nibbles, scale_2, count)
    for e in (0, 77, experts - 1):
        p_ref, c_ref, s2_ref, fb_ref = M.mxfp4_to_nvfp4(packed[e:e + 1], e8[e:e + 1])
        assert np.array_equal(codes[e:e + 1], c_ref)
        assert np.array_equal(p_dev[e:e + 1].cpu().numpy(), p_ref)
        assert float(s2[e]) == float(s2_ref[0]) and int(fb[e]) == int(fb_ref[0])
