"""GPU parity at the benchmark's full sizes, in the launch configurations that
bench.py times (same shapes, strides, entry points and chunking):

* the Hessian of both MLP calibration streams (K = 4096 and K = 12288), all
  16 device-drawn 65536-token chunks of each (2^20 tokens), every group
  against the oracle's float64 sum over the same tokens, and the fused amax
  over every element;
* the scale sweep of the full gate, up [12288, 4096] and down [4096, 12288]
  weights under those very Hessians (the GPU's fp32 H is the input on both
  sides), capped at one workgroup per CU as in the timed steps and uncapped
  as in the serial pass (identical outputs): every row against the oracle's
  full 127-code sweep (NVFP4MI_SWEEP_SAMPLE=n limits this to a seeded
  sample of n rows per weight, for quick runs), and for every block the
  nibbles at the GPU's code and the cost bound of the max-based code (one of
  the sweep's candidates);
* the Gemma-2B-like q_proj [2048, 2048]: H of its 4096 calibration tokens
  and the sweep of all 2048 rows against the oracle;
* the MXFP4 -> NVFP4 cast of all 128 expert pairs [2048, 7168], every expert
  bit for bit (codes, rewritten nibbles, scale_2, fallback count).

Inputs come from datagen (the C4 chunks drawn on the device, as the benchmark
draws them, and read back); expected values from the oracle only, run in a
pool of worker processes (tests/_pool.py)."""
import os

import numpy as np
import pytest
import torch

import datagen
from oracle import nvfp4 as N
from oracle import formats as F
import nvfp4_post_quantization_amd as nq

import _pool
from _gpu import DEV, need_gpu, note, to_dev_bf16, to_dev_u8, host, rel_frobenius, compare_sweep

pytestmark = pytest.mark.gpu

# rows of each C4 weight compared with the oracle's sweep: all of them,
# unless NVFP4MI_SWEEP_SAMPLE names a smaller seeded sample
SWEEP_SAMPLE = int(os.environ.get("NVFP4MI_SWEEP_SAMPLE", "0"))
HIN = {"gate": 0, "up": 0, "down": 1}


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.fixture(scope="module")
def pool():
    p = _pool.make_pool()
    yield p
    p.shutdown(cancel_futures=True)


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class _FullH:
    """Both calibration streams' Hessians over all 2^20 tokens, computed once
    per module: on the GPU by one chunk-list call over the 16 resident chunks
    as the benchmark does ("H", the sweeps' input below), and chunk by chunk
    ("H_single"); and by the oracle over (token, channel) pieces of the same
    chunks."""

    def __init__(self, pool):
        self.pool = pool
        self.res = {}

    def __call__(self, stream_id):
        if stream_id not in self.res:
            self.res[stream_id] = self._run(stream_id)
        return self.res[stream_id]

    def _run(self, s):
        k = datagen.C4_HIDDEN if s == 0 else datagen.C4_INTER
        groups = k // 16
        tp, cp = 16384, 1024                              # piece: 16384 tokens x 64 groups
        H1 = torch.zeros((groups, 16, 16), dtype=torch.float32, device=DEV)
        amax1 = torch.zeros(1, dtype=torch.float32, device=DEV)
        ws = torch.empty(nq.hessian_workspace_bytes(datagen.C4_CHUNK, k), dtype=torch.uint8, device=DEV)
        xs = []
        ref = np.zeros((groups, 16, 16))
        amax_ref = 0.0
        pending = []                                      # (chunk, [(c0, future)])

        def drain(item):
            nonlocal amax_ref
            for c0, fut in item[1]:
                h, a = fut.result()
                ref[c0 // 16:(c0 + cp) // 16] += h
                amax_ref = max(amax_ref, a)

        for chunk in range(datagen.C4_TOKENS // datagen.C4_CHUNK):
            note(f"full H stream={s} k={k} chunk={chunk}")
            x = datagen.config4_chunk_torch(s, chunk, DEV)
            nq.hessian_accum(x, H1, amax=amax1, workspace=ws)
            xb = _bits(x)
            xs.append(x)
            futs = [(c0, self.pool.submit(_pool.hessian_piece, np.ascontiguousarray(xb[t0:t0 + tp, c0:c0 + cp])))
                    for c0 in range(0, k, cp) for t0 in range(0, xb.shape[0], tp)]
            del xb
            pending.append((chunk, futs))
            if len(pending) > 2:                          # bound the host copies in flight
                drain(pending.pop(0))
        note(f"full H stream={s}: chunk-list call over {len(xs)} chunks")
        H = torch.zeros((groups, 16, 16), dtype=torch.float32, device=DEV)
        amax = torch.zeros(1, dtype=torch.float32, device=DEV)
        nq.hessian_accum_chunks(xs, H, amax)
        torch.cuda.synchronize()
        del xs
        torch.cuda.empty_cache()
        for item in pending:
            drain(item)
        return {"H": H, "amax": float(host(amax)[0]), "H_single": H1, "amax_single": float(host(amax1)[0]),
                "ref": ref, "amax_ref": amax_ref}


@pytest.fixture(scope="module")
def full_h(pool):
    return _FullH(pool)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("stream_id", [0, 1])
def test_hessian_all_chunks(full_h, stream_id):
    r = full_h(stream_id)
    for key, am in (("H", "amax"), ("H_single", "amax_single")):
        h = host(r[key]).astype(np.float64)
        err = rel_frobenius(h, r["ref"])
        assert err.max() <= 1e-5, f"{key}: max rel Frobenius error {err.max():.3e} (group {int(err.argmax())})"
        assert r[am] == r["amax_ref"]


def _every_block_checks(w_bits, h32, s2, packed, codes, cost):
    """For every block: nibbles equal the oracle's quantization at the GPU's
    code, and the GPU's choice costs no more than the max-based code's (a
    candidate of the sweep); the fp32 cost output is that cost within 1e-4."""
    rows, k = w_bits.shape
    g = k // 16
    w = F.bf16_bits_to_f64(w_bits).reshape(rows, g, 16)
    nib, wq = N.quantize_at_code(w, codes, s2)
    assert np.array_equal(packed, F.pack_nibbles(nib.reshape(rows, k))), "nibbles differ"
    del nib
    h64 = h32.astype(np.float64)

    def costs_of(wq_):
        e = (w - wq_).transpose(1, 0, 2)                  # [g, rows, 16]
        return np.sum(np.matmul(e, h64) * e, axis=2).T    # [rows, g]

    c_gpu = costs_of(wq)
    del wq
    _, wq_max = N.quantize_at_code(w, N.max_code(np.max(np.abs(w), axis=2), s2), s2)
    c_max = costs_of(wq_max)
    del wq_max
    wt = w.transpose(1, 0, 2)
    w0 = np.sum(np.matmul(wt, h64) * wt, axis=2).T
    assert np.all(c_gpu <= c_max + 1e-5 * np.maximum(c_max, 1e-6 * w0)), "worse than the max-based code"
    assert np.all(np.abs(cost - c_gpu) <= 1e-4 * np.maximum(c_gpu, 1e-6 * w0) + 1e-30), "cost output off"


@pytest.mark.timeout(900)
@pytest.mark.parametrize("which", ["gate", "up", "down"])
def test_sweep_full_weight_full_h(full_h, pool, which):
    r = full_h(HIN[which])
    note(f"sweep full weight {which} under the 2^20-token H")
    w_bits = datagen.config4_weights(which)
    rows, k = w_bits.shape
    w = to_dev_bf16(w_bits)
    s2_dev, am = nq.compute_scale2(w)
    amax_ref, s2 = N.tensor_scale(w_bits)
    assert float(host(s2_dev)[0]) == s2 and float(host(am)[0]) == amax_ref
    capped = nq.scale_sweep(w, r["H"], s2_dev, want_cost=True, wgs_per_cu=1)
    plain = nq.scale_sweep(w, r["H"], s2_dev, want_cost=True)
    packed, codes, cost = (host(t) for t in capped)
    for a, b, name in zip((packed, codes, cost), (host(t) for t in plain), ("packed", "codes", "cost")):
        assert np.array_equal(a, b), f"capped and uncapped sweeps differ in {name}"
    h32 = host(r["H"])

    # every row (or a seeded sample): the oracle's full 127-code sweep, in
    # slices of 1024 rows to bound the host memory of the cost tables
    if 0 < SWEEP_SAMPLE < rows:
        sr = np.sort(np.random.default_rng(7 + HIN[which] + (which == "up")).choice(
            rows, SWEEP_SAMPLE, replace=False))
    else:
        sr = np.arange(rows)
    n_mism = 0
    for i in range(0, len(sr), 1024):
        rs = sr[i:i + 1024]
        costs = _pool.sweep_costs(pool, w_bits[rs], h32.astype(np.float64), s2,
                                  rows_per_item=16 if k == 4096 else 8)
        n_mism += compare_sweep(w_bits[rs], h32, s2, packed[rs], codes[rs], cost[rs], costs=costs)
        del costs
    assert n_mism <= 1e-4 * len(sr) * (k // 16)
    _every_block_checks(w_bits, h32, s2, packed, codes, cost)


@pytest.mark.timeout(600)
def test_c2_hessian_and_sweep_all_rows(pool):
    """Gemma-2B-like q_proj [2048, 2048] with its 4096 calibration tokens:
    the GPU's H against the oracle, then every row of the sweep (under the
    GPU's H) against the oracle's full sweep."""
    note("C2 q_proj: H of 4096 tokens, sweep of all 2048 rows")
    w_bits, x_bits = datagen.config2()
    k = w_bits.shape[1]
    H = torch.zeros((k // 16, 16, 16), dtype=torch.float32, device=DEV)
    amax = torch.zeros(1, dtype=torch.float32, device=DEV)
    nq.hessian_accum(to_dev_bf16(x_bits), H, amax=amax)
    h32 = host(H)
    ref = N.hessian(x_bits)
    assert rel_frobenius(h32.astype(np.float64), ref).max() <= 1e-5
    assert float(host(amax)[0]) == N.tensor_scale(x_bits)[0]
    w = to_dev_bf16(w_bits)
    s2_dev, _ = nq.compute_scale2(w)
    s2 = N.tensor_scale(w_bits)[1]
    assert float(host(s2_dev)[0]) == s2
    packed, codes, cost = (host(t) for t in nq.scale_sweep(w, H, s2_dev, want_cost=True))
    capped = nq.scale_sweep(w, H, s2_dev, want_cost=True, wgs_per_cu=1)
    for a, b in zip((packed, codes, cost), (host(t) for t in capped)):
        assert np.array_equal(a, b), "capped and uncapped sweeps differ"
    costs = _pool.sweep_costs(pool, w_bits, h32.astype(np.float64), s2, rows_per_item=32)
    compare_sweep(w_bits, h32, s2, packed, codes, cost, costs=costs)


@pytest.mark.timeout(900)
def test_cast_all_experts_bit_exact(pool):
    note("cast all 128 expert pairs [2048, 7168]")
    packed, e8, forced = datagen.config5()
    p_dev = to_dev_u8(packed)
    codes, s2, fb = nq.mxfp4_to_nvfp4_cast(p_dev, to_dev_u8(e8))
    codes, s2, fb = host(codes), host(s2), host(fb)
    p_out = host(p_dev)
    del p_dev
    experts = packed.shape[0]
    # the generator's forced blocks are exactly the fallback blocks
    assert np.array_equal(fb, forced.reshape(experts, -1).sum(axis=1))
    p_ref, c_ref, s2_ref, fb_ref = _pool.cast(pool, packed, e8)
    for e in range(experts):
        assert np.array_equal(codes[e], c_ref[e]), f"codes differ in expert {e}"
        assert np.array_equal(p_out[e], p_ref[e]), f"nibbles differ in expert {e}"
    assert np.array_equal(s2.astype(np.float64), s2_ref)
    assert np.array_equal(fb, fb_ref)
