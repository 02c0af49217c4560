"""GPU parity: the W4A4 Hessian (H from the fake-quantized input, quantized in
registers inside the accumulation pass) against the oracle's
hessian_fakequant = hessian(dequant(quantize_dynamic(x))).

Bars:
* one token per launch: H_g is a single outer product xh^T xh, exact in fp32,
  so it must equal the oracle's bit for bit -- a wrong code, nibble or
  dequantized value anywhere shows up here;
* many tokens: relative Frobenius error <= 1e-5 per block (fp32 partial sums,
  as for the plain Hessian), bitwise reproducible;
* the fused amax is the raw max |x|, exact.
Every E2M1 decision path (fast, two-float, nudged, exact) meets the same bars.
Inputs come from datagen; expected values from the oracle only."""
import numpy as np
import pytest
import torch

import datagen
from oracle import nvfp4 as N
from oracle import formats as F
import nvfp4_post_quantization_amd as nq

from _gpu import DEV, need_gpu, note, to_dev_bf16, to_dev_f32, host, rel_frobenius

pytestmark = pytest.mark.gpu
TOL = 1e-5


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.fixture(params=["fast", "twofloat", "nudged", "exact"])
def path(request, monkeypatch):
    flag = {"fast": None, "twofloat": "2", "nudged": "3", "exact": "1"}[request.param]
    if flag is None:
        monkeypatch.delenv("NVFP4MI_FORCE_EXACT", raising=False)
    else:
        monkeypatch.setenv("NVFP4MI_FORCE_EXACT", flag)
    return request.param


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _run(bits: np.ndarray, s2: float, chunks=1, ld=None, h0=None):
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
    s2_dev = to_dev_f32([s2])
    bounds = np.linspace(0, t, chunks + 1).astype(int)
    for a, b in zip(bounds[:-1], bounds[1:]):
        nq.hessian_accum_fq(x[a:b], s2_dev, H, amax)
    return host(H), float(host(amax)[0])


def _check(bits, s2=None, **kw):
    if s2 is None:
        s2 = N.tensor_scale(bits)[1]
    h, am = _run(bits, s2, **kw)
    ref = N.hessian_fakequant(bits, s2, h_init=kw.get("h0"))
    err = rel_frobenius(h, ref)
    assert err.max() <= TOL, f"max rel Frobenius error {err.max():.3e}"
    assert am == float(np.max(np.abs(F.bf16_bits_to_f64(bits))))
    return h, ref


def _single_tokens(rng, n, k):
    """Rows of varied character: Laplace with outliers, normal, values packed
    around E2M1 rounding midpoints, a zero block, tiny and huge blocks."""
    rows = []
    for i in range(n):
        kind = i % 4
        if kind == 0:
            r = rng.laplace(0, 1, k)
            r[rng.choice(k, 8, replace=False)] *= 40.0
        elif kind == 1:
            r = rng.standard_normal(k) * 0.02
        elif kind == 2:
            mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
            r = rng.choice(mids, k) * rng.choice([-1.0, 1.0], k) * (1.0 + rng.uniform(-1e-3, 1e-3, k))
            r[::16] = 6.0 * np.sign(rng.standard_normal(k // 16) + 1e-9)       # block max 6
        else:
            r = rng.standard_normal(k)
            r[:16] = 0.0
            r[16:32] *= 1e-6
            r[32:48] *= 1e3
        rows.append(r)
    return datagen.f32_to_bf16_bits(np.array(rows, dtype=np.float32))


def test_fq_single_token_exact(path):
    """One token per launch: H must equal the oracle's outer products exactly."""
    note(f"hessian_fq single tokens path={path}")
    rng = np.random.default_rng(42)
    x = _single_tokens(rng, 8, 16384)
    s2 = N.tensor_scale(x)[1]
    for i in range(x.shape[0]):
        h, _ = _run(x[i:i + 1], s2)
        ref = N.hessian_fakequant(x[i:i + 1], s2)
        assert np.array_equal(h, ref.astype(np.float32)), f"row {i}: H differs from the oracle"
        assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref), "oracle not exact in fp32"


def test_fq_config1(path):
    note(f"hessian_fq config1 path={path}")
    _, x = datagen.config1()
    _check(x)


def test_fq_config2_chunked_and_reproducible(path):
    note(f"hessian_fq config2 chunked path={path}")
    _, x = datagen.config2()
    h1, ref = _check(x, chunks=3)
    s2 = N.tensor_scale(x)[1]
    h2, _ = _run(x, s2, chunks=3)
    assert np.array_equal(h1, h2), "accumulation must be bitwise reproducible"
    # the quantized input's Hessian is not the raw one
    assert rel_frobenius(ref, N.hessian(x)).max() > 1e-3


@pytest.mark.parametrize("t,k,ld", [(1, 16, None), (63, 48, None), (65, 144, 152), (1000, 272, None),
                                    (3, 4096, None), (777, 2064, 2072)])
def test_fq_ragged(t, k, ld):
    note(f"hessian_fq t={t} k={k} ld={ld}")
    rng = np.random.default_rng(t + k)
    x = datagen.f32_to_bf16_bits(rng.laplace(0, 1, (t, k)).astype(np.float32))
    _check(x, ld=ld)


def test_fq_accumulates_into_existing():
    note("hessian_fq accumulate into existing H")
    rng = np.random.default_rng(5)
    x = datagen.f32_to_bf16_bits(rng.standard_normal((200, 64)).astype(np.float32))
    h0 = N.hessian(datagen.f32_to_bf16_bits(rng.standard_normal((50, 64)).astype(np.float32)))
    _check(x, h0=h0.astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("factor", [1.0 / 64, 64.0, 4096.0])
def test_fq_scale_off_calibration(path, factor):
    """A tensor scale far below the input's (blocks saturate at code 126) or
    far above it (small blocks quantize to zero)."""
    note(f"hessian_fq scale x{factor} path={path}")
    rng = np.random.default_rng(9)
    x = datagen.f32_to_bf16_bits(rng.laplace(0, 1, (300, 512)).astype(np.float32))
    s2 = float(np.float32(N.tensor_scale(x)[1] * factor))
    _check(x, s2=s2)


@pytest.mark.parametrize("stream_id", [0, 1])
def test_fq_full_chunks(stream_id):
    """Two whole 65536-token chunks of a calibration stream (K = 4096 or
    12288), as the benchmark runs them: sampled groups against the oracle."""
    k = datagen.C4_HIDDEN if stream_id == 0 else datagen.C4_INTER
    note(f"hessian_fq full chunks stream={stream_id} k={k}")
    groups = k // 16
    rng = np.random.default_rng(300 + stream_id)
    gs = np.sort(rng.choice(groups, 8, replace=False))
    gs = np.unique(np.concatenate([gs, datagen.config4_outlier_channels(stream_id) // 16]))
    cols_dev = torch.as_tensor((gs[:, None] * 16 + np.arange(16)).reshape(-1), device=DEV)
    H = torch.zeros((groups, 16, 16), dtype=torch.float32, device=DEV)
    amax = torch.zeros(1, dtype=torch.float32, device=DEV)
    ws = torch.empty(nq.hessian_workspace_bytes(datagen.C4_CHUNK, k), dtype=torch.uint8, device=DEV)
    # the activations' tensor scale from step 1 over the first chunk (oracle)
    x = datagen.config4_chunk_torch(stream_id, 0, DEV)
    am0, s2 = 0.0, 0.0
    for r0 in range(0, x.shape[0], 8192):
        a, s = N.tensor_scale(_bits(x[r0:r0 + 8192]))
        if a > am0:
            am0, s2 = a, s
    del x
    s2_dev = to_dev_f32([s2])
    ref = np.zeros((len(gs), 16, 16))
    amax_ref = 0.0
    for chunk in range(2):
        x = datagen.config4_chunk_torch(stream_id, chunk, DEV)
        nq.hessian_accum_fq(x, s2_dev, H, amax=amax, workspace=ws)
        ref = N.hessian_fakequant(_bits(x.index_select(1, cols_dev)), s2, h_init=ref)
        for r0 in range(0, x.shape[0], 8192):
            amax_ref = max(amax_ref, N.tensor_scale(_bits(x[r0:r0 + 8192]))[0])
        del x
    err = rel_frobenius(host(H)[gs], ref)
    assert err.max() <= TOL, f"max rel Frobenius error {err.max():.3e}"
    assert float(host(amax)[0]) == amax_ref


@pytest.mark.parametrize("t,k", [(130, 132096), (200, 131200)])
def test_fq_wide_k_ranges_cross_slabs(t, k):
    """The fake-quant kernel's larger grid: more slabs than its workgroups,
    so work ranges cross slab boundaries (multi-slot partials)."""
    note(f"hessian_fq wide k t={t} k={k}")
    rng = np.random.default_rng(t * k)
    x = datagen.f32_to_bf16_bits(rng.laplace(0, 1, (t, k)).astype(np.float32))
    _check(x)


@pytest.mark.parametrize("t,k,chunks", [(1000, 272, 3), (4096, 2048, 5), (64, 512, 64)])
def test_fq_chunk_list(path, t, k, chunks):
    """Several chunks in one W4A4 call: H against the oracle over all chunks'
    tokens, bitwise reproducible, the raw amax over every chunk, and within
    the bound of the per-chunk calls."""
    note(f"hessian_fq chunk list t={t} k={k} chunks={chunks} path={path}")
    rng = np.random.default_rng(t + k + chunks)
    bits = [datagen.f32_to_bf16_bits(rng.laplace(0, 1, (t, k)).astype(np.float32)) for _ in range(chunks)]
    allbits = np.concatenate(bits, axis=0)
    s2 = N.tensor_scale(allbits)[1]
    xs = [to_dev_bf16(b) for b in bits]
    s2_dev = to_dev_f32([s2])
    runs = []
    for _ in range(2):
        H = torch.zeros((k // 16, 16, 16), dtype=torch.float32, device=DEV)
        amax = torch.zeros(1, dtype=torch.float32, device=DEV)
        nq.hessian_accum_fq_chunks(xs, s2_dev, H, amax)
        runs.append((host(H), float(host(amax)[0])))
    assert np.array_equal(runs[0][0], runs[1][0]), "chunk-list accumulation must be bitwise reproducible"
    ref = N.hessian_fakequant(allbits, s2)
    assert rel_frobenius(runs[0][0], ref).max() <= TOL
    assert runs[0][1] == float(np.max(np.abs(F.bf16_bits_to_f64(allbits))))
    Hs = torch.zeros((k // 16, 16, 16), dtype=torch.float32, device=DEV)
    for x in xs:
        nq.hessian_accum_fq(x, s2_dev, Hs)
    assert rel_frobenius(host(Hs), ref).max() <= TOL
