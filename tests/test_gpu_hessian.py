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


@pytest.mark.parametrize("fill", ["zero", "ones", "random"])
def test_hessian_workspace_contents_do_not_matter(fill):
    """Any workspace contents give the same H, bit for bit, call after call on
    one workspace (the W4A4 variant's calls in between): every partial slot
    the reduce reads is written earlier in the same call."""
    note(f"hessian workspace contents: {fill}")
    rng = np.random.default_rng(21)
    shapes = [(3000, 1024), (130, 66048), (4096, 2048)]
    xs = [to_dev_bf16(datagen.f32_to_bf16_bits(rng.laplace(0, 1, s).astype(np.float32))) for s in shapes]
    need = max(nq.hessian_workspace_bytes(*s) for s in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    if fill == "ones":
        ws.fill_(0xFF)
    elif fill == "random":
        ws.copy_(torch.from_numpy(rng.integers(0, 256, need, dtype=np.uint8)))
    s2 = torch.tensor([0.01], dtype=torch.float32, device=DEV)
    for rep in range(2):
        for x in xs:
            k = x.shape[1]
            ref = torch.zeros((k // 16, 16, 16), dtype=torch.float32, device=DEV)
            nq.hessian_accum(x, ref)                                # its own fresh workspace
            ref_fq = torch.zeros_like(ref)
            nq.hessian_accum_fq(x, s2, ref_fq)
            h = torch.zeros_like(ref)
            nq.hessian_accum(x, h, workspace=ws)
            h_fq = torch.zeros_like(ref)
            nq.hessian_accum_fq(x, s2, h_fq, workspace=ws)
            h2 = torch.zeros_like(ref)
            nq.hessian_accum(x, h2, workspace=ws)
            assert torch.equal(h, ref) and torch.equal(h2, ref) and torch.equal(h_fq, ref_fq)


@pytest.mark.parametrize("t,k,chunks,ld", [(1000, 272, 3, None), (4096, 2048, 5, 2056), (130, 66048, 2, None),
                                           (65536, 4096, 2, None), (64, 512, 64, None), (7, 16, 2, None)])
def test_hessian_chunk_list(t, k, chunks, ld):
    """Several chunks in one call: H against the oracle over all chunks'
    tokens (accumulated into an existing H), within the per-chunk calls'
    bound of them, bitwise reproducible, and amax over every chunk."""
    note(f"hessian chunk list t={t} k={k} chunks={chunks} ld={ld}")
    rng = np.random.default_rng(t + k + chunks)
    bits = [datagen.f32_to_bf16_bits(rng.laplace(0, 1, (t, k)).astype(np.float32)) for _ in range(chunks)]
    bits[1][:, :16] *= 0                                    # an all-zero group in one chunk
    def dev(b):
        if ld is None:
            return to_dev_bf16(b)
        full = np.zeros((t, ld), np.uint16)
        full[:, :k] = b
        return to_dev_bf16(full)[:, :k]
    xs = [dev(b) for b in bits]
    h0 = N.hessian(datagen.f32_to_bf16_bits(rng.standard_normal((50, k)).astype(np.float32))).astype(np.float32)
    runs = []
    for _ in range(2):
        H = torch.from_numpy(h0.copy()).to(DEV)
        amax = torch.zeros(1, dtype=torch.float32, device=DEV)
        nq.hessian_accum_chunks(xs, H, amax)
        runs.append((host(H), float(host(amax)[0])))
    assert np.array_equal(runs[0][0], runs[1][0]), "chunk-list accumulation must be bitwise reproducible"
    allbits = np.concatenate(bits, axis=0)
    ref = N.hessian(allbits, h_init=h0.astype(np.float64))
    err = rel_frobenius(runs[0][0], ref)
    assert err.max() <= TOL, f"max rel Frobenius error {err.max():.3e}"
    assert runs[0][1] == float(np.max(np.abs(F.bf16_bits_to_f64(allbits))))
    Hs = torch.from_numpy(h0.copy()).to(DEV)
    for x in xs:
        nq.hessian_accum(x, Hs)
    assert rel_frobenius(host(Hs), ref).max() <= TOL


def test_hessian_chunk_list_empty_chunks():
    """Chunks without tokens leave H and amax as they were."""
    note("hessian chunk list: empty chunks")
    xs = [torch.empty((0, 64), dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    H = torch.full((4, 16, 16), 1.5, dtype=torch.float32, device=DEV)
    amax = torch.full((1,), 2.0, dtype=torch.float32, device=DEV)
    nq.hessian_accum_chunks(xs, H, amax)
    assert torch.equal(H, torch.full_like(H, 1.5)) and float(host(amax)[0]) == 2.0
