"""GPU parity: FP8 E4M3 per-tensor static tier (scale, quantize, dequant)
against the oracle, bit for bit.

* every finite bf16 pattern, at scales from subnormal to huge (and 0), on
  both quantizer paths (certified hardware convert and exact thresholds);
* the C1-C3 tensors, ragged and strided shapes;
* the full C3 activation tensor [8192, 4096]: every element against the
  oracle's code table for all 65,536 patterns at that scale;
* dequant of all 256 codes (NaN codes compared as NaN).
Inputs come from datagen; expected values from the oracle only."""
import numpy as np
import pytest
import torch

import datagen
from oracle import fp8 as P8
from oracle import formats as F
import nvfp4_post_quantization_amd as nq

from _gpu import DEV, need_gpu, note, to_dev_bf16, to_dev_u8, to_dev_f32, host, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.fixture(params=["fast", "exact"])
def path(request, monkeypatch):
    if request.param == "fast":
        monkeypatch.delenv("NVFP4MI_FORCE_EXACT", raising=False)
    else:
        monkeypatch.setenv("NVFP4MI_FORCE_EXACT", "1")
    return request.param


def _finite_patterns():
    b = np.arange(0x10000, dtype=np.uint32)
    b = b[(b & 0x7F80) != 0x7F80]                  # drop Inf / NaN
    return b.astype(np.uint16).reshape(-1, 256)    # 255 x 256


def _quantize(bits, s, ld=None):
    rows, k = bits.shape
    if ld is None:
        x = to_dev_bf16(bits)
    else:
        full = np.zeros((rows, ld), np.uint16)
        full[:, :k] = bits
        x = to_dev_bf16(full)[:, :k]
    return host(nq.fp8_quantize(x, to_dev_f32([s])))


SCALES = [1.0 / 3.0, 2.0 ** -3, 0.01234, 2.0 ** -20, 1e-30, 2.0 ** -130, 1e-44, 0.0, 1e30, 3.0e38]


@pytest.mark.parametrize("s", SCALES)
def test_fp8_quantize_every_pattern(path, s):
    s = float(np.float32(s))
    note(f"fp8 quantize all patterns s={s!r} path={path}")
    bits = _finite_patterns()
    assert np.array_equal(_quantize(bits, s), P8.fp8_quantize(bits, s))


def test_fp8_scale_exact():
    note("fp8 scale")
    w1, x1 = datagen.config1()
    w2, x2 = datagen.config2()
    cases = [w1, x1, w2, x2, datagen.config3()[:1024],
             np.array([0x3F80], np.uint16), np.zeros(40, np.uint16), x1.reshape(-1)[:13]]
    for c in cases:
        flat = np.ascontiguousarray(c.reshape(-1))
        s, am = nq.fp8_compute_scale(to_dev_bf16(flat))
        a_ref, s_ref = P8.fp8_tensor_scale(flat)
        assert float(host(am)[0]) == a_ref
        assert float(host(s)[0]) == s_ref


@pytest.mark.parametrize("which", ["c1w", "c1x", "c2w", "c2x"])
def test_fp8_quantize_tensors(path, which):
    note(f"fp8 quantize {which} path={path}")
    w1, x1 = datagen.config1()
    w2, x2 = datagen.config2()
    bits = {"c1w": w1, "c1x": x1, "c2w": w2, "c2x": x2}[which]
    _, s = P8.fp8_tensor_scale(bits)
    q = _quantize(bits, s)
    assert np.array_equal(q, P8.fp8_quantize(bits, s))
    d = to_host_bits(nq.fp8_dequant(to_dev_u8(q), to_dev_f32([s])))
    assert np.array_equal(d, P8.fp8_dequant(q, s))


@pytest.mark.parametrize("rows,k,ld", [(1, 8, None), (333, 24, None), (7, 4104, 4112), (65, 264, 272),
                                       (1000, 16, 24)])
def test_fp8_ragged_and_strided(rows, k, ld):
    note(f"fp8 rows={rows} k={k} ld={ld}")
    rng = np.random.default_rng(rows * 7 + k)
    bits = datagen.f32_to_bf16_bits(rng.laplace(0, 1, (rows, k)).astype(np.float32))
    _, s = P8.fp8_tensor_scale(bits)
    q = _quantize(bits, s, ld=ld)
    assert np.array_equal(q, P8.fp8_quantize(bits, s))
    assert np.array_equal(to_host_bits(nq.fp8_dequant(to_dev_u8(q), to_dev_f32([s]))), P8.fp8_dequant(q, s))


@pytest.mark.parametrize("s", [0.0123, 1.0, 2.0 ** -133, 1e36, 0.0])
def test_fp8_dequant_all_codes(s):
    s = float(np.float32(s))
    note(f"fp8 dequant all codes s={s!r}")
    codes = np.tile(np.arange(256, dtype=np.uint8), (3, 1))
    got = to_host_bits(nq.fp8_dequant(to_dev_u8(codes), to_dev_f32([s])))
    with np.errstate(over="ignore", invalid="ignore"):
        want = P8.fp8_dequant(codes, s)
    nan = (codes & 0x7F) == 0x7F
    assert np.array_equal(got[~nan], want[~nan])
    g = got[nan].astype(np.uint32)
    assert np.all(((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0)), "NaN codes must decode to NaN"


def test_fp8_full_activation_tensor():
    """C3 X [8192, 4096] in the launch shape the benchmark times: the scale
    exactly, and every element's code against the oracle's table of all
    65,536 patterns at that scale; dequant likewise through the oracle."""
    note("fp8 full C3 tensor")
    xb = datagen.config3()
    x = to_dev_bf16(xb)
    s_dev, am = nq.fp8_compute_scale(x)
    a_ref, s = P8.fp8_tensor_scale(xb)
    assert float(host(am)[0]) == a_ref and float(host(s_dev)[0]) == s
    q = nq.fp8_quantize(x, s_dev)
    with np.errstate(invalid="ignore"):                     # the table includes the NaN patterns
        table = P8.fp8_quantize(np.arange(0x10000, dtype=np.uint32).astype(np.uint16), s)
    assert np.array_equal(host(q), table[xb])
    dq_table = P8.fp8_dequant(np.arange(256, dtype=np.uint8), s)
    got = to_host_bits(nq.fp8_dequant(q, s_dev))
    assert np.array_equal(got, dq_table[host(q)])


def test_fp8_empty():
    note("fp8 empty")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    s = to_dev_f32([1.0])
    assert nq.fp8_quantize(x, s).shape == (0, 64)
    assert nq.fp8_dequant(torch.empty((0, 64), dtype=torch.uint8, device=DEV), s).shape == (0, 64)
    sc, am = nq.fp8_compute_scale(torch.empty(0, dtype=torch.bfloat16, device=DEV))
    assert float(host(sc)[0]) == 0.0 and float(host(am)[0]) == 0.0
