"""The measurement entry points (include/nvfp4mi_probe.h) on the GPU:
* the HBM probes do what they say (write fills, copy copies, read leaves its
  sink alone on zeros and stores the fold when it equals the marker);
* the sweep's counting build gives nvfp4_scale_sweep's outputs bit for bit,
  and its counters are consistent: blocks and waves exact, every block
  evaluates code 0, no block more than all 127 codes, evaluations within the
  wave steps' lane slots, forms and screens within the steps."""
import numpy as np
import pytest
import torch

import datagen
from oracle import nvfp4 as N
import nvfp4_post_quantization_amd as nq

from _gpu import DEV, need_gpu, note, to_dev_bf16, host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _sp():
    return torch.cuda.current_stream(DEV).cuda_stream


def test_probe_write_copy_read():
    lib = nq.load()
    note("probes: write, copy, read on 1 MiB + 48 B")
    n = (1 << 20) + 48
    a = torch.empty(n, dtype=torch.uint8, device=DEV)
    assert lib.nvfp4_probe_write(a.data_ptr(), n, 0x01020304, 7, _sp()) == 0
    words = host(a).view(np.uint32)
    assert np.all(words == 0x01020304)
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device=DEV)
    dst = torch.zeros(n, dtype=torch.uint8, device=DEV)
    assert lib.nvfp4_probe_copy(src.data_ptr(), dst.data_ptr(), n, 3, _sp()) == 0
    assert torch.equal(host_t(src), host_t(dst))
    sink = torch.full((4,), 7, dtype=torch.int32, device=DEV)
    z = torch.zeros(n, dtype=torch.uint8, device=DEV)
    assert lib.nvfp4_probe_read(z.data_ptr(), n, sink.data_ptr(), 0, _sp()) == 0
    assert host(sink).tolist() == [7, 7, 7, 7]
    # one 16-byte word holding the marker: the fold equals it and is stored
    m = torch.zeros(n, dtype=torch.uint8, device=DEV)
    m[:4] = torch.tensor(list((0x9E3779B9).to_bytes(4, "little")), dtype=torch.uint8, device=DEV)
    assert lib.nvfp4_probe_read(m.data_ptr(), n, sink.data_ptr(), 5, _sp()) == 0
    assert host(sink).view(np.uint32)[0] == 0x9E3779B9


def host_t(t):
    torch.cuda.synchronize()
    return t.cpu()


@pytest.mark.parametrize("case", ["c1", "c2", "ragged", "zero_scale"])
def test_sweep_stats_matches_sweep(case):
    note(f"sweep stats {case}")
    if case == "c1":
        w_bits, x_bits = datagen.config1()
    elif case == "c2":
        w_bits, x_bits = datagen.config2()
    else:
        rng = np.random.default_rng(11)
        w_bits = datagen.normal_bf16(rng, (97, 336), 0.02)
        x_bits = datagen.laplace_bf16(rng, (300, 336), 1.0)
    if case == "zero_scale":
        w_bits = np.zeros_like(w_bits)
    rows, k = w_bits.shape
    H = torch.from_numpy(N.hessian(x_bits).astype(np.float32)).to(DEV)
    w = to_dev_bf16(w_bits)
    s2, _ = nq.compute_scale2(w)
    p0, c0, _ = nq.scale_sweep(w, H, s2)
    p1, c1, st = nq.scale_sweep_stats(w, H, s2)
    assert torch.equal(p0, p1) and torch.equal(c0, c1)
    evals, steps, forms, screens, blocks, waves = (int(v) for v in host(st))
    groups = k // 16
    assert blocks == rows * groups
    assert groups <= waves <= groups * ((rows + 63) // 64)     # a wave per group and row range
    assert blocks <= evals <= 127 * blocks
    assert evals <= 64 * steps
    assert forms <= steps and screens <= steps
    if case == "zero_scale":
        assert evals == blocks                              # code 0 only: cost 0 ends every search
    # a second call accumulates
    _, _, st2 = nq.scale_sweep_stats(w, H, s2, stats=st.clone())
    assert np.array_equal(host(st2), 2 * host(st))
