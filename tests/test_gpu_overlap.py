"""GPU: the sweep's occupancy cap and concurrent execution beside the Hessian.

* nvfp4_scale_sweep_ex with one workgroup per CU gives the same packed
  nibbles, codes and costs as the uncapped sweep, bit for bit;
* a Hessian accumulation on one stream and capped sweeps on another stream,
  running at the same time, give exactly the results each gives alone (the
  schedule bench.py times).
Inputs come from datagen; the sweep itself is checked against the oracle in
test_gpu_sweep.py and test_gpu_fullsize.py."""
import numpy as np
import pytest
import torch

import datagen
from oracle import nvfp4 as N
import nvfp4_post_quantization_amd as nq

from _gpu import DEV, need_gpu, note, to_dev_bf16, host, compare_sweep

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _equal(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


def test_capped_sweep_equals_uncapped_config2():
    note("capped sweep config2")
    w, x = datagen.config2()
    h32 = N.hessian(x).astype(np.float32)
    wd = to_dev_bf16(w)
    H = torch.from_numpy(h32).to(DEV)
    s2, _ = nq.compute_scale2(wd)
    ref = nq.scale_sweep(wd, H, s2, want_cost=True)
    cap = nq.scale_sweep(wd, H, s2, want_cost=True, wgs_per_cu=1)
    assert _equal(ref, cap)
    rows = 32
    compare_sweep(w[:rows], h32, float(host(s2)[0]), host(cap[0])[:rows], host(cap[1])[:rows], host(cap[2])[:rows])


def test_sweeps_beside_hessian_on_another_stream():
    """Two 65536-token K = 12288 chunks accumulate on one stream while the
    gate and up weights are swept, capped, on a second stream; then the down
    weight is swept, capped, beside two K = 4096 chunks."""
    note("capped sweeps beside the Hessian")
    W = {n: to_dev_bf16(datagen.config4_weights(n)) for n in ("gate", "up")}
    x0 = datagen.config4_chunk_torch(0, 0, DEV)
    H0 = torch.zeros((256, 16, 16), dtype=torch.float32, device=DEV)
    nq.hessian_accum(x0, H0)
    del x0
    X1 = [datagen.config4_chunk_torch(1, c, DEV) for c in range(2)]
    s2 = {n: nq.compute_scale2(w)[0] for n, w in W.items()}
    ws = torch.empty(max(nq.hessian_workspace_bytes(65536, k) for k in (4096, 12288)), dtype=torch.uint8, device=DEV)

    # alone, one after the other
    H1_ref = torch.zeros((768, 16, 16), dtype=torch.float32, device=DEV)
    for x in X1:
        nq.hessian_accum(x, H1_ref, workspace=ws)
    sw_ref = {n: nq.scale_sweep(w, H0, s2[n], want_cost=True) for n, w in W.items()}
    torch.cuda.synchronize()

    # together: the Hessian on the current stream, the capped sweeps on a side stream
    side = torch.cuda.Stream(device=DEV)
    main = torch.cuda.current_stream(DEV)
    H1 = torch.zeros((768, 16, 16), dtype=torch.float32, device=DEV)
    out = {n: tuple(torch.empty_like(t) for t in sw_ref[n]) for n in W}
    ready = torch.cuda.Event()
    ready.record(main)
    side.wait_event(ready)
    for n, w in W.items():
        nq.scale_sweep(w, H0, s2[n], want_cost=True, out=out[n], wgs_per_cu=1, stream=side)
    for x in X1:
        nq.hessian_accum(x, H1, workspace=ws)
    done = torch.cuda.Event()
    done.record(side)
    main.wait_event(done)
    torch.cuda.synchronize()
    assert torch.equal(H1, H1_ref)
    for n in W:
        assert _equal(out[n], sw_ref[n]), n

    # as in the pipelined step: the down weight's capped sweep (under the
    # second stream's H) on the side stream while the first stream's H of
    # the next step accumulates into a fresh buffer
    del X1
    wd = to_dev_bf16(datagen.config4_weights("down"))
    s2d = nq.compute_scale2(wd)[0]
    down_ref = nq.scale_sweep(wd, H1_ref, s2d, want_cost=True)
    X0 = [datagen.config4_chunk_torch(0, c, DEV) for c in range(2)]
    H0_ref = torch.zeros_like(H0)
    for x in X0:
        nq.hessian_accum(x, H0_ref, workspace=ws)
    torch.cuda.synchronize()
    H0b = torch.zeros_like(H0)
    down = tuple(torch.empty_like(t) for t in down_ref)
    ready = torch.cuda.Event()
    ready.record(main)
    side.wait_event(ready)
    nq.scale_sweep(wd, H1_ref, s2d, want_cost=True, out=down, wgs_per_cu=1, stream=side)
    for x in X0:
        nq.hessian_accum(x, H0b, workspace=ws)
    done = torch.cuda.Event()
    done.record(side)
    main.wait_event(done)
    torch.cuda.synchronize()
    assert torch.equal(H0b, H0_ref)
    assert _equal(down, down_ref)


@pytest.mark.parametrize("rows,k", [(1, 16), (65, 48), (333, 272), (130, 4096)])
def test_capped_sweep_ragged(rows, k):
    """Row counts off the 64-row blocks and narrow or single-group widths:
    the capped launch gives the uncapped outputs, costs included."""
    note(f"capped sweep rows={rows} k={k}")
    rng = np.random.default_rng(rows * 7 + k)
    w = datagen.f32_to_bf16_bits(rng.normal(0.0, 0.02, (rows, k)).astype(np.float32))
    x = datagen.f32_to_bf16_bits(rng.laplace(0.0, 1.0, (256, k)).astype(np.float32))
    h32 = N.hessian(x).astype(np.float32)
    wd = to_dev_bf16(w)
    H = torch.from_numpy(h32).to(DEV)
    s2, _ = nq.compute_scale2(wd)
    ref = nq.scale_sweep(wd, H, s2, want_cost=True)
    cap = nq.scale_sweep(wd, H, s2, want_cost=True, wgs_per_cu=1)
    assert _equal(ref, cap)
    compare_sweep(w, h32, float(host(s2)[0]), host(cap[0]), host(cap[1]), host(cap[2]))
