#!/usr/bin/env python3
"""Benchmark of the NVFP4 post-training-quantization hot path on one MI355X.

One step is one pass of every stage of the path over resident synthetic
inputs:
  * the hybrid-model MLP set (gate/up W [12288, 4096], down W [4096, 12288];
    2^20 calibration tokens streamed as 16 chunks of 65536 per Linear input):
      a1 tensor amax -> scale_2 of each weight,
      a2 block-diagonal Hessian of both input streams (32 chunk calls, the
         activation amax fused into the same read),
      a3 the Hessian-weighted E4M3 scale sweep of all three weights
         (9,437,184 blocks);
  * activations X [8192, 4096]: a1 amax, a4 dynamic NVFP4 quantization and
    a5 the dequant round trip;
  * 128 MoE experts x (w1, w3) [2048, 7168] MXFP4: a6 the MXFP4->NVFP4 cast
    (in place on the nibbles, so each step first restores the original
    nibbles of the fallback blocks, ~9 MB, inside the timed step).
After the timed steps, two neighbouring pieces are timed on their own and
reported under stages (not part of the step): the W4A4 form of a2 (Hessian
of the fake-quantized calibration streams, next_w4a4_hessian), the FP8 E4M3
per-tensor static tier on the C3 activations (next_fp8_static), the
block-Hadamard rotation with the sweep under it and its cost against the
plain sweep's (next_block_hadamard), and the fake-quant QuantLinear forward
of one calibration chunk through the swept gate weight
(next_quantlinear_forward).

The headline value is weight blocks swept per second of whole-step time.
In the timed steps one HIP stream accumulates the Hessians and a second runs
everything else: a1 and a4-a6, the gate/up sweeps once the first
calibration stream's H is done (beside the second stream's Hessian), and
the down sweep once the second H is done (beside the next step's first
Hessian: consecutive steps alternate between two sets of H, amax and
scale_2 buffers).  Every sweep there is capped at one workgroup per CU so
that the Hessian keeps its own workgroups resident beside it.  Both buffer
sets must hold identical results, and one serial step afterwards must
reproduce every output bit for bit.  Per-stage times come from HIP events
over the same work in stage order on one stream.
The roofline entry is the stage with the largest share of the step; for the
Hessian it gives the live per-call rate in the timed steps and, under
"alone", the rate of the same calls in the serial pass.  The
cpu_baseline leg times the float64 oracle on a bounded sample of the same
work on the host cores and extrapolates to the whole job.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, spec
FP32_PEAK_TFLOPS = 157.3         # MI355X fp32 matrix (and packed vector), spec
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, spec
SWEEP_FLOP_PER_BLOCK = 127 * (304 + 64)      # minimal method work per 16-element block
C5_FALLBACK_BYTES = 32           # a fallback MX block reads and writes 16 bytes of nibbles


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle CPU baseline leg")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a 4 GiB device copy (known bytes, for HBM counter scaling)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported. The library has no "
              "multi-GPU path: the Hessian would shard over tokens with one all-reduce of H, and the sweep, "
              "quantizers and cast over rows or experts with no exchange.", file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import datagen
    import nvfp4_post_quantization_amd as nq

    lib = nq.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ------------------------------------------------------------ inputs (untimed)
    t0 = time.time()
    W = {n: dev_bf16(datagen.config4_weights(n)) for n in ("gate", "up", "down")}
    log(f"weights ready ({time.time() - t0:.1f}s)")
    X = [[datagen.config4_chunk_torch(s, c, dev) for c in range(16)] for s in (0, 1)]
    torch.cuda.synchronize()
    log(f"calibration chunks ready: {sum(x.numel() for xs in X for x in xs) * 2 / 2**30:.1f} GiB ({time.time() - t0:.1f}s)")
    x3 = dev_bf16(datagen.config3())
    p5_host, e5_host, forced5 = datagen.config5()
    P5 = torch.from_numpy(p5_host).to(dev)
    E5 = torch.from_numpy(e5_host).to(dev)
    n_forced = int(forced5.sum())
    # The cast rewrites the nibbles of its fallback blocks in place; each step
    # first puts back their original 16 bytes so that every step casts the
    # same input (fallback: k_max - k_j > 17 within an expert's pair).
    k5 = e5_host.astype(np.int16) - 127
    kmax5 = k5.reshape(k5.shape[0], -1).max(axis=1)
    fb_idx = torch.from_numpy(np.flatnonzero((kmax5[:, None, None, None] - k5).reshape(-1) > 17)).to(dev)
    P5_blocks = P5.view(torch.int64).view(-1, 2)                # one row = one MX block's 16 nibble bytes
    P5_fb_orig = P5_blocks.index_select(0, fb_idx)
    del p5_host, e5_host, forced5, k5
    log(f"all inputs resident ({time.time() - t0:.1f}s)")

    # ------------------------------------------------------------ outputs / state
    f32 = dict(dtype=torch.float32, device=dev)
    u8 = dict(dtype=torch.uint8, device=dev)
    NB = 2
    Hb = [{0: torch.zeros((256, 16, 16), **f32), 1: torch.zeros((768, 16, 16), **f32)} for _ in range(NB)]
    amax_xb = [{0: torch.zeros(1, **f32), 1: torch.zeros(1, **f32)} for _ in range(NB)]
    H, amax_x = Hb[0], amax_xb[0]
    ws_bytes = max(nq.hessian_workspace_bytes(datagen.C4_CHUNK, k) for k in (4096, 12288))
    ws = torch.empty(ws_bytes, **u8)
    s2wb = [{n: torch.zeros(1, **f32) for n in W} for _ in range(NB)]
    amwb = [{n: torch.zeros(1, **f32) for n in W} for _ in range(NB)]
    s2w, amw = s2wb[0], amwb[0]
    sw_out = {n: (torch.empty((w.shape[0], w.shape[1] // 2), **u8),
                  torch.empty((w.shape[0], w.shape[1] // 16), **u8)) for n, w in W.items()}
    s2x3, amx3 = torch.zeros(1, **f32), torch.zeros(1, **f32)
    q3 = (torch.empty((8192, 2048), **u8), torch.empty((8192, 256), **u8))
    dq3 = torch.empty((8192, 4096), dtype=torch.bfloat16, device=dev)
    c5 = (torch.empty((128, 2, 2048, 448), **u8), torch.empty(128, **f32), torch.empty(128, dtype=torch.int64, device=dev))

    def chk(name, st):
        if st != 0:
            raise RuntimeError(f"{name}: {lib.nvfp4_status_string(st).decode()}")

    stages = ["a1_scale2", "a2_hessian", "a3_sweep", "a4_quantize", "a5_dequant", "a6_cast"]
    marks = stages[:5] + ["a6_restore", "a6_cast"]              # serial-pass event marks
    hin = {"gate": 0, "up": 0, "down": 1}

    side = torch.cuda.Stream(device=dev)                         # default priority
    sptr_b = side.cuda_stream
    streams = {sptr: stream, sptr_b: side}

    def stage_calls(name, sp, b=0):
        """The calls of one stage (all but a2), enqueued on stream pointer sp."""
        if name == "a1_scale2":
            for n, w in W.items():
                chk("scale2", lib.nvfp4_compute_scale2(w.data_ptr(), w.numel(), s2wb[b][n].data_ptr(),
                                                       amwb[b][n].data_ptr(), sp))
            chk("scale2", lib.nvfp4_compute_scale2(x3.data_ptr(), x3.numel(), s2x3.data_ptr(), amx3.data_ptr(), sp))
        elif name == "a4_quantize":
            chk("quantize", lib.nvfp4_quantize_dynamic(x3.data_ptr(), 8192, 4096, 4096, s2x3.data_ptr(),
                                                       q3[0].data_ptr(), q3[1].data_ptr(), sp))
        elif name == "a5_dequant":
            chk("dequant", lib.nvfp4_dequant(q3[0].data_ptr(), q3[1].data_ptr(), s2x3.data_ptr(), 8192, 4096,
                                             dq3.data_ptr(), sp))
        elif name == "a6_restore":                             # benchmark only: the cast's input back
            with torch.cuda.stream(streams[sp]):
                P5_blocks.index_copy_(0, fb_idx, P5_fb_orig)
        elif name == "a6_cast":
            chk("cast", lib.mxfp4_to_nvfp4_cast(P5.data_ptr(), E5.data_ptr(), 128, 2, 2048, 7168, c5[0].data_ptr(),
                                                c5[1].data_ptr(), c5[2].data_ptr(), sp))

    def sweep(n, sp, wgs_per_cu=0, b=0):
        w = W[n]
        p, c = sw_out[n]
        chk("sweep", lib.nvfp4_scale_sweep_ex(w.data_ptr(), w.shape[0], w.shape[1], w.shape[1],
                                              Hb[b][hin[n]].data_ptr(), s2wb[b][n].data_ptr(), p.data_ptr(),
                                              c.data_ptr(), None, wgs_per_cu, sp))

    def hessian_stream(s, evh, b=0):
        """The 16 chunk calls of calibration stream s, bracketed by one event
        pair (an event between calls would leave the GPU idle ~10 us each)."""
        evh[s][0].record(stream)
        for x in X[s]:
            chk("hessian", lib.nvfp4_hessian_accum(x.data_ptr(), x.shape[0], x.shape[1], x.shape[1],
                                                   Hb[b][s].data_ptr(), amax_xb[b][s].data_ptr(), ws.data_ptr(),
                                                   ws.numel(), sptr))
        evh[s][1].record(stream)

    def step_serial(ev):
        """Every stage in order on one stream (per-stage timing)."""
        ev["start"].record(stream)
        stage_calls("a1_scale2", sptr)
        ev["a1_scale2"].record(stream)
        for s in (0, 1):
            H[s].zero_()
            amax_x[s].zero_()
        hessian_stream(0, ev["h"])
        hessian_stream(1, ev["h"])
        ev["a2_hessian"].record(stream)
        for n in W:
            sweep(n, sptr)
        ev["a3_sweep"].record(stream)
        for k in ("a4_quantize", "a5_dequant", "a6_restore", "a6_cast"):
            stage_calls(k, sptr)
            ev[k].record(stream)

    def step(ev, b, wait_ev):
        """The timed step, on buffer set b (H, amax and scale_2 alternate
        between consecutive steps).  The first HIP stream accumulates both
        calibration streams' H; the second takes a1 and a4-a6, the gate/up
        sweeps once the first H is done and the down sweep once the second
        is, every sweep capped at one workgroup per CU.  So the down sweep of
        one step runs beside the next step's first Hessian; wait_ev (the
        second stream's end of the step two back, the last reader of set b)
        guards the reuse of set b."""
        ev["start"].record(stream)
        stage_calls("a1_scale2", sptr_b, b)
        for k in ("a4_quantize", "a5_dequant", "a6_restore", "a6_cast"):
            stage_calls(k, sptr_b)
        if wait_ev is not None:
            stream.wait_event(wait_ev)
        for s in (0, 1):
            Hb[b][s].zero_()
            amax_xb[b][s].zero_()
        hessian_stream(0, ev["h"], b)
        ev["h0_done"].record(stream)
        side.wait_event(ev["h0_done"])
        for n in ("gate", "up"):
            sweep(n, sptr_b, 1, b)
        hessian_stream(1, ev["h"], b)
        ev["h1_done"].record(stream)
        side.wait_event(ev["h1_done"])
        sweep("down", sptr_b, 1, b)
        ev["side_done"].record(side)

    def new_events(serial=False):
        E = lambda: torch.cuda.Event(enable_timing=True)
        h = [(E(), E()) for s in (0, 1)]
        if serial:
            return dict({k: E() for k in ["start"] + marks}, h=h)
        return {"start": E(), "h0_done": E(), "h1_done": E(), "side_done": E(), "h": h}

    log(f"warmup {args.warmup} step(s)")
    wev = [new_events() for _ in range(args.warmup)]
    for i in range(args.warmup):
        step(wev[i], i % NB, wev[i - NB]["side_done"] if i >= NB else None)
    torch.cuda.synchronize()
    fb = int(c5[2].sum().item())

    evs = [new_events() for _ in range(args.steps)]
    log(f"timing {args.steps} step(s)")
    torch.cuda.synchronize()
    t_begin = time.perf_counter()
    for i in range(args.steps):
        step(evs[i], i % NB, evs[i - NB]["side_done"] if i >= NB else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_begin
    ms_per_step = wall * 1e3 / args.steps
    # mean Hessian call (partial + reduce) on its stream inside the timed steps
    h_call_ms = sum(a.elapsed_time(b) for ev in evs for a, b in ev["h"]) / (args.steps * 32)

    # the overlapped schedule must produce exactly what the serial order does
    def outputs(b=0):
        d = {"H0": Hb[b][0], "H1": Hb[b][1], "amax_x0": amax_xb[b][0], "amax_x1": amax_xb[b][1],
             "s2w_gate": s2wb[b]["gate"], "s2w_up": s2wb[b]["up"], "s2w_down": s2wb[b]["down"], "q3_packed": q3[0],
             "q3_codes": q3[1], "dq3": dq3, "c5_codes": c5[0], "c5_scale2": c5[1], "c5_fallbacks": c5[2]}
        for n in W:
            d[f"{n}_packed"], d[f"{n}_codes"] = sw_out[n]
        return d

    bl = (args.steps - 1) % NB
    snap = {k: t.clone() for k, t in outputs(bl).items()}
    if args.steps >= NB:
        other = outputs(1 - bl)
        diff2 = [k for k in ("H0", "H1", "amax_x0", "amax_x1", "s2w_gate", "s2w_up", "s2w_down")
                 if not torch.equal(other[k], snap[k])]
        if diff2:
            raise RuntimeError(f"the two buffer sets differ: {diff2}")
    # per-stage times from the same work in stage order on one stream
    n_serial = max(1, min(args.steps, 5))
    evs_serial = [new_events(serial=True) for _ in range(n_serial + 1)]
    torch.cuda.synchronize()
    step_serial(evs_serial.pop())                               # one untimed serial step first
    for i in range(n_serial):
        step_serial(evs_serial[i])
    torch.cuda.synchronize()
    differ = {k: int((t != snap[k]).sum().item()) for k, t in outputs().items() if not torch.equal(t, snap[k])}
    if differ:
        raise RuntimeError(f"overlapped step differs from the serial step (differing elements: {differ})")

    # per-stage times (ms per step, averaged over the serial steps)
    st_ms = {k: 0.0 for k in marks}
    step_ms = 0.0
    for ev in evs_serial:
        prev = ev["start"]
        for k in marks:
            st_ms[k] += prev.elapsed_time(ev[k]) / n_serial
            prev = ev[k]
        step_ms += ev["start"].elapsed_time(ev["a6_cast"]) / n_serial
    h_call_serial_ms = sum(a.elapsed_time(b) for ev in evs_serial for a, b in ev["h"]) / (n_serial * 32)

    # algorithmic work per step
    blocks = sum(w.numel() // 16 for w in W.values())
    x_bytes = sum(x.numel() * 2 for xs in X for x in xs)
    a1_bytes = sum(w.numel() * 2 for w in W.values()) + x3.numel() * 2
    q_bytes = x3.numel() * 2.5625
    cast_bytes = E5.numel() + c5[0].numel() + fb * C5_FALLBACK_BYTES     # the restore of the inputs not counted
    flops = blocks * SWEEP_FLOP_PER_BLOCK
    info = {
        "a1_scale2": dict(launches=4, bytes=a1_bytes),
        "a2_hessian": dict(launches=32, bytes=x_bytes),
        "a3_sweep": dict(launches=3, flops=flops, blocks=blocks),
        "a4_quantize": dict(launches=1, bytes=q_bytes),
        "a5_dequant": dict(launches=1, bytes=q_bytes),
        "a6_cast": dict(launches=1, bytes=cast_bytes),
    }
    stage_rep = {}
    for k in stages:
        t = st_ms[k] / 1e3
        d = {"ms_per_step": round(st_ms[k], 4), "launches_per_step": info[k]["launches"],
             "share": round(st_ms[k] / step_ms, 4)}
        if "bytes" in info[k]:
            gbs = info[k]["bytes"] / t / 1e9
            d.update(algorithmic_GB=round(info[k]["bytes"] / 1e9, 4), GBps=round(gbs, 1),
                     frac_hbm_peak=round(gbs / HBM_PEAK_GBS, 4))
        else:
            tf = info[k]["flops"] / t / 1e12
            d.update(blocks=info[k]["blocks"], blocks_per_s=round(info[k]["blocks"] / t, 1),
                     TFLOPs=round(tf, 2), frac_fp32_peak=round(tf / FP32_PEAK_TFLOPS, 4))
        stage_rep[k] = d
    stage_rep["a3_sweep"]["note"] = ("algorithmic flops count all 127 codes of every block; the pruned search "
                                     "evaluates about 15 per block, so this fraction is not a VALU utilisation")
    stage_rep["a6_cast"]["fallback_mx_blocks"] = fb
    stage_rep["a6_cast"]["forced_by_generator"] = n_forced
    stage_rep["a6_cast"]["input_restore_ms"] = round(st_ms["a6_restore"], 4)   # in the step, not in this stage

    dom = max(("a2_hessian", "a3_sweep"), key=lambda k: st_ms[k])
    if dom == "a3_sweep":
        per_launch_s = st_ms[dom] / 1e3 / 3
        achieved = flops / 3 / per_launch_s / 1e12
        roof = {"kernel": "sweep_kernel", "bound": "alu", "achieved": round(achieved, 3), "peak": FP32_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / FP32_PEAK_TFLOPS, 4),
                "per_launch": f"{blocks // 3} blocks x {SWEEP_FLOP_PER_BLOCK} flop, {per_launch_s * 1e3:.4f} ms avg"}
    else:
        per_launch_s = h_call_ms / 1e3                               # live, on its stream, in the timed steps
        achieved = x_bytes / 32 / per_launch_s / 1e9
        alone = x_bytes / 32 / (h_call_serial_ms / 1e3) / 1e9
        roof = {"kernel": "hessian_partial_kernel+hessian_reduce_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "per_launch": f"{x_bytes / 32 / 1e9:.4f} GB avg, {per_launch_s * 1e3:.4f} ms avg (events around "
                              f"each calibration stream's 16 calls, on their stream, in the timed steps, where they "
                              f"share the GPU with the side-stream sweeps)",
                "alone": {"ms_per_launch": round(h_call_serial_ms, 4), "achieved": round(alone, 1),
                          "frac": round(alone / HBM_PEAK_GBS, 4),
                          "note": "the same calls in the serial pass, with nothing else running"}}
    roof["traffic"] = traffic_from_profiles(roof["kernel"])

    # W4A4 form of a2, outside the step: the Hessian of the fake-quantized
    # calibration streams (activation scale_2 from max calibration of each
    # stream's first chunk), 32 chunk calls per pass
    s2a = {s: torch.zeros(1, **f32) for s in (0, 1)}
    Hq = {s: torch.zeros_like(H[s]) for s in (0, 1)}
    for s in (0, 1):
        chk("scale2", lib.nvfp4_compute_scale2(X[s][0].data_ptr(), X[s][0].numel(), s2a[s].data_ptr(), None, sptr))

    def fq_pass():
        for s in (0, 1):
            Hq[s].zero_()
            for x in X[s]:
                chk("hessian_fq", lib.nvfp4_hessian_accum_fq(x.data_ptr(), x.shape[0], x.shape[1], x.shape[1],
                                                             s2a[s].data_ptr(), Hq[s].data_ptr(), None,
                                                             ws.data_ptr(), ws.numel(), sptr))

    fq_pass()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        fq_pass()
    e1.record(stream)
    torch.cuda.synchronize()
    fq_ms = e0.elapsed_time(e1) / args.steps
    fq_gbs = x_bytes / (fq_ms / 1e3) / 1e9
    stage_rep["next_w4a4_hessian"] = {
        "outside_step": True, "ms_per_pass": round(fq_ms, 4), "launches_per_pass": 32,
        "algorithmic_GB": round(x_bytes / 1e9, 4), "GBps": round(fq_gbs, 1),
        "frac_hbm_peak": round(fq_gbs / HBM_PEAK_GBS, 4),
        "kernel": "hessian_fq_partial_kernel+hessian_reduce_kernel"}

    # FP8 E4M3 per-tensor static tier, outside the step: scale, quantize and
    # dequant of the C3 activations [8192, 4096]
    s8, am8 = torch.zeros(1, **f32), torch.zeros(1, **f32)
    q8 = torch.empty((8192, 4096), **u8)
    dq8 = torch.empty((8192, 4096), dtype=torch.bfloat16, device=dev)
    ev8 = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def fp8_pass(ev):
        ev[0].record(stream)
        chk("fp8 scale", lib.fp8e4m3_compute_scale(x3.data_ptr(), x3.numel(), s8.data_ptr(), am8.data_ptr(), sptr))
        ev[1].record(stream)
        chk("fp8 quantize", lib.fp8e4m3_quantize(x3.data_ptr(), 8192, 4096, 4096, s8.data_ptr(), q8.data_ptr(), sptr))
        ev[2].record(stream)
        chk("fp8 dequant", lib.fp8e4m3_dequant(q8.data_ptr(), s8.data_ptr(), 8192, 4096, dq8.data_ptr(), sptr))
        ev[3].record(stream)

    fp8_pass(ev8)
    t8 = [0.0, 0.0, 0.0]
    for _ in range(args.steps):
        fp8_pass(ev8)
        torch.cuda.synchronize()
        for i in range(3):
            t8[i] += ev8[i].elapsed_time(ev8[i + 1]) / args.steps
    e8 = x3.numel()
    stage_rep["next_fp8_static"] = {"outside_step": True, "workload": "X [8192, 4096] bf16"}
    for name, ms, nbytes in (("scale", t8[0], 2 * e8), ("quantize", t8[1], 3 * e8), ("dequant", t8[2], 3 * e8)):
        gbs = nbytes / (ms / 1e3) / 1e9
        stage_rep["next_fp8_static"][name] = {"ms": round(ms, 4), "algorithmic_GB": round(nbytes / 1e9, 4),
                                              "GBps": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}

    # Block-Hadamard rotation under the sweep, outside the step: W' = W R for
    # the three weights, H' = R^T H R for both streams, then the sweep of
    # (W', H') at scale_2(W'); its total cost is compared with the plain
    # sweep's (both are the Hessian-weighted error in the original basis)
    Wr = {n: torch.empty_like(w) for n, w in W.items()}
    Hr = {s: torch.empty_like(H[s]) for s in (0, 1)}
    s2r = {n: torch.zeros(1, **f32) for n in W}
    cost_p = {n: torch.empty((w.shape[0], w.shape[1] // 16), **f32) for n, w in W.items()}
    cost_r = {n: torch.empty((w.shape[0], w.shape[1] // 16), **f32) for n, w in W.items()}
    evr = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def rot_pass(ev):
        ev[0].record(stream)
        for n, w in W.items():
            chk("hadamard", lib.nvfp4_block_hadamard(w.data_ptr(), w.shape[0], w.shape[1], w.shape[1],
                                                     Wr[n].data_ptr(), w.shape[1], sptr))
        ev[1].record(stream)
        for s in (0, 1):
            chk("hessian hadamard", lib.nvfp4_hessian_hadamard(H[s].data_ptr(), H[s].shape[0], Hr[s].data_ptr(), sptr))
        for n, w in W.items():
            chk("scale2", lib.nvfp4_compute_scale2(Wr[n].data_ptr(), w.numel(), s2r[n].data_ptr(), None, sptr))
        ev[2].record(stream)
        for n, w in W.items():
            p, c = sw_out[n]
            chk("sweep", lib.nvfp4_scale_sweep(Wr[n].data_ptr(), w.shape[0], w.shape[1], w.shape[1],
                                               Hr[hin[n]].data_ptr(), s2r[n].data_ptr(), p.data_ptr(),
                                               c.data_ptr(), cost_r[n].data_ptr(), sptr))
        ev[3].record(stream)

    for n, w in W.items():                                      # plain sweep with costs, for the comparison
        p, c = sw_out[n]
        chk("sweep", lib.nvfp4_scale_sweep(w.data_ptr(), w.shape[0], w.shape[1], w.shape[1], H[hin[n]].data_ptr(),
                                           s2w[n].data_ptr(), p.data_ptr(), c.data_ptr(), cost_p[n].data_ptr(), sptr))
    rot_pass(evr)
    tr = [0.0, 0.0, 0.0]
    reps = max(1, min(args.steps, 3))
    for _ in range(reps):
        rot_pass(evr)
        torch.cuda.synchronize()
        for i in range(3):
            tr[i] += evr[i].elapsed_time(evr[i + 1]) / reps
    w_elems = sum(w.numel() for w in W.values())
    rot_gbs = 4 * w_elems / (tr[0] / 1e3) / 1e9
    stage_rep["next_block_hadamard"] = {
        "outside_step": True,
        "rotate_weights": {"ms": round(tr[0], 4), "launches": 3, "algorithmic_GB": round(4 * w_elems / 1e9, 4),
                           "GBps": round(rot_gbs, 1), "frac_hbm_peak": round(rot_gbs / HBM_PEAK_GBS, 4)},
        "rotate_hessians_and_scale2_ms": round(tr[1], 4),
        "rotated_sweep": {"ms": round(tr[2], 4), "blocks_per_s": round(blocks / (tr[2] / 1e3), 1)},
        "total_cost_rotated_over_plain": {n: round(float(cost_r[n].double().sum() / cost_p[n].double().sum()), 5)
                                          for n in W},
    }

    # Fake-quant QuantLinear forward, outside the step: one 65536-token chunk
    # [65536, 4096] through the gate weight after the sweep (w_hat = two-DQ of
    # the swept NVFP4 weight, [12288, 4096]); the activation's scale_2 from max
    # calibration of that chunk
    xq = X[0][0]
    wq_hat = torch.empty_like(W["gate"])
    p, c = sw_out["gate"]
    chk("dequant", lib.nvfp4_dequant(p.data_ptr(), c.data_ptr(), s2w["gate"].data_ptr(), W["gate"].shape[0],
                                     W["gate"].shape[1], wq_hat.data_ptr(), sptr))
    s2q = torch.zeros(1, **f32)
    chk("scale2", lib.nvfp4_compute_scale2(xq.data_ptr(), xq.numel(), s2q.data_ptr(), None, sptr))
    tq, kq, oq = xq.shape[0], xq.shape[1], wq_hat.shape[0]
    yq = torch.empty((tq, oq), dtype=torch.bfloat16, device=dev)
    wsq = torch.empty(lib.nvfp4_quantlinear_workspace_bytes(tq, kq), **u8)
    xhq = torch.empty_like(xq)
    evq = [torch.cuda.Event(enable_timing=True) for _ in range(6)]

    def ql_pass(ev):
        ev[0].record(stream)
        chk("fakequant", lib.nvfp4_fakequant(xq.data_ptr(), tq, kq, kq, s2q.data_ptr(), xhq.data_ptr(), kq, sptr))
        ev[1].record(stream)
        chk("forward", lib.nvfp4_quantlinear_forward(xq.data_ptr(), tq, kq, kq, s2q.data_ptr(), wq_hat.data_ptr(),
                                                     oq, kq, yq.data_ptr(), oq, wsq.data_ptr(), wsq.numel(), sptr))
        ev[2].record(stream)
        torch.matmul(xhq, wq_hat.t(), out=yq)                  # torch's GEMM on the same operands, for context
        ev[3].record(stream)

    ql_pass(evq)
    tq_ms = [0.0, 0.0, 0.0]
    reps = max(1, min(args.steps, 5))
    for _ in range(reps):
        ql_pass(evq)
        torch.cuda.synchronize()
        for i in range(3):
            tq_ms[i] += evq[i].elapsed_time(evq[i + 1]) / reps
    flop = 2.0 * tq * kq * oq
    fq_b = 4.0 * tq * kq
    stage_rep["next_quantlinear_forward"] = {
        "outside_step": True,
        "workload": f"x [{tq}, {kq}] bf16 through w_hat [{oq}, {kq}] (C4 gate, swept then dequantized)",
        "fakequant": {"ms": round(tq_ms[0], 4), "algorithmic_GB": round(fq_b / 1e9, 4),
                      "GBps": round(fq_b / (tq_ms[0] / 1e3) / 1e9, 1),
                      "frac_hbm_peak": round(fq_b / (tq_ms[0] / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
        "forward": {"ms": round(tq_ms[1], 4), "TFLOPs": round(flop / (tq_ms[1] / 1e3) / 1e12, 1),
                    "frac_bf16_peak": round(flop / (tq_ms[1] / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "torch_matmul_same_operands": {"ms": round(tq_ms[2], 4),
                                       "TFLOPs": round(flop / (tq_ms[2] / 1e3) / 1e12, 1)},
    }
    del yq, wsq, xhq

    if args.copy_probe:
        # an elementwise kernel of known traffic (4 GiB read + 4 GiB written per
        # launch): the reference for scaling the HBM byte counters
        a = torch.zeros(1 << 31, dtype=torch.int16, device=dev)
        b = torch.empty_like(a)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.neg(a, out=b)
        e0.record(stream)
        for _ in range(5):
            torch.neg(a, out=b)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        stage_rep["hbm_copy_probe"] = {"kernel": "elementwise neg int16, 2^31 elements",
                                       "bytes_read": a.numel() * 2, "bytes_written": a.numel() * 2,
                                       "GBps": round(2 * a.numel() * 2 / (ms / 1e3) / 1e9, 1)}
        del a, b

    value = blocks / (ms_per_step / 1e3)
    out = {
        "metric": "weight blocks/sec (Hessian scale sweep) + accumulate/quant GB/s vs HBM peak",
        "value": round(value, 1),
        "unit": "weight blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "hybrid-model MLP set calibration (gate/up [12288,4096], down [4096,12288], "
                        "2^20 tokens in 16 x 65536-token chunks: scale_2, Hessian, sweep) + activation "
                        "quantize/dequant [8192,4096] + MXFP4->NVFP4 cast of 128 experts x (w1,w3) [2048,7168]",
            "weight_blocks_per_step": blocks,
            "calibration_tokens": datagen.C4_TOKENS,
            "chunk_tokens": datagen.C4_CHUNK,
            "parallelism": "single GPU",
            "schedule": "timed steps: a2 of both calibration streams on one HIP stream; a1, a4-a6 and the three "
                        "sweeps (capped at one workgroup per CU) on a second stream, the gate/up sweeps beside the "
                        "second calibration stream's Hessian and the down sweep beside the next step's first "
                        "(two alternating sets of H/amax/scale_2 buffers; checked bit-exact against the serial "
                        "order); stages: the same work in stage order on one stream",
            "serial_step_ms": round(step_ms, 4),
        },
        "roofline": roof,
        "cpu_baseline": None,
        "stages": stage_rep,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(W, X, H, s2w, blocks)
    print(json.dumps(out), flush=True)


def traffic_from_profiles(kernel: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by the copy
    probe) from the committed counter summary; null unless every kernel of
    `kernel` ("a+b" sums them) was measured on its current source."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.txt")
    srcs = {"sweep_kernel": "sweep.hip", "hessian_partial_kernel": "hessian.hip",
            "hessian_reduce_kernel": "hessian.hip"}
    total = 0.0
    try:
        lines = [dict(kv.split("=", 1) for kv in ln.split() if "=" in kv)
                 for ln in open(path) if ln.startswith("kernel=")]
        for name in kernel.split("+"):
            src = os.path.join(ROOT, "nvfp4_post_quantization_amd", "csrc", srcs[name])
            sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
            hit = [f for f in lines if f.get("kernel") == name and f.get("src_sha") == sha]
            if not hit:
                return None
            total += float(hit[0]["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None
    return round(total, 1)


def cpu_baseline(W, X, H, s2w, blocks):
    """Time the float64 oracle on a bounded sample of the same job and
    extrapolate to the whole step (Hessian of both streams + all sweeps)."""
    import numpy as np
    import torch
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    n_chunks = 2                                   # whole 65536-token chunks per stream
    t_tok = n_chunks * X[0][0].shape[0]
    t0 = time.perf_counter()
    hs = {}
    for s in (0, 1):
        hs[s] = 0.0
        h = None
        for c in range(n_chunks):
            xs = X[s][c].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            a = time.perf_counter()
            h = oracle.hessian(xs, h)
            hs[s] += time.perf_counter() - a
            del xs
    rows = {"gate": 288, "down": 96}
    sweep_t, sweep_blocks = 0.0, 0
    for n, r in rows.items():
        wb = W[n][:r].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        h = H[0 if n != "down" else 1].cpu().numpy().astype(np.float64)
        s2 = float(s2w[n].cpu().numpy()[0])
        a = time.perf_counter()
        oracle.scale_sweep(wb, h, s2)
        sweep_t += time.perf_counter() - a
        sweep_blocks += wb.size // 16
    wall = time.perf_counter() - t0
    full_tokens = 1 << 20
    t_hess = (hs[0] + hs[1]) * (full_tokens / t_tok)
    t_sweep = sweep_t / sweep_blocks * blocks
    est = t_hess + t_sweep
    return {
        "value": round(blocks / est, 1),
        "unit": "weight blocks/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"float64 oracle on {t_tok} tokens of each calibration stream (Hessian) and "
                   f"{rows['gate']} gate rows + {rows['down']} down rows ({sweep_blocks} blocks, sweep), "
                   f"extrapolated to 2^20 tokens and {blocks} blocks: est. {est:.0f} s per step "
                   f"(Hessian {t_hess:.0f} s, sweep {t_sweep:.0f} s); sample wall {wall:.1f} s; "
                   f"host cores visible {len(os.sched_getaffinity(0))}"),
    }


if __name__ == "__main__":
    main()
