#!/usr/bin/env python3
"""Benchmark of the NVFP4 post-training-quantization hot path on one MI355X.

One step is one pass of every stage of the path over resident synthetic
inputs:
  * the hybrid-model MLP set (gate/up W [12288, 4096], down W [4096, 12288];
    2^20 calibration tokens streamed as 16 chunks of 65536 per Linear input):
      a1 tensor amax -> scale_2 of each weight (one batched call with the
         activations' a1 below),
      a2 block-diagonal Hessian of both input streams (one call per stream
         over its 16 resident chunks, the activation amax fused into the same
         read),
      a3 the Hessian-weighted E4M3 scale sweep of all three weights
         (9,437,184 blocks);
  * activations X [8192, 4096]: a1 amax, a4 dynamic NVFP4 quantization and
    a5 the dequant round trip;
  * 128 MoE experts x (w1, w3) [2048, 7168] MXFP4: a6 the MXFP4->NVFP4 cast
    (in place on the nibbles, so each step first restores the original
    nibbles of the fallback blocks, ~9 MB, inside the timed step).
After the timed steps, the neighbouring pieces are timed on their own and
reported under stages (not part of the step): the W4A4 form of a2 (Hessian
of the fake-quantized calibration streams, next_w4a4_hessian), the FP8 E4M3
per-tensor static tier on the C3 activations (next_fp8_static), the
block-Hadamard rotation with the sweep under it and its cost against the
plain sweep's (next_block_hadamard), and the fake-quant QuantLinear forward
of one calibration chunk through the swept gate weight
(next_quantlinear_forward).

The headline value is weight blocks swept per second of whole-step time.
In the timed steps one HIP stream runs a1, the Hessians and then a4-a6, and
a second runs the sweeps: gate/up once the first calibration stream's H is
done (beside the second stream's Hessian), down once the first stream's
step is done (beside the next step's a1 and first Hessian: consecutive
steps alternate between two sets of H, amax and scale_2 buffers).  Every
sweep there is capped at one workgroup per CU so that the Hessian keeps its
own workgroups resident beside it.  Both buffer
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
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, spec
FP32_PEAK_TFLOPS = 157.3         # MI355X fp32 matrix (and packed vector), spec
# the library is built without packed FP32 VALU forms, so its fp32 VALU
# ceiling is one FMA per lane per cycle: 256 CU x 4 SIMD x 16 lanes x 2 flop x 2.4 GHz
VALU_NONPACKED_TFLOPS = 78.6
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, spec
# the method's work per 16-element block and code, by one convention: the
# symmetric quadratic form (136 distinct H entries + a 16-term dot, each an
# FMA of 2 flop) plus quantize / dequantize / subtract (4 per element)
FORM_FLOP, QUANT_FLOP, SCREEN_FLOP = 304, 64, 32
SWEEP_FLOP_PER_BLOCK = 127 * (FORM_FLOP + QUANT_FLOP)   # all 127 codes of a block
C5_FALLBACK_BYTES = 32           # a fallback MX block reads and writes 16 bytes of nibbles
C5_MX_BLOCKS_PER_GROUP = 2 * 2048 * (7168 // 32)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    # 30 timed steps: the pipeline restarts after the synchronize that opens
    # the timed region, and its first steps run slower (the side stream lags
    # for about four steps); over 10 steps that start-up added about 0.1 ms
    # per step on MI355X (6.15-6.17 against 6.06 ms over 30)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle CPU baseline leg")
    p.add_argument("--no-extras", action="store_true",
                   help="time the step only: skip the measured ceilings, the rotated-buffer stage timings, "
                        "the C2 leg and the pieces outside the step")
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
    # per buffer set, both calibration streams' H and amax in one allocation,
    # so the step clears them with one fill kernel instead of four
    hz = [torch.zeros((256 + 768) * 256 + 8, **f32) for _ in range(NB)]
    Hb = [{0: z[:65536].view(256, 16, 16), 1: z[65536:262144].view(768, 16, 16)} for z in hz]
    amax_xb = [{0: z[262144:262145], 1: z[262148:262149]} for z in hz]
    H, amax_x = Hb[0], amax_xb[0]
    ws_bytes = max(nq.hessian_workspace_bytes(datagen.C4_CHUNK, k) for k in (4096, 12288))
    ws = torch.empty(ws_bytes, **u8)
    # the chunk-list accumulate: one call per calibration stream over its 16 chunks
    wsc_bytes = max(nq.hessian_chunks_workspace_bytes(datagen.C4_CHUNK, k, 16) for k in (4096, 12288))
    wsc = torch.empty(wsc_bytes, **u8)
    x_ptrs = [(ctypes.c_void_p * len(X[s]))(*[x.data_ptr() for x in X[s]]) for s in (0, 1)]
    # step 1 of the three weights and the C3 activations in one batched call:
    # per buffer set, scale_2 and amax of [gate, up, down, X] in one array each
    s2_all = [torch.zeros(4, **f32) for _ in range(NB)]
    am_all = [torch.zeros(4, **f32) for _ in range(NB)]
    s2wb = [{n: s2_all[b][i:i + 1] for i, n in enumerate(W)} for b in range(NB)]
    amwb = [{n: am_all[b][i:i + 1] for i, n in enumerate(W)} for b in range(NB)]
    a1_in = list(W.values()) + [x3]
    a1_ptrs = (ctypes.c_void_p * 4)(*[t.data_ptr() for t in a1_in])
    a1_ns = (ctypes.c_int64 * 4)(*[t.numel() for t in a1_in])
    s2w, amw = s2wb[0], amwb[0]
    sw_out = {n: (torch.empty((w.shape[0], w.shape[1] // 2), **u8),
                  torch.empty((w.shape[0], w.shape[1] // 16), **u8)) for n, w in W.items()}
    s2x3b = [s2_all[b][3:4] for b in range(NB)]
    s2x3 = s2x3b[0]
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
            chk("scale2", lib.nvfp4_compute_scale2_batch(a1_ptrs, a1_ns, 4, s2_all[b].data_ptr(),
                                                         am_all[b].data_ptr(), sp))
        elif name == "a4_quantize":
            chk("quantize", lib.nvfp4_quantize_dynamic(x3.data_ptr(), 8192, 4096, 4096, s2x3b[b].data_ptr(),
                                                       q3[0].data_ptr(), q3[1].data_ptr(), sp))
        elif name == "a5_dequant":
            chk("dequant", lib.nvfp4_dequant(q3[0].data_ptr(), q3[1].data_ptr(), s2x3b[b].data_ptr(), 8192, 4096,
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
        """Calibration stream s's Hessian: one chunk-list call over its 16
        resident chunks (one accumulate launch per chunk, one reduce), bracketed by an
        event pair on its stream."""
        evh[s][0].record(stream)
        x0 = X[s][0]
        chk("hessian", lib.nvfp4_hessian_accum_chunks(x_ptrs[s], len(X[s]), x0.shape[0], x0.shape[1], x0.shape[1],
                                                      Hb[b][s].data_ptr(), amax_xb[b][s].data_ptr(), wsc.data_ptr(),
                                                      wsc.numel(), sptr))
        evh[s][1].record(stream)

    def step_serial(ev):
        """Every stage in order on one stream (per-stage timing)."""
        ev["start"].record(stream)
        stage_calls("a1_scale2", sptr)
        ev["a1_scale2"].record(stream)
        hz[0].zero_()
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
        between consecutive steps).  The first HIP stream runs a1, the
        Hessians of both calibration streams, then a4-a6; the second takes
        the gate/up sweeps once the first H is done and the down sweep once
        the first stream's step is done, every sweep capped at one workgroup
        per CU.  So the down sweep of one step runs beside the next step's a1
        and first Hessian; wait_ev (the second stream's end of the step two
        back, the last reader of set b) guards the reuse of set b.  The
        HBM-bound stages run in series with the HBM-bound accumulate rather
        than beside it (beside it they slowed its calls by about as much as
        their own time), and a4-a6 run where the second stream is idle: next
        to a capped sweep's 256-VGPR waves only one of their waves fits per
        SIMD, which had made them 1.5-3.5x slower."""
        ev["start"].record(stream)
        stage_calls("a1_scale2", sptr, b)
        if wait_ev is not None:
            stream.wait_event(wait_ev)
        hz[b].zero_()
        hessian_stream(0, ev["h"], b)
        ev["h0_done"].record(stream)
        side.wait_event(ev["h0_done"])
        for n in ("gate", "up"):
            sweep(n, sptr_b, 1, b)
        hessian_stream(1, ev["h"], b)
        for k in ("a4_quantize", "a5_dequant", "a6_restore", "a6_cast"):
            stage_calls(k, sptr, b)
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
    h_call_ms = sum(a.elapsed_time(b) for ev in evs for a, b in ev["h"]) / (args.steps * 2)

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
    h_call_serial_ms = sum(a.elapsed_time(b) for ev in evs_serial for a, b in ev["h"]) / (n_serial * 2)

    # algorithmic work per step
    blocks = sum(w.numel() // 16 for w in W.values())
    x_bytes = sum(x.numel() * 2 for xs in X for x in xs)
    a1_bytes = sum(w.numel() * 2 for w in W.values()) + x3.numel() * 2
    q_bytes = x3.numel() * 2.5625
    cast_bytes = E5.numel() + c5[0].numel() + fb * C5_FALLBACK_BYTES     # the restore of the inputs not counted
    info = {
        "a1_scale2": dict(launches=1, bytes=a1_bytes),
        "a2_hessian": dict(launches=2, bytes=x_bytes),
        "a3_sweep": dict(launches=3, blocks=blocks),
        "a4_quantize": dict(launches=1, bytes=q_bytes),
        "a5_dequant": dict(launches=1, bytes=q_bytes),
        "a6_cast": dict(launches=1, bytes=cast_bytes),
    }
    stage_rep = {}
    for k in stages:
        t = st_ms[k] / 1e3
        d = {"ms_per_step": round(st_ms[k], 4), "calls_per_step": info[k]["launches"],
             "share": round(st_ms[k] / step_ms, 4)}
        if "bytes" in info[k]:
            gbs = info[k]["bytes"] / t / 1e9
            d.update(algorithmic_GB=round(info[k]["bytes"] / 1e9, 4), GBps=round(gbs, 1),
                     frac_hbm_peak=round(gbs / HBM_PEAK_GBS, 4))
        else:
            d.update(blocks=info[k]["blocks"], blocks_per_s=round(info[k]["blocks"] / t, 1))
        stage_rep[k] = d
    stage_rep["a6_cast"]["fallback_mx_blocks"] = fb
    stage_rep["a6_cast"]["forced_by_generator"] = n_forced
    stage_rep["a6_cast"]["input_restore_ms"] = round(st_ms["a6_restore"], 4)   # in the step, not in this stage
    fb_groups = c5[2].cpu().numpy()
    stage_rep["a6_cast"]["lossless_block_share"] = round(1.0 - fb / (128 * C5_MX_BLOCKS_PER_GROUP), 6)
    stage_rep["a6_cast"]["lossless_group_share"] = round(float((fb_groups == 0).mean()), 6)
    stage_rep["a6_cast"]["lossless_note"] = (
        "an MX block is lossless when it stays inside the 17-exponent window (its nibbles and dequantized "
        "values are unchanged); a group (expert pair w1/w3) is lossless when none of its blocks falls back. "
        "The generator forces 0.5% of the blocks of every expert out of the window, so no group is lossless")

    # the sweep's executed work: the counting build of the same kernel on the
    # serial pass's inputs (outputs must equal the serial sweep's)
    sw_stats = {n: sweep_work(lib, chk, W[n], H[hin[n]], s2w[n], sw_out[n], sptr) for n in W}
    stage_rep["a3_sweep"].update(sweep_work_report(sw_stats, st_ms["a3_sweep"] / 1e3))

    dom = max(("a2_hessian", "a3_sweep"), key=lambda k: st_ms[k])
    if dom == "a3_sweep":
        achieved = stage_rep["a3_sweep"]["executed_TFLOPs"]
        roof = {"kernel": "sweep_kernel", "bound": "alu", "achieved": achieved, "peak": VALU_NONPACKED_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / VALU_NONPACKED_TFLOPS, 4),
                "per_launch": f"{blocks // 3} blocks, executed work counted by nvfp4_scale_sweep_stats, "
                              f"{st_ms[dom] / 3:.4f} ms avg"}
    else:
        per_launch_s = h_call_ms / 1e3                               # live, on its stream, in the timed steps
        achieved = x_bytes / 2 / per_launch_s / 1e9
        alone = x_bytes / 2 / (h_call_serial_ms / 1e3) / 1e9
        roof = {"kernel": "hessian_partial_kernel+hessian_reduce_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "per_launch": f"{x_bytes / 2 / 1e9:.4f} GB avg, {per_launch_s * 1e3:.4f} ms avg (one "
                              f"nvfp4_hessian_accum_chunks call per calibration stream over its 16 chunks: events "
                              f"around each call, on its stream, in the timed steps, where they "
                              f"share the GPU with the second stream's sweeps)",
                "alone": {"ms_per_launch": round(h_call_serial_ms, 4), "achieved": round(alone, 1),
                          "frac": round(alone / HBM_PEAK_GBS, 4),
                          "note": "the same calls in the serial pass, with nothing else running"}}
    roof["traffic"] = traffic_from_profiles(roof["kernel"])

    if not args.no_extras:
        # measured HBM ceilings of this device, and every HBM stage against them
        ceil = measure_ceilings(lib, chk, dev, stream, sptr)
        stage_rep["hbm_ceilings"] = ceil
        roof["measured_peak"] = ceil["read_GBps"]
        roof["frac_of_measured"] = round(roof["achieved"] / ceil["read_GBps"], 4)
        roof["measured_peak_note"] = ("streaming-read ceiling measured in this run (nvfp4_probe_read, 2 GiB, best "
                                      "of four workgroup counts)")
        if "alone" in roof:
            roof["alone"]["frac_of_measured"] = round(roof["alone"]["achieved"] / ceil["read_GBps"], 4)
        rw = {"a1_scale2": (1, 0), "a2_hessian": (1, 0), "a4_quantize": (2.0, 0.5625),
              "a5_dequant": (0.5625, 2.0), "a6_cast": (E5.numel() + fb * 16, c5[0].numel() + fb * 16)}
        for k, (r_, w_) in rw.items():
            if "GBps" in stage_rep[k]:
                stage_rep[k]["frac_of_measured"] = round(stage_rep[k]["GBps"] / ceiling_for(ceil, r_, w_), 4)
                if r_ and w_:
                    stage_rep[k]["frac_of_copy"] = round(stage_rep[k]["GBps"] / ceil["copy_GBps"], 4)
        # each HBM stage again, over rotating distinct buffers (MALL defeated,
        # launch gaps included, one event pair per rotation)
        rot = rotated_stage_times(lib, chk, dev, stream, sptr, W, x3, s2x3, q3, P5, E5, c5, fb, ceil)
        for k, v in rot.items():
            stage_rep[k]["rotated"] = v
        # the read-and-write stages against a plain copy of the same number of
        # bytes, timed the same way (a size-matched ceiling: short kernels do
        # not reach the 2 GiB streaming rates)
        for k in ("a4_quantize", "a5_dequant", "a6_cast"):
            r = rot[k]
            nbytes = r["GBps"] * 1e9 * r["ms_per_call"] / 1e3
            cu = copy_same_bytes_us(lib, chk, dev, stream, sptr, nbytes)
            r["copy_same_bytes_us"] = round(cu, 2)
            # a time ratio, not a utilisation: above 1 the stage beats a 1:1 copy
            # of its byte count (a write-heavy mix can)
            r["copy_time_over_stage_time"] = round(cu / (r["ms_per_call"] * 1e3), 4)
        stage_rep["c2_qproj"] = c2_leg(lib, chk, dev, stream, sptr, ceil)

    if not args.no_extras:
        # W4A4 form of a2, outside the step: the Hessian of the fake-quantized
        # calibration streams (activation scale_2 from max calibration of each
        # stream's first chunk), one chunk-list call per stream and pass
        s2a = {s: torch.zeros(1, **f32) for s in (0, 1)}
        Hq = {s: torch.zeros_like(H[s]) for s in (0, 1)}
        for s in (0, 1):
            chk("scale2", lib.nvfp4_compute_scale2(X[s][0].data_ptr(), X[s][0].numel(), s2a[s].data_ptr(), None, sptr))

        def fq_pass():
            for s in (0, 1):
                Hq[s].zero_()
                x0 = X[s][0]
                chk("hessian_fq", lib.nvfp4_hessian_accum_fq_chunks(x_ptrs[s], len(X[s]), x0.shape[0], x0.shape[1],
                                                                    x0.shape[1], s2a[s].data_ptr(), Hq[s].data_ptr(),
                                                                    None, wsc.data_ptr(), wsc.numel(), sptr))

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
            "outside_step": True, "ms_per_pass": round(fq_ms, 4), "calls_per_pass": 2, "launches_per_pass": 34,
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
            "schedule": "timed steps: a1, a2 of both calibration streams, then a4-a6 on one HIP stream; the "
                        "three sweeps (capped at one workgroup per CU) on a second stream, the gate/up sweeps beside "
                        "the second calibration stream's Hessian and the down sweep beside the next step's a1 and "
                        "first Hessian (two alternating sets of H/amax/scale_2 buffers; checked bit-exact against "
                        "the serial order); stages: the same work in stage order on one stream",
            "serial_step_ms": round(step_ms, 4),
        },
        "roofline": roof,
        "cpu_baseline": None,
        "stages": stage_rep,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(W, X, H, s2w, blocks)
    print(json.dumps(out), flush=True)


def ev_ms(stream, fn, reps, warm=1):
    """Mean ms per fn() over `reps` calls between one HIP event pair on `stream`."""
    import torch
    for _ in range(warm):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def measure_ceilings(lib, chk, dev, stream, sptr, reps=5):
    """HBM read, write and copy rates of this device from plain streaming
    kernels (nvfp4_probe_*: 16 B per lane, 1 KiB per wave instruction) over
    2 GiB buffers, eight times the 256 MB MALL; each at a few workgroup
    counts, keeping the best (a ceiling is the most the box was seen to do)."""
    import torch
    n = 1 << 31
    a = torch.zeros(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    half = n // 2
    grids = (256, 512, 1024, 2048)
    best = {}
    for g in grids:
        tr = ev_ms(stream, lambda: chk("probe read", lib.nvfp4_probe_read(a.data_ptr(), n, sink.data_ptr(), g,
                                                                            sptr)), reps)
        tw = ev_ms(stream, lambda: chk("probe write", lib.nvfp4_probe_write(b.data_ptr(), n, 0, g, sptr)), reps)
        tc = ev_ms(stream, lambda: chk("probe copy", lib.nvfp4_probe_copy(a.data_ptr(), b.data_ptr() + half, half,
                                                                            g, sptr)), reps)
        for name, v in (("read", n / tr), ("write", n / tw), ("copy", 2 * half / tc)):
            gbs = v / 1e6
            if gbs > best.get(name, (0, 0))[0]:
                best[name] = (gbs, g)
    del a, b
    torch.cuda.empty_cache()
    return {"read_GBps": round(best["read"][0], 1), "write_GBps": round(best["write"][0], 1),
            "copy_GBps": round(best["copy"][0], 1),
            "best_workgroups": {k: v[1] for k, v in best.items()},
            "kernels": "nvfp4_probe_read / _write / _copy: 2 GiB read, 2 GiB written, 1 GiB copied "
                       "(copy counts read + written bytes); 5 calls each between one event pair, at "
                       f"{', '.join(str(g) for g in grids)} workgroups, best kept",
            "frac_of_measured_rule": "a stage that reads R and writes W bytes is compared with "
                                     "(R + W) / (R / read_GBps + W / write_GBps)",
            "frac_of_copy_rule": "a stage that both reads and writes is also compared with copy_GBps: "
                                 "interleaved read and write streams on this device reach about the copy "
                                 "rate, not the serial read-then-write rate"}


def copy_same_bytes_us(lib, chk, dev, stream, sptr, nbytes, nrot=8, reps=4):
    """Microseconds of nvfp4_probe_copy moving nbytes in all (nbytes / 2 read,
    nbytes / 2 written), rotating over nrot buffer pairs so that no call finds
    its source in the MALL; best of four workgroup counts."""
    import torch
    half = (int(nbytes) // 2 + 15) // 16 * 16
    src = [torch.zeros(half, dtype=torch.uint8, device=dev) for _ in range(nrot)]
    dst = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(nrot)]
    best = float("inf")
    for g in (256, 512, 1024, 2048):
        def one(g=g):
            for i in range(nrot):
                chk("probe copy", lib.nvfp4_probe_copy(src[i].data_ptr(), dst[i].data_ptr(), half, g, sptr))
        one()
        best = min(best, ev_ms(stream, one, reps, warm=0) / nrot * 1e3)
    del src, dst
    torch.cuda.empty_cache()
    return best


def ceiling_for(ceil, r, w):
    """Rate of a read of r bytes followed by a write of w bytes at the measured ceilings."""
    return (r + w) / (r / ceil["read_GBps"] + w / ceil["write_GBps"])


def sweep_work(lib, chk, w, H, s2, ref_out, sptr):
    """Counters of the sweep's search (nvfp4_scale_sweep_stats) on one weight;
    its outputs must equal ref_out (packed, codes) bit for bit."""
    import torch
    st = torch.zeros(6, dtype=torch.int64, device=w.device)
    p = torch.empty_like(ref_out[0])
    c = torch.empty_like(ref_out[1])
    chk("sweep stats", lib.nvfp4_scale_sweep_stats(w.data_ptr(), w.shape[0], w.shape[1], w.shape[1], H.data_ptr(),
                                                   s2.data_ptr(), p.data_ptr(), c.data_ptr(), st.data_ptr(), sptr))
    torch.cuda.synchronize()
    if not (torch.equal(p, ref_out[0]) and torch.equal(c, ref_out[1])):
        raise RuntimeError("the counting sweep's outputs differ from the sweep's")
    return [int(v) for v in st.cpu().tolist()]


# the sources each profiled kernel's device code comes from (common.hpp holds
# host-side declarations only); a committed counter line applies while their
# hashes (first 16 hex digits of sha256, joined by "+") match the ones it was
# taken on
KERNEL_SOURCES = {
    "sweep_kernel": ("sweep_kernel.hpp", "sweep.hip", "nvfp4_device.hpp"),
    "hessian_partial_kernel": ("hessian.hip", "nvfp4_device.hpp"),
    "hessian_reduce_kernel": ("hessian.hip", "nvfp4_device.hpp"),
}


def src_sha(files):
    csrc = os.path.join(ROOT, "nvfp4_post_quantization_amd", "csrc")
    return "+".join(hashlib.sha256(open(os.path.join(csrc, f), "rb").read()).hexdigest()[:16] for f in files)


def valu_issue_from_profiles():
    """VALU issue utilisation of the uncapped sweep from the committed SQ
    counter summary, if it was taken on the current sweep sources."""
    path = os.path.join(ROOT, "profiles", "sweep_valu_counters.txt")
    try:
        sha = src_sha(KERNEL_SOURCES["sweep_kernel"])
        for ln in open(path):
            if ln.startswith("kernel=sweep_kernel"):
                kv = dict(x.split("=", 1) for x in ln.split() if "=" in x)
                if kv.get("src_sha") == sha:
                    return {k: float(v) for k, v in kv.items() if k not in ("kernel", "src_sha")}
    except (OSError, ValueError):
        pass
    return None


def sweep_work_report(stats, seconds):
    """Executed-work figures of a set of sweeps that took `seconds` in all."""
    tot = [sum(v[i] for v in stats.values()) for i in range(6)]
    evals, steps, forms, screens, nblk, waves = tot
    executed = 64 * (steps * QUANT_FLOP + forms * FORM_FLOP + screens * SCREEN_FLOP)
    useful = evals * (QUANT_FLOP + FORM_FLOP)
    ex_tf = executed / seconds / 1e12
    out = {
        "evaluated_codes_per_block": round(evals / nblk, 3),
        "evaluated_codes_per_block_by_weight": {n: round(v[0] / v[4], 3) for n, v in stats.items()},
        "lane_utilisation": round(evals / (64 * steps), 4),
        "full_form_step_share": round(forms / steps, 4),
        "executed_TFLOPs": round(ex_tf, 2),
        "frac_valu_nonpacked_peak": round(ex_tf / VALU_NONPACKED_TFLOPS, 4),
        "useful_TFLOPs": round(useful / seconds / 1e12, 2),
        "exhaustive_roofline_blocks_per_s": round(FP32_PEAK_TFLOPS * 1e12 / SWEEP_FLOP_PER_BLOCK, 1),
        "valu_issue_from_counters": valu_issue_from_profiles(),
        "work_note": (f"counted by nvfp4_scale_sweep_stats (same kernel body, same outputs): each wave step is one "
                      f"code slot for all 64 lanes; executed flop = 64 x (steps x {QUANT_FLOP} + full-form steps "
                      f"x {FORM_FLOP} + screen steps x {SCREEN_FLOP}), useful flop = evaluated codes x "
                      f"{QUANT_FLOP + FORM_FLOP}, against the {VALU_NONPACKED_TFLOPS} TFLOP/s non-packed fp32 VALU "
                      f"ceiling of the library as compiled (packed fp32 forms off); the exhaustive roofline is the spec-peak rate of a search that "
                      f"evaluates all 127 codes ({SWEEP_FLOP_PER_BLOCK} flop per block)"),
    }
    return out


def rotated_stage_times(lib, chk, dev, stream, sptr, W, x3, s2x3, q3, P5, E5, c5, fb, ceil, reps=3):
    """Per-call time of a1, a4, a5 and a6 over rotating distinct buffers, so
    that no call finds its input in the 256 MB MALL: eight copies of the C3
    activations (512 MiB) and their outputs for a1/a4/a5 (a1 also over the
    three C4 weights), two copies of the C5 experts for a6.  One event pair
    per rotation; launch gaps between the calls are included."""
    import torch
    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    nrot = 8
    xs = [x3.clone() for _ in range(nrot)]
    qs = [(torch.empty_like(q3[0]), torch.empty_like(q3[1])) for _ in range(nrot)]
    ds = [torch.empty_like(x3) for _ in range(nrot)]
    rows, k = x3.shape
    a1_in = list(W.values()) + xs

    a1_s2 = torch.zeros(len(a1_in), **f32)
    a1_am = torch.zeros(len(a1_in), **f32)
    a1_ptrs = (ctypes.c_void_p * len(a1_in))(*[t.data_ptr() for t in a1_in])
    a1_ns = (ctypes.c_int64 * len(a1_in))(*[t.numel() for t in a1_in])

    def a1():
        chk("scale2", lib.nvfp4_compute_scale2_batch(a1_ptrs, a1_ns, len(a1_in), a1_s2.data_ptr(),
                                                     a1_am.data_ptr(), sptr))

    def a4():
        for i in range(nrot):
            chk("quantize", lib.nvfp4_quantize_dynamic(xs[i].data_ptr(), rows, k, k, s2x3.data_ptr(),
                                                       qs[i][0].data_ptr(), qs[i][1].data_ptr(), sptr))

    def a5():
        for i in range(nrot):
            chk("dequant", lib.nvfp4_dequant(qs[i][0].data_ptr(), qs[i][1].data_ptr(), s2x3.data_ptr(), rows, k,
                                             ds[i].data_ptr(), sptr))

    P5b, E5b = P5.clone(), E5.clone()
    c5b = tuple(torch.empty_like(t) for t in c5)
    sets = [(P5, E5, c5), (P5b, E5b, c5b)]

    def a6():
        for p, e, c in sets:
            chk("cast", lib.mxfp4_to_nvfp4_cast(p.data_ptr(), e.data_ptr(), 128, 2, 2048, 7168, c[0].data_ptr(),
                                                c[1].data_ptr(), c[2].data_ptr(), sptr))

    n_el = x3.numel()
    a1_bytes = sum(t.numel() * 2 for t in a1_in)
    jobs = {
        "a1_scale2": (a1, 1, a1_bytes, (a1_bytes, 0),
                      "one batched call over the 3 C4 weights + 8 copies of X [8192, 4096] (0.84 GB; 3 launches)"),
        "a4_quantize": (a4, nrot, n_el * 2.5625, (n_el * 2, n_el * 0.5625), "8 copies of X [8192, 4096]"),
        "a5_dequant": (a5, nrot, n_el * 2.5625, (n_el * 0.5625, n_el * 2), "8 packed/code sets -> 8 outputs"),
        "a6_cast": (a6, 2, E5.numel() + c5[0].numel() + fb * C5_FALLBACK_BYTES,
                    (E5.numel() + fb * 16, c5[0].numel() + fb * 16), "2 copies of the 128 expert pairs"),
    }
    out = {}
    for name, (fn, calls, nbytes, (r_, w_), what) in jobs.items():
        ms = ev_ms(stream, fn, reps) / calls
        gbs = nbytes / (ms / 1e3) / 1e9
        out[name] = {"ms_per_call": round(ms, 4), "rotation": what, "GBps": round(gbs, 1),
                     "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                     "frac_of_measured": round(gbs / ceiling_for(ceil, r_, w_), 4)}
        if r_ and w_:
            out[name]["frac_of_copy"] = round(gbs / ceil["copy_GBps"], 4)
    # the cast rewrote fallback nibbles in place; put the originals back is not
    # needed after this point (nothing reads P5 again)
    del xs, qs, ds, P5b, E5b, c5b
    torch.cuda.empty_cache()
    return out


def c2_leg(lib, chk, dev, stream, sptr, ceil, reps=20):
    """The Gemma-2B-like q_proj [2048, 2048] with 4096 calibration tokens
    [4096, 2048], outside the step: a1 (scale_2 of W), a2 (H of the 4096
    tokens; 16 MiB, MALL-resident across the repeated calls, reported, not
    graded) and a3 (sweep of all 2048 rows, 262,144 blocks)."""
    import numpy as np
    import torch
    import datagen
    f32 = dict(dtype=torch.float32, device=dev)
    wb, xb = datagen.config2()
    w = torch.from_numpy(np.ascontiguousarray(wb).view(np.int16)).view(torch.bfloat16).to(dev)
    x = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).to(dev)
    (rows, k), t = w.shape, x.shape[0]
    s2, am = torch.zeros(1, **f32), torch.zeros(1, **f32)
    H, Hacc, amx = torch.zeros((k // 16, 16, 16), **f32), torch.zeros((k // 16, 16, 16), **f32), torch.zeros(1, **f32)
    ws = torch.empty(lib.nvfp4_hessian_workspace_bytes(t, k), dtype=torch.uint8, device=dev)
    packed = torch.empty((rows, k // 2), dtype=torch.uint8, device=dev)
    codes = torch.empty((rows, k // 16), dtype=torch.uint8, device=dev)
    a1 = lambda: chk("scale2", lib.nvfp4_compute_scale2(w.data_ptr(), w.numel(), s2.data_ptr(), am.data_ptr(), sptr))
    a2 = lambda: chk("hessian", lib.nvfp4_hessian_accum(x.data_ptr(), t, k, k, Hacc.data_ptr(), amx.data_ptr(),
                                                        ws.data_ptr(), ws.numel(), sptr))
    a3 = lambda: chk("sweep", lib.nvfp4_scale_sweep(w.data_ptr(), rows, k, k, H.data_ptr(), s2.data_ptr(),
                                                    packed.data_ptr(), codes.data_ptr(), None, sptr))
    a1()
    chk("hessian", lib.nvfp4_hessian_accum(x.data_ptr(), t, k, k, H.data_ptr(), None, ws.data_ptr(), ws.numel(),
                                           sptr))
    t1, t2, t3 = ev_ms(stream, a1, reps), ev_ms(stream, a2, reps), ev_ms(stream, a3, reps)
    blocks = rows * k // 16
    work = sweep_work(lib, chk, w, H, s2, (packed, codes), sptr)
    roof_us = blocks * SWEEP_FLOP_PER_BLOCK / (FP32_PEAK_TFLOPS * 1e12) * 1e6
    a3_rep = {"ms": round(t3, 4), "blocks": blocks, "blocks_per_s": round(blocks / (t3 / 1e3), 1),
              "exhaustive_roofline_us": round(roof_us, 1), "target_ms": round(2 * roof_us / 1e3, 4),
              "target_met": bool(t3 <= 2 * roof_us / 1e3)}
    a3_rep.update(sweep_work_report({"q_proj": work}, t3 / 1e3))
    a3_rep["target_note"] = ("target: half the spec-peak rate of the exhaustive 127-code search, i.e. at most "
                             "twice the exhaustive roofline time")
    g2 = x.numel() * 2 / (t2 / 1e3) / 1e9
    return {"outside_step": True, "workload": f"W [{rows}, {k}] bf16, X [{t}, {k}] bf16 (one call each)",
            "a1_scale2": {"ms": round(t1, 4), "GBps": round(w.numel() * 2 / (t1 / 1e3) / 1e9, 1)},
            "a2_hessian": {"ms": round(t2, 4), "GBps": round(g2, 1), "frac_hbm_peak": round(g2 / HBM_PEAK_GBS, 4),
                           "mall_resident": True,
                           "note": "16 MiB of X stays in the MALL across the repeated calls: not an HBM figure"},
            "a3_sweep": a3_rep}


def traffic_from_profiles(kernel: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by the copy
    probe) from the committed counter summary, times each kernel's launches
    per call where the summary states them; null unless every kernel of
    `kernel` ("a+b" sums them) was measured on its current source."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.txt")
    total = 0.0
    try:
        lines = [dict(kv.split("=", 1) for kv in ln.split() if "=" in kv)
                 for ln in open(path) if ln.startswith("kernel=")]
        for name in kernel.split("+"):
            sha = src_sha(KERNEL_SOURCES[name])
            hit = [f for f in lines if f.get("kernel") == name and f.get("src_sha") == sha]
            if not hit:
                return None
            total += float(hit[0]["hbm_bytes_per_launch"]) * float(hit[0].get("launches_per_call", 1))
    except (OSError, KeyError, ValueError):
        return None
    return round(total, 1)


def _cpu_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _cpu_hessian_piece(x_bits):
    import oracle
    oracle.hessian(x_bits)
    return x_bits.shape[0] * x_bits.shape[1]


def _cpu_sweep_rows(w_bits, h, s2):
    import oracle
    oracle.scale_sweep(w_bits, h, s2)
    return w_bits.size // 16


def cpu_baseline(W, X, H, s2w, blocks):
    """Time the float64 oracle on a bounded sample of the same job, spread
    over a pool of worker processes (one per host core, up to 16, one BLAS
    thread each: Hessian pieces of 16384 tokens x 64 groups, sweep tiles of
    16 rows), and extrapolate to the whole step (Hessian of both calibration
    streams + the three sweeps).  The inputs are copied to the host before
    the clock starts; the pool is started and warmed up before it too."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import numpy as np
    import torch
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    pool = cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"),
                                  initializer=_cpu_worker_init)
    warm = np.zeros((64, 16), dtype=np.uint16)
    list(pool.map(_cpu_hessian_piece, [warm] * workers))
    n_chunks = 2                                   # whole 65536-token chunks per stream
    t_tok = n_chunks * X[0][0].shape[0]
    pieces = []
    for s in (0, 1):
        for c in range(n_chunks):
            xs = X[s][c].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            pieces += [np.ascontiguousarray(xs[t0:t0 + 16384, c0:c0 + 1024])
                       for c0 in range(0, xs.shape[1], 1024) for t0 in range(0, xs.shape[0], 16384)]
            del xs
    rows = {"gate": 1536, "down": 512}
    tiles = []
    for n, r in rows.items():
        wb = W[n][:r].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        h = H[0 if n != "down" else 1].cpu().numpy().astype(np.float64)
        s2 = float(s2w[n].cpu().numpy()[0])
        tiles += [(np.ascontiguousarray(wb[i:i + 16]), h, s2) for i in range(0, r, 16)]
    a = time.perf_counter()
    list(pool.map(_cpu_hessian_piece, pieces))
    t_h = time.perf_counter() - a
    a = time.perf_counter()
    sweep_blocks = sum(pool.map(_cpu_sweep_rows, *zip(*tiles)))
    t_s = time.perf_counter() - a
    pool.shutdown()
    full_tokens = 1 << 20
    t_hess = t_h * (full_tokens / t_tok)
    t_sweep = t_s / sweep_blocks * blocks
    est = t_hess + t_sweep
    return {
        "value": round(blocks / est, 1),
        "unit": "weight blocks/s",
        "cores": workers,
        "kind": "oracle",
        "sample": (f"float64 oracle in {workers} worker processes x 1 BLAS thread (Hessian: {t_tok} tokens of "
                   f"each calibration stream in 16384-token x 64-group pieces, {t_h:.1f} s; sweep: "
                   f"{rows['gate']} gate rows + {rows['down']} down rows = {sweep_blocks} blocks in 16-row tiles, "
                   f"{t_s:.1f} s), extrapolated to 2^20 tokens and {blocks} blocks: est. {est:.0f} s per step "
                   f"(Hessian {t_hess:.0f} s, sweep {t_sweep:.0f} s); host cores visible "
                   f"{len(os.sched_getaffinity(0))}"),
        "threads": {"hessian_leg": workers, "sweep_leg": workers, "per_worker_blas_threads": 1},
    }


if __name__ == "__main__":
    main()
