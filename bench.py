#!/usr/bin/env python3
"""Bench: the BitNet b1.58 BitLinear forward on one MI355X.

Headline (`value`): weight-stream throughput of the M = 1 decode path over the
210 matrices of one decode step of 30 distinct 2.4B-shaped transformer layers
-- per layer q (2560->2560), k and v (2560->640), o (2560->2560), gate and up
(2560->6912), down (6912->2560): 2,084,044,800 ternary weights, 521,011,200
packed bytes (about twice the 256 MB on-chip cache).  The 210 problems are
treated as independent and run as ONE fused launch per step: every workgroup
quantizes its token row (int8 absmax) while staging it, then streams its rows
of packed weights through the ternary GEMV and the fp32 rescale.  A real
decode step has dependencies (q/k/v -> attention -> o -> gate/up -> down ->
next layer), so the figure is the sustained weight-stream rate of the path,
not a reachable per-token step time; the `deporder` leg times the same
matrices in dependency order, one launch per stage, for context.  Weight
ternarization / packing is the offline step and runs once before timing.
Inputs are seeded synthetic tensors generated in HBM before the timed region.

value = packed weight bytes per step / wall time per step (GB/s, 1 GB = 1e9 B).

Also reported: the roofline of the dominant kernel (gemv_fused_grouped_kernel)
from HIP events recorded on its stream inside the timed region, next to the
in-run achievable ceilings (a streaming read of a 4 GiB buffer, int8 MFMAs from
registers); the single 2560 x 2560 GEMV hot and HBM-cold; the prefill GEMM
(M = 2048) in int8 TOPS; the batched-decode sweep hot and HBM-cold; the CPU
oracle timed on the whole decode step with all host threads and with one.
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, TOPS


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("gemv.hip", "device_common.h"):
        with open(os.path.join(ROOT, "ternary_weight_token_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, or None
    when the counters were taken on different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(f"{kernel}|{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def settle(torch, fn, seconds: float = 0.1) -> None:
    """Untimed calls of fn() for a fixed wall time before a leg is timed: after the
    host-side set-up between legs the GPU's clocks have dropped, and they take tens
    of milliseconds of load to come back."""
    t0 = time.perf_counter()
    while True:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return


def graph_us(torch, fn, reps: int = 20, replays: int = 5) -> float:
    """Device time per call of fn(): reps calls captured in one HIP graph, replayed
    (removes the host cost of one launch per call from the figure)."""
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (reps * replays)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--legs", default="achievable,config0,two_launch,deporder,rmsnorm,prefill,sweep,decode_m8,"
                                      "ffn100b,scales,encodings",
                    help="secondary legs to run (comma-separated subset of the default)")
    ap.add_argument("--clock-ramp-ms", type=float, default=300.0,
                    help="untimed launches of the step for this wall time before the warmup steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling PMC byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    from synth import workloads as W
    import ternary_weight_token_amd as tw

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    tw.lib()
    dev = "cuda:0"
    stream = torch.cuda.current_stream()

    # ------------------------------------------------------------ headline setup
    t0 = time.time()
    mats = W.decode_step_2p4b(30)
    packed, sws = [], []
    for m in mats:
        w = W.weights(m, dev)
        p, s = tw.pack_weights(w, 1e-5)
        packed.append(p)
        sws.append(s)
        del w
    xs = [W.decode_step_activations(l, dev) for l in range(30)]
    ys = [torch.empty((1, m.N), dtype=torch.float32, device=dev) for m in mats]
    # the step: one fused launch (activation quantization inside the GEMV workgroups)
    fplan = tw.bitnet_grouped_plan_fused(
        [(xs[m.layer][m.slot], packed[i], sws[i], ys[i], None, None, None) for i, m in enumerate(mats)])
    torch.cuda.synchronize()
    weight_bytes = sum(m.N * m.K // 4 for m in mats)
    n_weights = sum(m.N * m.K for m in mats)
    # algorithmic bytes of one fused launch: 0.25 B per weight, 2 B per x element read
    # (once per matrix), 4 B per output, 4 B per s_w read
    fused_bytes = weight_bytes + sum(2 * m.K + 4 * m.N + 4 for m in mats)
    log(f"decode step ready in {time.time() - t0:.1f}s: {len(mats)} matrices, {weight_bytes} packed bytes")

    # ------------------------------------------------------------ timed region
    # One launch per step and nothing else on the stream, so the HIP event pair
    # around the timed region divided by the step count is the launch's average
    # duration (inter-launch gaps included).  Events around every launch would add
    # their own dispatch overhead to both the wall time and the launch (~5 us here).
    # Before the warmup steps the step runs untimed for a fixed wall time: an idle GPU
    # takes tens of milliseconds of load to leave its low clocks, longer than a few
    # warmup steps last.
    ramp_s = max(args.clock_ramp_ms, 0.0) * 1e-3
    r0 = time.perf_counter()
    while time.perf_counter() - r0 < ramp_s:
        for _ in range(64):
            fplan.launch(stream)
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        fplan.launch(stream)
    torch.cuda.synchronize()
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e_start.record(stream)
    for _ in range(args.steps):
        fplan.launch(stream)
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = wall * 1e3 / args.steps
    kern_ms = e_start.elapsed_time(e_end) / args.steps
    value = weight_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = fused_bytes / (kern_ms * 1e-3) / 1e9
    log(f"step {ms_per_step * 1e3:.1f} us wall, fused quant + GEMV launch {kern_ms * 1e3:.1f} us (events) "
        f"-> {achieved:.0f} GB/s")
    # sanity: outputs of the last step are finite
    for y in ys:
        assert torch.isfinite(y).all()

    line = {
        "metric": "BitLinear M=1 weight-stream GB/s (% HBM peak); int8 TOPS at M=2048",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_ramp_ms": args.clock_ramp_ms,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded SplitMix64 inputs generated in HBM)",
        "config": {
            "workload": "decode step: 30 x 2.4B-shaped layers {q,k,v,o,gate,up,down}, M=1, "
                        "one fused launch per step (activation quantization + ternary GEMV + rescale)",
            "matrices": len(mats), "weights": n_weights, "packed_bytes": weight_bytes,
            "hbm_frac_of_value": round(value / HBM_PEAK_GBS, 4),
            "weights_per_s": round(n_weights / (ms_per_step * 1e-3), 1),
        },
        "roofline": {
            "kernel": "gemv_fused_grouped_kernel",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": committed_traffic("gemv_fused_grouped_kernel", "decode_step_2p4b"),
            "algorithmic_bytes_per_launch": fused_bytes,
            "avg_launch_us": round(kern_ms * 1e3, 2),
        },
    }

    # ------------------------------------------------------------ secondary legs
    if not args.no_secondary:
        sec = {}
        legs = set(args.legs.split(","))
        if "achievable" in legs:
            # in-run ceilings beside the spec peaks: one streaming read of a 4 GiB buffer
            # (16x the on-chip cache; 16-byte non-temporal lane-linear loads) and int8
            # MFMAs from registers only (v_mfma_i32_16x16x64_i8, 8 chains per wavefront)
            sink = torch.zeros(1, dtype=torch.int32, device=dev)
            buf = torch.randint(-(1 << 31), (1 << 31) - 1, (1 << 30,), dtype=torch.int32, device=dev)
            nbytes = buf.numel() * 4
            best = {}
            for blocks in (2048, 4096, 8192, 16384, 32768):
                for _ in range(2):
                    tw.probe_stream_read(buf, sink, blocks)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(10):
                    tw.probe_stream_read(buf, sink, blocks)
                b.record(stream)
                torch.cuda.synchronize()
                best[blocks] = nbytes / (a.elapsed_time(b) * 1e-3 / 10) / 1e9
            del buf
            sr_blocks = max(best, key=best.get)
            mfma = {}
            for blocks in (256, 512, 1024):
                tw.probe_mfma_i8(sink, blocks, 200)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                ops = 0.0
                for _ in range(5):
                    ops += tw.probe_mfma_i8(sink, blocks, 4000)
                b.record(stream)
                torch.cuda.synchronize()
                mfma[blocks] = ops / (a.elapsed_time(b) * 1e-3) / 1e12
            mf_blocks = max(mfma, key=mfma.get)
            sec["achievable"] = {
                "stream_read_GBs": round(best[sr_blocks], 1), "stream_read_frac_of_spec": round(best[sr_blocks] / HBM_PEAK_GBS, 4),
                "stream_read": f"4 GiB once per launch, {sr_blocks} workgroups of 256 threads (best of "
                               f"{sorted(best)}: {[round(best[k]) for k in sorted(best)]} GB/s)",
                "mfma_i8_TOPS": round(mfma[mf_blocks], 1), "mfma_i8_frac_of_spec": round(mfma[mf_blocks] / INT8_PEAK_TOPS, 4),
                "mfma_i8": f"{mf_blocks} workgroups x 8 wavefronts x 8 chains x 4000 rounds (best of "
                           f"{sorted(mfma)}: {[round(mfma[k]) for k in sorted(mfma)]} TOPS)"}
            line["roofline"]["achievable"] = round(best[sr_blocks], 1)
            line["roofline"]["frac_of_achievable"] = round(achieved / best[sr_blocks], 4)
            log(f"achievable: stream read {best[sr_blocks]:.0f} GB/s, int8 MFMA {mfma[mf_blocks]:.0f} TOPS")
            del sink
        if "config0" in legs:
            # the single 2560 x 2560 GEMV (M = 1, 0.1% x20 outliers): the whole path per call
            # (quantization + GEMV launches) and the GEMV alone, hot (the same 1.6 MB of
            # weights every call, cache-resident) and HBM-cold (320 distinct copies, 524 MB,
            # twice the on-chip cache, called in turn); device time from HIP graphs
            x0, w0 = W.single_gemv(dev)
            p0, s0 = tw.pack_weights(w0, 1e-5)
            del w0
            q0, sx0 = tw.quant_act(x0)
            y0 = torch.empty((1, 2560), dtype=torch.float32, device=dev)
            path_us = graph_us(torch, lambda: (tw.bitnet_quant_act(x0, q0, sx0), tw.bitnet_linear(q0, sx0, p0, s0, y0)),
                               reps=50)
            hot_us = graph_us(torch, lambda: tw.bitnet_linear(q0, sx0, p0, s0, y0), reps=50)
            copies = [p0.clone() for _ in range(320)]

            def cold_calls():
                for c in copies:
                    tw.bitnet_linear(q0, sx0, c, s0, y0)
            cold_us = graph_us(torch, cold_calls, reps=1, replays=5) / len(copies)
            wb = p0.numel()
            sec["config0_single_gemv_2560"] = {
                "path_us": round(path_us, 2), "hot_us": round(hot_us, 2), "hot_weight_GBs": round(wb / (hot_us * 1e-6) / 1e9, 1),
                "cold_us": round(cold_us, 2), "cold_weight_GBs": round(wb / (cold_us * 1e-6) / 1e9, 1),
                "cold_copies": len(copies), "cold_bytes": wb * len(copies)}
            log(f"config 0: path {path_us:.2f} us, GEMV hot {hot_us:.2f} us, cold {cold_us:.2f} us")
            del copies
        if "two_launch" in legs:
            # the same step as two launches: grouped quantization, then grouped GEMV on q
            qs = [[torch.empty((1, x.shape[1]), dtype=torch.int8, device=dev) for x in xl] for xl in xs]
            sxs = [[torch.empty(1, dtype=torch.float32, device=dev) for _ in xl] for xl in xs]
            qplan = tw.bitnet_grouped_plan_quant([(xs[l][j], qs[l][j], sxs[l][j]) for l in range(30) for j in range(4)])
            lplan = tw.bitnet_grouped_plan_linear(
                [(qs[m.layer][m.slot], sxs[m.layer][m.slot], packed[i], sws[i], ys[i], None) for i, m in enumerate(mats)])
            gemv_bytes = weight_bytes + sum(m.K + 4 * m.N + 8 for m in mats)
            settle(torch, lambda: (qplan.launch(stream), lplan.launch(stream)))
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i in range(100):
                qplan.launch(stream)
                lplan.launch(stream)
            b.record(stream)
            torch.cuda.synchronize()
            step_us = a.elapsed_time(b) * 1e3 / 100
            a.record(stream)
            for i in range(100):
                lplan.launch(stream)
            b.record(stream)
            torch.cuda.synchronize()
            g_us = a.elapsed_time(b) * 1e3 / 100
            sec["decode_step_2p4b_two_launches"] = {
                "us": round(step_us, 1), "weight_GBs": round(weight_bytes / (step_us * 1e-6) / 1e9, 1),
                "gemv_grouped_kernel_us": round(g_us, 2),
                "gemv_grouped_kernel_GBs": round(gemv_bytes / (g_us * 1e-6) / 1e9, 1)}
            log(f"two-launch step: {step_us:.1f} us (grouped GEMV {g_us:.1f} us)")
            del qs, sxs, qplan, lplan
        if "deporder" in legs:
            # the same 210 matrices in dependency order: per layer one fused launch each for
            # {q, k, v}, {o}, {gate, up} and {down} (120 launches per step, in stream order,
            # captured in one HIP graph).  Inputs are not chained through attention and the
            # SwiGLU, which are outside the path: this times the launch granularity of a
            # real step, not its arithmetic
            stage_of = {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3}
            plans = []
            for l in range(30):
                for st_ in range(4):
                    probs = [(xs[m.layer][m.slot], packed[i], sws[i], ys[i], None, None, None)
                             for i, m in enumerate(mats) if m.layer == l and stage_of[m.name] == st_]
                    plans.append(tw.bitnet_grouped_plan_fused(probs))

            def dep_step():
                for pl in plans:
                    pl.launch(torch.cuda.current_stream())
            d_us = graph_us(torch, dep_step, reps=1, replays=20)
            sec["decode_step_2p4b_dependency_order"] = {
                "us": round(d_us, 1), "weight_GBs": round(weight_bytes / (d_us * 1e-6) / 1e9, 1),
                "launches": len(plans), "vs_one_launch_us": round(d_us - kern_ms * 1e3, 1)}
            log(f"dependency-order step: {d_us:.1f} us in {len(plans)} launches")
            del plans
        if "rmsnorm" in legs:
            # the same fused step with the RMSNorm of the attention and FFN inputs folded
            # into the q / k / v and gate / up problems (their workgroups normalize the
            # token row with the layer's gain before quantizing it)
            gains = [W.decode_step_gains(l, dev) for l in range(30)]
            nys = [torch.empty_like(y) for y in ys]
            nplan = tw.bitnet_grouped_plan_fused(
                [(xs[m.layer][m.slot], packed[i], sws[i], nys[i], None, None, None,
                  gains[m.layer].get(m.slot), 1e-6) for i, m in enumerate(mats)])
            for _ in range(200):
                nplan.launch(stream)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(200):
                nplan.launch(stream)
            b.record(stream)
            torch.cuda.synchronize()
            n_us = a.elapsed_time(b) * 1e3 / 200
            for y in nys:
                assert torch.isfinite(y).all()
            sec["decode_step_2p4b_rmsnorm_fused"] = {
                "us": round(n_us, 1), "weight_GBs": round(weight_bytes / (n_us * 1e-6) / 1e9, 1),
                "normed_matrices": sum(1 for m in mats if m.slot in W.NORMED_SLOTS_2P4B),
                "vs_plain_fused_us": round(n_us - kern_ms * 1e3, 1)}
            log(f"fused step with RMSNorm: {n_us:.1f} us ({n_us - kern_ms * 1e3:+.1f} us vs without)")
            # and SwiGLU at both ends: each layer's gate / up as one pair problem whose
            # epilogue writes silu(y_gate) y_up (RMSNorm-ed input), and the down
            # projection taking an fp32 row (the SwiGLU output) as its input
            hidden = [W.decode_step_ffn_hidden(l, dev) for l in range(30)]
            sprobs = []
            for i, m in enumerate(mats):
                if m.name == "up":
                    continue
                if m.name == "gate":
                    iu = next(j for j, o in enumerate(mats) if o.layer == m.layer and o.name == "up")
                    sprobs.append((xs[m.layer][m.slot], (packed[i], packed[iu]), (sws[i], sws[iu]), nys[i], None,
                                   None, None, gains[m.layer].get(m.slot), 1e-6))
                elif m.slot == W.SWIGLU_SLOT_2P4B:
                    sprobs.append((hidden[m.layer], packed[i], sws[i], nys[i], None, None, None))
                else:
                    sprobs.append((xs[m.layer][m.slot], packed[i], sws[i], nys[i], None, None, None,
                                   gains[m.layer].get(m.slot), 1e-6))
            splan = tw.bitnet_grouped_plan_fused(sprobs)
            for _ in range(200):
                splan.launch(stream)
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(200):
                splan.launch(stream)
            b.record(stream)
            torch.cuda.synchronize()
            s_us = a.elapsed_time(b) * 1e3 / 200
            for y in nys:
                assert torch.isfinite(y).all()
            sec["decode_step_2p4b_rmsnorm_swiglu_fused"] = {
                "us": round(s_us, 1), "weight_GBs": round(weight_bytes / (s_us * 1e-6) / 1e9, 1),
                "gate_up_pairs": sum(1 for m in mats if m.name == "gate"),
                "fp32_input_matrices": sum(1 for m in mats if m.slot == W.SWIGLU_SLOT_2P4B),
                "vs_rmsnorm_fused_us": round(s_us - n_us, 1)}
            log(f"fused step with RMSNorm and SwiGLU: {s_us:.1f} us ({s_us - n_us:+.1f} us vs RMSNorm only)")
            del nplan, splan, nys, gains, hidden
        if "prefill" in legs:
            # prefill GEMM, M = 2048
            reps = 50
            for name in ("up", "down"):
                for density in (None, 0.3, 0.5, 0.7):
                    x, w = W.prefill_inputs(name, density, dev)
                    p, s = tw.pack_weights(w, 1e-5)
                    del w
                    q, sx = tw.quant_act(x)
                    N, K = p.shape[0], q.shape[1]
                    y = torch.empty((2048, N), dtype=torch.float32, device=dev)
                    settle(torch, lambda: tw.bitnet_linear(q, sx, p, s, y))
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    for _ in range(reps):
                        tw.bitnet_linear(q, sx, p, s, y)
                    b.record(stream)
                    torch.cuda.synchronize()
                    us = a.elapsed_time(b) * 1e3 / reps
                    tops = 2.0 * 2048 * N * K / (us * 1e-6) / 1e12
                    key = f"prefill_{name}_M2048" + ("" if density is None else f"_density{int(density * 100)}")
                    sec[key] = {"us": round(us, 2), "int8_tops": round(tops, 1),
                                "frac_of_int8_peak": round(tops / INT8_PEAK_TOPS, 4)}
                    log(f"{key}: {us:.1f} us, {tops:.0f} TOPS")
                    if density is None:
                        # the same GEMM with the layer bias and a bf16 output
                        bias = torch.linspace(-1.0, 1.0, N, dtype=torch.float32, device=dev)
                        yb = torch.empty((2048, N), dtype=torch.bfloat16, device=dev)
                        for _ in range(5):
                            tw.bitnet_linear_ex(q, sx, p, s, bias, yb)
                        a.record(stream)
                        for _ in range(reps):
                            tw.bitnet_linear_ex(q, sx, p, s, bias, yb)
                        b.record(stream)
                        torch.cuda.synchronize()
                        us = a.elapsed_time(b) * 1e3 / reps
                        tops = 2.0 * 2048 * N * K / (us * 1e-6) / 1e12
                        sec[key + "_bias_bf16"] = {"us": round(us, 2), "int8_tops": round(tops, 1),
                                                   "frac_of_int8_peak": round(tops / INT8_PEAK_TOPS, 4)}
                        log(f"{key}_bias_bf16: {us:.1f} us, {tops:.0f} TOPS")
                        del yb, bias
        if "sweep" in legs:
            # batched-decode sweep K=2560 N=6912: every kernel at every M, one launch
            # per call, device time (graph-captured)
            p, s = tw.pack_weights(W.sweep_weights(dev), 1e-5)
            # hot: the same 4.4 MB of weights every call (cache-resident); cold: 128 distinct
            # copies (566 MB, twice the on-chip cache) called in turn, so that every call
            # streams its weights from HBM
            copies = [p.clone() for _ in range(128)]
            sweep, cold = {}, {}
            for M in (1, 2, 4, 8, 16, 32, 64, 128, 256):
                q, sx = tw.quant_act(W.sweep_activations(M, dev))
                y = torch.empty((M, p.shape[0]), dtype=torch.float32, device=dev)
                row, crow = {}, {}
                for kname, kid in (("gemv", 1), ("mfma_decode", 4), ("gemm", 2), ("auto", 0)):
                    us = graph_us(torch, lambda: tw.bitnet_linear_select(q, sx, p, s, y, None, kid))
                    row[kname] = {"us": round(us, 2), "weight_GBs": round(p.numel() / (us * 1e-6) / 1e9, 1)}

                    def cold_calls(kid=kid):
                        for c in copies:
                            tw.bitnet_linear_select(q, sx, c, s, y, None, kid)
                    us = graph_us(torch, cold_calls, reps=1, replays=3) / len(copies)
                    crow[kname] = {"us": round(us, 2), "weight_GBs": round(p.numel() / (us * 1e-6) / 1e9, 1)}
                sweep[f"M{M}"] = row
                cold[f"M{M}"] = crow
            sec["sweep_K2560_N6912"] = sweep
            sec["sweep_K2560_N6912_cold"] = dict(cold, copies=len(copies), bytes=p.numel() * len(copies))
            log(f"sweep (hot): {json.dumps(sweep)}")
            log(f"sweep (cold): {json.dumps(cold)}")
            del copies

        if "decode_m8" in legs:
            # batched decode step: the same 210 matrices with 8 sequences decoding together
            # (grouped quant + grouped linear, which runs the MFMA decode kernel)
            M8 = 8
            xs8 = [W.decode_step_activations(l, dev, M8) for l in range(30)]
            qs8 = [[torch.empty((M8, x.shape[1]), dtype=torch.int8, device=dev) for x in xl] for xl in xs8]
            sxs8 = [[torch.empty(M8, dtype=torch.float32, device=dev) for _ in xl] for xl in xs8]
            ys8 = [torch.empty((M8, m.N), dtype=torch.float32, device=dev) for m in mats]
            qplan8 = tw.bitnet_grouped_plan_quant([(xs8[l][j], qs8[l][j], sxs8[l][j]) for l in range(30) for j in range(4)])
            lplan8 = tw.bitnet_grouped_plan_linear(
                [(qs8[m.layer][m.slot], sxs8[m.layer][m.slot], packed[i], sws[i], ys8[i], None)
                 for i, m in enumerate(mats)])
            settle(torch, lambda: (qplan8.launch(stream), lplan8.launch(stream)))
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(100):
                qplan8.launch(stream)
                lplan8.launch(stream)
            b.record(stream)
            torch.cuda.synchronize()
            us = a.elapsed_time(b) * 1e3 / 100
            sec["decode_step_2p4b_M8"] = {"us": round(us, 1), "weight_GBs": round(weight_bytes / (us * 1e-6) / 1e9, 1),
                                          "tokens_per_s": round(M8 / (us * 1e-6), 1), "launches": 2}
            log(f"decode step M=8: {us:.1f} us, {sec['decode_step_2p4b_M8']['weight_GBs']} GB/s")
            del xs8, qs8, sxs8, ys8, qplan8, lplan8

        if "ffn100b" in legs:
            # 100B-scale FFN stream: 8 layers x {gate, up 8192->28672; down 28672->8192},
            # 1,409,286,144 packed bytes (5.5x the on-chip cache)
            fmats = W.ffn_100b(8)
            fpacked, fsw = [], []
            for m in fmats:
                p_, s_ = tw.pack_weights(W.weights(m, dev), 1e-5)
                fpacked.append(p_)
                fsw.append(s_)
            fbytes = sum(p_.numel() for p_ in fpacked)
            for M in (1, 8):
                xs8 = [W.ffn_100b_activations(l, M, dev) for l in range(8)]
                qx = [[tw.quant_act(x) for x in xl] for xl in xs8]
                fys = [torch.empty((M, m.N), dtype=torch.float32, device=dev) for m in fmats]
                plan = tw.bitnet_grouped_plan_linear(
                    [(qx[m.layer][m.slot][0], qx[m.layer][m.slot][1], fpacked[i], fsw[i], fys[i], None)
                     for i, m in enumerate(fmats)])
                run = lambda: plan.launch(stream)
                settle(torch, run)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(20):
                    run()
                b.record(stream)
                torch.cuda.synchronize()
                us = a.elapsed_time(b) * 1e3 / 20
                key = f"ffn100b_8layers_M{M}"
                sec[key] = {"us": round(us, 1), "weight_GBs": round(fbytes / (us * 1e-6) / 1e9, 1),
                            "launches": 1, "kernel": "gemv_grouped_kernel" if M == 1 else "skinny2_grouped_kernel"}
                log(f"{key}: {us:.1f} us, {sec[key]['weight_GBs']} GB/s")
            # one GPU's share of an 8-way column split of the 100B gate matrix (K=8192, N=3584)
            shard = fpacked[0][:3584].contiguous()
            q1, s1 = tw.quant_act(W.ffn_100b_activations(0, 1, dev)[0])
            y1 = torch.empty((1, 3584), dtype=torch.float32, device=dev)
            us = graph_us(torch, lambda: tw.bitnet_linear(q1, s1, shard, fsw[0], y1), reps=50)
            sec["colsplit8_gate_shard_M1"] = {"us": round(us, 2), "weight_GBs": round(shard.numel() / (us * 1e-6) / 1e9, 1)}
            del fpacked
        if "encodings" in legs:
            # the decode step with its weights as sign / mask bitplanes (the same 2 bits
            # per weight, converted from the packed codes): one fused launch of the
            # bit-serial kernel, quantization inside the workgroups as in the timed step
            planes = [tw.pack_bitplanes(p_, m.K) for p_, m in zip(packed, mats)]
            bys = [torch.empty_like(y) for y in ys]
            bplan = tw.bitnet_grouped_plan_fused(
                [(xs[m.layer][m.slot], planes[i], sws[i], bys[i], None, None, None) for i, m in enumerate(mats)])
            for _ in range(300):
                bplan.launch(stream)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(500):
                bplan.launch(stream)
            b.record(stream)
            torch.cuda.synchronize()
            b_us = a.elapsed_time(b) * 1e3 / 500
            for y_, yb_ in zip(ys, bys):
                assert torch.isfinite(yb_).all()
            sec["decode_step_2p4b_bitplanes_fused"] = {
                "us": round(b_us, 1), "weight_GBs": round(weight_bytes / (b_us * 1e-6) / 1e9, 1),
                "kernel": "gemv_bits_fused_grouped_kernel", "vs_codes_fused_us": round(b_us - kern_ms * 1e3, 1)}
            log(f"fused step over bitplanes: {b_us:.1f} us ({b_us - kern_ms * 1e3:+.1f} us vs the 2-bit codes)")
            del planes, bys, bplan
            # the same 100B-scale FFN stream (M = 1, 24 GEMV launches in one graph) with
            # the weights as 2-bit codes, as sign / mask bitplanes (same bytes, another
            # contraction) and as b1.0 binary bits (half the bytes)
            fmats = W.ffn_100b(8)
            enc = {"two_bit_codes": [], "bitplanes": [], "binary": []}
            for m in fmats:
                w = W.weights(m, dev)
                p_, s_ = tw.pack_weights(w, 1e-5)
                enc["two_bit_codes"].append((p_, s_))
                enc["bitplanes"].append((tw.pack_bitplanes(p_, m.K), s_))
                enc["binary"].append(tw.pack_weights_binary(w))
                del w
            xq = [[tw.quant_act(x) for x in W.ffn_100b_activations(l, 1, dev)] for l in range(8)]
            fys = [torch.empty((1, m.N), dtype=torch.float32, device=dev) for m in fmats]
            nweights = sum(m.N * m.K for m in fmats)
            res = {}
            for v in enc:
                def stream_fn(v=v):
                    for i, m in enumerate(fmats):
                        q_, s_ = xq[m.layer][m.slot]
                        wb, sw_ = enc[v][i]
                        if v == "two_bit_codes":
                            tw.bitnet_linear(q_, s_, wb, sw_, fys[i])
                        else:
                            tw.bitnet_linear_bits(q_, s_, wb, tw.FMT_BINARY if v == "binary" else tw.FMT_BITPLANES,
                                                  sw_, fys[i], None, 2)
                us = graph_us(torch, stream_fn, reps=2, replays=5)
                wbytes = sum(e[0].numel() for e in enc[v])
                res[v] = {"us": round(us, 1), "weight_bytes": wbytes,
                          "weight_GBs": round(wbytes / (us * 1e-6) / 1e9, 1),
                          "gweights_per_s": round(nweights / (us * 1e-6) / 1e9, 1), "launches": len(fmats)}
                log(f"ffn100b M=1 encoding {v}: {us:.1f} us, {res[v]['weight_GBs']} GB/s, "
                    f"{res[v]['gweights_per_s']} G weights/s")
            # one launch over the 8 gate matrices stacked (N = 229376, K = 8192): the
            # per-launch ramp and drain no longer weigh on the comparison
            big_w = {}
            for v in enc:
                big_w[v] = torch.cat([enc[v][i][0] for i, m in enumerate(fmats) if m.name == "gate"], 0)
            q0, s0 = xq[0][0]
            yb = torch.empty((1, big_w["binary"].shape[0]), dtype=torch.float32, device=dev)
            one = {}
            for v in enc:
                sw_ = enc[v][0][1]
                if v == "two_bit_codes":
                    fn = lambda: tw.bitnet_linear(q0, s0, big_w[v], sw_, yb)
                else:
                    f_ = tw.FMT_BINARY if v == "binary" else tw.FMT_BITPLANES
                    fn = lambda v=v, f_=f_, sw_=sw_: tw.bitnet_linear_bits(q0, s0, big_w[v], f_, sw_, yb, None, 2)
                us = graph_us(torch, fn, reps=10, replays=5)
                wbytes = big_w[v].numel()
                one[v] = {"us": round(us, 1), "weight_GBs": round(wbytes / (us * 1e-6) / 1e9, 1),
                          "gweights_per_s": round(229376 * 8192 / (us * 1e-6) / 1e9, 1)}
                log(f"stacked gate 229376x8192 M=1 encoding {v}: {us:.1f} us, {one[v]['weight_GBs']} GB/s, "
                    f"{one[v]['gweights_per_s']} G weights/s")
            res["one_launch_229376x8192"] = one
            # the same stacked matrix with 8 tokens, the library's choice for each format: the
            # MFMA decode kernel on the codes, the matrix-core kernel on the planes and on the
            # binary bits (weights read once); and, for comparison, the multi-token bit-serial
            # kernel on both (weights read once per 2 / 4 tokens)
            q8, s8 = tw.quant_act(W.ffn_100b_activations(0, 8, dev)[0])
            y8 = torch.empty((8, big_w["binary"].shape[0]), dtype=torch.float32, device=dev)
            one8 = {}
            for v in enc:
                sw_ = enc[v][0][1]
                if v == "two_bit_codes":
                    fn = lambda: tw.bitnet_linear(q8, s8, big_w[v], sw_, y8)
                else:
                    f_ = tw.FMT_BINARY if v == "binary" else tw.FMT_BITPLANES
                    fn = lambda v=v, f_=f_, sw_=sw_: tw.bitnet_linear_bits(q8, s8, big_w[v], f_, sw_, y8, None, 0)
                us = graph_us(torch, fn, reps=5, replays=3)
                wbytes = big_w[v].numel()
                one8[v] = {"us": round(us, 1), "weight_GBs": round(wbytes / (us * 1e-6) / 1e9, 1),
                           "gweights_per_s": round(229376 * 8192 / (us * 1e-6) / 1e9, 1),
                           "kernel": "skinny2_kernel" if v == "two_bit_codes" else "bits_lds_kernel"}
                log(f"stacked gate 229376x8192 M=8 encoding {v}: {us:.1f} us, {one8[v]['weight_GBs']} GB/s")
                if v != "two_bit_codes":
                    fn3 = lambda v=v, f_=f_, sw_=sw_: tw.bitnet_linear_bits(q8, s8, big_w[v], f_, sw_, y8, None, 3)
                    us3 = graph_us(torch, fn3, reps=5, replays=3)
                    one8[f"{v}_bit_serial"] = {"us": round(us3, 1),
                                               "weight_GBs": round(wbytes / (us3 * 1e-6) / 1e9, 1),
                                               "kernel": "bits_mt_kernel"}
                    log(f"stacked gate 229376x8192 M=8 {v}, bit-serial kernel: {us3:.1f} us")
            res["one_launch_229376x8192_M8"] = one8
            sec["ffn100b_8layers_M1_encodings"] = res
            del enc, big_w
        if "scales" in legs:
            # weight-scale granularity on the 100B-scale FFN stream at M = 1 (HBM-bound):
            # one scale per tensor, per output channel, per group of 128 weights; 24
            # GEMV launches per stream, captured in one graph
            fmats = W.ffn_100b(8)
            variants = {"per_tensor": 0, "per_channel": -1, "group128": 128}
            packs = {v: [] for v in variants}
            for m in fmats:
                w = W.weights(m, dev)
                packs["per_tensor"].append(tw.pack_weights(w, 1e-5))
                packs["per_channel"].append(tw.pack_weights_grouped(w, m.K, 1e-5))
                packs["group128"].append(tw.pack_weights_grouped(w, 128, 1e-5))
                del w
            xq = [[tw.quant_act(x) for x in W.ffn_100b_activations(l, 1, dev)] for l in range(8)]
            fys = [torch.empty((1, m.N), dtype=torch.float32, device=dev) for m in fmats]
            wbytes = sum(m.N * m.K // 4 for m in fmats)
            res = {}
            for v, g in variants.items():
                def stream_fn(v=v, g=g):
                    for i, m in enumerate(fmats):
                        q_, s_ = xq[m.layer][m.slot]
                        p_, sw_ = packs[v][i]
                        tw.bitnet_linear_ex(q_, s_, p_, sw_, None, fys[i], None, 0, w_group=(m.K if g < 0 else g))
                us = graph_us(torch, stream_fn, reps=2, replays=5)
                sbytes = sum(p_[1].numel() * 4 for p_ in packs[v])
                res[v] = {"us": round(us, 1), "weight_GBs": round(wbytes / (us * 1e-6) / 1e9, 1),
                          "scale_bytes": sbytes, "launches": len(fmats)}
                log(f"ffn100b M=1 scales {v}: {us:.1f} us, {res[v]['weight_GBs']} GB/s")
            sec["ffn100b_8layers_M1_weight_scales"] = res
            del packs
            # the decode step as two launches (grouped quantization, grouped GEMV), with
            # one scale per tensor and with group-128 scales
            qs2 = [[torch.empty((1, x.shape[1]), dtype=torch.int8, device=dev) for x in xl] for xl in xs]
            sx2 = [[torch.empty(1, dtype=torch.float32, device=dev) for _ in xl] for xl in xs]
            qplan2 = tw.bitnet_grouped_plan_quant([(xs[l][j], qs2[l][j], sx2[l][j]) for l in range(30) for j in range(4)])
            gpk = []
            for m in mats:
                w = W.weights(m, dev)
                gpk.append(tw.pack_weights_grouped(w, 128, 1e-5))
                del w
            dres = {}
            for v, plan_probs in (
                    ("per_tensor", [(qs2[m.layer][m.slot], sx2[m.layer][m.slot], packed[i], sws[i], ys[i], None)
                                    for i, m in enumerate(mats)]),
                    ("group128", [(qs2[m.layer][m.slot], sx2[m.layer][m.slot], gpk[i][0], gpk[i][1], ys[i], None, 128)
                                  for i, m in enumerate(mats)])):
                lp = tw.bitnet_grouped_plan_linear(plan_probs)
                for _ in range(50):
                    qplan2.launch(stream)
                    lp.launch(stream)
                torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(100):
                    qplan2.launch(stream)
                    lp.launch(stream)
                b.record(stream)
                torch.cuda.synchronize()
                us = a.elapsed_time(b) * 1e3 / 100
                dres[v] = {"us": round(us, 1), "weight_GBs": round(weight_bytes / (us * 1e-6) / 1e9, 1),
                           "scale_bytes": (4 if v == "per_tensor" else sum(p_[1].numel() * 4 for p_ in gpk))}
                log(f"decode step two launches, scales {v}: {us:.1f} us")
            sec["decode_step_2p4b_weight_scales"] = dres
            # the same at 8 tokens (grouped quant + grouped linear): the line-granular MFMA
            # decode kernel, with its group-wise path for group-128 scales
            xs8 = [W.decode_step_activations(l, dev, 8) for l in range(30)]
            qs8 = [[torch.empty((8, x.shape[1]), dtype=torch.int8, device=dev) for x in xl] for xl in xs8]
            sx8 = [[torch.empty(8, dtype=torch.float32, device=dev) for _ in xl] for xl in xs8]
            ys8 = [torch.empty((8, m.N), dtype=torch.float32, device=dev) for m in mats]
            qplan8 = tw.bitnet_grouped_plan_quant([(xs8[l][j], qs8[l][j], sx8[l][j]) for l in range(30) for j in range(4)])
            dres8 = {}
            for v, plan_probs in (
                    ("per_tensor", [(qs8[m.layer][m.slot], sx8[m.layer][m.slot], packed[i], sws[i], ys8[i], None)
                                    for i, m in enumerate(mats)]),
                    ("group128", [(qs8[m.layer][m.slot], sx8[m.layer][m.slot], gpk[i][0], gpk[i][1], ys8[i], None, 128)
                                  for i, m in enumerate(mats)])):
                lp = tw.bitnet_grouped_plan_linear(plan_probs)
                settle(torch, lambda: (qplan8.launch(stream), lp.launch(stream)))
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(30):
                    qplan8.launch(stream)
                    lp.launch(stream)
                b.record(stream)
                torch.cuda.synchronize()
                us = a.elapsed_time(b) * 1e3 / 30
                kern = {1: "skinny2_grouped_kernel<false, true>",
                        4: f"skinny2_grouped_kernel<true, {'true' if lp.flags & 1 else 'false'}>"}.get(
                    lp.variant, f"gemv_grouped_kernel (plan variant {lp.variant})")
                dres8[v] = {"us": round(us, 1), "weight_GBs": round(weight_bytes / (us * 1e-6) / 1e9, 1), "kernel": kern}
                log(f"decode step M=8 two launches, scales {v}: {us:.1f} us")
            sec["decode_step_2p4b_M8_weight_scales"] = dres8
            del gpk, xs8, qs8, sx8, ys8
            # prefill M = 2048 with one scale per tensor and per group of 128 weights (the
            # pipelined GEMM's group-wise path: fp32 accumulators per group)
            pres = {}
            for name in ("up", "down"):
                x, w = W.prefill_inputs(name, None, dev)
                q, sx = tw.quant_act(x)
                N, K = w.shape
                y = torch.empty((2048, N), dtype=torch.float32, device=dev)
                row = {}
                for v, g in (("per_tensor", 0), ("group128", 128)):
                    p_, s_ = tw.pack_weights(w, 1e-5) if g == 0 else tw.pack_weights_grouped(w, g, 1e-5)
                    fn = lambda: tw.bitnet_linear_ex(q, sx, p_, s_, None, y, None, 0, w_group=g)
                    settle(torch, fn)
                    a.record(stream)
                    for _ in range(30):
                        fn()
                    b.record(stream)
                    torch.cuda.synchronize()
                    us = a.elapsed_time(b) * 1e3 / 30
                    tops = 2.0 * 2048 * N * K / (us * 1e-6) / 1e12
                    row[v] = {"us": round(us, 2), "int8_tops": round(tops, 1),
                              "frac_of_int8_peak": round(tops / INT8_PEAK_TOPS, 4)}
                    log(f"prefill {name} M=2048 scales {v}: {us:.1f} us")
                pres[name] = row
                del w, x
            sec["prefill_M2048_weight_scales"] = pres
        line["secondary"] = sec

    # ------------------------------------------------------------ CPU baseline
    if not args.no_cpu_baseline:
        # the oracle (plain C, OpenMP over output rows) on the whole decode step: quant of
        # the 120 activation vectors and the 210 ternary GEMVs over 521 MB of packed
        # weights (more than the host's last-level cache), with every host thread and
        # with one thread; packed on the host by the oracle itself beforehand
        import oracle
        threads = len(os.sched_getaffinity(0))
        oracle.set_threads(threads)
        c_pack = time.perf_counter()
        host_inputs = []
        for m in mats:
            w = W.weights(m, dev).cpu().numpy()
            p_ref, sw_ref = oracle.pack(w, 1e-5)
            del w
            host_inputs.append((m, p_ref, sw_ref))
        xs_host = {(l, s_): synth.bf16_bits(xs[l][s_].cpu()).numpy().view(np.uint16)
                   for l in range(30) for s_ in range(4)}
        log(f"cpu oracle: whole step packed on the host in {time.perf_counter() - c_pack:.1f}s")

        def cpu_steps(min_seconds: float):
            steps = 0
            c0 = time.perf_counter()
            while True:
                qcache = {k: oracle.quant_act(v) for k, v in xs_host.items()}
                for m, p_ref, sw_ref in host_inputs:
                    qv, sv = qcache[(m.layer, m.slot)]
                    oracle.linear(qv, sv, p_ref, sw_ref)
                steps += 1
                if time.perf_counter() - c0 >= min_seconds:
                    return steps, time.perf_counter() - c0

        steps_n, sec_n = cpu_steps(args.cpu_seconds)
        cores_n = oracle.get_threads()
        oracle.set_threads(1)
        steps_1, sec_1 = cpu_steps(args.cpu_seconds / 2)
        oracle.set_threads(threads)
        line["cpu_baseline"] = {
            "value": round(steps_n * weight_bytes / sec_n / 1e9, 3),
            "unit": "GB/s",
            "cores": cores_n,
            "kind": "oracle",
            "sample": f"the whole decode step (quant of 120 vectors + 210 ternary GEMVs, {weight_bytes} packed "
                      f"bytes), {steps_n} steps in {sec_n:.1f}s on {cores_n} threads",
            "one_thread": {"value": round(steps_1 * weight_bytes / sec_1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                           "sample": f"{steps_1} whole steps in {sec_1:.1f}s"},
        }
        log(f"cpu oracle: {line['cpu_baseline']['value']} GB/s on {cores_n} threads, "
            f"{line['cpu_baseline']['one_thread']['value']} GB/s on 1")

    if args.copy_calibration:
        # a plain elementwise kernel of known traffic: reads 1 GiB, writes 1 GiB
        src = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log("copy calibration: 3 x (read 1 GiB + write 1 GiB) elementwise kernels done")

    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
