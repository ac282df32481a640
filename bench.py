#!/usr/bin/env python3
"""Benchmark of the Switch top-1 MoE layer on one MI355X (forward; backward alongside).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one whole-layer forward (route -> capacity/slots -> dispatch ->
expert FFN -> combine, plus the shared dense expert where the workload has
one) over one batch of synthetic tokens already resident in HBM.  The default
workload is the large layer (T=16384, d_model=5120, d_ff=8192, N=128 routed
experts, cf=1.25, plus one always-on shared FFN of width 8192, bf16); the
others run with --workload.  Prints one JSON line with:
  value          tokens/s of the whole layer (T * K / wall time of K steps);
                 value_median / ms_per_step_median from one event per step
                 boundary (median over the K steps)
  roofline       the routed expert-FFN GEMM (2 launches per step, bound by the
                 HBM bytes of the expert weights it touches): algorithmic bytes
                 per launch (touched weights + kept rows in and out; the hidden
                 matrix is listed apart) / average launch time, the latter from
                 HIP events that the library records around the routed FFN
                 inside every 8th timed step (switch_moe_forward_timed, on the
                 launch stream); `traffic` = HBM bytes per launch from rocprofv3
                 FETCH_SIZE / WRITE_SIZE counters, kept below together with a
                 fingerprint of the kernel sources they were taken on (null when
                 the sources have changed since)
  layer_roofline the sum over stages of max(bytes / 8 TB/s, FLOPs / 2.5166
                 PFLOP/s) against the median step, and the bound with every
                 stage overlapped
  stages         per-stage time from the same stage events over extra steps:
                 HBM GB/s and % of peak for route, dispatch, combine; TFLOP/s
                 and % of the bf16 MFMA peak for the expert GEMMs
  cpu_baseline   the fp64 CPU oracle timed on the host on the same batch (for
                 the large layer: a bounded, scaled sample, described in the
                 record)
  backward       the layer backward on the same batch (switch_moe_backward after
                 a training forward): tokens/s, the roofline of its dominant
                 weight pass (read w + write dw, timed with HIP events inside
                 the timed steps), per-stage times, and the fp64 backward
                 oracle timed on the host
  host, gpu_clocks  CPU model and cores; amd-smi clocks after the timed steps
Inputs are the seeded synthetic workload (x ~ N(0,1), Gaussian weights), no
dataset.  Only one GPU is supported.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA
METRIC = "MoE-layer tokens/sec at 1 MI355X; expert-GEMM MFMA % and route/dispatch HBM % of peak"
ROOT = os.path.dirname(os.path.abspath(__file__))

# Sources of the expert-FFN GEMM kernels.  HBM traffic measured with rocprofv3
# counters is reported only while these files are byte-identical to the ones
# the counters were taken on.
FFN_SOURCES = ("switch_top_routed_amd/csrc/expert_ffn.hip", "switch_top_routed_amd/csrc/expert_ffn_dma.hip",
               "switch_top_routed_amd/csrc/common.hpp", "switch_top_routed_amd/csrc/active_list.hpp")
# FETCH_SIZE / WRITE_SIZE (KiB per dispatch, as rocprofv3 prints them) of the two
# routed-FFN launches of one step, and the scale factors that a plain 1 GiB
# device copy gives those counters (bytes moved / bytes counted).  Source:
# profiles/*_hbm_traffic.md.
TRAFFIC = {
    "switch-base-uniform": {
        "sources_sha256": "007d29d65a7d5acacbdfd056b903734a3c5cd4b4a943ddde96d04425295288b1",
        "fetch_kib": [305813.3, 315572.1], "write_kib": [24108.6, 6027.0],
        "fetch_scale": 2.0, "write_scale": 1.0,
    },
    "switch-large-shared": {
        "sources_sha256": "007d29d65a7d5acacbdfd056b903734a3c5cd4b4a943ddde96d04425295288b1",
        "fetch_kib": [5365659.5, 5436823.2], "write_kib": [262159.4, 163840.0],
        "fetch_scale": 2.0, "write_scale": 1.0,
    },
}


# The same for the two fused weight passes of the backward (bwd_expert_fused: the
# pass over w2, then the pass over w1), fingerprinted by BWD_SOURCES.
BWD_SOURCES = ("switch_top_routed_amd/csrc/backward_fused.hip", "switch_top_routed_amd/csrc/common.hpp")
BWD_TRAFFIC = {
    "switch-base-uniform": {
        "sources_sha256": "5a1e0367bc876009e75bc64ae5e90adffbeb7467d853bb1863d91e8be95643ae",
        "fetch_kib": [322809.5, 314250.8], "write_kib": [614951.2, 601878.7],
        "fetch_scale": 2.0, "write_scale": 1.0,
    },
    "switch-large-shared": {
        "sources_sha256": "5a1e0367bc876009e75bc64ae5e90adffbeb7467d853bb1863d91e8be95643ae",
        "fetch_kib": [6231961.5, 5842643.3], "write_kib": [10775498.7, 10813449.6],
        "fetch_scale": 2.0, "write_scale": 1.0,
    },
}


def say(msg):
    """Progress line on stderr (stdout carries only the JSON record)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="switch-large-shared")
    ap.add_argument("--capacity-factor", type=float, default=None, help="override the workload's capacity factor")
    ap.add_argument("--priority", choices=("token", "gate"), default=None, help="override the overflow priority")
    ap.add_argument("--no-gate-scale", action="store_true", help="combine without the gate multiplier")
    ap.add_argument("--top-k", type=int, default=1, help="token choice with K experts per token")
    ap.add_argument("--routing", choices=("token", "expert"), default="token", help="token choice or expert choice")
    ap.add_argument("--renorm", action="store_true", help="top-K: divide each token's gates by their sum")
    ap.add_argument("--expand", type=int, default=1, metavar="M",
                    help="Expanded Drop: re-route overflow tokens over their M highest-logit experts (M >= 2)")
    ap.add_argument("--weights", choices=("native", "mxfp4"), default="native",
                    help="expert weights in the layer dtype, or MXFP4 (quantized on the device before timing)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the layer backward measurement")
    ap.add_argument("--grad-accumulate", action="store_true",
                    help="backward with SWITCH_ACCUM_EXPERT_GRADS: the routed experts' weight gradients accumulate "
                         "into the gradient buffers and idle experts are not touched")
    ap.add_argument("--backward-steps", type=int, default=None,
                    help="timed backward steps (default: min(steps, 50); 5 with a shared expert)")
    ap.add_argument("--stage-steps", type=int, default=20, help="extra steps with every stage boundary timed")
    ap.add_argument("--ffn-event-every", type=int, default=8,
                    help="timed steps between the ones that record HIP events around the routed FFN")
    ap.add_argument("--flush-mall", action="store_true",
                    help="write a 512 MB scratch buffer between timed steps (outside each step's events), so no "
                         "step reuses what the previous one left in the 256 MB memory-side cache; value then comes "
                         "from the per-step events")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat oracle layer passes until this much CPU time has elapsed (at most 30 passes)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a device-to-device copy of BYTES bytes (5 times): the reference kernel whose "
                         "FETCH_SIZE / WRITE_SIZE counters scale the measured HBM traffic")
    ap.add_argument("--sources-sha", action="store_true",
                    help="print the fingerprints of the FFN and backward kernel sources")
    return ap.parse_args()


def sources_sha256(files=None):
    h = hashlib.sha256()
    for rel in files or FFN_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def main():
    args = parse()
    if args.sources_sha:
        print(sources_sha256(), sources_sha256(BWD_SOURCES))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this layer is built and measured on one GPU; --gpus must be 1",
                          "requested_gpus": args.gpus}), flush=True)
        sys.exit(2)

    helper = None if (args.calibrate_copy or args.sources_sha) else clock_helper()  # before the GPU is touched
    import numpy as np
    import torch

    if args.calibrate_copy:
        src = torch.ones(args.calibrate_copy, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": args.calibrate_copy}), flush=True)
        return

    import switch_top_routed_amd as sw
    import workloads

    wl = workloads.WORKLOADS[args.workload]
    over = {}
    if args.capacity_factor is not None:
        over["capacity_factor"] = args.capacity_factor
    if args.priority is not None:
        over["priority"] = args.priority
    if args.no_gate_scale:
        over["gate_scale"] = False
    if over:
        wl = wl.with_(**over)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    esz = 2 if wl.dtype == "bf16" else 4
    weight_bytes = 2 * wl.N * wl.d_model * wl.d_ff * esz
    on_device = weight_bytes > (4 << 30)  # draw very large weight sets on the GPU
    say(f"inputs for {wl.name}")
    inp = workloads.make_inputs(wl, weights=not on_device)

    def dev(a):
        if a is None:
            return None
        if wl.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    x, wg = dev(inp.x), dev(inp.w_gate)
    if on_device:
        W = workloads.make_device_weights(wl)
        w1, w2, ws1, ws2 = W["w1"], W["w2"], W.get("ws1"), W.get("ws2")
    else:
        w1, w2, ws1, ws2 = dev(inp.w1), dev(inp.w2), dev(inp.ws1), dev(inp.ws2)
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).cuda()
    variant = args.top_k > 1 or args.routing != "token"
    if variant:
        over["top_k"] = args.top_k
        over["routing"] = args.routing
    xd = args.expand > 1
    if xd:
        over["expand"] = args.expand
    mxw = args.weights == "mxfp4"
    w1s = w2s = None
    if mxw:
        over["weights"] = "mxfp4"
        w1, w1s = sw.switch_quantize_mxfp4(w1)
        w2, w2s = sw.switch_quantize_mxfp4(w2)
        torch.cuda.synchronize()
    layer = sw.SwitchMoE(wl.T, wl.d_model, wl.d_ff, wl.N, dtype=dt, capacity_factor=wl.capacity_factor,
                         priority=wl.priority, gate_scale=wl.gate_scale, residual_all=wl.residual_all,
                         d_ff_shared=wl.d_ff_shared, top_k=args.top_k, routing=args.routing, renorm=args.renorm,
                         weight_format=args.weights, expand=args.expand)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        layer(x, wg, w1, w2, bias=bias, ws1=ws1, ws2=ws2, stream=stream, stage_events=ev, w1_scale=w1s,
              w2_scale=w2s)

    say("warmup")
    for _ in range(args.warmup):
        step()
    say(f"{args.steps} timed steps")
    # every ffn_event_every-th timed step records the two events around the routed FFN (each
    # event record costs ~2.5 us of GPU time, so they are not put into every step); the other
    # timed steps run the plain forward.  One torch event per step boundary gives the per-step
    # times whose median is reported beside the wall-clock mean.
    every = max(1, args.ffn_event_every)
    ffn_ev = {i: sw.StageEvents(which=(3, 4)) for i in range(0, args.steps, every)}
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)] if args.flush_mall else None
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") if args.flush_mall else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if flush is not None:
            flush.fill_(i & 0xFF)
        bounds[i].record(stream)
        step(ffn_ev.get(i))
        if ends is not None:
            ends[i].record(stream)
    bounds[args.steps].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    clocks = gpu_clocks(helper)
    if ends is not None:
        step_ms = [bounds[i].elapsed_time(ends[i]) for i in range(args.steps)]
    else:
        step_ms = [bounds[i].elapsed_time(bounds[i + 1]) for i in range(args.steps)]
    ms_median = float(np.median(step_ms))
    ms_per_step = elapsed / args.steps * 1e3
    value = wl.T * args.steps / elapsed if flush is None else wl.T / (ms_median * 1e-3)
    ffn_stage_ms = [e.ms(3, 4) for e in ffn_ev.values()]

    # every stage boundary, over extra (untimed) steps
    full_ev = [sw.StageEvents() for _ in range(args.stage_steps)]
    for e in full_ev:
        step(e)
    torch.cuda.synchronize()
    names = ["route", "assign", "dispatch", "expert_ffn", "shared_ffn", "combine"]
    st_s = {n: float(np.median([e.ms(i, i + 1) for e in full_ev])) * 1e-3 for i, n in enumerate(names)}

    out = layer.out
    kept = int(out["kept_count"].sum().item())
    n_active = int((out["kept_count"] > 0).sum().item())
    T, d, F, N, C = wl.T, wl.d_model, wl.d_ff, wl.N, layer.C
    dropped = T - kept
    Fs = wl.d_ff_shared
    # the library's forward folds the dispatch into GEMM 1 when x fits 32-bit offsets (same rule as its workspace layout)
    gathered = T * d * esz < 2 ** 31
    wbytes_per = (0.5 + 1.0 / 32) if mxw else esz  # bytes per weight: MXFP4 codes + E8M0 scales
    # algorithmic work of each stage of the layer (HBM bytes, FLOPs)
    work = {
        # x, W_g, bias, ids + gates out; slots, token_of_slot
        "route": (T * d * esz + N * d * esz + 4 * N + 8 * T + 12 * T + 4 * N * C, 2.0 * T * d * N),
        "dispatch": (2 * kept * d * esz + 4 * kept, 0.0),
        # touched weights once + the kept rows in and out (H is not algorithmic)
        "expert_ffn": (2 * n_active * d * F * wbytes_per + 2 * kept * d * esz, 4.0 * kept * d * F),
        # one row read per token (expert output or x), one written, plus the shared row; ids, slots, gates
        "combine": (2 * T * d * esz + (T * d * esz if Fs else 0) + 12 * T, float(kept * d)),
    }
    if variant:  # every kept pick's expert row, every x row, every y row
        work["combine"] = ((kept + 2 * T) * d * esz + (T * d * esz if Fs else 0), float(kept * d))
    if Fs:
        work["shared_ffn"] = (2 * d * Fs * esz + 2 * T * d * esz, 4.0 * T * d * Fs)
    ffn_launch_bytes = work["expert_ffn"][0] / 2  # per GEMM launch (each streams one weight matrix)
    h_launch_bytes = kept * F * esz  # hidden matrix: written by GEMM 1, read by GEMM 2 (reported, not algorithmic)
    ffn_flops = work["expert_ffn"][1]

    # the library's rule for the combine done by the shared expert's second GEMM (top-1 token choice,
    # bf16, the shared FFN on the LDS-tiled GEMM)
    fused_combine = bool(Fs) and not variant and wl.dtype == "bf16" and T > 64 and d % 256 == 0 and Fs % 256 == 0

    def gbs(b, t):
        return b / t / 1e9

    def bound_s(b, f):
        return max(b / (HBM_PEAK_GBS * 1e9), f / (MFMA_BF16_PEAK_TFLOPS * 1e12))

    stages = {
        "route": {"us": st_s["route"] * 1e6, "GB_s": gbs(work["route"][0], st_s["route"]),
                  "hbm_frac": gbs(work["route"][0], st_s["route"]) / HBM_PEAK_GBS},
        "assign": {"us": st_s["assign"] * 1e6},
        "dispatch": ({"us": st_s["dispatch"] * 1e6, "folded_into_gemm1": True,
                      "note": "GEMM 1 gathers the x rows; the span is the event pair alone"}
                     if gathered else
                     {"us": st_s["dispatch"] * 1e6, "GB_s": gbs(work["dispatch"][0], st_s["dispatch"]),
                      "hbm_frac": gbs(work["dispatch"][0], st_s["dispatch"]) / HBM_PEAK_GBS}),
        "expert_ffn": {"us": st_s["expert_ffn"] * 1e6, "launches": 2,
                       "GB_s": gbs(work["expert_ffn"][0], st_s["expert_ffn"]),
                       "hbm_frac": gbs(work["expert_ffn"][0], st_s["expert_ffn"]) / HBM_PEAK_GBS,
                       "TFLOP_s": ffn_flops / st_s["expert_ffn"] / 1e12,
                       "mfma_frac": ffn_flops / st_s["expert_ffn"] / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                       "h_bytes_per_launch": h_launch_bytes},
        "combine": ({"us": st_s["combine"] * 1e6, "folded_into_shared_gemm2": True,
                     "note": "the shared expert's second GEMM writes y (the combine) instead of its output; the span "
                             "is the event pair alone"}
                    if fused_combine else
                    {"us": st_s["combine"] * 1e6, "GB_s": gbs(work["combine"][0], st_s["combine"]),
                     "hbm_frac": gbs(work["combine"][0], st_s["combine"]) / HBM_PEAK_GBS}),
        "n_active": n_active, "kept": kept, "dropped": dropped, "stage_steps": args.stage_steps,
        "timing": "median over the stage_steps extra steps of the HIP events at the stage boundaries",
    }
    if Fs:
        sh_flops = work["shared_ffn"][1]
        stages["shared_ffn"] = {"us": st_s["shared_ffn"] * 1e6, "launches": 2,
                                "TFLOP_s": sh_flops / st_s["shared_ffn"] / 1e12,
                                "mfma_frac": sh_flops / st_s["shared_ffn"] / 1e12 / MFMA_BF16_PEAK_TFLOPS}
        if fused_combine:
            stages["shared_ffn"]["includes_combine"] = True

    # layer roofline: the sum of the stage bounds, each max(bytes / HBM peak, FLOPs / MFMA peak),
    # against the median step; and the bound with every stage overlapped (total bytes vs total FLOPs)
    bsum = sum(bound_s(b, f) for b, f in work.values())
    tot_b = sum(b for b, _ in work.values())
    tot_f = sum(f for _, f in work.values())
    boverlap = bound_s(tot_b, tot_f)
    layer_roofline = {
        "bound_us": bsum * 1e6, "step_us_median": ms_median * 1e3, "frac": bsum / (ms_median * 1e-3),
        "overlap_bound_us": boverlap * 1e6, "frac_overlap": boverlap / (ms_median * 1e-3),
        "peaks": {"hbm_GB_s": HBM_PEAK_GBS, "mfma_bf16_TFLOP_s": MFMA_BF16_PEAK_TFLOPS},
        "stages": {k: {"bytes": b, "flops": f, "bound_us": bound_s(b, f) * 1e6,
                       "bound_by": "hbm" if b / (HBM_PEAK_GBS * 1e9) >= f / (MFMA_BF16_PEAK_TFLOPS * 1e12) else "mfma"}
                   for k, (b, f) in work.items()},
        "note": "dispatch is counted as its own stage although GEMM 1 gathers the rows itself" if gathered else "",
    }

    launch_s = float(np.mean(ffn_stage_ms)) * 1e-3 / 2
    achieved = gbs(ffn_launch_bytes, launch_s)
    if wl.dtype != "bf16":
        kernel = "ffn_gemm_f32"
    elif mxw:
        kernel = "ffn_mx_stream"
    else:
        kernel = "ffn_tile_dma" if C > 64 and d % 256 == 0 and F % 256 == 0 else "ffn_gemm_bf16"
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None if over else traffic_bytes(wl.name),
                "kernel": f"{kernel} (routed expert FFN GEMM, 2 launches per step)",
                "bytes_per_launch": ffn_launch_bytes, "h_bytes_per_launch": h_launch_bytes,
                "bytes_rule": "touched experts' weight matrix + kept rows in + kept rows out, per launch; "
                              "the hidden matrix H (written by GEMM 1, read by GEMM 2) is listed apart",
                "launch_us": launch_s * 1e6,
                "launch_timing": f"HIP events around the routed FFN in {len(ffn_stage_ms)} of the {args.steps} timed steps"}

    cpu = None
    if not args.no_cpu_baseline:
        say("cpu baseline")
        if on_device:
            cpu = cpu_baseline_sampled(inp, {"w1": w1, "w2": w2, "ws1": ws1, "ws2": ws2}, layer.C,
                                       args.cpu_seconds)
        else:
            cpu = cpu_baseline(inp, args.cpu_seconds, args.top_k, args.routing, args.renorm, args.weights,
                               args.expand)

    backward = None
    if not args.no_backward and not variant and not mxw and not xd:  # the backward: top-1, native weights
        say("backward")
        backward = measure_backward(args, wl, inp, layer.C, x, wg, w1, w2, bias, ws1, ws2, stream, on_device)

    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "ms_per_step_median": ms_median,
        "value_median": wl.T / (ms_median * 1e-3),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic (seeded Gaussian tokens and weights)",
        "config": {"workload": wl.name, "T": T, "d_model": d, "d_ff": F, "N": N,
                   "capacity_factor": wl.capacity_factor, "C": C, "priority": wl.priority,
                   "gate_scale": wl.gate_scale, "d_ff_shared": wl.d_ff_shared, "parallelism": "single GPU",
                   "routing": ("expert choice" if args.routing == "expert" else
                               f"top-1 + Expanded Drop over {args.expand} candidates" if xd else
                               f"top-{max(1, args.top_k)}"),
                   "expert_weights": "MXFP4 (E2M1 + E8M0 per 32)" if mxw else wl.dtype,
                   "mall_flush": bool(args.flush_mall)},
        "roofline": roofline, "layer_roofline": layer_roofline, "stages": stages, "cpu_baseline": cpu,
        "backward": backward, "host": host_info(), "gpu_clocks": clocks,
    }
    print(json.dumps(line), flush=True)



def host_info():
    """CPU model and the cores this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count()
    return {"cpu_model": model, "affinity_cores": cores}


_CLOCK_HELPER = r"""
import json, subprocess, sys
sys.stdin.readline()  # asked for the clocks once the timed steps are done
out = None
for cmd in (["amd-smi", "metric", "-g", "0", "--clock", "--json"], ["amd-smi", "metric", "--clock", "--json"]):
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=20)
    except (OSError, subprocess.TimeoutExpired):
        continue
    if r.returncode == 0 and r.stdout.strip():
        out = r.stdout
        break
print(json.dumps(out))
"""


def clock_helper():
    """A child process that runs amd-smi when asked.  It is started before this
    process touches the GPU, so the tool it starts is never launched from a
    process that holds a GPU context.  None under a profiler (whose preloaded
    library initialises the GPU in every child) or when it cannot start."""
    import subprocess
    if any(k.startswith("ROCPROF") for k in os.environ) or "rocprof" in os.environ.get("LD_PRELOAD", ""):
        return None
    try:
        return subprocess.Popen([sys.executable, "-c", _CLOCK_HELPER], stdin=subprocess.PIPE, stdout=subprocess.PIPE,
                                stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return None


def gpu_clocks(helper):
    """Current GPU clocks as amd-smi reports them right after the timed steps
    (best effort: None when the helper is missing or prints nothing usable)."""
    if helper is None:
        return None
    try:
        raw, _ = helper.communicate("go\n", timeout=60)
        raw = json.loads(raw.strip() or "null")
    except Exception:  # noqa: BLE001 -- the clocks are informative only
        helper.kill()
        return None
    if not raw:
        return None
    try:
        data = json.loads(raw)
    except ValueError:
        return {"raw": raw[:400]}
    if isinstance(data, dict) and isinstance(data.get("gpu_data"), list):
        data = data["gpu_data"]
    if isinstance(data, list) and data:
        data = data[0]
    clk = data.get("clock", data) if isinstance(data, dict) else {}

    def mhz(v):
        return v.get("value") if isinstance(v, dict) else v
    picked = {}
    if isinstance(clk, dict):
        for k, v in clk.items():
            if isinstance(v, dict) and k.lower().startswith(("gfx_", "mem_", "fclk_", "socclk_")):
                picked[k] = mhz(v.get("clk"))
    if picked:
        gfx = [x for k, x in picked.items() if k.startswith("gfx_") and isinstance(x, (int, float))]
        return {"MHz": picked, "gfx_mean_MHz": sum(gfx) / len(gfx) if gfx else None,
                "note": "amd-smi right after the timed steps (the GPU may already be idling); the clock each kernel "
                        "ran at is in the MFMA counter profiles (GRBM_GUI_ACTIVE / time)"}
    return {"raw": json.dumps(clk)[:400]}


def measure_backward(args, wl, inp, C, x, wg, w1, w2, bias, ws1, ws2, stream, on_device):
    """The layer backward (switch_moe_backward) after one training forward on the
    same batch, with a seeded upstream gradient dy ~ N(0, 1) and dl_aux = 1e-2.
    One step = one backward.  The two weight passes (the fused MFMA kernels over
    w2 and w1) are timed with HIP events inside every timed step; the other
    stages over extra steps with every boundary recorded."""
    import numpy as np
    import torch

    import switch_top_routed_amd as sw
    import workloads

    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    esz = 2 if wl.dtype == "bf16" else 4
    T, d, F, N = wl.T, wl.d_model, wl.d_ff, wl.N
    tl = sw.SwitchMoE(T, d, F, N, dtype=dt, capacity_factor=wl.capacity_factor, priority=wl.priority,
                      gate_scale=wl.gate_scale, residual_all=wl.residual_all, d_ff_shared=wl.d_ff_shared,
                      train=True, accumulate_expert_grads=args.grad_accumulate)
    tl.forward_train(x, wg, w1, w2, bias=bias, ws1=ws1, ws2=ws2, stream=stream)
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed + 17)
    dy = torch.randn((T, d), generator=g, device="cuda").to(dt)
    dla = torch.full((1,), workloads.DL_AUX, dtype=torch.float32, device="cuda")

    def bstep(ev=None):
        tl.backward(x, wg, w1, w2, dy, dla, bias=bias, ws1=ws1, ws2=ws2, stream=stream, stage_events=ev)

    steps = args.backward_steps or (5 if wl.d_ff_shared else min(args.steps, 50))
    for _ in range(3):
        bstep()
    pass_ev = [sw.StageEvents(which=(1, 2, 3), n=6) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        bstep(pass_ev[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    w2_s = float(np.mean([e.ms(1, 2) for e in pass_ev])) * 1e-3
    w1_s = float(np.mean([e.ms(2, 3) for e in pass_ev])) * 1e-3
    full = [sw.StageEvents(n=6) for _ in range(min(args.stage_steps, steps))]
    for e in full:
        bstep(e)
    torch.cuda.synchronize()
    names = ["zero_idle", "w2_pass", "w1_pass", "shared", "router_dx"]
    st_us = {n: float(np.mean([e.ms(i, i + 1) for e in full])) * 1e3 for i, n in enumerate(names)}

    kc = tl.out["kept_count"]
    kept = int(kc.sum().item())
    n_active = int((kc > 0).sum().item())
    wbytes = n_active * d * F * esz  # one weight matrix of the active experts
    # algorithmic bytes: weight read + gradient write, plus the kept token rows each pass reads
    # and writes (w2 pass: dY rows, H, dZ, dg partials; w1 pass: dZ, x rows, dX_e in fp32)
    w2_bytes = 2 * wbytes + kept * (d + 2 * F) * esz + kept * (F // 64) * 4
    w1_bytes = 2 * wbytes + kept * (F + d) * esz + kept * d * 4
    flops = 8.0 * kept * d * F  # four GEMMs of 2 kept d F each
    dom, dom_s, dom_b = ("w2_pass", w2_s, w2_bytes) if w2_s >= w1_s else ("w1_pass", w1_s, w1_bytes)
    achieved = dom_b / dom_s / 1e9
    fused = wl.dtype == "bf16" and C <= 160 and T * d * esz < 2 ** 31
    kname = ("bwd_expert_fused" if fused else "gemm_generic") + f" ({'w2' if dom == 'w2_pass' else 'w1'} pass)"
    out = {
        "value": T * steps / elapsed, "unit": "tokens/s", "ms_per_step": elapsed / steps * 1e3, "steps": steps,
        "step": "one layer backward (switch_moe_backward) after a training forward on the same batch"
                + (", expert weight gradients accumulated (idle experts untouched)" if args.grad_accumulate else ""),
        "dl_aux": workloads.DL_AUX,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": bwd_traffic_bytes(wl.name, dom) if wl == workloads.WORKLOADS.get(wl.name) else None,
                     "kernel": kname,
                     "bytes_per_launch": dom_b, "launch_us": dom_s * 1e6,
                     "launch_timing": f"HIP events around each weight pass in the {steps} timed steps"},
        "passes": {"w2_pass_us": w2_s * 1e6, "w1_pass_us": w1_s * 1e6,
                   "w2_pass_GB_s": w2_bytes / w2_s / 1e9, "w1_pass_GB_s": w1_bytes / w1_s / 1e9,
                   "expert_TFLOP_s": flops / (w2_s + w1_s) / 1e12},
        "stages_us": st_us,
    }
    if wl.d_ff_shared:
        out["stages_us"]["shared_TFLOP_s"] = 8.0 * T * d * wl.d_ff_shared / (st_us["shared"] * 1e-6) / 1e12
    if not args.no_cpu_baseline and not on_device:
        out["cpu_baseline"] = cpu_backward_baseline(inp, dy)
    return out


def cpu_backward_baseline(inp, dy_dev):
    """The fp64 backward oracle, as it stands: one training forward plus one
    backward pass over the same batch with the same upstream gradient."""
    import numpy as np
    import torch

    import oracle
    import workloads
    from oracle import backward as ob
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    wl = inp.wl
    dt = wl.dtype
    dy = dy_dev.float().cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    ref = oracle.moe_forward_stored(inp)
    x, wgt = oracle.widen(inp.x, dt), oracle.widen(inp.w_gate, dt)
    ws1 = oracle.widen(inp.ws1, dt) if inp.ws1 is not None else None
    ws2 = oracle.widen(inp.ws2, dt) if inp.ws2 is not None else None
    ob.moe_backward(ref, x, wgt, lambda e: oracle.widen(inp.w1[e], dt), lambda e: oracle.widen(inp.w2[e], dt),
                    wl.N, dy, workloads.DL_AUX, gate_scale=wl.gate_scale, residual_all=wl.residual_all, ws1=ws1,
                    ws2=ws2)
    el = time.perf_counter() - t0
    return {"value": wl.T / el, "unit": "tokens/s", "cores": cores, "kind": "oracle", "seconds": el,
            "sample": f"one fp64 training forward + backward over the {wl.name} batch (T={wl.T} tokens)"}


def bwd_traffic_bytes(workload, which):
    """HBM bytes of one backward weight pass ("w2_pass" / "w1_pass") from the
    stored counter readings, or None (no readings, or changed sources)."""
    t = BWD_TRAFFIC.get(workload)
    if t is None or t["sources_sha256"] != sources_sha256(BWD_SOURCES):
        return None
    i = 0 if which == "w2_pass" else 1
    return t["fetch_kib"][i] * 1024 * t["fetch_scale"] + t["write_kib"][i] * 1024 * t["write_scale"]


def traffic_bytes(workload):
    """HBM bytes per routed-FFN launch from the stored counter readings, or None
    if there are none for this workload or the kernel sources have changed."""
    t = TRAFFIC.get(workload)
    if t is None or t["sources_sha256"] != sources_sha256():
        return None
    per = [f * 1024 * t["fetch_scale"] + w * 1024 * t["write_scale"] for f, w in zip(t["fetch_kib"], t["write_kib"])]
    return sum(per) / len(per)


def cpu_baseline(inp, seconds, top_k=1, routing="token", renorm=False, weights="native", expand=1):
    """The fp64 oracle, as it stands, on the same workload (and routing): whole
    layer passes over the batch, repeated until `seconds` have elapsed (at most
    30 passes)."""
    import oracle
    from oracle import expanded as ox
    from oracle import mxfp4 as mx
    from oracle import routing as orr

    def one_pass():
        if top_k <= 1 and routing == "token" and weights == "native" and expand <= 1:
            return oracle.moe_forward_stored(inp)
        wl, dt = inp.wl, inp.wl.dtype
        x, wg = oracle.widen(inp.x, dt), oracle.widen(inp.w_gate, dt)
        w1_of, w2_of = (lambda e: oracle.widen(inp.w1[e], dt)), (lambda e: oracle.widen(inp.w2[e], dt))
        if weights == "mxfp4":  # the oracle's own MXFP4 encoding of each expert, decoded exactly
            w1_of = lambda e: mx.dequantize(*mx.quantize(oracle.widen(inp.w1[e:e + 1], dt)))[0]  # noqa: E731
            w2_of = lambda e: mx.dequantize(*mx.quantize(oracle.widen(inp.w2[e:e + 1], dt)))[0]  # noqa: E731
            if top_k <= 1 and routing == "token" and expand <= 1:
                return oracle.moe_forward(x, wg, inp.bias, w1_of, w2_of, wl.N, wl.capacity_factor,
                                          priority=wl.priority, gate_scale=wl.gate_scale,
                                          residual_all=wl.residual_all)
        ws1 = oracle.widen(inp.ws1, dt) if inp.ws1 is not None else None
        ws2 = oracle.widen(inp.ws2, dt) if inp.ws2 is not None else None
        if expand > 1:
            return ox.moe_forward_expanded(x, wg, inp.bias, w1_of, w2_of, wl.N, M=expand,
                                           capacity_factor=wl.capacity_factor, priority=wl.priority,
                                           gate_scale=wl.gate_scale, residual_all=wl.residual_all, ws1=ws1, ws2=ws2)
        if routing == "expert":
            return orr.moe_forward_expert_choice(x, wg, inp.bias, w1_of, w2_of, wl.N, wl.capacity_factor,
                                                 gate_scale=wl.gate_scale, residual_all=wl.residual_all,
                                                 ws1=ws1, ws2=ws2)
        C = min(wl.T, orr.capacity_topk(wl.T, wl.N, top_k, wl.capacity_factor))
        return orr.moe_forward_topk(x, wg, inp.bias, w1_of, w2_of, wl.N, K=top_k, C=C, priority=wl.priority,
                                    gate_scale=wl.gate_scale, residual_all=wl.residual_all, renorm=renorm,
                                    ws1=ws1, ws2=ws2)
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    def timed(budget):
        passes = 0
        t0 = time.perf_counter()
        while True:
            one_pass()
            passes += 1
            el = time.perf_counter() - t0
            if el >= budget or passes >= 30:
                return passes, el

    passes, el = timed(seconds)
    one = None
    if inp.wl.T * inp.wl.d_model <= 4096 * 768:  # small layers: also on one thread (BLAS limited to 1)
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                p1, e1 = timed(seconds / 2)
            one = {"value": inp.wl.T * p1 / e1, "unit": "tokens/s", "cores": 1, "seconds": e1, "passes": p1}
        except Exception:  # pragma: no cover -- informative only
            one = None
    return {"value": inp.wl.T * passes / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "one_thread": one,
            "seconds": el, "sample": f"{passes} full fp64 layer passes over the {inp.wl.name} batch "
                                     f"(T={inp.wl.T} tokens each, "
                                     f"{'expert choice' if routing == 'expert' else f'top-{max(1, top_k)}'}"
                                     f"{f', Expanded Drop over {expand} candidates' if expand > 1 else ''}"
                                     f"{', MXFP4 experts' if weights == 'mxfp4' else ''})"}


def cpu_baseline_sampled(inp, W, C, seconds):
    """The fp64 oracle, as it stands, on a bounded sample of a layer whose
    weights exist only on the device (the 22 GB large layer).  The router,
    load statistics, capacity, slots, dispatch and combine run over the whole
    batch; the expert FFN runs for active experts in a seeded order until
    about `seconds` / 2 of it have elapsed, and is scaled by n_active / experts
    done; the shared FFN runs on 512 seeded tokens and is scaled by T / 512
    (its weights are widened once, counted in full).  Each sampled expert's
    weights are copied to the host before its timed step (input marshalling,
    not oracle work).  value = T / (sum of the full and scaled step times)."""
    import numpy as np
    import torch

    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    wl, dt = inp.wl, inp.wl.dtype

    def host_u16(t):
        return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)

    tm = {}
    t0 = time.perf_counter()
    x = oracle.widen(inp.x, dt)
    _, p, e, g = oracle.route(x, oracle.widen(inp.w_gate, dt), inp.bias)
    oracle.aux_loss(e, p, wl.N)
    a = oracle.assign_slots(e, g, wl.N, C, wl.priority)
    tm["route_assign"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    buf = oracle.dispatch(x, a["token_of_slot"], a["kept_count"])
    tm["dispatch"] = time.perf_counter() - t0
    active = np.asarray(a["active"])
    order = np.random.default_rng(wl.seed + 5).permutation(active)
    out = np.full(buf.shape, np.nan)
    done, t_ffn = 0, 0.0
    for ex in order:
        w1h, w2h = host_u16(W["w1"][int(ex)]), host_u16(W["w2"][int(ex)])
        k = int(a["kept_count"][ex])
        t0 = time.perf_counter()
        out[ex, :k] = oracle.ffn(buf[ex, :k], oracle.widen(w1h, dt), oracle.widen(w2h, dt))
        t_ffn += time.perf_counter() - t0
        done += 1
        if t_ffn >= seconds / 2:
            break
    tm["expert_ffn_scaled"] = t_ffn * active.size / max(done, 1)
    shared = None
    ns = 0
    if W.get("ws1") is not None:
        ns = min(512, wl.T)
        rows = np.sort(np.random.default_rng(wl.seed + 6).choice(wl.T, size=ns, replace=False))
        s1h, s2h = host_u16(W["ws1"]), host_u16(W["ws2"])
        t0 = time.perf_counter()
        s1, s2 = oracle.widen(s1h, dt), oracle.widen(s2h, dt)
        t_w = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.ffn(x[rows], s1, s2)
        t_mm = time.perf_counter() - t0
        tm["shared_ffn_scaled"] = t_w + t_mm * wl.T / ns
        shared = np.zeros_like(x)
    t0 = time.perf_counter()
    oracle.combine(out, x, e, a["slot"], g, wl.gate_scale, wl.residual_all, shared)
    tm["combine"] = time.perf_counter() - t0
    total = sum(tm.values())
    return {"value": wl.T / total, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "seconds": total, "step_seconds": tm,
            "sample": f"fp64 oracle over the {wl.name} batch (T={wl.T}): router, statistics, slots, dispatch and "
                      f"combine in full; expert FFN on {done} of {active.size} active experts, scaled by "
                      f"{active.size}/{done}"
                      + (f"; shared FFN on {ns} of {wl.T} tokens, scaled by {wl.T}/{ns} (weights widened once, in full)"
                         if ns else "")}


if __name__ == "__main__":
    main()
