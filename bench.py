#!/usr/bin/env python3
"""Benchmark of the Switch top-1 MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one whole-layer forward (route -> capacity/slots -> dispatch ->
expert FFN -> combine) over one batch of synthetic tokens already resident in
HBM.  Prints one JSON line with:
  value          tokens/s of the whole layer (T * K / wall time of K steps)
  roofline       the expert-FFN GEMM kernel (2 launches per step, HBM-bound on
                 the expert weights it touches): algorithmic bytes per launch /
                 average launch time from HIP events on the launch stream
  stages         per-stage time, HBM GB/s and % of peak (route, assign,
                 dispatch, expert FFN, combine) and MFMA % for the expert FFN
  cpu_baseline   the fp64 CPU oracle timed on the host on the same workload
Inputs are the seeded synthetic workload (x ~ N(0,1), Gaussian weights), no
dataset.  Only one GPU is supported.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA
METRIC = "MoE-layer tokens/sec at 1 MI355X; expert-GEMM MFMA % and route/dispatch HBM % of peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="switch-base-uniform")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stage-iters", type=int, default=50)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a device-to-device copy of BYTES bytes (5 times): the reference kernel whose "
                         "FETCH_SIZE / WRITE_SIZE counters scale the measured HBM traffic")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this layer is built and measured on one GPU; --gpus must be 1",
                          "requested_gpus": args.gpus}), flush=True)
        sys.exit(2)

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
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    weight_bytes = 2 * wl.N * wl.d_model * wl.d_ff * (2 if wl.dtype == "bf16" else 4)
    on_device = weight_bytes > (4 << 30)  # draw very large weight sets on the GPU
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
    layer = sw.SwitchMoE(wl.T, wl.d_model, wl.d_ff, wl.N, dtype=dt, capacity_factor=wl.capacity_factor,
                         priority=wl.priority, gate_scale=wl.gate_scale, residual_all=wl.residual_all,
                         d_ff_shared=wl.d_ff_shared)
    stream = torch.cuda.current_stream()

    def step():
        layer(x, wg, w1, w2, bias=bias, ws1=ws1, ws2=ws2, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    value = wl.T * args.steps / elapsed

    # ---- per-stage timing through the per-stage entry points (HIP events on the launch stream)
    C = layer.C
    esz = 2 if wl.dtype == "bf16" else 4
    r = sw.switch_route(x, wg, bias, stream=stream)
    a = sw.switch_assign_capacity(r["expert_id"], r["gate"], wl.N, C, wl.priority, stream=stream)
    xin = sw.switch_dispatch(x, a["token_of_slot"], a["kept_count"], wl.N, C, stream=stream)
    xout = sw.switch_expert_ffn(xin, w1, w2, a["kept_count"], a["active"], a["n_active"], stream=stream)
    torch.cuda.synchronize()
    kept = int(a["kept_count"].sum().item())
    n_active = int(a["n_active"].item())
    flags = sw.GATE_SCALE if wl.gate_scale else 0

    def timed(fn, iters):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        fn()
        ev0.record(stream)
        for _ in range(iters):
            fn()
        ev1.record(stream)
        ev1.synchronize()
        return ev0.elapsed_time(ev1) / iters * 1e-3  # seconds per call

    it = args.stage_iters
    rws = torch.empty(max(1, sw.lib().switch_route_workspace_bytes(wl.T, wl.d_model, wl.N, 1 if esz == 2 else 0)),
                      dtype=torch.uint8, device="cuda")
    t_route = timed(lambda: sw.switch_route(x, wg, bias, ws=rws, stream=stream), it)
    t_assign = timed(lambda: sw.switch_assign_capacity(r["expert_id"], r["gate"], wl.N, C, wl.priority,
                                                       stream=stream), it)
    t_disp = timed(lambda: sw.switch_dispatch(x, a["token_of_slot"], a["kept_count"], wl.N, C, expert_in=xin,
                                              stream=stream), it)
    fws = torch.empty(sw.lib().switch_expert_ffn_workspace_bytes(wl.N, C, wl.d_model, wl.d_ff, 1 if esz == 2 else 0),
                      dtype=torch.uint8, device="cuda")
    t_ffn = timed(lambda: sw.switch_expert_ffn(xin, w1, w2, a["kept_count"], a["active"], a["n_active"],
                                               expert_out=xout, ws=fws, stream=stream), it)
    yb = torch.empty_like(x)
    t_comb = timed(lambda: sw.switch_combine(xout, x, r["expert_id"], a["slot"], r["gate"], flags, y=yb,
                                             stream=stream), it)

    T, d, F, N = wl.T, wl.d_model, wl.d_ff, wl.N
    dropped = T - kept
    route_bytes = T * d * esz + N * d * esz + T * 8 + N * 16
    disp_bytes = 2 * kept * d * esz + 4 * kept
    comb_bytes = (kept + T) * d * esz + dropped * 0 + T * d * esz + T * 12
    ffn_launch_bytes = n_active * d * F * esz + kept * (d + F) * esz  # one GEMM launch
    ffn_flops = 4.0 * kept * d * F

    def gbs(b, t):
        return b / t / 1e9

    stages = {
        "route": {"us": t_route * 1e6, "GB_s": gbs(route_bytes, t_route), "hbm_frac": gbs(route_bytes, t_route) / HBM_PEAK_GBS},
        "assign": {"us": t_assign * 1e6},
        "dispatch": {"us": t_disp * 1e6, "GB_s": gbs(disp_bytes, t_disp), "hbm_frac": gbs(disp_bytes, t_disp) / HBM_PEAK_GBS},
        "expert_ffn": {"us": t_ffn * 1e6, "launches": 2, "GB_s": gbs(2 * ffn_launch_bytes, t_ffn),
                       "hbm_frac": gbs(2 * ffn_launch_bytes, t_ffn) / HBM_PEAK_GBS,
                       "TFLOP_s": ffn_flops / t_ffn / 1e12,
                       "mfma_frac": ffn_flops / t_ffn / 1e12 / MFMA_BF16_PEAK_TFLOPS},
        "combine": {"us": t_comb * 1e6, "GB_s": gbs(comb_bytes, t_comb), "hbm_frac": gbs(comb_bytes, t_comb) / HBM_PEAK_GBS},
        "n_active": n_active, "kept": kept, "dropped": dropped,
    }
    launch_s = t_ffn / 2
    achieved = gbs(ffn_launch_bytes, launch_s)
    roofline = {"bound": "hbm", "kernel": "ffn_gemm_bf16 (expert FFN GEMM, 2 launches per step)",
                "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                "traffic": None, "bytes_per_launch": ffn_launch_bytes, "launch_us": launch_s * 1e6}

    cpu = None
    if not args.no_cpu_baseline and not on_device:
        cpu = cpu_baseline(inp)

    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic (seeded Gaussian tokens and weights)",
        "config": {"workload": wl.name, "T": T, "d_model": d, "d_ff": F, "N": N,
                   "capacity_factor": wl.capacity_factor, "C": C, "priority": wl.priority,
                   "gate_scale": wl.gate_scale, "d_ff_shared": wl.d_ff_shared, "parallelism": "single GPU"},
        "roofline": roofline, "stages": stages, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(inp):
    """The fp64 oracle, as it stands, on the same workload (one full layer pass)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    t0 = time.perf_counter()
    oracle.moe_forward_stored(inp)
    el = time.perf_counter() - t0
    return {"value": inp.wl.T / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "seconds": el, "sample": f"one full fp64 layer pass over the {inp.wl.name} batch (T={inp.wl.T})"}


if __name__ == "__main__":
    main()
