#!/usr/bin/env python3
"""Throughput of the per-token NVFP4 routed-MoE hot path on one MI355X.

One step = pmoe_moe_forward on BF16 activations (per-token quantization
overlapped with the routing, FC1 + activation, requantization, FC2,
fixed-order finalize) over one batch of
synthetic tokens already resident in HBM, with weights prepared beforehand
(preparation is timed separately and reported as `prepare`).

Default workload: the one-GPU share of an EP4 MoE layer -- E=96 local experts,
H=7168, I=3072, SwiGLU, top-6, T=1024 tokens, two hot experts (router logits
+2 on experts 0 and 48); inputs from the seeded generator in synth/.

Prints one JSON line. `roofline` is the dominant kernel (FC1 grouped GEMM):
algorithmic bytes per launch over its average duration, measured here with
HIP events around that step on the stream it runs on. `cpu_baseline` times
the CPU oracle on a bounded sample (all routes of the first --cpu-experts
experts). `device` reports this device's own ceilings: the bandwidth of a plain
1 GiB device-to-device copy, and the graphics clock and socket power sampled
while the step runs back to back.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed-MoE tokens/s + effective TFLOPS (% MFMA peak), H7168/I3072 top-6, 1 GPU"
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_F16_TFLOPS = 2500.0     # MI355X dense FP16/BF16 MFMA
NOMINAL_MHZ = 2400.0         # MI355X peak engine clock the MFMA peak is quoted at
NVFP4_BYTES = 9.0 / 16.0     # packed E2M1 + one E4M3 scale per 16 elements


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="ep4_t1024")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stage-reps", type=int, default=20)
    ap.add_argument("--cpu-experts", type=int, default=20,
                    help="the CPU oracle baseline runs all routes of this many experts")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes 5 times "
                         "(calibrates the HBM byte counters) and exit")
    return ap.parse_args()


def algorithmic_bytes(w, counts, T, R):
    """Bytes each step must move at least (weights of active experts once, activations once)."""
    active = int(np.count_nonzero(counts))
    fc1_w = active * w.N1 * w.H * NVFP4_BYTES + active * 4
    fc2_w = active * w.H * w.I * NVFP4_BYTES + active * 4
    xq = T * w.H * NVFP4_BYTES + 4 * T
    hq = R * w.I * NVFP4_BYTES + 4 * R
    z = R * w.H * 2
    return {
        "quantize": T * w.H * 2 + xq,
        "route": T * w.K * 4 * 3,
        "fc1": fc1_w + xq + hq,
        "requant": 2 * hq,
        "fc2": fc2_w + hq + z,
        "finalize": z + T * w.K * 8 + T * w.H * 2,
        "step": fc1_w + fc2_w + T * w.H * 2 + 2 * xq + 2 * hq + 2 * z + T * w.K * 8 + T * w.H * 2,
    }


def cpu_baseline(w, ids, wts, n_experts):
    """Oracle throughput on all routes of the first n_experts experts (expert 0 is hot)."""
    import synth
    from oracle import moe as om
    from oracle import quant as oq
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    experts = list(range(n_experts))
    W = om.LazyWeights(lambda e: synth.expert_weights(w, e), w.E, w.N1, w.H, w.I)
    for e in experts:
        W.expert(e)                                   # preparation is outside the timed region
    x = synth.activations(w)
    t0 = time.perf_counter()
    xq, xs, xg = oq.quantize_input_per_token(x)
    res = om.routed_moe(xq, xs, xg, ids, wts, W, w.act, experts=experts)
    dt = time.perf_counter() - t0
    rows = int(res.computed_rows.sum())
    return {"value": rows / w.K / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"all {rows} routes of experts {experts} (of T*K={w.T * w.K}) incl. per-token "
                      f"quantization of all {w.T} tokens; tokens/s = routes/K/s; {dt:.1f} s",
            "seconds": dt}


def stream_copy_gbs(torch, nbytes=1 << 30, reps=10):
    """Bytes read + written per second by a plain 1 GiB device-to-device copy: the
    achievable streaming bandwidth of this device, next to the 8 TB/s nominal peak."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2.0 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def clock_under_load(torch, fn, seconds=1.0):
    """Median graphics clock (MHz) and socket power (W) sampled from the GPU's metrics table
    while fn() runs back to back for about `seconds`; None where the metrics are unavailable."""
    import threading
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception as exc:  # no metrics interface: report the gap, do not guess
        return {"gfx_mhz": None, "socket_w": None, "samples": 0, "note": f"amdsmi unavailable: {exc}"}

    def num(v):
        if isinstance(v, (list, tuple)):
            v = [x for x in v if isinstance(x, (int, float)) and 0 < x < 65535]
            return sum(v) / len(v) if v else None
        return float(v) if isinstance(v, (int, float)) and 0 < v < 65535 else None

    clocks, watts, stop = [], [], threading.Event()

    def sample():
        while not stop.is_set():
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
                c = num(m.get("current_gfxclks")) or num(m.get("current_gfxclk")) or \
                    num(m.get("average_gfxclk_frequency"))
                pw = num(m.get("current_socket_power")) or num(m.get("average_socket_power"))
                if c:
                    clocks.append(c)
                if pw:
                    watts.append(pw)
            except Exception:
                pass
            stop.wait(0.01)

    for _ in range(20):
        fn()
    torch.cuda.synchronize()
    t = threading.Thread(target=sample, daemon=True)
    t0 = time.perf_counter()
    t.start()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
    stop.set()
    t.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass
    med = lambda v: float(np.median(v)) if v else None
    return {"gfx_mhz": med(clocks), "socket_w": med(watts), "samples": len(clocks),
            "note": "amdsmi GPU metrics, median over the samples taken while the step ran"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(expert parallelism is described in the design notes); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import precision_moe_amd as pm
    from precision_moe_amd import profiling
    import synth

    if args.copy_bytes:
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.copy_bytes} bytes 5 times")
        return

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] workload {w.name}: T={w.T} H={w.H} I={w.I} E={w.E} K={w.K} act={w.act}")

    # ---------------------------------------------------------------- weights
    w1, w2 = synth.all_weights(w, device=dev)
    w1 = w1.view(torch.bfloat16)
    w2 = w2.view(torch.bfloat16)
    P = pm.prepare_weights(w1, w2)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 3
    e0.record()
    for _ in range(reps):
        pm.prepare_weights(w1, w2, out=P)
    e1.record()
    torch.cuda.synchronize()
    prep_ms = e0.elapsed_time(e1) / reps
    elems = w.E * (w.N1 * w.H + w.H * w.I)
    prepare = {"ms": prep_ms, "GB/s": elems * (2 + NVFP4_BYTES) / (prep_ms * 1e-3) / 1e9,
               "note": "reads BF16 once (algorithmic; the kernel reads it twice) and writes NVFP4"}
    log(f"[bench] prepare_weights {prep_ms:.2f} ms")

    # ---------------------------------------------------------------- inputs
    x = synth.activations(w, device=dev).view(torch.bfloat16)
    ids_np, wts_np = synth.router(w)
    ids = torch.from_numpy(ids_np).to(dev)
    wts = torch.from_numpy(wts_np).to(dev)
    T = w.T
    xq = torch.empty((T, w.H // 2), dtype=torch.uint8, device=dev)
    xs = torch.empty((T, w.H // 16), dtype=torch.uint8, device=dev)
    xg = torch.empty((T,), dtype=torch.float32, device=dev)
    ws = torch.empty(pm.moe_workspace_bytes(T, w.K, w.E, w.H, w.I, P.act), dtype=torch.uint8, device=dev)
    out = torch.empty((T, w.H), dtype=torch.bfloat16, device=dev)

    def step():
        pm.moe_forward(x, ids, wts, P, workspace=ws, out=out)

    def step_separate_quantize():
        pm.quantize_input_per_token(x, out=(xq, xs, xg))
        pm.routed_moe(xq, xs, xg, ids, wts, P, workspace=ws, out=out)

    # ---------------------------------------------------------------- timed region
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for _ in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    log(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.1f} us/step (wall {wall / args.steps * 1e6:.1f} us/step)")

    # ---------------------------------------------------------------- FC1 alone
    # Inside a step the two expert halves run FC1 on two streams, overlapped
    # with the other half's work; the roofline figure times the whole FC1
    # kernel (one launch over all experts, the same code) with HIP events on
    # the stream it runs on, over as many launches as the timed region had.
    fc1_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    for a, b in fc1_evs:
        a.record()
        pm.routed_moe(xq, xs, xg, ids, wts, P, workspace=ws, out=out, steps=(pm.STEP_FC1, pm.STEP_FC1))
        b.record()
    torch.cuda.synchronize()
    fc1_ms_timed = float(np.mean([a.elapsed_time(b) for a, b in fc1_evs]))

    # ---------------------------------------------------------------- per-step events
    names = ["quantize", "route", "fc1", "requant", "fc2", "finalize"]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
    acc = np.zeros(len(names))
    for _ in range(args.stage_reps):
        evs[0].record()
        pm.quantize_input_per_token(x, out=(xq, xs, xg))
        evs[1].record()
        for s in range(5):
            pm.routed_moe(xq, xs, xg, ids, wts, P, workspace=ws, out=out, steps=(s, s))
            evs[s + 2].record()
        torch.cuda.synchronize()
        acc += [evs[i].elapsed_time(evs[i + 1]) for i in range(len(names))]
    stage_ms = acc / args.stage_reps

    views = pm.workspace_views(ws, T, w.K, w.E, w.H, w.I, P.act)

    # ---------------------------------------------------------------- other recipes
    # The per-tensor NVFP4 and W4A16 variants of the same layer, on the same
    # inputs: static scales calibrated as 2688 / amax of the FC1 input and of
    # the per-token run's intermediate (setup, outside the timed region).
    R_rows = int(views["counters"][0].item())
    a1 = (2688.0 / x.float().abs().max()).reshape(1).float()
    a2 = (2688.0 / views["h"][:R_rows].abs().max()).reshape(1).float()
    P_pt = pm.prepare_weights(w1, w2, input_scales=(a1, a2))
    del w1, w2
    torch.cuda.empty_cache()
    xq_pt = torch.empty_like(xq)
    xs_pt = torch.empty_like(xs)

    def step_per_tensor():
        pm.quantize_input_per_tensor(x, a1, out=(xq_pt, xs_pt))
        pm.routed_moe_per_tensor(xq_pt, xs_pt, ids, wts, P_pt, a2, workspace=ws, out=out)

    def step_w4a16():
        pm.routed_moe_w4a16(x, ids, wts, P, workspace=ws, out=out)

    def step_one_stream():
        pm.moe_forward(x, ids, wts, P, streams=1, workspace=ws, out=out)

    def step_fused():
        pm.moe_forward(x, ids, wts, P, finalize="fused", workspace=ws, out=out)

    logits = torch.from_numpy(synth.router_logits(w)).to(dev)
    r_ids = torch.empty_like(ids)
    r_w = torch.empty_like(wts)

    def step_router():
        pm.router_topk(logits, w.K, w.renormalize, out=(r_ids, r_w))

    recipes = {}
    flops_step = 2.0 * R_rows * (w.N1 * w.H + w.H * w.I)
    for name, fn in (("per_tensor", step_per_tensor), ("weight_only_w4a16", step_w4a16),
                     ("per_token_ordered_finalize", step),
                     ("per_token_separate_quantize", step_separate_quantize),
                     ("per_token_one_stream", step_one_stream),
                     ("per_token_fused_finalize", step_fused),
                     ("router_topk", step_router)):
        for _ in range(max(args.warmup // 2, 2)):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        recipes[name] = {"ms_per_step": ms, "tokens/s": T / (ms * 1e-3)}
        if name != "router_topk":
            recipes[name]["TFLOP/s"] = flops_step / (ms * 1e-3) / 1e12
        log(f"[bench] {name}: {ms * 1e3:.1f} us/step")
    # the fixed-order finalize's cost over the order-free one (same inputs, same process)
    recipes["determinism_cost"] = (recipes["per_token_ordered_finalize"]["ms_per_step"] /
                                   recipes["per_token_fused_finalize"]["ms_per_step"] - 1.0)
    del P_pt

    # ---------------------------------------------------------------- ceilings of this device
    copy_gbs = stream_copy_gbs(torch)
    clock = clock_under_load(torch, step)
    log(f"[bench] device copy {copy_gbs:.0f} GB/s; clock under load {clock['gfx_mhz']} MHz, "
        f"{clock['socket_w']} W ({clock['samples']} samples)")

    counts = np.diff(views["expert_offsets"].cpu().numpy())
    R = int(counts.sum())
    ab = algorithmic_bytes(w, counts, T, R)
    kernels = {n: {"us": float(stage_ms[i] * 1e3),
                   "GB/s": float(ab[n] / (stage_ms[i] * 1e-3) / 1e9)} for i, n in enumerate(names)}
    for k in kernels.values():
        k["hbm_frac"] = k["GB/s"] / PEAK_HBM_GBS
    flops = 2.0 * R * (w.N1 * w.H + w.H * w.I)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    fc1_flops = 2.0 * R * w.N1 * w.H
    kernels["fc1"]["TFLOP/s"] = float(fc1_flops / (stage_ms[2] * 1e-3) / 1e12)
    kernels["fc2"]["TFLOP/s"] = float(2.0 * R * w.H * w.I / (stage_ms[4] * 1e-3) / 1e12)
    for n in ("fc1", "fc2"):
        kernels[n]["mfma_frac"] = kernels[n]["TFLOP/s"] / PEAK_F16_TFLOPS
    fc1_gbs = ab["fc1"] / (fc1_ms_timed * 1e-3) / 1e9
    traffic = profiling.read_traffic(os.path.join(ROOT, "profiles", f"fc1_{w.name}_hbm_traffic.txt"), w.name)

    result = {
        "metric": METRIC,
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "T": T, "H": w.H, "I": w.I, "E": w.E, "top_k": w.K,
                   "act": w.act, "routed_rows": R, "parallelism": "none (1 GPU)"},
        "tflops": tflops,
        "mfma_frac": tflops / PEAK_F16_TFLOPS,
        "hbm_frac_step": ab["step"] / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "roofline": {"bound": "hbm", "kernel": "fc1 grouped GEMM (SwiGLU epilogue)" if w.gated else
                     "fc1 grouped GEMM (squared-ReLU epilogue)",
                     "achieved": fc1_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": fc1_gbs / PEAK_HBM_GBS, "traffic": traffic,
                     "algorithmic_bytes": ab["fc1"], "avg_launch_us": fc1_ms_timed * 1e3,
                     "device_copy_GBps": copy_gbs, "frac_of_device_copy": fc1_gbs / copy_gbs},
        "device": {"copy_GBps": copy_gbs, "gfx_mhz_under_load": clock["gfx_mhz"],
                   "socket_w_under_load": clock["socket_w"], "clock_samples": clock["samples"],
                   "clock_note": clock["note"], "nominal_mhz": NOMINAL_MHZ,
                   "mfma_frac_at_measured_clock": (tflops / (PEAK_F16_TFLOPS * clock["gfx_mhz"] / NOMINAL_MHZ)
                                                   if clock["gfx_mhz"] else None)},
        "kernels": kernels,
        "prepare": prepare,
        "recipes": recipes,
    }
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline ...")
        result["cpu_baseline"] = cpu_baseline(w, ids_np, wts_np, args.cpu_experts)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
