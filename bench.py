#!/usr/bin/env python3
"""Throughput of the per-token NVFP4 routed-MoE hot path on one MI355X.

One step = pmoe_moe_forward on BF16 activations (per-token quantization in
the same launch as the routing, FC1 + activation, requantization, FC2,
fixed-order finalize) over one batch of synthetic tokens already resident in
HBM, with weights prepared beforehand (preparation is timed separately and
reported as `prepare`).

Default workload: the one-GPU share of an EP4 MoE layer -- E=96 local experts,
H=7168, I=3072, SwiGLU, top-6, T=1024 tokens, two hot experts (router logits
+2 on experts 0 and 48); inputs from the seeded generator in synth/.

Prints one JSON line. `value` is tokens/s over the K bracketed steps; `step_us`
gives the median and p10/p90 of K more steps timed one by one. `roofline` is
the dominant kernel, the FC1 grouped GEMM as the step runs it: two launches
(one per part of the experts) on two streams; its algorithmic bytes over the
span from the first launch's start to the last launch's end, measured with
HIP events recorded on the stream each launch runs on (the library records
them around its own launches). `other_workloads` gives the same figures for
further workloads, `cpu_baseline` the CPU oracle on a bounded sample (all routes
of the first --cpu-experts experts), and `device` this device's own ceilings:
the bandwidth of a plain 1 GiB device-to-device copy, and the graphics clock
and socket power sampled while the step runs back to back.
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
    ap.add_argument("--other-workloads", default="ep4_t512,large,relu2,swiglu,tiny",
                    help="comma-separated further workloads timed in the same run ('' for none)")
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


def percentiles_us(ms_list):
    a = np.asarray(ms_list, np.float64) * 1e3
    return {"mean": float(a.mean()), "median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


def source_id():
    """The git commit when run from a checkout, and a hash of the library and bench sources
    (the GPU host gets a copy of the tree without its history)."""
    import hashlib
    import subprocess
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "precision_moe_amd", "csrc")
    for p in sorted(os.listdir(csrc)) + ["../../include/pmoe.h", "../../bench.py"]:
        with open(os.path.join(csrc, p), "rb") as f:
            h.update(f.read())
    try:
        sha = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True,
                             timeout=10).stdout.strip() or None
    except Exception:
        sha = None
    return {"git_sha": sha, "source_sha256": h.hexdigest()[:16]}


def timed_steps(torch, fn, steps):
    """K calls of fn, each between two events on torch's current stream: per-step ms."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        fn()
        evs[i + 1].record()
    torch.cuda.synchronize()
    return [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]


def gemm_spans(torch, pm, fn, steps):
    """K steps with the library's step events: per step, the FC1 span (first FC1 launch's
    start to the last one's end, over both streams), the FC2 span, and each part's own FC1
    and FC2 launch times (ms)."""
    per = [[torch.cuda.Event(enable_timing=True) for _ in range(pm.STEP_EVENTS)] for _ in range(steps)]
    for evs in per:
        for e in evs:
            e.record()                      # creates the events; the library records them again
    torch.cuda.synchronize()
    for evs in per:
        fn(evs)
    torch.cuda.synchronize()
    out = {"fc1_span": [], "fc2_span": [], "fc1_part1": [], "fc1_part2": [], "fc2_part1": [],
           "fc2_part2": []}
    for e in per:
        t = lambda i, j: e[i].elapsed_time(e[j])           # ms from event i to event j
        out["fc1_span"].append(max(t(0, 1), t(0, 3)) - min(0.0, t(0, 2)))
        out["fc2_span"].append(max(t(4, 5), t(4, 7)) - min(0.0, t(4, 6)))
        out["fc1_part1"].append(t(0, 1))
        out["fc1_part2"].append(t(2, 3))
        out["fc2_part1"].append(t(4, 5))
        out["fc2_part2"].append(t(6, 7))
    return out


def run_workload(torch, pm, synth, w, P, dev, steps, warmup):
    """Step time distribution, throughput and in-step GEMM figures of one workload."""
    x = synth.activations(w, device=dev).view(torch.bfloat16)
    ids_np, wts_np = synth.router(w)
    ids = torch.from_numpy(ids_np).to(dev)
    wts = torch.from_numpy(wts_np).to(dev)
    ws = torch.empty(pm.moe_workspace_bytes(w.T, w.K, w.E, w.H, w.I, P.act), dtype=torch.uint8, device=dev)
    out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)

    def step(step_events=None):
        pm.moe_forward(x, ids, wts, P, workspace=ws, out=out, step_events=step_events)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    dist = timed_steps(torch, step, steps)
    spans = gemm_spans(torch, pm, step, steps)
    views = pm.workspace_views(ws, w.T, w.K, w.E, w.H, w.I, P.act)
    counts = np.diff(views["expert_offsets"].cpu().numpy())
    R = int(counts.sum())
    ab = algorithmic_bytes(w, counts, w.T, R)
    ms = float(np.mean(dist))
    flops = 2.0 * R * (w.N1 * w.H + w.H * w.I)
    fc1 = float(np.mean(spans["fc1_span"]))
    fc2 = float(np.mean(spans["fc2_span"]))
    res = {
        "workload": w.name, "T": w.T, "H": w.H, "I": w.I, "E": w.E, "top_k": w.K, "act": w.act,
        "routed_rows": R, "step_us": percentiles_us(dist), "tokens/s": w.T / (ms * 1e-3),
        "TFLOP/s": flops / (ms * 1e-3) / 1e12, "mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
        "fc1_in_step": {"span_us": fc1 * 1e3, "GB/s": ab["fc1"] / (fc1 * 1e-3) / 1e9,
                        "hbm_frac": ab["fc1"] / (fc1 * 1e-3) / 1e9 / PEAK_HBM_GBS,
                        "TFLOP/s": 2.0 * R * w.N1 * w.H / (fc1 * 1e-3) / 1e12,
                        "mfma_frac": 2.0 * R * w.N1 * w.H / (fc1 * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
                        "algorithmic_bytes": ab["fc1"]},
        "fc2_in_step": {"span_us": fc2 * 1e3, "GB/s": ab["fc2"] / (fc2 * 1e-3) / 1e9,
                        "hbm_frac": ab["fc2"] / (fc2 * 1e-3) / 1e9 / PEAK_HBM_GBS,
                        "TFLOP/s": 2.0 * R * w.H * w.I / (fc2 * 1e-3) / 1e12,
                        "mfma_frac": 2.0 * R * w.H * w.I / (fc2 * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
                        "algorithmic_bytes": ab["fc2"]},
        "launch_us": {k: float(np.mean(v)) * 1e3 for k, v in spans.items() if "part" in k},
    }
    return res, dict(x=x, ids=ids, wts=wts, ids_np=ids_np, wts_np=wts_np, ws=ws, out=out, step=step,
                     views=views, counts=counts, R=R, ab=ab, spans=spans)


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

    def step(step_events=None):
        pm.moe_forward(x, ids, wts, P, workspace=ws, out=out, step_events=step_events)

    def step_separate_quantize():
        pm.quantize_input_per_token(x, out=(xq, xs, xg))
        pm.routed_moe(xq, xs, xg, ids, wts, P, workspace=ws, out=out)

    # ---------------------------------------------------------------- weight refresh
    # In-place re-preparation of the weights (timed on its own), right before the
    # forward steps, as a weight refit is followed by forwards.
    prep_ms = timed_steps(torch, lambda: pm.prepare_weights(w1, w2, out=P), 3)
    prep = float(np.mean(prep_ms))
    elems = w.E * (w.N1 * w.H + w.H * w.I)
    prepare = {"ms": prep, "GB/s": elems * (2 + NVFP4_BYTES) / (prep * 1e-3) / 1e9,
               "note": "reads BF16 once (algorithmic; the kernel reads it twice) and writes NVFP4"}
    log(f"[bench] prepare_weights {prep:.2f} ms")

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

    # ---------------------------------------------------------------- step distribution
    # K more steps, each between two events: median and p10/p90 of the step time
    dist = timed_steps(torch, step, args.steps)
    # K more steps with the library's step events: the grouped GEMMs as the step runs them
    spans = gemm_spans(torch, pm, step, args.steps)
    log(f"[bench] step median {np.median(dist) * 1e3:.1f} us; in-step FC1 span "
        f"{np.mean(spans['fc1_span']) * 1e3:.1f} us, FC2 span {np.mean(spans['fc2_span']) * 1e3:.1f} us")

    # ---------------------------------------------------------------- whole FC1 launch
    # Secondary figure: FC1 over all experts as one launch (fc_kernel, the one-stream
    # path's kernel) on the quantized activations of this workload, timed alone.
    pm.quantize_input_per_token(x, out=(xq, xs, xg))
    pm.routed_moe(xq, xs, xg, ids, wts, P, workspace=ws, out=out, steps=(pm.STEP_ROUTE, pm.STEP_ROUTE))
    fc1_whole = timed_steps(torch, lambda: pm.routed_moe(xq, xs, xg, ids, wts, P, workspace=ws, out=out,
                                                         steps=(pm.STEP_FC1, pm.STEP_FC1)), args.steps)

    # ---------------------------------------------------------------- per-step events
    names = ["quantize", "route", "fc1", "requant", "fc2", "finalize"]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
    acc = np.zeros(len(names))
    for _ in range(args.stage_reps):
        evs[0].record()
        pm.quantize_input_per_token(x, out=(xq, xs, xg))
        evs[1].record()
        for st in range(5):
            pm.routed_moe(xq, xs, xg, ids, wts, P, workspace=ws, out=out, steps=(st, st))
            evs[st + 2].record()
        torch.cuda.synchronize()
        acc += [evs[i].elapsed_time(evs[i + 1]) for i in range(len(names))]
    stage_ms = acc / args.stage_reps

    views = pm.workspace_views(ws, T, w.K, w.E, w.H, w.I, P.act)

    # ---------------------------------------------------------------- other recipes
    # The per-tensor NVFP4 and W4A16 variants of the same layer, on the same
    # inputs: static scales calibrated as 2688 / amax of the FC1 input and of
    # the per-token run's intermediate (setup, outside the timed region).
    pm.routed_moe(xq, xs, xg, ids, wts, P, workspace=ws, out=out)
    R_rows = int(views["counters"][0].item())
    a1 = (2688.0 / x.float().abs().max()).reshape(1).float()
    a2 = (2688.0 / views["h"][:R_rows].abs().max()).reshape(1).float()
    P_pt = pm.prepare_weights(w1, w2, input_scales=(a1, a2))
    del w1, w2
    torch.cuda.empty_cache()

    def step_per_tensor():  # the one-call forward, as the per-token step
        pm.moe_forward(x, ids, wts, P_pt, recipe="per_tensor", a1=a1, a2=a2, workspace=ws, out=out)

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
        # each recipe starts from a steady device: after idle or memory-bound
        # work (the per-tensor weight preparation above) the first ~25-40 steps
        # of any GPU work run slower
        for _ in range(max(args.warmup, 30)):
            fn()
        torch.cuda.synchronize()
        ms = float(np.mean(timed_steps(torch, fn, args.steps)))
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
    kernels["fc1"]["TFLOP/s"] = float(2.0 * R * w.N1 * w.H / (stage_ms[2] * 1e-3) / 1e12)
    kernels["fc2"]["TFLOP/s"] = float(2.0 * R * w.H * w.I / (stage_ms[4] * 1e-3) / 1e12)
    for n in ("fc1", "fc2"):
        kernels[n]["mfma_frac"] = kernels[n]["TFLOP/s"] / PEAK_F16_TFLOPS
    fc1_span = float(np.mean(spans["fc1_span"]))
    fc2_span = float(np.mean(spans["fc2_span"]))
    fc1_gbs = ab["fc1"] / (fc1_span * 1e-3) / 1e9
    fc1_whole_ms = float(np.mean(fc1_whole))
    traffic = profiling.read_traffic(os.path.join(ROOT, "profiles", f"fc1_{w.name}_hbm_traffic.txt"), w.name)
    kern = ("pmoe::fc_half_kernel<1, 0>" if w.gated else "pmoe::fc_half_kernel<0, 0>")

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
        "dtype": "nvfp4",
        "compute": "NVFP4 W4A4 (E2M1 codes, E4M3 block scales per 16, FP32 per-token / per-expert "
                   "scales) decoded exactly to FP16 operands of v_mfma_f32_16x16x32_f16, FP32 "
                   "accumulation; BF16 output",
        "data": "synthetic",
        "config": {"workload": w.name, "T": T, "H": w.H, "I": w.I, "E": w.E, "top_k": w.K,
                   "act": w.act, "routed_rows": R, "parallelism": "none (1 GPU)"},
        "source": source_id(),
        "step_us": percentiles_us(dist),
        "tflops": tflops,
        "mfma_frac": tflops / PEAK_F16_TFLOPS,
        "hbm_frac_step": ab["step"] / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "roofline": {"bound": "hbm", "kernel": kern,
                     "what": "FC1 grouped GEMM as the step runs it: one launch per part of the "
                             "experts, on two streams; achieved = algorithmic bytes of the whole FC1 "
                             "over the span from the first launch's start to the last one's end "
                             "(HIP events recorded by the library on each launch's stream), mean over "
                             "the steps",
                     "achieved": fc1_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": fc1_gbs / PEAK_HBM_GBS, "traffic": traffic,
                     "traffic_what": "HBM bytes of the step's launches of this kernel (both parts): "
                                     "rocprofv3 FETCH_SIZE and WRITE_SIZE, each scaled by what it "
                                     "reads for a plain device copy; null once the GEMM sources "
                                     "differ from the ones measured",
                     "algorithmic_bytes": ab["fc1"], "span_us": fc1_span * 1e3,
                     "span_us_median": float(np.median(spans["fc1_span"])) * 1e3,
                     "launch_us": {"part1": float(np.mean(spans["fc1_part1"])) * 1e3,
                                   "part2": float(np.mean(spans["fc1_part2"])) * 1e3},
                     "whole_launch": {"kernel": "pmoe::fc_kernel (all experts, one launch, alone)",
                                      "avg_launch_us": fc1_whole_ms * 1e3,
                                      "GB/s": ab["fc1"] / (fc1_whole_ms * 1e-3) / 1e9,
                                      "frac": ab["fc1"] / (fc1_whole_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
                     "device_copy_GBps": copy_gbs, "frac_of_device_copy": fc1_gbs / copy_gbs},
        "fc2_in_step": {"span_us": fc2_span * 1e3, "GB/s": ab["fc2"] / (fc2_span * 1e-3) / 1e9,
                        "hbm_frac": ab["fc2"] / (fc2_span * 1e-3) / 1e9 / PEAK_HBM_GBS,
                        "algorithmic_bytes": ab["fc2"],
                        "launch_us": {"part1": float(np.mean(spans["fc2_part1"])) * 1e3,
                                      "part2": float(np.mean(spans["fc2_part2"])) * 1e3}},
        "device": {"copy_GBps": copy_gbs, "gfx_mhz_under_load": clock["gfx_mhz"],
                   "socket_w_under_load": clock["socket_w"], "clock_samples": clock["samples"],
                   "clock_note": clock["note"], "nominal_mhz": NOMINAL_MHZ,
                   "mfma_frac_at_measured_clock": (tflops / (PEAK_F16_TFLOPS * clock["gfx_mhz"] / NOMINAL_MHZ)
                                                   if clock["gfx_mhz"] else None)},
        "kernels": kernels,
        "prepare": prepare,
        "recipes": recipes,
    }

    # ---------------------------------------------------------------- other workloads
    others = {}
    del ws, out, views
    torch.cuda.empty_cache()
    for name in [n for n in args.other_workloads.split(",") if n]:
        ow = synth.WORKLOADS[name]
        same = (ow.index, ow.weight_epoch, ow.E, ow.N1, ow.H, ow.I) == (w.index, w.weight_epoch, w.E,
                                                                        w.N1, w.H, w.I)
        if same and P is not None:
            OP = P
        else:  # other weights, or the main ones after an earlier workload freed them
            P = None
            torch.cuda.empty_cache()
            a, b = synth.all_weights(ow, device=dev)
            OP = pm.prepare_weights(a.view(torch.bfloat16), b.view(torch.bfloat16))
            del a, b
            torch.cuda.empty_cache()
        # after this workload's weight preparation: warmed to a steady device first
        res, _ = run_workload(torch, pm, synth, ow, OP, dev, args.steps, max(args.warmup, 30))
        others[name] = res
        log(f"[bench] {name}: median {res['step_us']['median']:.1f} us/step, "
            f"{res['tokens/s'] / 1e6:.3f} M tokens/s, FC1 span {res['fc1_in_step']['span_us']:.1f} us")
        del OP
        torch.cuda.empty_cache()
    result["other_workloads"] = others

    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline ...")
        result["cpu_baseline"] = cpu_baseline(w, ids_np, wts_np, args.cpu_experts)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
