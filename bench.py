#!/usr/bin/env python3
"""Throughput benchmark of the MI355X routed-MoE expert layer.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME ...]

A step is one full MoE-layer call (router GEMV/GEMM, top-k + renormalised
softmax, token->expert permutation, dequantising gate/up + SwiGLU, down,
weighted combine) over one batch of seeded synthetic tokens, with every
expert resident in HBM.  Decode workloads rotate over many resident layer
instances of the same shape (as consecutive layers of a stack would), so
repeated steps do not re-read one layer's experts from the on-die caches;
their timed region replays captured HIP graphs of exactly K steps.

With no --workload the run measures the metric's three configurations: the
4-token MTP verify (the headline line), the single-token decode and the
8192-token prefill chunk, each with its own step time, roofline and CPU
oracle baseline; the last two go under "also" in the same JSON line.

Prints ONE JSON line: the throughput (tokens/s), the roofline of the
dominant kernel from HIP events bound to each kernel's own dispatch on the
launch stream, the counter summaries committed under profiles/ when they
were taken on the current kernel sources, and the CPU oracle timed on a
bounded sample of the same workload.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 MFMA

METRIC = "MoE-layer tokens/s (decode, 8K prefill); % HBM peak (decode) / % MFMA peak"
DEFAULT_WORKLOADS = ["mtp_verify_t4_q2", "decode_t1_q2", "prefill_t8192_q2"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0, help="timed steps per workload (0: workload default)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", action="append", default=None,
                    help="workload to time (repeatable; default: " + ", ".join(DEFAULT_WORKLOADS) + ")")
    ap.add_argument("--layers", type=int, default=0, help="resident layer instances to rotate over")
    ap.add_argument("--seed", type=int, default=2026)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replay")
    ap.add_argument("--route", choices=("auto", "fused", "split"), default="auto",
                    help="grouped-path routing: the library's choice, one launch, or the multi-launch sequence")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB 4 times (reference for HBM counters)")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: every workload of this layer fits one MI355X and the "
              "multi-GPU (expert-parallel) path is not built; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    torch.cuda.set_device(torch.device("cuda:0"))
    names = args.workload or DEFAULT_WORKLOADS
    results, baselines = [], []
    # every GPU measurement first (back to back, so the clocks stay up), then
    # the CPU oracle baselines
    for name in names:
        r, cpu_job = run_workload(args, name)
        results.append(r)
        baselines.append(cpu_job)
        torch.cuda.empty_cache()
    for r, job in zip(results, baselines):
        r["cpu_baseline"] = job() if job is not None else None
    res = dict(results[0])
    res["metric"] = METRIC
    props = torch.cuda.get_device_properties(0)
    res["system"] = {"gpu": props.name, "arch": getattr(props, "gcnArchName", None),
                     "compute_units": props.multi_processor_count, "hip": torch.version.hip,
                     "torch": torch.__version__}
    if len(results) > 1:
        res["also"] = {r["config"]["workload"]: {k: v for k, v in r.items() if k not in ("metric",)}
                       for r in results[1:]}
    print(json.dumps(res), flush=True)


def run_workload(args, name):
    import torch
    from moe_synth import WORKLOADS, generate as G, canonical_block_bytes
    from quantized_moe_expert_gemv_amd import binding as B
    from quantized_moe_expert_gemv_amd import prof_summary

    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    stack = w.n_layers > 1
    decode = w.tokens <= B.STRATA_DECODE_MAX_T
    # skinny batches (up to 64 tokens) take the grouped-GEMM path but, like
    # decode, are bound by reading the touched experts once: timed the same way
    skinny = not decode and w.tokens <= 64
    T = w.tokens
    if args.layers:
        n_inst = args.layers
    elif stack:
        n_inst = w.n_layers
    elif decode or skinny:
        n_inst = 48 if w.hidden <= 2560 else 8
    else:
        n_inst = 2
    steps = args.steps or (1920 if (decode and not stack) else 640 if skinny else (64 if stack else 40))

    # ------------------------------------------------------------ resident layers
    t_setup = time.time()
    cfg = B.make_config(w.hidden, w.inter, w.n_experts, w.top_k, w.n_shared, w.fmt, T)
    layers, host0 = [], None
    for l in range(n_inst):
        wr = torch.from_numpy(G.router_weights(args.seed, l, w.hidden, w.n_experts)).to(dev)
        b = torch.from_numpy(G.router_bias(args.seed, l, w.n_experts, w.zipf_s)).to(dev) if w.biased else None
        canon_h = G.layer_canonical(args.seed, l, w.hidden, w.inter, w.n_experts, w.fmt, w.d_sigma)
        sh_h = G.shared_canonical(args.seed, l, w.hidden, w.inter, w.fmt, w.d_sigma) if w.n_shared else None
        canon = torch.from_numpy(canon_h.reshape(-1)).to(dev)
        sh = torch.from_numpy(sh_h).to(dev) if sh_h is not None else None
        layers.append(B.StrataMoE(cfg, wr, b, canon, sh))
        if l == 0:
            host0 = (canon_h, sh_h)
        del canon, sh, canon_h
    torch.cuda.synchronize()
    log(f"{n_inst} layer instances of {name} resident in "
        f"{sum(l.packed.numel() for l in layers) / 1e9:.1f} GB ({time.time() - t_setup:.0f} s)")

    # token batches (bf16, seeded)
    n_batches = 64 if (decode or skinny) else 1
    xs_h = [np.stack([G.token_candidates(args.seed, 1000 + bi, t, w.hidden) for t in range(T)])
            for bi in range(n_batches)]
    xs = [torch.from_numpy(x.astype(np.int16)).to(dev).view(torch.bfloat16) for x in xs_h]
    outs = [torch.empty((T, w.hidden), dtype=torch.float32, device=dev) for _ in range(2)]
    tmp = torch.empty((T, w.hidden), dtype=torch.float32, device=dev)

    flags = {"auto": 0, "fused": B.STRATA_FUSED_ROUTE, "split": B.STRATA_SPLIT_ROUTE}[args.route]
    one_launch_route = (not decode and T <= 64 and w.n_experts <= 512 and w.top_k <= 64 and
                        (args.route == "fused" or (args.route == "auto" and T <= B.STRATA_FUSED_ROUTE_DEFAULT_T)))

    def step(i, trace_events=None):
        x = xs[i % n_batches]
        if stack:
            if trace_events is not None:
                B.strata_moe_trace_next_call(layers[0].handle, trace_events)
            B.stack_forward(layers, x, out=outs[0], tmp=tmp)
        else:
            layer = layers[i % n_inst]
            if trace_events is not None:
                B.strata_moe_trace_next_call(layer.handle, trace_events)
            layer.forward(x, out=outs[i % 2], flags=flags)

    # ------------------------------------------------------------ routing statistics (for bytes)
    # unique experts per step, from the library's own routing of each (layer, batch) pair
    period = int(np.lcm(n_inst if not stack else 1, n_batches))
    uniq = []
    if not stack:
        for i in range(min(period, steps)):
            _, _, _, offs = layers[i % n_inst].route(xs[i % n_batches])
            uniq.append(int((offs[1:] - offs[:-1] > 0).sum().item()))
    else:
        uniq = [w.top_k]          # per layer of a single-token stack step
    u_mean = float(np.mean(uniq))

    # ------------------------------------------------------------ throughput
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # decode and skinny steps are graph replays; the prefill chunks launch
    # eagerly: replaying their eight kernels from a graph measured 1.5-5%
    # slower (8192 tokens 913 against 869 us on one box)
    use_graph = (decode or skinny) and not args.eager
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    if use_graph:
        # exactly `steps` steps: a captured rotation of g_len steps (the whole
        # (layer, batch) period, 8 stack passes, or all the steps when fewer)
        # replayed steps // g_len times, plus a graph of the remainder
        g_len = min(steps, 8 if stack else period)
        reps, rem = divmod(steps, g_len)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(3):
                step(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(g_len):
                step(i)
        tail = None
        if rem:
            tail = torch.cuda.CUDAGraph()
            with torch.cuda.graph(tail):
                for i in range(rem):
                    step(i)
        graph.replay()
        if tail is not None:
            tail.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for _ in range(reps):
            graph.replay()
        if tail is not None:
            tail.replay()
        e1.record()
        torch.cuda.synchronize()
    else:
        t0 = time.perf_counter()
        e0.record()
        for i in range(steps):
            step(i)
        e1.record()
        torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    ms_per_step = gpu_ms / steps
    value = T * steps / (gpu_ms / 1e3)
    log(f"{name}: {steps} steps in {gpu_ms:.2f} ms GPU ({wall * 1e3:.1f} ms wall): {ms_per_step * 1e3:.2f} us/step")

    # ------------------------------------------------------------ per-kernel durations (HIP events)
    if decode:                                              # (stack: layer 0 of each pass)
        knames = ["route_gemv", "topk", "gateup", "down_combine"]
    else:
        knames = ["router_gemm", "topk", "colscan", "scan", "scatter", "gateup_gemm", "down_gemm", "combine"]
        if one_launch_route:               # router, top-k and permutation in one launch
            knames = ["route_one_launch", "gateup_gemm", "down_gemm", "combine"]
        elif T <= 32:                      # one top-k chunk also scans and scatters
            knames = ["router_gemm", "topk_scan_scatter", "gateup_gemm", "down_gemm", "combine"]
    # each kernel's own dispatch start/end, bound to a pair of events on the
    # launch stream (eager launches of the same steps, after the timed region)
    n_trace = min(steps, 256)
    ev_sets = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * len(knames))]
               for _ in range(n_trace)]
    torch.cuda.synchronize()
    for i in range(n_trace):
        step(i, trace_events=ev_sets[i])
    torch.cuda.synchronize()
    dur = np.array([[ev[2 * j].elapsed_time(ev[2 * j + 1]) for j in range(len(knames))] for ev in ev_sets])
    # the median over the traced steps: single dispatches launched one at a
    # time with their own events now and then run several microseconds long
    # (the mean of a decode kernel moved by up to 3 us from run to run)
    kern_us = np.median(dur, axis=0) * 1e3

    # algorithmic work per launch
    bq = canonical_block_bytes(w.fmt)
    gu_bytes = 2 * w.inter * (w.hidden // 32) * bq
    dn_bytes = w.hidden * (w.inter // 32) * bq
    x_bytes = T * w.hidden * 2
    out_bytes = T * w.hidden * 4
    router_bytes = w.n_experts * w.hidden * 4
    kernels = {}
    counters = None
    if decode:
        ue = u_mean + w.n_shared
        alg = {"route_gemv": router_bytes + x_bytes,
               "topk": T * w.n_experts * 4,
               "gateup": ue * gu_bytes + x_bytes,
               "down_combine": ue * dn_bytes + out_bytes}
        for j, n in enumerate(knames):
            kernels[n] = {"us": round(float(kern_us[j]), 3), "alg_bytes": int(alg[n]),
                          "GBps": round(alg[n] / (kern_us[j] * 1e-6) / 1e9, 1)}
        dom = max(knames, key=lambda n: kernels[n]["us"])
        achieved = kernels[dom]["GBps"]
        # HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE summary,
        # if it was taken on the current kernel sources
        measured = prof_summary.read_traffic(os.path.join(ROOT, "profiles", f"decode_hbm_traffic_{name}.md"))
        roofline = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": int(measured[dom]) if dom in measured else None,
                    "alg_bytes": kernels[dom]["alg_bytes"]}
        layer_bytes = router_bytes + ue * (gu_bytes + dn_bytes) + x_bytes + out_bytes
        if stack:                 # every layer of the pass moves the same algorithmic bytes
            layer_bytes *= w.n_layers
        layer_frac = layer_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9)
    else:
        P = T * w.top_k
        fl = {"router_gemm": 2.0 * T * w.hidden * w.n_experts, "route_one_launch": 2.0 * T * w.hidden * w.n_experts,
              "gateup_gemm": 2.0 * (P + w.n_shared * T) * w.hidden * 2 * w.inter,
              "down_gemm": 2.0 * (P + w.n_shared * T) * w.inter * w.hidden}
        for j, n in enumerate(knames):
            kernels[n] = {"us": round(float(kern_us[j]), 3)}
            if n in fl:
                kernels[n]["TFLOPs"] = round(fl[n] / (kern_us[j] * 1e-6) / 1e12, 1)
        dom = max(knames, key=lambda n: kernels[n]["us"])
        achieved = kernels[dom].get("TFLOPs", 0.0)
        # HBM bytes per launch of that kernel (FETCH_SIZE + WRITE_SIZE summary
        # taken on the current kernel sources), for reference next to the flops
        measured = prof_summary.read_traffic(os.path.join(ROOT, "profiles", f"prefill_hbm_traffic_{name}.md"))
        roofline = {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": MFMA_F16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                    "traffic": int(measured[dom]) if dom in measured else None}
        # matrix-core busy fraction from the committed SQ counter summary
        counters = prof_summary.read_mfma(os.path.join(ROOT, "profiles", f"prefill_mfma_counters_{name}.md")) or None
        if counters and dom in counters:
            roofline["mfma_busy_frac_counter"] = counters[dom]["busy_frac"]
        layer_flops = sum(fl.values())
        layer_frac = layer_flops / (ms_per_step * 1e-3) / (MFMA_F16_PEAK_TFLOPS * 1e12)
        layer_bytes = None
        if skinny:
            # bound by reading the touched experts once: the expert GEMMs
            # against the HBM peak (algorithmic bytes: the unique experts'
            # packed gate/up or down bytes plus the tokens in / rows out)
            ue = u_mean + w.n_shared
            alg = {"gateup_gemm": ue * gu_bytes + x_bytes,
                   "down_gemm": ue * dn_bytes + (P + w.n_shared * T) * w.hidden * 2}
            for n in alg:
                j = knames.index(n)
                kernels[n]["alg_bytes"] = int(alg[n])
                kernels[n]["GBps"] = round(alg[n] / (kern_us[j] * 1e-6) / 1e9, 1)
            dom = max(alg, key=lambda n: kernels[n]["us"])
            achieved = kernels[dom]["GBps"]
            roofline = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                        "alg_bytes": kernels[dom]["alg_bytes"]}
            layer_bytes = router_bytes + ue * (gu_bytes + dn_bytes) + x_bytes + out_bytes
            layer_frac = layer_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9)

    # the CPU oracle baseline, run by the caller once every GPU measurement is done
    cpu_job = None if args.no_cpu else (lambda: cpu_baseline(args, w, host0, xs_h, G))

    del layers, xs, outs, tmp
    return {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32" if decode else "fp16",
        "data": "synthetic",
        "config": {"workload": name, "tokens_per_step": T, "hidden": w.hidden,
                   "inter": w.inter, "experts": w.n_experts, "top_k": w.top_k,
                   "shared": w.n_shared, "format": ("MXFP4" if w.fmt == 5 else f"Q{w.fmt}"), "layers_rotated": n_inst,
                   "stack_layers": w.n_layers, "launch": "hip_graph" if use_graph else "eager",
                   "routing": None if decode else ("one_launch" if one_launch_route else "multi_launch"),
                   "unique_experts_per_step": round(u_mean, 2)},
        "roofline": roofline,
        "layer_roofline_frac": None if layer_frac is None else round(layer_frac, 4),
        "step_alg_bytes": None if layer_bytes is None else int(layer_bytes),
        "kernels": kernels,
        "mfma_counters": counters,
        "cpu_baseline": None,
    }, cpu_job


def copy_calibration(mib):
    """A plain copy of known size: what the HBM read/write counters report for
    it scales the counters of the layer's kernels to bytes."""
    import torch
    n = mib << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(4):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 4
    print(json.dumps({"copy_bytes_each_way": n, "copies": 4, "ms_per_copy": round(ms, 4),
                      "GBps_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def cpu_baseline(args, w, host0, xs_h, G):
    """The fp64 oracle, as it stands, on layer 0 of the same workload."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas = None
    canon_h, sh_h = host0
    wr = G.router_weights(args.seed, 0, w.hidden, w.n_experts)
    b = G.router_bias(args.seed, 0, w.n_experts, w.zipf_s) if w.biased else None
    rec = (lambda e: canon_h[e])
    t0 = time.perf_counter()
    n_tok, n_calls = 0, 0
    if w.tokens <= 8 and w.n_layers == 1:
        while True:
            x = G.bf16_bits_to_f32(xs_h[n_calls % len(xs_h)]).astype(np.float64)
            O.moe_layer(x, wr, b, rec, w.hidden, w.inter, w.top_k, w.fmt, shared_record=sh_h)
            n_tok += x.shape[0]
            n_calls += 1
            if time.perf_counter() - t0 > args.cpu_seconds:
                break
        sample = f"{n_calls} calls of {w.tokens} token(s) on layer 0"
    elif w.n_layers == 1:
        # a slice of the chunk: the oracle's cost is per token and per touched expert
        x = G.bf16_bits_to_f32(xs_h[0]).astype(np.float64)
        n = 64
        O.moe_layer(x[:n], wr, b, rec, w.hidden, w.inter, w.top_k, w.fmt, shared_record=sh_h)
        n_tok, n_calls = n, 1
        sample = f"first {n} tokens of the {w.tokens}-token chunk on layer 0"
    else:
        x = G.bf16_bits_to_f32(xs_h[0]).astype(np.float64)
        O.moe_layer(x, wr, b, rec, w.hidden, w.inter, w.top_k, w.fmt)
        n_tok, n_calls = x.shape[0] / w.n_layers, 1
        sample = "one token through layer 0 of the stack, scaled to the full stack"
    dt = time.perf_counter() - t0
    return {"value": round(n_tok / dt, 3), "unit": "tokens/s", "cores": blas, "kind": "oracle",
            "sample": sample, "seconds": round(dt, 2),
            "host_cpus": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
