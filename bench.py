"""Benchmark of the MoE layer hot path on one MI355X.

Default workload: single-token decode through one GLM-5.2-scale MoE layer
(T=1, hidden 6144, expert intermediate 2048, 256 routed experts in 8 groups,
top-4 groups, top-8 experts, 1 shared expert, int4 weights with per-row
scales): ~171 MB of expert weights per token, HBM-bound.

A step is one moe_layer_forward over one token input; the inputs rotate over
64 distinct tokens (so the routed experts change step to step) and a 1 GiB
buffer is rewritten between steps, outside the timed events, so the weights
come from HBM, not from the 256 MB Infinity Cache or the L2s.  The flush
only reads (a sum over the buffer): a flush that writes would leave dirty
lines whose write-back the next kernel pays for.  HIP events on
the launch stream time each step; a second pass times each kernel of the
path alone (MOE_STAGE) for the roofline of the dominant kernel.  The oracle
is timed on the host cores on a bounded sample of the same workload.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + effective weight GB/s vs HBM peak (int4 decode)"
HBM_PEAK_GBS = 8000.0
N_INPUTS = 64


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_moe_noaux_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources (else None)."""
    p = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_source_hash") != kernel_source_hash() or d.get("kernel") != kernel:
        return None
    return d.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_int4")
    ap.add_argument("--no-flush", action="store_true", help="keep caches warm between steps")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    from quantized_moe_noaux_amd import moe

    dev = "cuda:0"
    torch.cuda.set_device(0)
    wl = synth.workload(args.workload)
    T = wl.T
    sh = moe.shape_of(wl)
    log("bench: %s T=%d H=%d I=%d E=%d k=%d int%d" % (wl.name, T, wl.hidden, wl.inter, wl.n_experts,
                                                      wl.top_k, wl.wbits))

    # ---------------------------------------------------------------- inputs
    host = synth.HostLayer(wl)
    gate_w = torch.from_numpy(host.gate_w).to(dev)
    bias = torch.from_numpy(host.bias).to(dev)
    routed = synth.device_weights(wl, 0, 0, wl.n_experts, dev)
    shared = synth.device_weights(wl, 0, wl.n_experts, 1, dev) if wl.n_shared else None
    xs = torch.stack([torch.from_numpy(
        synth.host_normals(wl.seed + i, synth.stream_id(0, synth.X), T * wl.hidden, 1.0).reshape(T, wl.hidden))
        for i in range(N_INPUTS)]).to(dev)
    y = torch.empty((T, wl.hidden), dtype=torch.float32, device=dev)
    idx = torch.empty((T, wl.top_k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, wl.top_k), dtype=torch.float32, device=dev)
    ws = moe.workspace(moe.moe_workspace_bytes(sh, T), dev)
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB, read to flush
    stream = torch.cuda.current_stream()
    n_stages = moe.moe_layer_stage_count(sh, T)
    torch.cuda.synchronize()

    def flush():
        if not args.no_flush:
            flush_buf.sum()

    def step(i, flags=0):
        moe.moe_layer_forward(sh, xs[i % N_INPUTS], gate_w, bias, routed, shared, y, ws, idx, wts, flags=flags)

    # union of the selected experts per input, for the bytes actually read
    union_sizes = []
    for i in range(N_INPUTS):
        step(i)
        torch.cuda.synchronize()
        union_sizes.append(len(np.unique(idx.cpu().numpy())))
    for i in range(args.warmup):
        flush()
        step(i)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush()
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = np.array([a.elapsed_time(b) for a, b in ev])
    ms = float(step_ms.mean())

    # ---------------------------------------------------------------- per-kernel
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_stages + 1)] for _ in range(args.steps)]
    for i in range(args.steps):
        flush()
        for s in range(n_stages):
            sev[i][s].record(stream)
            step(i, flags=moe.MOE_STAGE(s))
        sev[i][n_stages].record(stream)
    torch.cuda.synchronize()
    stage_ms = np.array([[sev[i][s].elapsed_time(sev[i][s + 1]) for s in range(n_stages)]
                         for i in range(args.steps)]).mean(0)

    # algorithmic bytes: each unique routed expert of the batch and the shared
    # expert once (codes + fp32 row scales); router weights counted apart
    gate_up_bytes = 2 * (wl.gate_bytes + 4 * wl.inter)
    down_bytes = wl.down_bytes + 4 * wl.hidden
    n_exp = float(np.mean(union_sizes)) + wl.n_shared
    layer_bytes = n_exp * (gate_up_bytes + down_bytes)
    router_bytes = 4 * wl.n_experts * wl.hidden
    tok_s = T / (ms * 1e-3)
    kernels = ["router+quant", "plan", "gate_up_swiglu_quant", "down_combine"]
    kbytes = [router_bytes, 0, n_exp * gate_up_bytes, n_exp * down_bytes]
    dom = int(np.argmax(stage_ms))
    dom_bytes = kbytes[dom] if dom < len(kbytes) else None
    dom_gbs = dom_bytes / (stage_ms[dom] * 1e-3) / 1e9 if dom_bytes else None
    traffic = traffic_from_profiles(wl.name, kernels[dom] if dom < len(kernels) else "stage%d" % dom)
    log("bench: step %.2f us (p10 %.2f p90 %.2f), %.0f tok/s, layer %.0f GB/s = %.1f%% of HBM peak" %
        (ms * 1e3, np.percentile(step_ms, 10) * 1e3, np.percentile(step_ms, 90) * 1e3, tok_s,
         layer_bytes / (ms * 1e-3) / 1e9, 100 * layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS))
    log("bench: stages (us): %s" % ", ".join("%.2f" % (v * 1e3) for v in stage_ms))

    # ---------------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        osh = oracle.shape_of(wl)
        done, spent, tokens = 0, 0.0, 0
        t_start = time.perf_counter()
        while spent < args.cpu_seconds and done < N_INPUTS:
            x = xs[done].cpu().numpy()
            ridx, _ = oracle.route(osh, x, host.gate_w, host.bias)
            experts = oracle.layer_experts(host, ridx)       # generated outside the timing
            c0 = time.perf_counter()
            oracle.layer_forward(osh, x, host.gate_w, host.bias, experts, host.shared)
            spent += time.perf_counter() - c0
            tokens += T
            done += 1
            host._experts = {k: v for k, v in host._experts.items() if k == wl.n_experts}
            if time.perf_counter() - t_start > 4 * args.cpu_seconds:
                break
        cpu = {"value": tokens / spent, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": "%d of the %d rotating %s inputs (T=%d each), full layer forward per input, "
                         "expert generation excluded" % (done, N_INPUTS, wl.name, T),
               "seconds": round(spent, 2)}
        log("bench: oracle %.3f tok/s on %d threads (%d inputs, %.1f s)" %
            (cpu["value"], cpu["cores"], done, spent))

    out = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic (seeded SplitMix64 weights and N(0,1) tokens, %d rotating inputs%s)" %
                (N_INPUTS, "" if args.no_flush else ", caches flushed between steps"),
        "config": {"workload": wl.name, "T": T, "hidden": wl.hidden, "inter": wl.inter,
                   "n_experts": wl.n_experts, "n_group": wl.n_group, "topk_group": wl.topk_group,
                   "top_k": wl.top_k, "n_shared": wl.n_shared, "wbits": wl.wbits, "rsf": wl.rsf},
        "effective_weight_GBps": layer_bytes / (ms * 1e-3) / 1e9,
        "effective_weight_frac": layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm", "kernel": kernels[dom] if dom < len(kernels) else "stage%d" % dom,
                     "achieved": dom_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dom_gbs / HBM_PEAK_GBS if dom_gbs else None,
                     "traffic": traffic, "algorithmic_bytes_per_launch": dom_bytes,
                     "avg_launch_us": float(stage_ms[dom] * 1e3)},
        "detail": {"stage_us": [float(v * 1e3) for v in stage_ms], "stage_names": kernels[:n_stages],
                   "step_us_p10_p50_p90": [float(np.percentile(step_ms, p) * 1e3) for p in (10, 50, 90)],
                   "mean_experts_read": n_exp, "layer_weight_bytes": layer_bytes,
                   "router_weight_bytes": router_bytes, "wall_s_timed_loop_incl_flush": wall},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
