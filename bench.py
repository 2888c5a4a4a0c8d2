"""Benchmark of the MoE layer hot path on one MI355X.

Default workload: single-token decode through one GLM-5.2-scale MoE layer
(T=1, hidden 6144, expert intermediate 2048, 256 routed experts in 8 groups,
top-4 groups, top-8 experts, 1 shared expert, int4 weights with per-row
scales): ~171 MB of expert weights per token, HBM-bound.  Other workloads
(--workload): verify_int8 (3 tokens, int8 weights), prefill_int4 (2048
tokens through the expert-grouped int8-MFMA path), stack_int2 (75 layers),
mtp_int4 (draft verification and acceptance), tier_int4 and tier_stack_int4
(experts over HBM and host memory).  The default run also records the
workloads in SECONDARY, each run by a child process with its defaults, under
"secondary" in its JSON line (--no-secondary skips them).

A step is one moe_layer_forward over one input batch; the inputs rotate
(64 distinct tokens for decode and verify, 4 batches for prefill) so the
routed experts change step to step, and a 1 GiB buffer is read between
steps, outside the timed events, so the weights come from HBM rather than
the 256 MB Infinity Cache or the L2s.  The flush only reads: a flush that
writes would leave dirty lines whose write-back the next kernel pays for.
HIP events on the launch stream time each step; a second pass times each
kernel of the path alone (MOE_STAGE flags) for the roofline of the dominant
kernel.  The oracle is timed on the host cores on a bounded sample of the
same workload.

Prints ONE JSON line on stdout; progress goes to stderr.

Two helper modes serve the HBM-traffic figure (rocprofv3 counters):
  --copy-calibration   a plain 1 GiB device copy, run under
                       `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` to
                       scale the counters to bytes
  --write-traffic      parses the four counter runs (kernel of a workload,
                       copy) and writes profiles/traffic_<workload>.json,
                       tagged with a hash of the kernel sources
"""
import argparse
import csv
import glob
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
MFMA_I8_PEAK_TOPS = 5000.0     # dense int8 MFMA, MI355X
FP64_PEAK_TFLOPS = 78.6        # fp64 vector
COPY_BYTES = 1 << 30

# kernels of each path, in stage order, with the substring that names them in
# a rocprofv3 trace
GEMV_STAGES = [("router+quant", "k_router_logits_small"), ("plan", "k_plan"),
               ("gate_up_swiglu_quant", "k_gate_up"), ("down_combine", "k_down")]


def gemv_stages(n_stages):
    """The GEMV path's stages of one call: a one-token call of the production
    row widths routes inside its gate/up launch and has no plan launch."""
    return GEMV_STAGES if n_stages == len(GEMV_STAGES) else [s for s in GEMV_STAGES if s[0] != "plan"]
GROUPED_STAGES = [("router_logits_fp64", "k_router_logits_mfma"), ("topk", "k_topk"),
                  ("quant_x", "k_gg_quant"), ("permute", "k_perm_"),
                  ("gate_up_swiglu_quant", "k_gg_gate_up"), ("down", "k_gg_down"),
                  ("combine", "k_gg_combine")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# sources (and build script) that make the kernels of each path
PATH_SOURCES = {"gemv": ["gemv.hip", "route.hip", "moe_dev.h", "topk_dev.h", "moe_internal.h", "slot_record.h"],
                "grouped": ["grouped.hip", "route.hip", "misc.hip", "moe_dev.h", "topk_dev.h", "moe_internal.h"]}


def kernel_source_hash(path):
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "quantized_moe_noaux_amd")
    for f in PATH_SOURCES[path]:
        h.update(open(os.path.join(pkg, "csrc", f), "rb").read())
    h.update(open(os.path.join(pkg, "_build.py"), "rb").read())
    return h.hexdigest()[:16]


def path_of(workload):
    return "grouped" if workload == "prefill_int4" else "gemv"


def stages_of(workload):
    if workload == "prefill_int4":
        return GROUPED_STAGES
    if workload == "stack_int2":
        return stack_stages(GEMV_STAGES)
    return GEMV_STAGES


def stack_stages(stages):
    """In the stack the router launch also forms the layer's RMSNorm."""
    return [("rmsnorm+router+quant", m) if n == "router+quant" else (n, m) for n, m in stages]


def traffic_from_profiles(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources (else None)."""
    p = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_source_hash") != kernel_source_hash(path_of(workload)) or d.get("kernel") != kernel:
        return None
    return d.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------- counter helpers
def _counter_rows(d):
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit("no counter_collection.csv under %s" % d)
    return rows


def _per_dispatch(rows, counter, match=None):
    """{kernel name: [value per dispatch]} for one counter (KiB per dispatch)."""
    out = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        name = r.get("Kernel_Name", "")
        if match and match not in name:
            continue
        out.setdefault(name, []).append(float(r["Counter_Value"]))
    return out


def _copy_kib(d, counter):
    per = _per_dispatch(_counter_rows(d), counter)
    # the copy kernel (by name), else the kernel with the most bytes per dispatch
    named = {k: v for k, v in per.items() if "copy" in k.lower()}
    name, vals = max((named or per).items(), key=lambda kv: sum(kv[1]) / len(kv[1]))
    return name, sum(vals) / len(vals)


def write_traffic(args):
    kernel, match = [s for s in stages_of(args.workload) if s[0] == args.kernel][0]
    res = {"workload": args.workload, "kernel": kernel, "kernel_source_hash": kernel_source_hash(path_of(args.workload))}
    total = 0.0
    for counter, kdir, cdir in (("FETCH_SIZE", args.pmc_fetch, args.copy_fetch),
                                ("WRITE_SIZE", args.pmc_write, args.copy_write)):
        per = _per_dispatch(_counter_rows(kdir), counter, match)
        vals = [v for vs in per.values() for v in vs]
        if not vals:
            raise SystemExit("no %s dispatches of %s in %s" % (counter, match, kdir))
        copy_name, copy_kib = _copy_kib(cdir, counter)
        factor = COPY_BYTES / (copy_kib * 1024.0)
        kib = sum(vals) / len(vals)
        res[counter.lower()] = {"kib_per_dispatch": kib, "dispatches": len(vals),
                                "copy_kernel": copy_name[:80], "copy_kib_per_dispatch": copy_kib,
                                "bytes_per_counted_byte": factor, "bytes_per_launch": kib * 1024.0 * factor}
        total += kib * 1024.0 * factor
    res["hbm_bytes_per_launch"] = total
    res["commands"] = args.commands
    p = os.path.join(ROOT, "profiles", "traffic_%s.json" % args.workload)
    with open(p, "w") as fh:
        json.dump(res, fh, indent=1)
        fh.write("\n")
    log("bench: wrote %s: %.1f MB per launch of %s" % (p, total / 1e6, kernel))


# The default run (the int4 decode layer) also records the other workloads,
# each in a child process of its own with its default steps, so that one run
# carries every configuration's figure; the headline line is unaffected.
SECONDARY = ["prefill_int4", "stack_int2", "verify_int8", "mtp_int4", "tier_int4"]
SECONDARY_TIMEOUT_S = 300


def run_secondary():
    import subprocess
    res = {}
    for w in SECONDARY:
        log("bench: secondary workload %s" % w)
        t0 = time.time()
        try:
            p = subprocess.run([sys.executable, os.path.abspath(__file__), "--workload", w, "--no-cpu-baseline",
                                "--no-secondary"], stdout=subprocess.PIPE, text=True, timeout=SECONDARY_TIMEOUT_S)
        except subprocess.TimeoutExpired:
            res[w] = {"error": "timed out after %d s" % SECONDARY_TIMEOUT_S}
            continue
        lines = [ln for ln in p.stdout.splitlines() if ln.startswith("{")]
        if p.returncode != 0 or not lines:
            res[w] = {"error": "exit status %d" % p.returncode}
            continue
        j = json.loads(lines[-1])
        rf = j.get("roofline") or {}
        det = j.get("detail") or {}
        rec = {k: j.get(k) for k in ("value", "unit", "ms_per_step", "steps", "warmup", "higher_is_better", "dtype")}
        rec["config"] = j.get("config")
        rec["roofline"] = {k: rf.get(k) for k in ("bound", "kernel", "achieved", "peak", "unit", "frac", "traffic")}
        for k in ("stage_us", "per_layer_us", "tokens_per_step", "hit_rate"):
            if k in det:
                rec[k] = det[k]
        rec["wall_s"] = time.time() - t0
        res[w] = rec
    return res


def copy_calibration():
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 10}), flush=True)


def stream_ceiling():
    """The read bandwidth a plain stream reaches on this GPU, with the
    decode kernels' load pattern (moe_stream_read): 1 GiB, four times the
    memory-side cache, read 20 times back to back; and a 128 MiB region,
    which the memory-side cache can hold, read 20 times back to back."""
    import torch
    from quantized_moe_noaux_amd import moe
    dev = "cuda:0"
    sink = torch.empty(moe.MOE_STREAM_SINK_WORDS, dtype=torch.int32, device=dev)
    big = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    region = big[: (128 << 20) // 4]
    stream = torch.cuda.current_stream()
    out = {}
    for name, buf in (("hbm_1GiB", big), ("region_128MiB", region)):
        for _ in range(3):
            moe.moe_stream_read(buf, sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(20):
            moe.moe_stream_read(buf, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        gbps = 20 * buf.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        out[name + "_GBps"] = gbps
        log("bench: stream read %s: %.0f GB/s = %.1f%% of %d GB/s" % (name, gbps, 100 * gbps / HBM_PEAK_GBS,
                                                                     HBM_PEAK_GBS))
    out["hbm_frac_of_peak"] = out["hbm_1GiB_GBps"] / HBM_PEAK_GBS
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------- the layer benchmark
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode_int4",
                    choices=["decode_int4", "verify_int8", "prefill_int4", "stack_int2", "mtp_int4", "tier_int4",
                             "tier_stack_int4"])
    ap.add_argument("--no-flush", action="store_true", help="keep caches warm between steps")
    ap.add_argument("--graph", action="store_true", help="launch each step as a captured HIP graph")
    ap.add_argument("--top-p", type=float, default=0.0, help="adaptive expert top-p (decode / verify)")
    ap.add_argument("--stack-eager", action="store_true", help="stack: launch directly instead of a graph")
    ap.add_argument("--draft", type=int, default=4, help="mtp_int4: drafts per verify step")
    ap.add_argument("--tokens", type=int, default=None,
                    help="decode_int4 / verify_int8: tokens per step (the verify batch 1 + drafts)")
    ap.add_argument("--temp", type=float, default=0.7, help="mtp_int4: sampling temperature (0 = greedy)")
    ap.add_argument("--slots", type=int, default=32, help="tier_int4: HBM slots for routed experts (of 256)")
    ap.add_argument("--repin", type=int, default=16, help="tier_int4: tokens between live repins")
    ap.add_argument("--layers", type=int, default=4, help="tier_stack_int4: layers")
    ap.add_argument("--lookahead", type=int, default=0,
                    help="stack_int2: router lookahead, N workgroups per prefetched expert (0 = off)")
    ap.add_argument("--lookahead-ranks", type=int, default=None,
                    help="tier_stack_int4: prefetch only the first N ranks of each predicted selection")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    ap.add_argument("--no-secondary", action="store_true",
                    help="default run: skip the other workloads' records (see SECONDARY)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--stream-ceiling", action="store_true",
                    help="measure the plain streaming-read bandwidth (the HBM kernels' practical ceiling)")
    ap.add_argument("--write-traffic", action="store_true")
    ap.add_argument("--kernel", default="gate_up_swiglu_quant")
    ap.add_argument("--pmc-fetch")
    ap.add_argument("--pmc-write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--commands", nargs="*", default=[])
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.write_traffic:
        return write_traffic(args)
    if args.copy_calibration:
        return copy_calibration()
    if args.stream_ceiling:
        return stream_ceiling()

    import numpy as np
    import torch
    import synth
    from quantized_moe_noaux_amd import moe

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.workload == "mtp_int4":
        return bench_mtp(args)
    if args.workload == "tier_int4":
        return bench_tier(args)
    if args.workload == "tier_stack_int4":
        return bench_tier_stack(args)
    wl = synth.workload(args.workload)
    if args.top_p:
        if wl.layers > 1 or args.workload == "prefill_int4":
            raise SystemExit("--top-p applies to the one-layer GEMV workloads (decode_int4, verify_int8)")
        wl = synth.workload(args.workload, top_p=args.top_p)
    if args.tokens is not None:
        if wl.layers > 1 or args.workload == "prefill_int4" or not 1 <= args.tokens <= 8:
            raise SystemExit("--tokens takes 1..8 on the one-layer GEMV workloads (decode_int4, verify_int8)")
        from dataclasses import replace
        wl = replace(wl, T=args.tokens)
    if wl.layers > 1:
        return bench_stack(args, wl)
    T = wl.T
    grouped = wl.name == "prefill_int4"
    n_inputs = 4 if grouped else 64
    steps = args.steps if args.steps is not None else (50 if grouped else 200)
    warmup = args.warmup if args.warmup is not None else (5 if grouped else 20)
    flags = moe.MOE_PATH_GROUPED if grouped else moe.MOE_PATH_GEMV
    sh = moe.shape_of(wl)
    n_stages = moe.moe_layer_stage_count(sh, T, flags)
    stages = GROUPED_STAGES if grouped else gemv_stages(n_stages)
    log("bench: %s T=%d H=%d I=%d E=%d k=%d int%d (%s path)" %
        (wl.name, T, wl.hidden, wl.inter, wl.n_experts, wl.top_k, wl.wbits, "grouped" if grouped else "GEMV"))

    # ---------------------------------------------------------------- inputs
    host = synth.HostLayer(wl)
    gate_w = torch.from_numpy(host.gate_w).to(dev)
    bias = torch.from_numpy(host.bias).to(dev)
    routed = synth.device_weights(wl, 0, 0, wl.n_experts, dev)
    shared = synth.device_weights(wl, 0, wl.n_experts, 1, dev) if wl.n_shared else None
    xs = torch.stack([torch.from_numpy(
        synth.host_normals(wl.seed + i, synth.stream_id(0, synth.X), T * wl.hidden, 1.0).reshape(T, wl.hidden))
        for i in range(n_inputs)]).to(dev)
    y = torch.empty((T, wl.hidden), dtype=torch.float32, device=dev)
    idx = torch.empty((T, wl.top_k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, wl.top_k), dtype=torch.float32, device=dev)
    ws = moe.workspace(moe.moe_workspace_bytes(sh, T, flags), dev)
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB, read to flush
    stream = torch.cuda.current_stream()
    assert n_stages == len(stages), (n_stages, len(stages))
    torch.cuda.synchronize()

    def flush():
        if not args.no_flush:
            flush_buf.sum()

    def step(i, f=0):
        moe.moe_layer_forward(sh, xs[i % n_inputs], gate_w, bias, routed, shared, y, ws, idx, wts, flags=flags | f)

    # union of the selected experts per input, for the bytes actually read
    # (through moe_route, so that every launch of the layer's kernels in this
    # run is a timed one or a warmup, all on flushed caches)
    union_sizes = []
    rws = moe.workspace(moe.moe_route_workspace_bytes(sh, T), dev)
    for i in range(n_inputs):
        moe.moe_route(sh, xs[i], gate_w, bias, idx, wts, rws)
        torch.cuda.synchronize()
        sel = idx.cpu().numpy()
        union_sizes.append(len(np.unique(sel[sel >= 0])))        # top-p drops slots (-1)
    for i in range(warmup):
        flush()
        step(i)
    torch.cuda.synchronize()
    log("bench: inputs ready, %d warmup steps done" % warmup)

    # With --graph the step is launched as a HIP graph (one captured per
    # rotating input).  Measured on MI355X with ROCm 7, replaying the
    # three-launch decode layer as a graph costs ~7 us more per step than
    # launching its kernels directly, so direct launch is the default.
    graphs = []
    if args.graph:
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        for i in range(n_inputs):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                step(i)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(warmup):
            flush()
            graphs[i % n_inputs].replay()
        torch.cuda.synchronize()
        log("bench: %d step graphs captured" % n_inputs)

    run = (lambda i: graphs[i % n_inputs].replay()) if graphs else step

    # ---------------------------------------------------------------- timed steps
    # Every interval is one pair of events with a cache flush inside, right
    # before the work: [flush] alone, and [flush, stages 0..s] for every s
    # (MOE_STAGE masks; the last prefix is the whole step), interleaved on
    # each rotating input.  A flush-only interval carries the same event
    # overhead and flush as the others, so the differences are the work's
    # GPU time (each kernel starts right after its predecessor, as in a
    # serving loop) and stage s's duration is prefix s minus prefix s-1.
    def prefix_flags(s):
        f = 0
        for j in range(s + 1):
            f |= moe.MOE_STAGE(j)
        return f

    def ev_pair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    fev = [ev_pair() for _ in range(steps)]
    sev = [[ev_pair() for _ in range(n_stages)] for _ in range(steps)]
    rev = [ev_pair() for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fev[i][0].record(stream)
        flush()
        fev[i][1].record(stream)
        rev[i][0].record(stream)
        flush()
        run(i)
        rev[i][1].record(stream)
        for s in range(n_stages - 1):
            sev[i][s][0].record(stream)
            flush()
            step(i, prefix_flags(s))
            sev[i][s][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    f_ms = np.array([a.elapsed_time(b) for a, b in fev])
    flush_ms = float(f_ms.mean())
    step_ms = np.array([a.elapsed_time(b) for a, b in rev]) - f_ms
    ms = float(step_ms.mean())
    per = np.array([[sev[i][s][0].elapsed_time(sev[i][s][1]) for s in range(n_stages - 1)]
                    + [step_ms[i] + f_ms[i]] for i in range(steps)]) - f_ms[:, None]
    prefix_ms = per.mean(0)
    stage_ms = np.diff(np.concatenate([[0.0], prefix_ms]))
    # standard error of each stage's mean (per-step differences of prefixes):
    # a stage much shorter than the step's own spread is not resolved
    stage_se = np.diff(np.concatenate([np.zeros((steps, 1)), per], 1), axis=1).std(0) / np.sqrt(steps)
    log("bench: step and per-stage timing done (%d steps, %.1f us of flush subtracted per interval)" %
        (steps, flush_ms * 1e3))

    # algorithmic work.  Weight bytes: each unique routed expert of the batch
    # and the shared expert once (codes + fp32 row scales); router weights
    # counted apart.
    gate_up_bytes = 2 * (wl.gate_bytes + 4 * wl.inter)
    down_bytes = wl.down_bytes + 4 * wl.hidden
    n_exp = float(np.mean(union_sizes)) + wl.n_shared
    layer_bytes = n_exp * (gate_up_bytes + down_bytes)
    router_bytes = 4 * wl.n_experts * wl.hidden
    rows = T * (wl.top_k + wl.n_shared)            # (token, expert) pairs, no padding
    tok_s = T / (ms * 1e-3)
    names = [s[0] for s in stages]
    # per stage: (bound, algorithmic amount per launch, peak, unit)
    if grouped:
        work = [("alu", 2.0 * T * wl.n_experts * wl.hidden / 1e12, FP64_PEAK_TFLOPS, "TFLOP/s"),
                None, None, None,
                ("mfma", 2.0 * rows * 2 * wl.inter * wl.hidden / 1e12, MFMA_I8_PEAK_TOPS, "TOP/s"),
                ("mfma", 2.0 * rows * wl.hidden * wl.inter / 1e12, MFMA_I8_PEAK_TOPS, "TOP/s"),
                ("hbm", (rows + T) * wl.hidden * 4 / 1e9, HBM_PEAK_GBS, "GB/s")]
    else:
        by_name = {"router+quant": ("hbm", router_bytes / 1e9, HBM_PEAK_GBS, "GB/s"),
                   "gate_up_swiglu_quant": ("hbm", n_exp * gate_up_bytes / 1e9, HBM_PEAK_GBS, "GB/s"),
                   "down_combine": ("hbm", n_exp * down_bytes / 1e9, HBM_PEAK_GBS, "GB/s")}
        work = [by_name.get(n) for n in names]
    dom = int(np.argmax(stage_ms))
    bound, amount, peak, unit = work[dom] if work[dom] else ("hbm", None, HBM_PEAK_GBS, "GB/s")
    achieved = amount / (stage_ms[dom] * 1e-3) if amount else None
    # counters are taken on the plain selection; a top-p run reads fewer bytes
    traffic = None if wl.top_p else traffic_from_profiles(wl.name, names[dom])
    log("bench: step %.2f us (p10 %.2f p90 %.2f%s), %.0f tok/s, weights %.0f GB/s = %.1f%% of HBM peak" %
        (ms * 1e3, np.percentile(step_ms, 10) * 1e3, np.percentile(step_ms, 90) * 1e3,
         ", graph" if graphs else "", tok_s,
         layer_bytes / (ms * 1e-3) / 1e9, 100 * layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS))
    log("bench: stages (us): %s" % ", ".join("%s %.2f" % (n, v * 1e3) for n, v in zip(names, stage_ms)))

    # ---------------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, wl, host, xs, n_inputs)

    out = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic (seeded SplitMix64 weights and N(0,1) tokens, %d rotating inputs%s)" %
                (n_inputs, "" if args.no_flush else ", caches flushed between steps"),
        "config": {"workload": wl.name + ("_topp%g" % wl.top_p if wl.top_p else "") +
                               ("_T%d" % T if args.tokens is not None else ""), "T": T,
                   "top_p": wl.top_p, "hidden": wl.hidden, "inter": wl.inter,
                   "n_experts": wl.n_experts, "n_group": wl.n_group, "topk_group": wl.topk_group,
                   "top_k": wl.top_k, "n_shared": wl.n_shared, "wbits": wl.wbits, "rsf": wl.rsf,
                   "path": "grouped" if grouped else "gemv", "graph": bool(graphs)},
        "effective_weight_GBps": layer_bytes / (ms * 1e-3) / 1e9,
        "effective_weight_frac": layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "roofline": {"bound": bound, "kernel": names[dom], "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak if achieved else None, "traffic": traffic,
                     "algorithmic_per_launch": amount, "avg_launch_us": float(stage_ms[dom] * 1e3)},
        "detail": {"stage_us": {n: float(v * 1e3) for n, v in zip(names, stage_ms)},
                   "stage_us_stderr": {n: float(v * 1e3) for n, v in zip(names, stage_se)},
                   "stage_roofline_frac": {n: (w[1] / (v * 1e-3) / w[2] if w else None)
                                           for n, v, w in zip(names, stage_ms, work)},
                   "step_us_p10_p50_p90": [float(np.percentile(step_ms, p) * 1e3) for p in (10, 50, 90)],
                   "flush_us": flush_ms * 1e3,
                   "mean_experts_read": n_exp, "layer_weight_bytes": layer_bytes,
                   "router_weight_bytes": router_bytes, "wall_s_timed_loop_incl_flush": wall},
        "cpu_baseline": cpu,
    }
    default_run = (wl.name == "decode_int4" and args.tokens is None and not args.top_p and not args.graph
                   and not args.no_flush)
    if default_run and not args.no_secondary:
        del routed, shared, xs, flush_buf, ws, rws
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        out["secondary"] = run_secondary()
    print(json.dumps(out), flush=True)


def bench_stack(args, wl):
    """One token through the whole decode stack per step (graph replay of one
    moe_stack_forward call); per-kernel figures from single layers."""
    import numpy as np
    import torch
    import synth
    from quantized_moe_noaux_amd import moe

    dev = "cuda:0"
    eps = 1e-6
    n_inputs = 64
    steps = args.steps if args.steps is not None else 20
    warmup = args.warmup if args.warmup is not None else 3
    sh = moe.shape_of(wl)
    log("bench: %s, %d layers, H=%d I=%d E=%d k=%d int%d; generating the layers in HBM" %
        (wl.name, wl.layers, wl.hidden, wl.inter, wl.n_experts, wl.top_k, wl.wbits))
    hosts, layers = synth.device_stack(wl, dev)
    arr = moe.layers(layers)
    la = moe.MOE_LOOKAHEAD(args.lookahead)
    ws = moe.workspace(moe.moe_stack_workspace_bytes(sh, 1, la), dev)
    xs = torch.stack([torch.from_numpy(synth.host_normals(wl.seed + i, synth.stream_id(0, synth.X), wl.hidden, 1.0)
                                       .reshape(1, wl.hidden)) for i in range(n_inputs)]).to(dev)
    x = torch.empty((1, wl.hidden), dtype=torch.float32, device=dev)
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def flush():
        if not args.no_flush:
            flush_buf.sum()

    # the step: the token's residual stream through every layer, as one
    # captured graph (or, with --stack-eager, launched directly)
    graph = None
    if not args.stack_eager:
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            moe.moe_stack_forward(sh, x, arr, eps, ws, flags=la)
        torch.cuda.synchronize()

    def step(i):
        x.copy_(xs[i % n_inputs])
        if graph is not None:
            graph.replay()
        else:
            moe.moe_stack_forward(sh, x, arr, eps, ws, flags=la)

    for i in range(warmup):
        flush()
        step(i)
    torch.cuda.synchronize()
    log("bench: %s, %d warmup steps done" % ("graph captured" if graph is not None else "direct launch", warmup))
    # timed as the layer benchmark does: one pair of events per interval,
    # each with a flush right before the work, minus an interleaved
    # flush-only interval
    def ev_pair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def prefix_flags(s):
        f = 0
        for j in range(s + 1):
            f |= moe.MOE_STAGE(j)
        return f

    fev = [ev_pair() for _ in range(steps)]
    rev = [ev_pair() for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fev[i][0].record(stream)
        flush()
        fev[i][1].record(stream)
        rev[i][0].record(stream)
        flush()
        step(i)
        rev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = np.array([a.elapsed_time(b) for a, b in rev]) - np.array([a.elapsed_time(b) for a, b in fev])
    ms = float(step_ms.mean())

    # per kernel: one layer (layer i % L) of the stack at a time; stage s's
    # duration is the time of stages 0..s minus that of stages 0..s-1
    n_stages = moe.moe_layer_stage_count(sh, 1)
    names = [s_[0] for s_ in stack_stages(gemv_stages(n_stages))]
    one = [moe.layers([L]) for L in layers]
    xt = xs[0].clone()
    reps = 4 * wl.layers
    fev = [ev_pair() for _ in range(reps)]
    sev = [[ev_pair() for _ in range(n_stages)] for _ in range(reps)]
    for i in range(reps):
        fev[i][0].record(stream)
        flush()
        fev[i][1].record(stream)
        for s_ in range(n_stages):
            sev[i][s_][0].record(stream)
            flush()
            moe.moe_stack_forward(sh, xt, one[i % wl.layers], eps, ws, flags=prefix_flags(s_))
            sev[i][s_][1].record(stream)
    torch.cuda.synchronize()
    flush_ms = float(np.mean([a.elapsed_time(b) for a, b in fev]))
    prefix_ms = np.array([np.mean([sev[i][s_][0].elapsed_time(sev[i][s_][1]) for i in range(reps)])
                          for s_ in range(n_stages)]) - flush_ms
    stage_ms = np.diff(np.concatenate([[0.0], prefix_ms]))
    log("bench: per-kernel pass done (%d layers per stage prefix, flush %.1f us subtracted)" % (reps, flush_ms * 1e3))

    n_exp = wl.top_k + wl.n_shared
    gate_up_bytes = 2 * (wl.gate_bytes + 4 * wl.inter)
    down_bytes = wl.down_bytes + 4 * wl.hidden
    token_bytes = wl.layers * n_exp * (gate_up_bytes + down_bytes)
    router_bytes = wl.layers * 4 * wl.n_experts * wl.hidden
    by_name = {"rmsnorm+router+quant": ("hbm", 4 * wl.n_experts * wl.hidden / 1e9),
               "gate_up_swiglu_quant": ("hbm", n_exp * gate_up_bytes / 1e9),
               "down_combine": ("hbm", n_exp * down_bytes / 1e9)}
    work = [by_name.get(n) for n in names]
    cand = [j for j in range(len(names)) if work[j]]
    dom = max(cand, key=lambda j: stage_ms[j])
    amount = work[dom][1]
    achieved = amount / (stage_ms[dom] * 1e-3)
    tok_s = 1.0 / (ms * 1e-3)
    log("bench: step %.1f us per token (%.2f us per layer), %.1f tok/s, weights %.0f GB/s = %.1f%% of HBM peak" %
        (ms * 1e3, ms * 1e3 / wl.layers, tok_s, token_bytes / (ms * 1e-3) / 1e9,
         100 * token_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS))
    log("bench: per layer (us): %s" % ", ".join("%s %.2f" % (n, v * 1e3) for n, v in zip(names, stage_ms)))

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        osh = oracle.shape_of(wl)
        ones = np.ones(wl.hidden, np.float32)
        spent, tokens, t_start = 0.0, 0, time.perf_counter()
        while spent < args.cpu_seconds and time.perf_counter() - t_start < 4 * args.cpu_seconds:
            xh = xs[tokens % n_inputs].cpu().numpy()
            for H in hosts:
                nh = oracle.rmsnorm(xh, ones, eps)
                ridx, _ = oracle.route(osh, nh, H.gate_w, H.bias)
                experts = oracle.layer_experts(H, ridx)      # generated outside the timing
                c0 = time.perf_counter()
                nh = oracle.rmsnorm(xh, ones, eps)
                yh, _, _ = oracle.layer_forward(osh, nh, H.gate_w, H.bias, experts, H.shared)
                xh = (xh + yh).astype(np.float32)
                spent += time.perf_counter() - c0
                H._experts = {}
            tokens += 1
        cpu = {"value": tokens / spent, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": "%d tokens through all %d layers (RMSNorm, layer forward, residual add), expert "
                         "generation excluded" % (tokens, wl.layers), "seconds": round(spent, 2)}
        cpu.update(host_info())
        log("bench: oracle %.3f tok/s on %d threads (%d tokens, %.1f s)" % (cpu["value"], cpu["cores"], tokens, spent))

    out = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic (seeded SplitMix64 weights for %d layers and N(0,1) tokens, %d rotating inputs%s)" %
                (wl.layers, n_inputs, "" if args.no_flush else ", caches flushed between steps"),
        "config": {"workload": wl.name, "T": 1, "layers": wl.layers, "hidden": wl.hidden, "inter": wl.inter,
                   "n_experts": wl.n_experts, "n_group": wl.n_group, "topk_group": wl.topk_group,
                   "top_k": wl.top_k, "n_shared": wl.n_shared, "wbits": wl.wbits, "rsf": wl.rsf,
                   "path": "gemv", "graph": graph is not None, "lookahead_wgs": args.lookahead},
        "effective_weight_GBps": token_bytes / (ms * 1e-3) / 1e9,
        "effective_weight_frac": token_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm", "kernel": names[dom], "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_from_profiles(wl.name, names[dom]),
                     "algorithmic_per_launch": amount, "avg_launch_us": float(stage_ms[dom] * 1e3)},
        "detail": {"per_layer_us": {n: float(v * 1e3) for n, v in zip(names, stage_ms)},
                   "step_us_p10_p50_p90": [float(np.percentile(step_ms, p) * 1e3)
                                                           for p in (10, 50, 90)],
                   "token_weight_bytes": token_bytes, "router_weight_bytes": router_bytes,
                   "wall_s_timed_loop_incl_flush": wall},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


MTP_VOCAB = 320000   # the order of the pages' 320k-merge BPE vocabulary


def bench_mtp(args):
    """One MTP verify step per timed step: the int4 decode layer at T = 1 + D
    (batch-union GEMV path) and the acceptance step over D+1 target and D
    draft logit rows of the vocabulary (moe_mtp_accept), beside the same layer
    at T = 1 for plain decode.  Tokens per step are the kernel's own kept
    drafts + 1 on the synthetic verify inputs (draft logits = target + noise,
    tuned into the pages' 39-59% per-draft acceptance)."""
    import numpy as np
    import torch
    import synth
    from quantized_moe_noaux_amd import moe

    dev = "cuda:0"
    D, V, tau = args.draft, MTP_VOCAB, args.temp
    T = 1 + D
    wl = synth.workload("decode_int4", T=T)
    wl1 = synth.workload("decode_int4")
    n_inputs = 16
    steps = args.steps if args.steps is not None else 100
    warmup = args.warmup if args.warmup is not None else 10
    sh, sh1 = moe.shape_of(wl), moe.shape_of(wl1)
    flags = moe.MOE_PATH_GEMV
    log("bench: mtp_int4 verify T=%d (D=%d drafts) + acceptance over V=%d, tau=%g" % (T, D, V, tau))
    host = synth.HostLayer(wl)
    gate_w = torch.from_numpy(host.gate_w).to(dev)
    bias = torch.from_numpy(host.bias).to(dev)
    routed = synth.device_weights(wl, 0, 0, wl.n_experts, dev)
    shared = synth.device_weights(wl, 0, wl.n_experts, 1, dev)
    xs = torch.stack([torch.from_numpy(
        synth.host_normals(wl.seed + i, synth.stream_id(0, synth.X), T * wl.hidden, 1.0).reshape(T, wl.hidden))
        for i in range(n_inputs)]).to(dev)
    mi = [synth.mtp_inputs(1000 + i, 1, D, V, tau) for i in range(n_inputs)]
    to = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to(dev)
    drafts = [to(a[0], np.int32) for a in mi]
    pls = [to(a[1], np.float32) for a in mi]
    qls = [to(a[2], np.float32) for a in mi]
    us = [to(a[3], np.float64) for a in mi]
    y = torch.empty((T, wl.hidden), dtype=torch.float32, device=dev)
    ws = moe.workspace(moe.moe_workspace_bytes(sh, T, flags), dev)
    ws1 = moe.workspace(moe.moe_workspace_bytes(sh1, 1, flags), dev)
    aws = moe.workspace(moe.moe_mtp_accept_workspace_bytes(1, D, V), dev)
    n_acc = torch.empty((n_inputs,), dtype=torch.int32, device=dev)
    nxt = torch.empty((n_inputs,), dtype=torch.int32, device=dev)
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def flush():
        flush_buf.sum()

    def layer(i):
        moe.moe_layer_forward(sh, xs[i % n_inputs], gate_w, bias, routed, shared, y, ws, flags=flags)

    def accept(i):
        k = i % n_inputs
        moe.moe_mtp_accept(drafts[k], pls[k], qls[k], tau, us[k], n_acc[k:k + 1], nxt[k:k + 1], aws)

    def decode(i):
        moe.moe_layer_forward(sh1, xs[i % n_inputs][:1], gate_w, bias, routed, shared, y[:1], ws1, flags=flags)

    for i in range(warmup):
        flush(); layer(i); accept(i); flush(); decode(i)
    torch.cuda.synchronize()
    ev = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    E = [[ev() for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        for k, work in enumerate((lambda: None, lambda: decode(i), lambda: layer(i),
                                  lambda: (layer(i), accept(i)))):
            E[i][k][0].record(stream)
            flush()
            work()
            E[i][k][1].record(stream)
    torch.cuda.synchronize()
    t = np.array([[a.elapsed_time(b) for a, b in row] for row in E])  # ms
    t = t[:, 1:] - t[:, :1]
    dec_ms, lay_ms, ver_ms = (float(v) for v in t.mean(0))
    acc_ms = ver_ms - lay_ms
    na = n_acc.cpu().numpy()
    tok_step = float(np.mean(na + 1))
    per_draft = float(sum((na > j).sum() for j in range(D)) / max(1, sum((na >= j).sum() for j in range(D))))
    value = tok_step / (ver_ms * 1e-3)
    dec_tok_s = 1.0 / (dec_ms * 1e-3)
    log("bench: decode layer %.2f us; verify layer (T=%d) %.2f us + acceptance %.2f us = %.2f us" %
        (dec_ms * 1e3, T, lay_ms * 1e3, acc_ms * 1e3, ver_ms * 1e3))
    log("bench: %.2f tokens per verify step (%.0f%% of drafts kept): %.0f tok/s vs %.0f tok/s plain decode" %
        (tok_step, 100 * per_draft, value, dec_tok_s))
    # acceptance step: logit bytes read once by the stats pass (the draw pass
    # rereads two rows); the layer's weights as in the decode line
    acc_bytes = 4.0 * V * (2 * D + 1)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0) or reps == 0:
            a = mi[reps % n_inputs]
            oracle.mtp_accept(a[0], a[1], a[2], tau, a[3])
            reps += 1
        el = time.perf_counter() - t0
        cpu = {"value": reps / el, "unit": "acceptance steps/s (oracle, one sequence, V=%d)" % V,
               "cores": oracle.lib().oracle_num_threads(), "kind": "oracle",
               "sample": "%d acceptance steps of the rotating inputs; the verify layer itself is in the "
                         "decode_int4 line's baseline" % reps}
        cpu.update(host_info())
    out = {
        "metric": "MTP verify tokens/s (one int4 MoE layer + acceptance, synthetic drafts)",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ver_ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8+f64", "data": "synthetic (seeded layer weights, N(0,1) tokens, target logits N(0,9), "
                                   "draft logits = target + N(0,1), %d rotating inputs, caches flushed)" % n_inputs,
        "config": {"workload": "mtp_int4", "T": T, "drafts": D, "vocab": V, "temperature": tau,
                   "hidden": wl.hidden, "inter": wl.inter, "n_experts": wl.n_experts, "top_k": wl.top_k,
                   "wbits": wl.wbits, "path": "gemv"},
        "roofline": {"bound": "hbm", "kernel": "mtp_accept", "achieved": acc_bytes / (acc_ms * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": acc_bytes / (acc_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_per_launch": acc_bytes / 1e9, "avg_launch_us": acc_ms * 1e3},
        "detail": {"tokens_per_step": tok_step, "draft_acceptance": per_draft,
                   "verify_layer_us": lay_ms * 1e3, "acceptance_us": acc_ms * 1e3,
                   "decode_layer_us": dec_ms * 1e3, "decode_tokens_per_s": dec_tok_s},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_tier(args):
    """Decode through the HBM / host expert tier: the int4 decode layer with
    every routed expert in pinned host memory and --slots of them in HBM,
    the live repin every --repin tokens inside the timed loop.  The router
    bias is the skewed N(0, 0.5) of the prefill workload, so that some
    experts are hotter than others.  A step is one token; the timed loop is
    back to back (no cache flush: the misses' host reads dominate), its time
    covers the layer and the repins (whose count read-back synchronises).
    The hit rate is measured afterwards over the same number of tokens with
    the resident set the timed loop left."""
    import numpy as np
    import torch
    import synth
    from quantized_moe_noaux_amd import moe

    dev = "cuda:0"
    wl = synth.workload("decode_int4", bias_sigma=math.sqrt(0.5))
    C, R = args.slots, args.repin
    n_inputs = 64
    steps = args.steps if args.steps is not None else 256
    warmup = args.warmup if args.warmup is not None else 64
    sh = moe.shape_of(wl)
    flags = moe.MOE_PATH_GEMV
    log("bench: tier_int4 decode, %d of %d routed experts in HBM, repin every %d tokens" % (C, wl.n_experts, R))
    host = synth.HostLayer(wl)
    gate_w = torch.from_numpy(host.gate_w).to(dev)
    bias = torch.from_numpy(host.bias).to(dev)
    routed = synth.device_weights(wl, 0, 0, wl.n_experts, dev)
    shared = synth.device_weights(wl, 0, wl.n_experts, 1, dev)
    pinned = []
    for f in ("gate", "up", "down", "gate_s", "up_s", "down_s"):
        d = getattr(routed, f)
        h = torch.empty(d.shape, dtype=d.dtype, pin_memory=True)
        h.copy_(d)
        pinned.append(h)
    hostw = synth.DeviceWeights(*pinned)
    tier = moe.Tier(sh, hostw, C)
    xs = torch.stack([torch.from_numpy(
        synth.host_normals(wl.seed + i, synth.stream_id(0, synth.X), wl.hidden, 1.0).reshape(1, wl.hidden))
        for i in range(n_inputs)]).to(dev)
    y = torch.empty((1, wl.hidden), dtype=torch.float32, device=dev)
    idx = torch.empty((1, wl.top_k), dtype=torch.int32, device=dev)
    wts = torch.empty((1, wl.top_k), dtype=torch.float32, device=dev)
    ws = moe.workspace(moe.moe_workspace_bytes(sh, 1, flags), dev)
    torch.cuda.synchronize()
    log("bench: pinned host copy of the routed experts ready (%.2f GB)" % (wl.n_experts * wl.expert_bytes / 1e9))

    def step(i):
        moe.moe_layer_forward_tiered(sh, xs[i % n_inputs], gate_w, bias, tier, shared, y, ws, idx, wts)

    def resident_step(i):
        moe.moe_layer_forward(sh, xs[i % n_inputs], gate_w, bias, routed, shared, y, ws, idx, wts, flags=flags)

    copied = 0
    for i in range(warmup):
        step(i)
        if (i + 1) % R == 0:
            copied += tier.repin()
    torch.cuda.synchronize()
    log("bench: %d warmup tokens, %d experts copied into HBM" % (warmup, copied))
    copied = 0
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i)
        if (i + 1) % R == 0:
            copied += tier.repin()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    # the same layer with every expert in HBM, timed the same way
    for i in range(warmup):
        resident_step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        resident_step(warmup + i)
    torch.cuda.synchronize()
    ms_res = (time.perf_counter() - t0) * 1e3 / steps
    # hit rate with the resident set the timed loop left (no repin)
    slot_of = tier.resident()
    hits = sel = 0
    for i in range(steps):
        step(warmup + steps + i)
        e = idx.cpu().numpy().ravel()
        e = e[e >= 0]
        sel += len(e)
        hits += sum(slot_of[k] >= 0 for k in e)
    hit = hits / max(sel, 1)
    tier.close()
    value = 1e3 / ms
    weight_bytes = (wl.top_k + 1) * wl.expert_bytes
    miss_bytes = wl.top_k * (1.0 - hit) * wl.expert_bytes
    log("bench: step %.1f us (%.0f tok/s), hit rate %.1f%%, %.1f experts copied per repin; "
        "all experts in HBM: %.1f us" % (ms * 1e3, value, 100 * hit, copied / max(1, steps // R), ms_res * 1e3))
    out = {
        "metric": "MoE-layer tokens/s, int4 decode through the HBM / host expert tier",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8", "data": "synthetic (seeded SplitMix64 weights, router bias N(0,0.5), N(0,1) tokens, "
                               "%d rotating inputs, no cache flush)" % n_inputs,
        "config": {"workload": "tier_int4", "T": 1, "hbm_slots": C, "repin_every": R, "hidden": wl.hidden,
                   "inter": wl.inter, "n_experts": wl.n_experts, "top_k": wl.top_k, "n_shared": wl.n_shared,
                   "wbits": wl.wbits, "path": "gemv"},
        "roofline": {"bound": "hbm", "kernel": "layer", "achieved": weight_bytes / (ms * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": weight_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_per_launch": weight_bytes / 1e9, "avg_launch_us": ms * 1e3},
        "detail": {"hit_rate": hit, "host_bytes_per_token": miss_bytes,
                   "host_read_GBps": miss_bytes / (ms * 1e-3) / 1e9, "experts_copied_timed": copied,
                   "resident_step_us": ms_res * 1e3},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def bench_tier_stack(args):
    """Decode through a stack of --layers int4 layers, each with its routed
    experts in pinned host memory and --slots of them in HBM (one tier per
    layer, the live repin every --repin tokens), x <- x + MoE_l(RMSNorm(x)),
    once without and once with the router lookahead: before layer l runs,
    layer l+1's router is applied to RMSNorm(x_l) on a side stream, its
    experts are read back and prefetched into layer l+1's tier on that
    stream, and layer l+1 waits for the prefetch (--lookahead-ranks N: only
    the first N ranks of each prediction are prefetched).  The router bias is the
    decode workload's N(0, 0.01), so no small hot set exists.  Each mode
    runs --warmup tokens, then --steps timed tokens (a step is one token
    through every layer, repins included)."""
    import numpy as np
    import torch
    import synth
    from quantized_moe_noaux_amd import moe

    dev = "cuda:0"
    Ln, C, R = args.layers, args.slots, args.repin
    steps = args.steps if args.steps is not None else 16
    warmup = args.warmup if args.warmup is not None else 16
    wl = synth.workload("decode_int4", layers=Ln)
    sh = moe.shape_of(wl)
    log("bench: tier_stack_int4, %d layers, %d of %d routed experts in HBM per layer, repin every %d tokens" %
        (Ln, C, wl.n_experts, R))
    layers = []
    for l in range(Ln):
        host = synth.HostLayer(wl, layer=l, T=1)
        routed = synth.device_weights(wl, l, 0, wl.n_experts, dev)
        pinned = []
        for f in ("gate", "up", "down", "gate_s", "up_s", "down_s"):
            d = getattr(routed, f)
            h = torch.empty(d.shape, dtype=d.dtype, pin_memory=True)
            h.copy_(d)
            pinned.append(h)
        del routed
        torch.cuda.synchronize()
        layers.append(dict(gate_w=torch.from_numpy(host.gate_w).to(dev), bias=torch.from_numpy(host.bias).to(dev),
                           g=torch.ones(wl.hidden, dtype=torch.float32, device=dev),
                           shared=synth.device_weights(wl, l, wl.n_experts, 1, dev),
                           host=synth.DeviceWeights(*pinned)))
        torch.cuda.empty_cache()
    log("bench: %d layers' routed experts in pinned host memory (%.1f GB)" %
        (Ln, Ln * wl.n_experts * wl.expert_bytes / 1e9))
    n_inputs = 64
    xs = torch.stack([torch.from_numpy(
        synth.host_normals(wl.seed + i, synth.stream_id(0, synth.X), wl.hidden, 1.0).reshape(1, wl.hidden))
        for i in range(n_inputs)]).to(dev)
    x0 = xs[0]
    x = torch.empty_like(x0)
    nrm = torch.empty_like(x0)
    lnrm = torch.empty_like(x0)
    idx = torch.empty((1, wl.top_k), dtype=torch.int32, device=dev)
    wts = torch.empty((1, wl.top_k), dtype=torch.float32, device=dev)
    pidx = torch.empty((1, wl.top_k), dtype=torch.int32, device=dev)
    pw = torch.empty((1, wl.top_k), dtype=torch.float32, device=dev)
    ws = moe.workspace(moe.moe_workspace_bytes(sh, 1, moe.MOE_PATH_GEMV), dev)
    rws = moe.workspace(moe.moe_route_workspace_bytes(sh, 1), dev)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()

    def run(lookahead, ntok, t0, record=None):
        tiers = [moe.Tier(sh, L["host"], C) for L in layers]
        evs = [torch.cuda.Event() for _ in range(Ln)]
        stats = {"pred": 0, "hit": 0, "sel": 0, "resident": 0, "copies": 0, "pre": 0, "pre_hit": 0}
        try:
            def token(t, measure):
                x.copy_(xs[t % n_inputs])   # rotating N(0, 1) tokens
                for l in range(Ln):
                    L = layers[l]
                    if lookahead and l + 1 < Ln:
                        side.wait_stream(main)
                        with torch.cuda.stream(side):
                            N = layers[l + 1]
                            moe.moe_rmsnorm(x, N["g"], 1e-6, lnrm, stream=side)
                            moe.moe_route(sh, lnrm, N["gate_w"], N["bias"], pidx, pw, rws, stream=side)
                            ids = pidx.cpu().numpy().ravel()       # read back on the side stream, after the route
                        pre = ids if args.lookahead_ranks is None else ids[:args.lookahead_ranks]
                        stats["copies"] += tiers[l + 1].prefetch(pre, stream=side)
                        evs[l + 1].record(side)
                    if lookahead and l > 0:
                        main.wait_event(evs[l])
                    moe.moe_rmsnorm(x, L["g"], 1e-6, nrm)
                    res = tiers[l].resident() if measure else None
                    moe.moe_layer_forward_tiered(sh, nrm, L["gate_w"], L["bias"], tiers[l], L["shared"], x, ws,
                                                 idx, wts, flags=moe.MOE_ACCUMULATE)
                    if measure:
                        sel = idx.cpu().numpy().ravel()
                        stats["sel"] += len(sel)
                        stats["resident"] += sum(res[e] != -1 for e in sel)
                        if lookahead and l > 0:
                            stats["pred"] += len(sel)
                            stats["hit"] += len(set(sel.tolist()) & set(prev_pred[l].tolist()))
                            stats["pre"] += len(prev_pre[l])
                            stats["pre_hit"] += len(set(sel.tolist()) & set(prev_pre[l].tolist()))
                    if lookahead and l + 1 < Ln and measure:
                        prev_pred[l + 1] = ids
                        prev_pre[l + 1] = pre
                if (t + 1) % R == 0:
                    for tr in tiers:
                        stats["copies"] += tr.repin()
            prev_pred, prev_pre = {}, {}
            for t in range(t0, t0 + warmup):
                token(t, False)
            torch.cuda.synchronize()
            stats["copies"] = 0
            tic = time.perf_counter()
            for t in range(t0 + warmup, t0 + warmup + ntok):
                token(t, False)
            torch.cuda.synchronize()
            ms = (time.perf_counter() - tic) * 1e3 / ntok
            copies = stats["copies"]
            for t in range(t0 + warmup + ntok, t0 + warmup + 2 * ntok):
                token(t, True)
            torch.cuda.synchronize()
            return ms, copies, stats
        finally:
            for tr in tiers:
                tr.close()

    ms0, cp0, st0 = run(False, steps, 0)
    log("bench: no lookahead: %.2f ms per token, hits %.1f%%, %d experts copied" %
        (ms0, 100 * st0["resident"] / max(1, st0["sel"]), cp0))
    ms1, cp1, st1 = run(True, steps, 0)
    recall = st1["hit"] / max(1, st1["pred"])
    log("bench: lookahead: %.2f ms per token, hits %.1f%%, lookahead recall %.1f%%, %d experts copied "
        "(prefetched ranks: %s, %.1f%% of them used)" %
        (ms1, 100 * st1["resident"] / max(1, st1["sel"]), 100 * recall, cp1,
         "all" if args.lookahead_ranks is None else "first %d" % args.lookahead_ranks,
         100 * st1["pre_hit"] / max(1, st1["pre"])))
    value = 1e3 / ms1
    weight_bytes = Ln * (wl.top_k + 1) * wl.expert_bytes
    out = {
        "metric": "decode tokens/s, %d-layer int4 stack through the HBM / host expert tier with router lookahead" % Ln,
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms1, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8", "data": "synthetic (seeded SplitMix64 weights, router bias N(0,0.01), %d rotating "
                               "N(0,1) tokens, one token a step)" % n_inputs,
        "config": {"workload": "tier_stack_int4", "layers": Ln, "T": 1, "hbm_slots": C, "prefetch_slots": 16,
                   "repin_every": R, "hidden": wl.hidden, "inter": wl.inter, "n_experts": wl.n_experts,
                   "top_k": wl.top_k, "wbits": wl.wbits, "path": "gemv"},
        "roofline": {"bound": "hbm", "kernel": "stack", "achieved": weight_bytes / (ms1 * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": weight_bytes / (ms1 * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_per_launch": weight_bytes / 1e9, "avg_launch_us": ms1 * 1e3},
        "detail": {"no_lookahead_ms": ms0, "lookahead_ms": ms1, "lookahead_recall": recall,
                   "hit_rate_no_lookahead": st0["resident"] / max(1, st0["sel"]),
                   "hit_rate_lookahead": st1["resident"] / max(1, st1["sel"]),
                   "copies_timed_no_lookahead": cp0, "copies_timed_lookahead": cp1},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def host_info():
    """The host the oracle ran on: CPU model, the CPUs this process may use,
    and the OpenMP thread setting it inherited."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count()
    return {"cpu_model": model, "nproc": nproc, "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline(args, wl, host, xs, n_inputs):
    """The oracle, as it stands, on a bounded sample of the same inputs:
    whole inputs for decode / verify (cycled until the time budget is spent),
    groups of 4 tokens of the first input for prefill (every token's output
    depends only on its own row).  Expert generation is excluded.  For the
    small batches (decode, verify) a second, shorter sample runs the oracle
    on one thread."""
    import oracle
    osh = oracle.shape_of(wl)
    per = 4 if wl.T > 64 else wl.T

    def sample(budget, first=0):
        done, spent, tokens = 0, 0.0, 0
        t_start = time.perf_counter()
        while done == 0 or (spent < budget and time.perf_counter() - t_start < 4 * budget):
            j = first + done
            if wl.T > 64:
                x = xs[0, (j * per) % wl.T:(j * per) % wl.T + per].cpu().numpy()
            else:
                x = xs[j % n_inputs].cpu().numpy()
            ridx, _ = oracle.route(osh, x, host.gate_w, host.bias)
            experts = oracle.layer_experts(host, ridx)       # generated outside the timing
            c0 = time.perf_counter()
            oracle.layer_forward(osh, x, host.gate_w, host.bias, experts, host.shared)
            spent += time.perf_counter() - c0
            tokens += x.shape[0]
            done += 1
            host._experts = {k: v for k, v in host._experts.items() if k == wl.n_experts}
        return tokens, spent, done

    threads = oracle.num_threads()
    tokens, spent, done = sample(args.cpu_seconds)
    sample_desc = ("%d forwards of %d-token slices of one %d-token %s input" % (done, per, wl.T, wl.name)
                   if wl.T > 64 else
                   "%d forwards cycling the %d rotating %s inputs (T=%d each)" % (done, n_inputs, wl.name, wl.T))
    cpu = {"value": tokens / spent, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": sample_desc + ", full layer forward (router, experts, combine), expert generation excluded",
           "seconds": round(spent, 2)}
    cpu.update(host_info())
    log("bench: oracle %.3f tok/s on %d threads (%d forwards, %.1f s)" % (cpu["value"], threads, done, spent))
    if wl.T <= 64:
        oracle.set_num_threads(1)
        try:
            t1, s1, d1 = sample(args.cpu_seconds / 3, first=done)
        finally:
            oracle.set_num_threads(threads)
        cpu["single_thread"] = {"value": t1 / s1, "unit": "tokens/s", "forwards": d1, "seconds": round(s1, 2)}
        log("bench: oracle %.3f tok/s on 1 thread (%d forwards, %.1f s)" % (t1 / s1, d1, s1))
    return cpu


if __name__ == "__main__":
    main()
