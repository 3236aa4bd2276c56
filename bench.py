"""Throughput of the MoE FFN layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill_fp8]
                    [--no-cpu-baseline] [--stages/--no-stages]

One step = one whole layer forward (route -> dispatch -> 1x128 FP8 quant -> grouped
GEMM1 + SwiGLU + requant -> grouped GEMM2 -> combine) through the C ABI call
moe_layer_fwd on seeded synthetic inputs already resident in HBM.  Prints one JSON
line.  `value` is the algorithmic FLOP rate of the layer (router + both expert GEMMs,
unpadded rows) in TFLOP/s; tokens/s is reported beside it.  The roofline entry is for
the dominant kernel (the grouped GEMM1), timed with HIP events on the launch stream.
The CPU baseline times the fp64 oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import synth  # noqa: E402

PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_BF16_TFLOPS = 2500.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def make_layer(w: synth.Workload, dev):
    import fp8_grouped_gemm_amd as M
    inp = synth.layer_inputs(w, device=dev)
    weights = {}
    if w.route == "score":
        weights["w_router"], weights["bias"] = inp["w_router"], inp["bias"]
    if w.mode == "fp8":
        # codes rearranged once, offline, into the layout the GEMM loads
        q, weights["s13"] = M.moe_quant_weight_fp8(inp["w13"])
        weights["w13"] = M.moe_pack_weight_fp8(q)
        q, weights["s2"] = M.moe_quant_weight_fp8(inp["w2"])
        weights["w2"] = M.moe_pack_weight_fp8(q)
        del q
    elif w.mode == "w4a16":
        weights["w13"], weights["s13"] = M.moe_quant_weight_int4(inp["w13"])
        weights["w2"], weights["s2"] = M.moe_quant_weight_int4(inp["w2"])
    else:
        weights["w13"], weights["w2"] = inp["w13"], inp["w2"]
    return inp, weights


def gemm_bytes_flops(w: synth.Workload, counts: np.ndarray):
    """Algorithmic work of the two expert GEMMs from the routed counts (unpadded rows):
    FLOPs 2*M*N*K each; bytes = weights (+ scales) of touched experts + activations in +
    outputs, each once."""
    R = int(counts.sum())
    touched = int(np.sum(counts > 0))
    d, I = w.d, w.I
    if w.mode == "fp8":
        wb13 = 2 * I * d + (2 * I // 128) * (d // 128) * 4
        wb2 = d * I + (d // 128) * (I // 128) * 4
        a1 = w.T * d + w.T * (d // 128) * 4               # token codes + scales
        h = R * I + R * (I // 128) * 4                     # requantised h
        o = R * d * 2                                      # bf16 expert rows
    elif w.mode == "w4a16":
        wb13 = 2 * I * d // 2 + 2 * I * (d // 128) * 4
        wb2 = d * I // 2 + d * (I // 128) * 4
        a1 = w.T * d * 2
        h = R * I * 2
        o = R * d * 2
    else:
        wb13, wb2 = 2 * I * d * 4, d * I * 4
        a1, h, o = w.T * d * 4, R * I * 4, R * d * 4
    f1 = 2.0 * R * (2 * I) * d
    f2 = 2.0 * R * d * I
    b1 = touched * wb13 + a1 + h
    b2 = touched * wb2 + h + o
    return {"gemm1_flops": f1, "gemm2_flops": f2, "gemm1_bytes": b1, "gemm2_bytes": b2,
            "rows": R, "touched": touched}


def layer_flops_bytes(w: synth.Workload, counts: np.ndarray):
    g = gemm_bytes_flops(w, counts)
    router = 2.0 * w.T * w.E * w.d if w.route == "score" else 0.0
    act = 4 if w.mode == "fp32" else 2
    touched_w = g["gemm1_bytes"] + g["gemm2_bytes"] - 2 * (g["rows"] * w.I) - \
        (g["rows"] * w.d * act)
    wr = w.E * w.d * act if w.route == "score" else 0
    total_bytes = touched_w + w.T * w.d * act * 2 + wr     # weights + x + y + router
    return router + g["gemm1_flops"] + g["gemm2_flops"], total_bytes, g


# ------------------------------------------------------------- CPU baseline

def cpu_baseline(w: synth.Workload, inp: dict, n_experts: int = 8):
    """Time the fp64 oracle on a bounded sample: routing + dispatch of the whole batch,
    then the expert FFN (dequantise, GEMM1, SwiGLU, requant, GEMM2) of the rows routed
    to ``n_experts`` experts.  Weight quantisation (offline) is outside the timer."""
    import oracle as O
    from oracle import codecs as OC
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    x = inp["x"].float().cpu().numpy()
    wr = inp["w_router"].float().cpu().numpy()
    b = inp["bias"].cpu().numpy()
    t0 = time.perf_counter()
    logits = O.router_logits(x, wr)
    idx, gw = O.topk_route(logits.astype(np.float32), b, w.k)
    counts, offsets, ros, sor = O.dispatch(idx, w.E, w.m_align)
    qx, sx = OC.quant_fp8_act(x)
    t_route = time.perf_counter() - t0
    order = np.argsort(-counts, kind="stable")
    experts = [int(e) for e in order[:n_experts // 2]] + \
              [int(e) for e in order[len(order) // 2:len(order) // 2 + n_experts - n_experts // 2]]
    flops = 2.0 * w.T * w.E * w.d
    t_exp = 0.0
    rows_done = 0
    for e in experts:
        w13 = inp["w13"][e:e + 1].cpu().numpy()
        w2 = inp["w2"][e:e + 1].cpu().numpy()
        q13, s13 = OC.quant_fp8_weight(w13)
        q2, s2 = OC.quant_fp8_weight(w2)
        rows = np.arange(offsets[e], offsets[e + 1])
        slots = sor[rows]
        slots = slots[slots >= 0]
        toks = slots // w.k
        t0 = time.perf_counter()
        a = OC.dequant_fp8_act(qx[toks], sx[toks])
        W13 = OC.dequant_fp8_weight(q13, s13)[0]
        W2 = OC.dequant_fp8_weight(q2, s2)[0]
        gu = a @ W13.T
        h = O.swiglu(gu[:, :w.I], gu[:, w.I:])
        qh, sh = OC.quant_fp8_act(h.astype(np.float32))
        _ = OC.dequant_fp8_act(qh, sh) @ W2.T
        t_exp += time.perf_counter() - t0
        rows_done += len(toks)
        flops += 2.0 * len(toks) * (2 * w.I * w.d + w.d * w.I)
    total = t_route + t_exp
    return {"value": flops / total / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"fp64 numpy oracle: routing+dispatch+token quant of all {w.T} tokens "
                       f"({t_route:.2f} s) + expert FFN of the {rows_done} rows routed to "
                       f"{len(experts)} experts ({t_exp:.2f} s); algorithmic FLOPs of that "
                       f"sample / wall time")}


# ---------------------------------------------------------------------- main

SETTLE_S = 1.5


def settle(fn, seconds):
    """Run fn() untimed for `seconds`: an idle GPU starts at a low engine clock and
    ramps up under load; timing from a cold start understates steady-state speed."""
    t_end = time.time() + seconds
    n = 0
    while time.time() < t_end:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed steps before the warm-up steps, so the engine "
                         "clock has left its idle state (it ramps up over tens of ms)")
    ap.add_argument("--workload", default="prefill_fp8",
                    choices=sorted(synth.WORKLOADS) + ["grouped_gemm_fp8", "dense_gemm_fp8",
                                                       "masked_gemm_fp8"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stages", action="store_true")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="print a per-kernel summary of a rocprofv3 --kernel-trace --stats "
                         "--output-format csv run written to DIR, then exit")
    ap.add_argument("--pmc-summary", metavar="DIR",
                    help="print per-kernel average counter values of a rocprofv3 --pmc "
                         "--output-format csv run written to DIR, then exit")
    a = ap.parse_args(argv)
    if a.trace_summary:
        print(trace_summary(a.trace_summary))
        return 0
    if a.pmc_summary:
        print(json.dumps(pmc_summary(a.pmc_summary), indent=1))
        return 0
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1 "
                                   "(multi-GPU expert parallelism is not built)"}))
        return 2

    import fp8_grouped_gemm_amd as M
    if a.workload == "grouped_gemm_fp8":
        print(json.dumps(bench_grouped_gemm(M, a.steps, a.warmup, a.settle)), flush=True)
        return 0
    if a.workload == "dense_gemm_fp8":
        print(json.dumps(bench_dense_gemm(M, a.steps, a.warmup, a.settle)), flush=True)
        return 0
    if a.workload == "masked_gemm_fp8":
        print(json.dumps(bench_masked_gemm(M, a.steps, a.warmup, a.settle)), flush=True)
        return 0
    w = synth.WORKLOADS[a.workload]
    if w.m_align != 16:
        w = synth.scaled(w, m_align=16)     # the kernels' row padding (output unaffected)
    dev = torch.device("cuda:0")
    log(f"workload {w}")
    t0 = time.time()
    inp, weights = make_layer(w, dev)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f} s")
    desc = M.LayerDesc(w.T, w.d, w.E, w.k, w.I, mode=w.mode, route=w.route, m_align=w.m_align)
    ws = torch.empty(M.moe_layer_workspace_size(desc), dtype=torch.uint8, device=dev)
    x = inp["x"]
    ids = inp.get("token_ids")
    y = torch.empty_like(x)
    counts = torch.empty(w.E, dtype=torch.int32, device=dev)

    def step():
        M.moe_layer_fwd(desc, weights, x, ids, workspace=ws, y=y, counts=counts)

    settle(step, a.settle)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(a.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / a.steps
    cnt = counts.cpu().numpy()
    flops, bytes_, g = layer_flops_bytes(w, cnt)
    log(f"layer {ms:.3f} ms/step; rows {g['rows']} touched experts {g['touched']}; "
        f"loads max {cnt.max()} median {int(np.median(cnt))} min {cnt.min()}")

    # per-stage times through the individual entry points (same kernels, same stream)
    stages = {}
    if not a.no_stages and w.mode == "fp8" and w.route == "score":
        stages = stage_times(M, w, inp, weights, a.steps)
    elif not a.no_stages and w.mode == "w4a16" and w.route == "hash":
        stages = stage_times_w4a16(M, w, inp, weights, a.steps)
    if stages:
        log("stages (ms): " + ", ".join(f"{k} {v:.3f}" for k, v in stages.items()))
    g1_ms = stages.get("gemm1")
    roofline = None
    traffic = measured_traffic("gemm1") if a.workload == "prefill_fp8" else None
    if g1_ms and w.mode == "w4a16":
        # int4 weights streamed once against T rows: ~430 FLOP/B, above the bf16 ridge
        # (2500 TFLOP/s / 8 TB/s = 312 FLOP/B), so the bound is the bf16 MFMA peak
        tf = g["gemm1_flops"] / (g1_ms * 1e-3) / 1e12
        roofline = {"kernel": "grouped_gemm_w4a16 (GEMM1: gate+up, SwiGLU)",
                    "bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                    "traffic": None, "avg_ms": round(g1_ms, 4),
                    "hbm_gbs": round(g["gemm1_bytes"] / (g1_ms * 1e-3) / 1e9, 1),
                    "flops_per_launch": g["gemm1_flops"]}
    elif g1_ms:
        achieved = g["gemm1_bytes"] / (g1_ms * 1e-3) / 1e9
        roofline = {"kernel": "grouped_gemm_fp8 (GEMM1: gate+up, SwiGLU, e4m3 requant)",
                    "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                    "traffic": traffic, "avg_ms": round(g1_ms, 4),
                    "tflops": round(g["gemm1_flops"] / (g1_ms * 1e-3) / 1e12, 1),
                    "bytes_per_launch": g["gemm1_bytes"]}
    out = {
        "metric": "MoE layer FP8 grouped-GEMM TFLOPS + tokens/s on 1 MI355X (% roofline)",
        "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "settle_s": a.settle,
        "ms_per_step": round(ms, 4),
        "tokens_per_s": round(w.T / (ms * 1e-3), 1),
        "layer_hbm_frac": round(bytes_ / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"fp8": "e4m3", "w4a16": "int4xbf16", "fp32": "f32"}[w.mode],
        "data": "synthetic",
        "config": {"workload": f"{w.name}: T={w.T} d={w.d} E={w.E} top-{w.k} I={w.I}",
                   "mode": w.mode, "route": w.route, "m_align": w.m_align,
                   "skew": f"+{w.skew_add} on {w.skew_frac:.0%} of experts" if w.skew_frac else None},
        "stages_ms": {k: round(v, 4) for k, v in stages.items()} or None,
        "roofline": roofline,
    }
    if not a.no_cpu_baseline and w.mode == "fp8" and w.route == "score":
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(out), flush=True)
    return 0


def measured_traffic(kernel):
    """HBM bytes per launch of a GEMM kernel from the committed rocprofv3 counter summary,
    or None when the kernel source changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemm_fp8_prefill_traffic.json")
    src = os.path.join(ROOT, "fp8_grouped_gemm_amd", "csrc", "gemm_fp8.hip")
    try:
        d = json.load(open(path))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256") != sha:
        return None
    return round(d[kernel]["hbm_bytes_per_launch"])


def _find(dirname, suffix):
    for root, _, files in os.walk(dirname):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {dirname}")


def trace_summary(dirname):
    """Per-kernel call count and average / total duration from rocprofv3's kernel
    stats csv (library kernels first)."""
    import csv
    rows = list(csv.DictReader(open(_find(dirname, "kernel_stats.csv"))))
    out = [f"{'kernel':<72} {'calls':>6} {'avg_us':>10} {'total_ms':>10} {'pct':>6}"]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    for r in rows:
        name = r["Name"]
        if len(name) > 70:
            name = name[:67] + "..."
        out.append(f"{name:<72} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} "
                   f"{float(r['TotalDurationNs']) / 1e6:>10.3f} {float(r['Percentage']):>6.2f}")
    return "\n".join(out)


def pmc_summary(dirname):
    """Average counter value per dispatch for every kernel in a --pmc csv run."""
    import csv
    import collections
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(_find(dirname, "counter_collection.csv"))):
        acc[r["Kernel_Name"][:90]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: {"dispatches": len(v), "avg": sum(v) / len(v)} for c, v in d.items()}
            for k, d in acc.items()}


def bench_grouped_gemm(M, steps, warmup, settle_s=SETTLE_S):
    """The standalone FP8 grouped GEMM: 16 groups with Zipf(1.1) sizes summing to 8192
    rows, each padded to 128; N=4096, K=7168; bf16 out.  A 512 MB write between timed
    launches (outside the events) evicts the weights from the last-level cache."""
    dev = torch.device("cuda:0")
    sizes = synth.zipf_group_sizes(8192, 16, 1.1, seed=0)
    N, K = 4096, 7168
    padded = -(-sizes // 128) * 128
    offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    R = int(offsets[-1])
    g = synth.gemm_inputs(sizes, N, K, seed=0, device=dev)
    dest = np.concatenate([np.arange(offsets[i], offsets[i] + sizes[i]) for i in range(16)])
    a = torch.zeros((R, K), dtype=torch.float32, device=dev)
    a[torch.from_numpy(dest).to(dev)] = g["a"]
    qa, sa = M.moe_quant_fp8(a)
    qb, sb = M.moe_quant_weight_fp8(g["b"])
    qb = M.moe_pack_weight_fp8(qb)
    off = torch.from_numpy(offsets).to(dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    settle(lambda: M.grouped_gemm_fp8(qa, sa, qb, sb, off, R, N), settle_s)
    for _ in range(warmup):
        M.grouped_gemm_fp8(qa, sa, qb, sb, off, R, N)
    torch.cuda.synchronize()
    tot = 0.0
    for _ in range(steps):
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        M.grouped_gemm_fp8(qa, sa, qb, sb, off, R, N)
        e1.record()
        torch.cuda.synchronize()
        tot += e0.elapsed_time(e1)
    ms = tot / steps
    flops = 2.0 * float(sizes.sum()) * N * K
    tflops = flops / (ms * 1e-3) / 1e12
    return {"metric": "FP8 grouped-GEMM TFLOPS on 1 MI355X (% roofline)", "value": round(tflops, 1),
            "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
            "settle_s": settle_s,
            "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "e4m3", "data": "synthetic",
            "config": {"workload": "grouped_gemm_fp8: 16 Zipf(1.1) groups sum 8192 (padded to "
                                   "128), N=4096, K=7168, bf16 out", "group_sizes": sizes.tolist()},
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP8_TFLOPS, 4),
                         "traffic": None}}


def _time_flushed(fn, steps, warmup, settle_s=SETTLE_S):
    """Average HIP-event time of fn() with a 512 MB write before each launch (outside the
    events), so that the weights do not stay in the last-level cache."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    settle(fn, settle_s)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    tot = 0.0
    for _ in range(steps):
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        tot += e0.elapsed_time(e1)
    return tot / steps


def bench_dense_gemm(M, steps, warmup, settle_s=SETTLE_S):
    """Dense block-scaled FP8 GEMM at the standalone grouped GEMM's size: M=8192, N=4096,
    K=7168, bf16 out."""
    dev = torch.device("cuda:0")
    Mr, N, K = 8192, 4096, 7168
    a = synth.normal((Mr, K), 0, "gemm_a", device=dev)
    b = synth.normal((1, N, K), 0, "gemm_b", device=dev, std=K ** -0.5)
    qa, sa = M.moe_quant_fp8(a)
    qb, sb = M.moe_quant_weight_fp8(b)
    qb = M.moe_pack_weight_fp8(qb)
    ms = _time_flushed(lambda: M.gemm_fp8(qa, sa, qb[0], sb[0]), steps, warmup, settle_s)
    tflops = 2.0 * Mr * N * K / (ms * 1e-3) / 1e12
    return {"metric": "FP8 dense GEMM TFLOPS on 1 MI355X (% roofline)", "value": round(tflops, 1),
            "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
            "settle_s": settle_s,
            "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "e4m3", "data": "synthetic",
            "config": {"workload": "dense_gemm_fp8: M=8192, N=4096, K=7168, bf16 out"},
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP8_TFLOPS, 4),
                         "traffic": None}}


def bench_masked_gemm(M, steps, warmup, settle_s=SETTLE_S):
    """GEMM1 of the decode layer over the fixed-capacity layout: the 128-token decode
    routing of 256 experts, capacity ceil(T k / E) * 2 rows per expert, SwiGLU + e4m3
    requant, N = I = 2048, K = d = 7168.  Bound by the touched experts' weight stream."""
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS["decode_fp8"]
    inp, weights = make_layer(w, dev)
    idx, _, _ = M.moe_route(inp["x"], inp["w_router"], inp["bias"], w.k)
    cap = M.moe_capacity(w.T, w.k, w.E, 2.0)
    counts = torch.bincount(idx.flatten().long(), minlength=w.E).to(torch.int32)
    qx, sx = M.moe_quant_fp8(inp["x"])
    rows = w.E * cap
    # each expert's block: its routed tokens first (any order serves the timing)
    order = torch.argsort(idx.flatten(), stable=True)
    e_sorted = idx.flatten()[order].long()
    first = torch.cumsum(counts.long(), 0) - counts.long()
    pos = torch.arange(order.numel(), device=dev) - first[e_sorted]
    keep = pos < cap
    src = torch.zeros(rows, dtype=torch.int64, device=dev)
    src[(e_sorted * cap + pos)[keep]] = (order // w.k)[keep]
    qa, sa = qx[src].contiguous(), sx[src].contiguous()
    cnt = torch.clamp(counts, max=cap)
    ms = _time_flushed(lambda: M.grouped_gemm_fp8_masked(qa, sa, weights["w13"], weights["s13"],
                                                          cnt, cap, w.I, swiglu=True),
                       steps, warmup, settle_s)
    touched = int((cnt > 0).sum().item())
    wbytes = touched * (2 * w.I * w.d + 2 * w.I // 128 * w.d // 128 * 4)
    gbs = wbytes / (ms * 1e-3) / 1e9
    tflops = 2.0 * float(cnt.sum().item()) * 2 * w.I * w.d / (ms * 1e-3) / 1e12
    return {"metric": "FP8 masked grouped-GEMM weight stream on 1 MI355X (% roofline)",
            "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps,
            "warmup": warmup, "settle_s": settle_s, "ms_per_step": round(ms, 4),
            "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "e4m3", "data": "synthetic",
            "tflops": round(tflops, 2),
            "config": {"workload": f"masked_gemm_fp8: decode GEMM1, E=256 x cap {cap}, "
                                   f"{touched} experts touched, N=2048 (SwiGLU), K=7168"},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}}


def stage_times(M, w, inp, weights, steps):
    """Average time of each step of the layer, run through the individual C entry points
    on torch's current stream and bracketed by HIP events."""
    dev = inp["x"].device
    x = inp["x"]
    names = ["route", "dispatch", "quant", "gemm1", "gemm2", "combine"]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
    acc = {n: 0.0 for n in names}
    R = M.moe_rows_bound(w.T, w.k, w.E, w.m_align)
    for it in range(steps + 1):
        ev[0].record()
        idx, gw, _ = M.moe_route(x, inp["w_router"], inp["bias"], w.k)
        ev[1].record()
        counts, offsets, ros, sor = M.moe_dispatch(idx, w.E, w.m_align)
        ev[2].record()
        qx, sx = M.moe_quant_fp8(x)
        ev[3].record()
        hq, sh = M.grouped_gemm_fp8(qx, sx, weights["w13"], weights["s13"], offsets, R, w.I,
                                    swiglu=True, a_rows=sor, a_row_div=w.k)
        ev[4].record()
        o = M.grouped_gemm_fp8(hq, sh, weights["w2"], weights["s2"], offsets, R, w.d)
        ev[5].record()
        M.moe_combine(o, ros, gw, w.T, w.k)
        ev[6].record()
        torch.cuda.synchronize()
        if it == 0:
            continue        # first pass warms the allocator
        for i, n in enumerate(names):
            acc[n] += ev[i].elapsed_time(ev[i + 1])
    return {n: acc[n] / steps for n in names}


def stage_times_w4a16(M, w, inp, weights, steps):
    """Stage times of the hash-routed W4A16 layer through the individual C entry points
    (route_hash -> dispatch -> GEMM1 with the token gather -> GEMM2 -> combine)."""
    x = inp["x"]
    names = ["route", "dispatch", "gemm1", "gemm2", "combine"]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
    acc = {n: 0.0 for n in names}
    R = M.moe_rows_bound(w.T, w.k, w.E, w.m_align)
    for it in range(steps + 1):
        ev[0].record()
        idx, gw = M.moe_route_hash(inp["token_ids"], w.E)
        ev[1].record()
        counts, offsets, ros, sor = M.moe_dispatch(idx, w.E, w.m_align)
        ev[2].record()
        h = M.grouped_gemm_w4a16(x, weights["w13"], weights["s13"], offsets, R, w.I,
                                 swiglu=True, a_rows=sor, a_row_div=w.k)
        ev[3].record()
        o = M.grouped_gemm_w4a16(h, weights["w2"], weights["s2"], offsets, R, w.d)
        ev[4].record()
        M.moe_combine(o, ros, gw, w.T, w.k)
        ev[5].record()
        torch.cuda.synchronize()
        if it == 0:
            continue
        for i, n in enumerate(names):
            acc[n] += ev[i].elapsed_time(ev[i + 1])
    return {n: acc[n] / steps for n in names}


if __name__ == "__main__":
    sys.exit(main())
