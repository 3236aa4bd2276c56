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
    elif w.mode == "w4a8":
        # 4-bit codes and scales rearranged once, offline, into the order the GEMM loads
        weights["w13"], weights["s13"] = M.moe_pack_weight_int4(*M.moe_quant_weight_int4(inp["w13"]))
        weights["w2"], weights["s2"] = M.moe_pack_weight_int4(*M.moe_quant_weight_int4(inp["w2"]))
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
    elif w.mode == "w4a8":
        wb13 = 2 * I * d // 2 + 2 * I * (d // 128) * 4
        wb2 = d * I // 2 + d * (I // 128) * 4
        a1 = w.T * d + w.T * (d // 128) * 4
        h = R * I + R * (I // 128) * 4
        o = R * d * 2
    else:
        wb13, wb2 = 2 * I * d * 4, d * I * 4
        a1, h, o = w.T * d * 4, R * I * 4, R * d * 4
    f1 = 2.0 * R * (2 * I) * d
    f2 = 2.0 * R * d * I
    b1 = touched * wb13 + a1 + h
    b2 = touched * wb2 + h + o
    # algorithmic bytes credited to each GEMM: the touched experts' weights and scales;
    # the activation codes, h and o round trips are implementation traffic (reported)
    return {"gemm1_flops": f1, "gemm2_flops": f2, "gemm1_bytes": b1, "gemm2_bytes": b2,
            "gemm1_wbytes": touched * wb13, "gemm2_wbytes": touched * wb2,
            "gemm1_ibytes": a1 + h, "gemm2_ibytes": h + o,
            "wbytes_per_expert": (wb13, wb2), "rows": R, "touched": touched}


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

def _blas_info():
    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    except Exception:
        blas = []
    if blas:
        p = blas[0]
        return int(p.get("num_threads", 1)), f"{p.get('internal_api')} {p.get('version')}"
    return os.cpu_count() or 1, "unknown"


def cpu_baseline(w: synth.Workload, inp: dict, sample_div: int = 16):
    """The fp64 oracle's layer forward, timed on the host on a bounded sample.

    Timed whole: routing of every token (router logits, biased top-k, dispatch, 1x128
    token quantisation) and the weighted combine of every token.  Timed on a sample: the
    expert FFN (dequantise the expert's weights, GEMM1, SwiGLU, requantise h, GEMM2 over
    every row routed to it), exactly as oracle.layer_forward runs it, for a random
    1/sample_div of the experts drawn uniformly within two strata (experts with more than
    32 routed rows, and the rest; at least one of each) and scaled per stratum by its
    size over its sample: an unbiased estimate of the full layer's expert time with less
    spread than one uniform draw.  The offline weight quantisation (the oracle's own
    128x128 quantiser) is outside the timers."""
    import concurrent.futures as cf
    import oracle as O
    from oracle import codecs as OC
    threads, blas = _blas_info()
    x = inp["x"].float().cpu().numpy()
    wr = inp["w_router"].float().cpu().numpy()
    b = inp["bias"].cpu().numpy()
    t0 = time.perf_counter()
    logits = O.router_logits(x, wr)
    idx, gw = O.topk_route(logits.astype(np.float32), b, w.k)
    counts, offsets, ros, sor = O.dispatch(idx, w.E, w.m_align)
    qx, sx = OC.quant_fp8_act(x)
    xin = OC.dequant_fp8_act(qx, sx)
    t_route = time.perf_counter() - t0
    n = max(1, w.E // sample_div)
    rng = np.random.default_rng(0)
    heavy = np.nonzero(counts > 32)[0]
    light = np.nonzero(counts <= 32)[0]
    picks, weight = [], {}
    for stratum in (heavy, light):
        if len(stratum) == 0:
            continue
        m = max(1, int(round(n * len(stratum) / w.E)))
        for e in rng.choice(stratum, m, replace=False):
            picks.append(int(e))
            weight[int(e)] = len(stratum) / m
    experts = sorted(picks)
    masters = [(inp["w13"][e:e + 1].cpu().numpy(), inp["w2"][e:e + 1].cpu().numpy())
               for e in experts]
    with cf.ThreadPoolExecutor(min(16, len(experts))) as ex:
        quant = list(ex.map(lambda m: (*OC.quant_fp8_weight(m[0]), *OC.quant_fp8_weight(m[1])),
                            masters))
    del masters
    t_exp, t_est, rows_done = 0.0, 0.0, 0
    for e, (q13, s13, q2, s2) in zip(experts, quant):
        t0 = time.perf_counter()
        rows = np.arange(offsets[e], offsets[e + 1])
        slots = sor[rows]
        slots = slots[slots >= 0]
        a = xin[slots // w.k]
        w13 = OC.dequant_fp8_weight(q13, s13)[0]
        w2 = OC.dequant_fp8_weight(q2, s2)[0]
        gu = a @ w13.T
        h = O.swiglu(gu[:, :w.I], gu[:, w.I:])
        qh, sh = OC.quant_fp8_act(h.astype(np.float32))
        _ = OC.dequant_fp8_act(qh, sh) @ w2.T
        dt = time.perf_counter() - t0
        t_exp += dt
        t_est += dt * weight[e]
        rows_done += len(slots)
    del quant
    o_rows = np.zeros((len(sor), w.d), np.float32)
    t0 = time.perf_counter()
    O.combine(o_rows, ros, gw, w.T, w.k)
    t_comb = time.perf_counter() - t0
    total = t_route + t_est + t_comb
    flops, _, _ = layer_flops_bytes(w, counts)
    return {"value": round(flops / total / 1e12, 4), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "tokens_per_s": round(w.T / total, 1),
            "layer_s_est": round(total, 2), "host_cpus": os.cpu_count(), "blas": blas,
            "sample": (f"fp64 numpy oracle, {threads} BLAS threads: routing + dispatch + token "
                       f"quant of all {w.T} tokens {t_route:.2f} s, combine of all tokens "
                       f"{t_comb:.2f} s, expert FFN of {len(experts)} of {w.E} experts drawn "
                       f"within the >32-row and <=32-row strata ({rows_done} rows) "
                       f"{t_exp:.2f} s, scaled per stratum to {t_est:.1f} s; full-layer "
                       f"time estimate {total:.1f} s")}


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


def measured_peaks(M, reps=5):
    """The rates this GPU reaches, from the library's two probes, timed with HIP events
    on the launch stream: the FP8 matrix core (16x16x128 e4m3 MFMAs, two waves per SIMD
    on every CU) and HBM reads (a 4 GiB buffer read once per call with 16-byte
    non-temporal loads; the better of one and sixteen 512-thread workgroups per CU, the
    two grid shapes that read fastest in a sweep of 1-16).  References beside the
    datasheet peaks."""
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 50000

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms = timed(lambda: M.moe_probe_mfma_fp8(cus, iters))
    mfma = cus * 8 * iters * 4 * 65536 / (ms * 1e-3) / 1e12
    buf = torch.randint(-2**31, 2**31 - 1, (1 << 30,), dtype=torch.int32, device=dev)
    ms_r = min(timed(lambda: M.moe_probe_hbm_read(buf, m * cus)) for m in (1, 16))
    del buf
    return {"mfma_fp8_tflops": round(mfma, 1),
            "hbm_read_gbs": round((4 << 30) / (ms_r * 1e-3) / 1e9, 1),
            "probes": f"FP8 MFMA loop ({cus} workgroups x 8 waves x {iters} x 4 16x16x128 "
                      f"MFMAs) and a 4 GiB non-temporal read (best of {cus} and {16 * cus} "
                      f"workgroups), {reps} timed calls each"}


def with_measured(roofline, peaks):
    """Add the measured peak of the roofline's bound (FP8 MFMA or HBM read) and the
    fraction of it achieved."""
    if not roofline or not peaks:
        return roofline
    if roofline["bound"] == "hbm":
        mp = peaks["hbm_read_gbs"]
    elif roofline["bound"] == "mfma" and roofline["peak"] == PEAK_FP8_TFLOPS:
        mp = peaks["mfma_fp8_tflops"]
    else:
        return roofline
    roofline["measured_peak"] = mp
    roofline["frac_of_measured"] = round(roofline["achieved"] / mp, 4)
    return roofline


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
                                                       "masked_gemm_fp8",
                                                       "decode_fp8_masked"])
    ap.add_argument("--chunk-tokens", type=int, default=0,
                    help="time the two-stream chunk pipeline (moe_layer_fwd_chunked) with "
                         "chunks of this many tokens instead of the single pass")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stages", action="store_true")
    ap.add_argument("--no-measured-peak", action="store_true",
                    help="skip the MFMA and HBM probes that give the measured peaks")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="print a per-kernel summary of a rocprofv3 --kernel-trace --stats "
                         "--output-format csv run written to DIR, then exit")
    ap.add_argument("--pmc-summary", metavar="DIR",
                    help="print per-kernel average counter values of a rocprofv3 --pmc "
                         "--output-format csv run written to DIR, then exit")
    ap.add_argument("--counters-md", nargs=5, metavar=("P1", "P2", "P3", "FETCH_DIR", "WRITE_DIR"),
                    help="print the markdown counter summary of the FP8 GEMM kernels of --workload "
                         "from the three COUNTER_PASSES runs and a FETCH_SIZE / WRITE_SIZE pair, "
                         "then exit")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print HBM bytes per dispatch of the GEMM kernels from a FETCH_SIZE "
                         "and a WRITE_SIZE rocprofv3 --pmc run of --workload (prefill_fp8, decode_fp8 or "
                         "grouped_gemm_fp8), calibrated on the weight quantiser, then exit")
    a = ap.parse_args(argv)
    if a.trace_summary:
        print(trace_summary(a.trace_summary))
        return 0
    if a.pmc_summary:
        print(json.dumps(pmc_summary(a.pmc_summary), indent=1))
        return 0
    if a.counters_md:
        print(counters_md(a.workload, a.counters_md[:3], *a.counters_md[3:]))
        return 0
    if a.traffic_summary:
        print(json.dumps(traffic_summary(*a.traffic_summary, a.workload), indent=1))
        return 0
    if a.gpus != 1:
        print(json.dumps({"error": "this implementation runs on exactly one GPU; --gpus must be 1 "
                                   "(multi-GPU expert parallelism is not built)"}))
        return 2

    import fp8_grouped_gemm_amd as M
    gemm_benches = {"grouped_gemm_fp8": bench_grouped_gemm, "dense_gemm_fp8": bench_dense_gemm,
                    "masked_gemm_fp8": bench_masked_gemm}
    if a.workload in gemm_benches:
        res = gemm_benches[a.workload](M, a.steps, a.warmup, a.settle)
        if not a.no_measured_peak:
            res["measured_peak"] = measured_peaks(M)
            with_measured(res.get("roofline"), res["measured_peak"])
        print(json.dumps(res), flush=True)
        return 0
    # the decode layer in the fixed-capacity layout: C = ceil(T k / E) * 2
    masked = a.workload == "decode_fp8_masked"
    cap_factor = 2.0 if masked else 0.0
    w = synth.WORKLOADS["decode_fp8" if masked else a.workload]
    if w.m_align != 16:
        w = synth.scaled(w, m_align=16)     # the kernels' row padding (output unaffected)
    dev = torch.device("cuda:0")
    log(f"workload {w}")
    t0 = time.time()
    inp, weights = make_layer(w, dev)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f} s")
    desc = M.LayerDesc(w.T, w.d, w.E, w.k, w.I, mode=w.mode, route=w.route, m_align=w.m_align,
                       capacity_factor=cap_factor, layout="masked" if masked else "contiguous")
    cap = M.moe_capacity(w.T, w.k, w.E, cap_factor)
    ws = torch.empty(M.moe_layer_workspace_size(desc), dtype=torch.uint8, device=dev)
    x = inp["x"]
    ids = inp.get("token_ids")
    y = torch.empty_like(x)
    counts = torch.empty(w.E, dtype=torch.int32, device=dev)

    def step():
        M.moe_layer_fwd(desc, weights, x, ids, workspace=ws, y=y, counts=counts)

    if a.chunk_tokens:
        step()                              # counts of the whole batch, for the accounting
        ws_c = torch.empty(M.moe_layer_chunked_workspace_size(desc, a.chunk_tokens),
                           dtype=torch.uint8, device=dev)
        aux = torch.cuda.Stream(device=dev)

        def step():                         # noqa: F811
            M.moe_layer_fwd_chunked(desc, weights, x, a.chunk_tokens, token_ids=ids,
                                    workspace=ws_c, y=y, aux_stream=aux)

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
    if cap > 0:
        cnt = np.minimum(cnt, cap)          # rows the capacity keeps
    flops, bytes_, g = layer_flops_bytes(w, cnt)
    log(f"layer {ms:.3f} ms/step; rows {g['rows']} touched experts {g['touched']}; "
        f"loads max {cnt.max()} median {int(np.median(cnt))} min {cnt.min()}")

    # per-stage times through the individual entry points (same kernels, same stream)
    stages = {}
    if a.chunk_tokens:
        pass                                # chunk pipeline: the layer time only
    elif not a.no_stages and masked:
        stages = stage_times_masked(M, w, inp, weights, a.steps, cap)
    elif not a.no_stages and w.mode == "fp8" and w.route == "score":
        stages = stage_times(M, w, inp, weights, a.steps)
    elif not a.no_stages and w.mode == "w4a16" and w.route == "hash":
        stages = stage_times_w4a16(M, w, inp, weights, a.steps)
    elif not a.no_stages and w.mode == "w4a8" and w.route == "hash":
        stages = stage_times_w4a8(M, w, inp, weights, a.steps)
    if stages:
        log("stages (ms): " + ", ".join(f"{k} {v:.3f}" for k, v in stages.items()))
    g1_ms = stages.get("gemm1")
    roofline = None
    traffic = (measured_traffic("gemm1", TRAFFIC_FILES[a.workload])
               if a.workload in ("prefill_fp8", "decode_fp8") and not masked else None)
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
    elif g1_ms and w.mode == "w4a8":
        # 4-bit weights (~860 FLOP per weight byte at this shape) on the FP8 matrix core:
        # the bound is the FP8 MFMA peak
        tf = g["gemm1_flops"] / (g1_ms * 1e-3) / 1e12
        roofline = {"kernel": "grouped_gemm_w4a8 (GEMM1: gate+up, SwiGLU, e4m3 requant)",
                    "bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_FP8_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                    "traffic": None, "avg_ms": round(g1_ms, 4),
                    "hbm_gbs": round(g["gemm1_bytes"] / (g1_ms * 1e-3) / 1e9, 1),
                    "flops_per_launch": g["gemm1_flops"]}
    elif g1_ms:
        # credited: touched experts' gate+up weights and their 128x128 scales
        achieved = g["gemm1_wbytes"] / (g1_ms * 1e-3) / 1e9
        roofline = {"kernel": "grouped_gemm_fp8 (GEMM1: gate+up, SwiGLU, e4m3 requant)",
                    "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                    "traffic": traffic, "avg_ms": round(g1_ms, 4),
                    "tflops": round(g["gemm1_flops"] / (g1_ms * 1e-3) / 1e12, 1),
                    "bytes_per_launch": g["gemm1_wbytes"],
                    "bytes_per_unit": g["wbytes_per_expert"][0], "units": g["touched"],
                    "intermediate_bytes": g["gemm1_ibytes"],
                    "gemm2": {"avg_ms": round(stages["gemm2"], 4),
                              "achieved": round(g["gemm2_wbytes"] / (stages["gemm2"] * 1e-3)
                                                / 1e9, 1),
                              "frac": round(g["gemm2_wbytes"] / (stages["gemm2"] * 1e-3) / 1e9
                                            / PEAK_HBM_GBS, 4),
                              "bytes_per_launch": g["gemm2_wbytes"],
                              "intermediate_bytes": g["gemm2_ibytes"]}}
    out = {
        "metric": "MoE layer FP8 grouped-GEMM TFLOPS + tokens/s on 1 MI355X (% roofline)",
        "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "settle_s": a.settle,
        "ms_per_step": round(ms, 4),
        "tokens_per_s": round(w.T / (ms * 1e-3), 1),
        "layer_hbm_frac": round(bytes_ / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"fp8": "e4m3", "w4a16": "int4xbf16", "w4a8": "int4xe4m3",
                  "fp32": "f32"}[w.mode],
        "data": "synthetic",
        "config": {"workload": (f"{w.name}{'_masked' if masked else ''}: T={w.T} d={w.d} "
                                f"E={w.E} top-{w.k} I={w.I}"
                                + (f", fixed-capacity layout C={cap}" if masked else "")
                                + (f", two-stream pipeline of {a.chunk_tokens}-token chunks"
                                   if a.chunk_tokens else "")),
                   "mode": w.mode, "route": w.route, "m_align": w.m_align,
                   "skew": f"+{w.skew_add} on {w.skew_frac:.0%} of experts" if w.skew_frac else None},
        "stages_ms": {k: round(v, 4) for k, v in stages.items()} or None,
        "roofline": roofline,
    }
    if not a.no_measured_peak:
        out["measured_peak"] = measured_peaks(M)
        with_measured(roofline, out["measured_peak"])
    if (not a.no_cpu_baseline and w.mode == "fp8" and w.route == "score" and not masked
            and not a.chunk_tokens):
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(out), flush=True)
    return 0


GEMM_SOURCES = ("gemm_fp8.hip", "gemm_fp8_kernel.hpp", "gemm_fp8_big.hip", "tiles.hpp",
                "dma.hpp", "common.hpp")


def gemm_source_sha256():
    """One digest over every source the FP8 GEMM kernels are built from."""
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(f.encode())
        h.update(open(os.path.join(ROOT, "fp8_grouped_gemm_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def measured_traffic(kernel, name="gemm_fp8_prefill_traffic.json"):
    """HBM bytes per launch of a GEMM kernel from a committed rocprofv3 counter summary
    (profiles/<name>), or None when the kernel sources changed since the counters were
    taken."""
    path = os.path.join(ROOT, "profiles", name)
    try:
        d = json.load(open(path))
        sha = gemm_source_sha256()
    except (OSError, ValueError):
        return None
    if d.get("gemm_source_sha256") != sha or kernel not in d.get("roles", {}):
        return None
    return round(d["roles"][kernel]["hbm_bytes_per_launch"])


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


# weight tensors moe_quant_weight_fp8 quantises in a workload's setup, [G, R, K] each: the
# calibration kernel of the traffic counters (reads 4 B and writes 1 B per element, plus
# one fp32 scale per 128 x 128 block)
CALIB_WEIGHTS = {"prefill_fp8": [(256, 4096, 7168), (256, 7168, 2048)],
                 "decode_fp8": [(256, 4096, 7168), (256, 7168, 2048)],
                 "grouped_gemm_fp8": [(16, 4096, 7168)]}
# committed traffic summary of each workload (profiles/)
TRAFFIC_FILES = {"prefill_fp8": "gemm_fp8_prefill_traffic.json",
                 "decode_fp8": "gemm_fp8_decode_traffic.json",
                 "grouped_gemm_fp8": "grouped_gemm_fp8_traffic.json"}
CALIB_KERNEL = "moe::quant_weight_fp8_kernel"


# the counter sets of the GEMM counter summaries, one rocprofv3 --pmc run each (within the
# per-run limits: at most 8 SQ, 4 TCC, 4 TCP, 2 TA and 2 GRBM counters)
COUNTER_PASSES = [
    "SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_LDS "
    "SQ_LDS_BANK_CONFLICT SQ_INSTS_MFMA GRBM_GUI_ACTIVE",
    "SQ_WAIT_INST_LDS SQ_WAIT_ANY SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VMEM SQ_ACTIVE_INST_VALU "
    "SQ_ACTIVE_INST_ANY SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_ANY",
    "TA_BUSY_avr TA_BUSY_max TCP_PENDING_STALL_CYCLES_sum TCP_TCR_TCP_STALL_CYCLES_sum "
    "SQ_INSTS_VMEM_RD SQ_INSTS_VALU SQ_INSTS_SALU GRBM_COUNT",
]
# bytes the roofline credits per launch of each GEMM role (weights and scales; the
# standalone GEMM: its operands and output)
CREDITED_BYTES = {"prefill_fp8": {"gemm1": 7518027776, "gemm2": 3759013888},
                  "grouped_gemm_fp8": {"gemm": 615493632}}


def counters_md(workload, pass_dirs, fetch_dir, write_dir, num_cus=256):
    """Markdown summary of the FP8 GEMM kernels' hardware counters: the three
    COUNTER_PASSES runs and the FETCH_SIZE / WRITE_SIZE pair of `workload`, averaged per
    dispatch, with the derived ratios (GRBM_GUI_ACTIVE summed over the 8 XCDs: / 8 is the
    kernel's length in shader cycles)."""
    merged = {}
    for d in list(pass_dirs) + [fetch_dir, write_dir]:
        for k, cs in pmc_summary(d).items():
            if "gemm_fp8_kernel" in k:
                merged.setdefault(k, {}).update(cs)
    tr = traffic_summary(fetch_dir, write_dir, workload)
    roles = {v["kernel"]: r for r, v in tr["roles"].items()}
    out = []
    for k, cs in merged.items():
        v = {c: x["avg"] for c, x in cs.items()}
        cyc = v["GRBM_GUI_ACTIVE"] / 8
        role = roles.get(k, "")
        rows = [
            ("MFMA pipe busy", f"SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE/8 x {num_cus} CU x 4 SIMD)",
             v["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * num_cus * 4)),
            ("TA busy", "TA_BUSY_avr / (GRBM_GUI_ACTIVE/8)", v["TA_BUSY_avr"] / cyc),
            ("TCP pending-request stall", f"TCP_PENDING_STALL_CYCLES_sum / ({num_cus} x GRBM_GUI_ACTIVE/8)",
             v["TCP_PENDING_STALL_CYCLES_sum"] / (num_cus * cyc)),
            ("wave time in s_waitcnt", "SQ_WAIT_ANY / SQ_WAVE_CYCLES", v["SQ_WAIT_ANY"] / v["SQ_WAVE_CYCLES"]),
            ("wave time waiting to issue", "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES",
             v["SQ_WAIT_INST_ANY"] / v["SQ_WAVE_CYCLES"]),
            ("VALU-active wave time", "SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES",
             v["SQ_ACTIVE_INST_VALU"] / v["SQ_WAVE_CYCLES"]),
            ("LDS bank-conflict share", "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE",
             v["SQ_LDS_BANK_CONFLICT"] / v["SQ_LDS_IDX_ACTIVE"]),
            ("MFMA instructions per LDS instruction", "SQ_INSTS_MFMA / SQ_INSTS_LDS",
             v["SQ_INSTS_MFMA"] / v["SQ_INSTS_LDS"]),
        ]
        out += [f"## `{k}` ({role or 'kernel'})", "", "| derived | formula | value |", "|---|---|---|"]
        out += [f"| {n} | {f} | {x:.3f} |" for n, f, x in rows]
        if k in tr["kernels"]:
            hb = tr["kernels"][k]["hbm_bytes_per_launch"]
            cal = tr["calibration"]
            cred = CREDITED_BYTES.get(workload, {}).get(role)
            extra = f" ({hb / cred:.2f}x the {cred / 1e9:.3f} GB credited)" if cred else ""
            out.append(f"| HBM-side bytes per launch | FETCH_SIZE x {cal['fetch_factor']:.4f} + "
                       f"WRITE_SIZE x {cal['write_factor']:.4f} (KiB) | {hb / 1e9:.3f} GB{extra} |")
        out += ["", "| counter | average per dispatch | dispatches |", "|---|---|---|"]
        out += [f"| {c} | {cs[c]['avg']:.6g} | {cs[c]['dispatches']} |" for c in sorted(cs)]
        out.append("")
    cal = tr["calibration"]
    out.append(f"Calibration of the traffic counters: `{cal['kernel']}` in the same runs reads "
               f"{cal['known_read_bytes_per_dispatch']:.0f} B and writes "
               f"{cal['known_write_bytes_per_dispatch']:.0f} B per dispatch (fp32 in, e4m3 codes and "
               f"block scales out); FETCH_SIZE read {cal['fetch_kib']:.1f} KiB (factor "
               f"{cal['fetch_factor']:.4f}), WRITE_SIZE {cal['write_kib']:.1f} KiB (factor "
               f"{cal['write_factor']:.4f}).  FETCH_SIZE counts L2 fills from the fabric, so "
               f"last-level (MALL) cache hits are included.  GEMM sources sha256 "
               f"{tr['gemm_source_sha256'][:16]}.")
    return "\n".join(out)


def traffic_summary(fetch_dir, write_dir, workload):
    """HBM-side bytes per dispatch of every kernel in a pair of rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each counter scaled by the factor that
    makes it read the known bytes of the calibration kernel in the same run."""
    fetch, write = pmc_summary(fetch_dir), pmc_summary(write_dir)
    shapes = CALIB_WEIGHTS[workload]
    known_r = sum(g * r * k * 4 for g, r, k in shapes) / len(shapes)
    known_w = sum(g * r * k + g * (r // 128) * (k // 128) * 4 for g, r, k in shapes) / len(shapes)
    cal = [k for k in fetch if k.startswith(CALIB_KERNEL)][0]
    fr = known_r / (fetch[cal]["FETCH_SIZE"]["avg"] * 1024)
    fw = known_w / (write[cal]["WRITE_SIZE"]["avg"] * 1024)
    out = {"calibration": {"kernel": CALIB_KERNEL, "dispatches": fetch[cal]["FETCH_SIZE"]["dispatches"],
                           "known_read_bytes_per_dispatch": known_r,
                           "fetch_kib": fetch[cal]["FETCH_SIZE"]["avg"], "fetch_factor": fr,
                           "known_write_bytes_per_dispatch": known_w,
                           "write_kib": write[cal]["WRITE_SIZE"]["avg"], "write_factor": fw},
           "kernels": {}}
    for k in fetch:
        if k in write and "gemm" in k:
            f, wv = fetch[k]["FETCH_SIZE"]["avg"], write[k]["WRITE_SIZE"]["avg"]
            out["kernels"][k] = {"dispatches": fetch[k]["FETCH_SIZE"]["dispatches"],
                                 "fetch_kib": f, "write_kib": wv,
                                 "hbm_bytes_per_launch": f * 1024 * fr + wv * 1024 * fw}
    # roles: the layer's GEMM1 (SwiGLU epilogue) and GEMM2, or the standalone GEMM
    roles = {}
    for k, v in out["kernels"].items():
        if workload in ("prefill_fp8", "decode_fp8") and "gemm_fp8_kernel" in k:
            roles["gemm1" if ", true" in k else "gemm2"] = dict(v, kernel=k)
        elif workload == "grouped_gemm_fp8" and "gemm_fp8_kernel" in k:
            roles["gemm"] = dict(v, kernel=k)
    out["roles"] = roles
    out["gemm_source_sha256"] = gemm_source_sha256()
    return out


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
                         "traffic": measured_traffic("gemm", TRAFFIC_FILES["grouped_gemm_fp8"]),
                         "algorithmic_bytes": int(R * K + R * (K // 128) * 4 + 16 * N * K
                                                  + 16 * (N // 128) * (K // 128) * 4
                                                  + R * N * 2)}}


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
    # the [E, C, d] layout filled by the library: masked dispatch, then the 1x128
    # quantiser gathering each row's token (empty rows zero)
    counts, ros, sor = M.moe_dispatch_masked(idx, w.E, cap)
    qa, sa = M.moe_quant_fp8(inp["x"], sor, w.k, w.E * cap)
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


def _stage_loop(names, one, steps):
    """Average HIP-event time of each named stage.  one(rec) runs the stages in order on
    torch's current stream and calls rec() after each.  After one warm pass and one
    synchronisation the timed passes are queued back to back and synchronised once at the
    end, so the host's launch time does not fall between the events of a short stage."""
    def run(evs):
        nxt = iter(evs[1:])
        evs[0].record()
        one(lambda: next(nxt).record())
    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]  # noqa: E731
    run(mk())                               # first pass warms the allocator
    torch.cuda.synchronize()
    passes = []
    for _ in range(steps):
        evs = mk()
        run(evs)
        passes.append(evs)
    torch.cuda.synchronize()
    return {n: sum(e[i].elapsed_time(e[i + 1]) for e in passes) / steps
            for i, n in enumerate(names)}


def stage_times(M, w, inp, weights, steps):
    """Average time of each step of the layer, run through the individual C entry points
    on torch's current stream and bracketed by HIP events."""
    x = inp["x"]
    R = M.moe_rows_bound(w.T, w.k, w.E, w.m_align)

    def one(rec):
        idx, gw, _ = M.moe_route(x, inp["w_router"], inp["bias"], w.k)
        rec()
        counts, offsets, ros, sor = M.moe_dispatch(idx, w.E, w.m_align)
        rec()
        qx, sx = M.moe_quant_fp8(x)
        rec()
        hq, sh = M.grouped_gemm_fp8(qx, sx, weights["w13"], weights["s13"], offsets, R, w.I,
                                    swiglu=True, a_rows=sor, a_row_div=w.k)
        rec()
        o = M.grouped_gemm_fp8(hq, sh, weights["w2"], weights["s2"], offsets, R, w.d)
        rec()
        M.moe_combine(o, ros, gw, w.T, w.k)
        rec()

    return _stage_loop(["route", "dispatch", "quant", "gemm1", "gemm2", "combine"], one, steps)


def stage_times_masked(M, w, inp, weights, steps, cap):
    """Stage times of the fixed-capacity decode layer through the individual C entry
    points: route -> masked dispatch -> quant-gather into [E, C, d] -> masked GEMM1 ->
    masked GEMM2 -> combine."""
    x = inp["x"]

    def one(rec):
        idx, gw, _ = M.moe_route(x, inp["w_router"], inp["bias"], w.k)
        rec()
        counts, ros, sor = M.moe_dispatch_masked(idx, w.E, cap)
        rec()
        qa, sa = M.moe_quant_fp8(x, sor, w.k, w.E * cap)
        rec()
        hq, sh = M.grouped_gemm_fp8_masked(qa, sa, weights["w13"], weights["s13"], counts, cap,
                                           w.I, swiglu=True)
        rec()
        o = M.grouped_gemm_fp8_masked(hq, sh, weights["w2"], weights["s2"], counts, cap, w.d)
        rec()
        M.moe_combine(o, ros, gw, w.T, w.k)
        rec()

    return _stage_loop(["route", "dispatch", "quant", "gemm1", "gemm2", "combine"], one, steps)


def stage_times_w4a8(M, w, inp, weights, steps):
    """Stage times of the hash-routed layer with 4-bit weights on the FP8 matrix core:
    route_hash -> dispatch -> 1x128 quant -> GEMM1 with the token gather -> GEMM2 ->
    combine."""
    x = inp["x"]
    R = M.moe_rows_bound(w.T, w.k, w.E, w.m_align)

    def one(rec):
        idx, gw = M.moe_route_hash(inp["token_ids"], w.E)
        rec()
        counts, offsets, ros, sor = M.moe_dispatch(idx, w.E, w.m_align)
        rec()
        qx, sx = M.moe_quant_fp8(x)
        rec()
        hq, sh = M.grouped_gemm_w4a8(qx, sx, weights["w13"], weights["s13"], offsets, R, w.I,
                                     swiglu=True, a_rows=sor, a_row_div=w.k)
        rec()
        o = M.grouped_gemm_w4a8(hq, sh, weights["w2"], weights["s2"], offsets, R, w.d)
        rec()
        M.moe_combine(o, ros, gw, w.T, w.k)
        rec()

    return _stage_loop(["route", "dispatch", "quant", "gemm1", "gemm2", "combine"], one, steps)


def stage_times_w4a16(M, w, inp, weights, steps):
    """Stage times of the hash-routed W4A16 layer through the individual C entry points
    (route_hash -> dispatch -> GEMM1 with the token gather -> GEMM2 -> combine)."""
    x = inp["x"]
    R = M.moe_rows_bound(w.T, w.k, w.E, w.m_align)

    def one(rec):
        idx, gw = M.moe_route_hash(inp["token_ids"], w.E)
        rec()
        counts, offsets, ros, sor = M.moe_dispatch(idx, w.E, w.m_align)
        rec()
        h = M.grouped_gemm_w4a16(x, weights["w13"], weights["s13"], offsets, R, w.I,
                                 swiglu=True, a_rows=sor, a_row_div=w.k)
        rec()
        o = M.grouped_gemm_w4a16(h, weights["w2"], weights["s2"], offsets, R, w.d)
        rec()
        M.moe_combine(o, ros, gw, w.T, w.k)
        rec()

    return _stage_loop(["route", "dispatch", "gemm1", "gemm2", "combine"], one, steps)


if __name__ == "__main__":
    sys.exit(main())
