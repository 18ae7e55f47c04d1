"""Benchmark of the causal GQA prefill hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Defaults: 100 warm-up steps (the engine clock takes about 100 ms of sustained
load to reach its steady value) and 50 timed steps.

One step = one attn_causal_prefill call (main kernel and, when the key range
is split, the combine kernel) over inputs already resident in HBM.  The
default workload is the long-context D=128 chunk: B=1, Hq=16, Hkv=2,
Lq=1024, Lkv=131072, end-aligned causal.  Throughput counts only unmasked
(query, key) pairs, 4*D FLOP each.  Prints ONE JSON line.

`value` is the step rate over exactly --steps back-to-back calls timed by
HIP events on the stream the kernels run on, after the --warmup calls and
after two measurement passes (timing_protocol: per-call events over 7
repetitions; roofline: the library's own events around the attention kernel,
and its clock sums), so nothing else is recorded inside the timed loop.  The
roofline object prices the attention kernel against the bf16 dense MFMA
peak.  The cpu_baseline object times the fp64 oracle on the same workload on
the host cores (all query rows where that takes under ~8 s, else an evenly
spaced row sample).  --workload d128_lq1k_lkv128k_rising is the metric's
shape with logits rising 150 nats in every 4096-key block, which the
reference refresh of the D = 128 kernel follows (without it every workgroup
would redo its key range with the exact running maximum); the
fixed_reference_pass object counts the workgroups that were redone.  Varlen
workloads (--workload varlen_pinned,
varlen_short) report HBM GB/s of algorithmic bytes instead; their step time
comes from replaying a captured graph of 10 back-to-back launches that
rotate over 8 copies of the store (more than the last-level cache holds).
--workload kv_write_pinned times the step's K/V slot write alone (GB/s) and
step_pinned the slot write followed by the varlen attention (us per step).

The roofline object also carries the average shader clock the timed
attention workgroups ran at (per XCD too) and, for the MFMA peak, the
fraction of the peak at that clock and at the slowest XCD's clock (every
XCD gets the same work, so the slowest sets the end).  timing_protocol gives
per-call median and min over 7 outer repetitions and the mean of
repetitions 3 to 7.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal GQA prefill TFLOP/s (unmasked pairs) + % bf16 MFMA peak, Lkv=131072"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 FLOP/clk x 2.4 GHz (AMD: 2.5 PFLOP/s dense)
PEAK_HBM_GBS = 8000.0
SRC = os.path.join(ROOT, "causal_gqa_prefill_flash_amd", "csrc", "attn.hip")


def prefill_pairs(B, Hq, Lq, Lkv, q_pos0, window):
    """Unmasked (query, key) pairs: row i at position q_pos0+i sees keys
    max(0, p-W+1) .. min(Lkv-1, p)."""
    p = torch.arange(Lq, dtype=torch.int64) + q_pos0
    hi = torch.clamp(p, max=Lkv - 1)
    lo = torch.clamp(p - window + 1, min=0) if window > 0 else torch.zeros_like(p)
    n = torch.clamp(hi - lo + 1, min=0)
    return int(n.sum()) * B * Hq


def varlen_pairs_and_bytes(info, attr, Hq, Hkv, D):
    """Unmasked pairs, and algorithmic HBM bytes (visible K/V rows once per
    KV head, Q read and O written once per covered row, uncovered rows
    written once) of a varlen step."""
    pairs = 0
    kv_rows = 0
    for s in range(info.shape[0]):
        q_start, q_len, col, kv_end = (int(x) for x in info[s])
        causal, W, _ = (int(x) for x in attr[s])
        lo_all, hi_all = None, 0
        for j in range(q_len):
            p = kv_end - q_len + j
            hi = min(kv_end - 1, p) if causal else kv_end - 1
            lo = max(0, p - W + 1) if W > 0 else 0
            pairs += max(0, hi - lo + 1)
            if hi >= lo:
                lo_all = lo if lo_all is None else min(lo_all, lo)
                hi_all = max(hi_all, hi + 1)
        if lo_all is not None:
            kv_rows += hi_all - lo_all
    return pairs * Hq, kv_rows


def src_digest():
    with open(SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, when they
    were taken on the kernel source that is built now; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("src_sha256_16") != src_digest():
        return None
    return t.get("bytes_per_launch")


def time_loop(fn, steps):
    """ms per step from events around `steps` back-to-back calls on the
    current stream (the stream the library launches on), nothing else
    recorded inside the loop."""
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_kernel(fn, steps):
    """(ms per launch of the attention kernel from the library's own events
    on its launch stream, the shader clock those launches ran at), over
    `steps` calls with the timing aid on."""
    import causal_gqa_prefill_flash_amd as attn
    torch.cuda.synchronize()
    attn.timing_begin()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    kernel_ms, launches = attn.timing_end()
    return kernel_ms / max(launches, 1), clock_info()


def time_calls(fn, steps, warmup):
    """(ms per step, ms per attention-kernel launch, its clock).  After the
    warm-up, the kernel pass (timing aid on) runs first; the step time is a
    separate loop of exactly `steps` calls with the aid off, so no event or
    clock atomic of the aid falls inside it."""
    for _ in range(warmup):
        fn()
    kms, clk = time_kernel(fn, steps)
    ms = time_loop(fn, steps)
    return ms, kms, clk


def clock_info():
    """Average shader clock of the last timed launches (per XCD too), from the
    library's cycle and reference-tick sums."""
    import causal_gqa_prefill_flash_amd as attn
    try:
        mhz, per = attn.timing_clock()
    except RuntimeError as e:
        return {"sclk_mhz": None, "error": str(e)}
    return {"sclk_mhz": round(mhz, 1), "sclk_per_xcd_mhz": [round(x, 1) for x in per]}


def with_clock(roof, clk, peak, peak_clock_mhz=2400.0):
    """Adds the measured clock and, for a compute peak (which scales with the
    clock), the fraction of that peak at the measured clock: at the mean of
    the timed workgroups, and at the slowest XCD's clock (the XCDs run at
    different clocks, equal work per XCD, so the slowest one sets the end)."""
    roof.update(clk)
    if peak and clk.get("sclk_mhz"):
        p = peak * clk["sclk_mhz"] / peak_clock_mhz
        roof["peak_at_sclk"] = round(p, 1)
        roof["frac_at_sclk"] = round(roof["achieved"] / p, 4)
        ran = [x for x in clk.get("sclk_per_xcd_mhz", []) if x > 0]
        if ran:
            pm = peak * min(ran) / peak_clock_mhz
            roof["frac_at_slowest_xcd_sclk"] = round(roof["achieved"] / pm, 4)
    return roof


def protocol_stats(fn, steps, reps=7):
    """Per-call times over `reps` outer repetitions of `steps` calls (events
    around each call): median and min over all calls, each repetition's mean,
    and the mean of repetitions 3..7."""
    evs = []
    for _ in range(reps):
        row = []
        for _ in range(steps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            row.append((a, b))
        evs.append(row)
    torch.cuda.synchronize()
    per = [[a.elapsed_time(b) for a, b in row] for row in evs]
    flat = sorted(x for row in per for x in row)
    means = [sum(row) / len(row) for row in per]
    return {"per_call_ms_median": round(flat[len(flat) // 2], 4),
            "per_call_ms_min": round(flat[0], 4),
            "rep_mean_ms": [round(m, 4) for m in means],
            "mean_of_reps_3_to_7_ms": round(sum(means[2:7]) / len(means[2:7]), 4),
            "reps": reps, "calls_per_rep": steps}


def time_graph(fns, steps, warmup):
    """ms per launch of the varlen path replayed from captured graphs: one
    graph of len(fns) back-to-back launches (fns[i] launches the i-th), plus
    one of steps % len(fns) launches, so exactly `steps` launches are timed."""
    n = len(fns)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    tail = None
    if steps % n:
        tail = torch.cuda.CUDAGraph()
        with torch.cuda.graph(tail):
            for f in fns[:steps % n]:
                f()
    torch.cuda.synchronize()
    for _ in range(max(1, (warmup + n - 1) // n)):
        g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps // n):
        g.replay()
    if tail is not None:
        tail.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def cpu_baseline_prefill(q, k, v, w, budget_s=30.0):
    """The oracle, as it stands, on a bounded sample of query rows."""
    import oracle
    B, Hq, Lq, D = q.shape
    Lkv = k.shape[2]
    q_pos0 = w["q_pos0"] if w["q_pos0"] is not None else Lkv - Lq
    n = 2
    while True:
        rows = sorted(set(int(x) for x in torch.linspace(0, Lq - 1, n).round().tolist()))
        t0 = time.perf_counter()
        oracle.prefill(q, k, v, 1.0 / math.sqrt(D), q_pos0=q_pos0, rows=rows)
        dt = time.perf_counter() - t0
        if dt > budget_s / 4 or n >= Lq:
            break
        n = min(Lq, max(n * 2, int(n * budget_s / 4 / max(dt, 1e-3))))
    p = torch.tensor(rows, dtype=torch.int64) + q_pos0
    vis = torch.clamp(torch.clamp(p, max=Lkv - 1) + 1, min=0)
    pairs = int(vis.sum()) * B * Hq
    if len(rows) == Lq:
        what = "full run: all %d query rows, all %d heads, fp64, %.1f s" % (Lq, Hq, dt)
    else:
        what = ("%d of %d query rows (evenly spaced), all %d heads, fp64, %.1f s"
                % (len(rows), Lq, Hq, dt))
    return {"value": 4.0 * D * pairs / dt / 1e12, "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle", "sample": what}


def bench_prefill(args, name):
    import causal_gqa_prefill_flash_amd as attn
    from causal_gqa_prefill_flash_amd import synth
    w = synth.PREFILL_WORKLOADS[name]
    B, Hq, Hkv, D, Lq, Lkv = w["B"], w["Hq"], w["Hkv"], w["D"], w["Lq"], w["Lkv"]
    q_pos0 = w["q_pos0"] if w["q_pos0"] is not None else Lkv - Lq
    qc, kc, vc = synth.prefill_inputs(B, Hq, Hkv, Lq, Lkv, D, wid=w["wid"])
    if w.get("logits") == "rising":
        qc, kc = synth.rising_logits(qc, kc, 1.0 / math.sqrt(D), 150.0, 4096)
    dev = torch.device("cuda:0")
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    out = torch.empty_like(q)
    device_bound = args.bound == "device"
    if device_bound:
        # the same call with (q_pos0, kv_len) read from device memory
        bounds = torch.tensor([q_pos0, Lkv], dtype=torch.int64, device=dev)
        ws_bytes = attn.prefill_dev_workspace_bytes(B, Hq, Hkv, Lq, Lkv, D)
    else:
        ws_bytes = attn.prefill_workspace_bytes(B, Hq, Hkv, Lq, Lkv, D)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def step():
        if device_bound:
            attn.causal_prefill_dev(q, k, v, bounds, out=out, workspace=ws)
        else:
            attn.causal_prefill(q, k, v, out=out, q_pos0=q_pos0, workspace=ws)

    for _ in range(args.warmup):
        step()
    # measurement passes first (they also keep the engine clock at its
    # loaded value), then the headline loop with nothing else inside it
    proto = protocol_stats(step, args.steps)
    kms, clk = time_kernel(step, args.steps)
    n_wg, n_redone = attn.timing_reruns()  # of that pass's launches
    ms = time_loop(step, args.steps)
    pairs = prefill_pairs(B, Hq, Lq, Lkv, q_pos0, 0)
    flops = 4.0 * D * pairs
    tflops = flops / (ms * 1e-3) / 1e12
    ktflops = flops / (kms * 1e-3) / 1e12
    line = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal GQA prefill %s%s" % (name, ", device bound" if device_bound
                                                               else ""),
                   "B": B, "Hq": Hq, "Hkv": Hkv, "D": D, "Lq": Lq, "Lkv": Lkv, "q_pos0": q_pos0,
                   "unmasked_pairs": pairs},
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": with_clock(
            {"bound": "mfma", "achieved": round(ktflops, 2), "peak": PEAK_BF16_TFLOPS,
             "unit": "TFLOP/s", "frac": round(ktflops / PEAK_BF16_TFLOPS, 4),
             "traffic": traffic_from_profile(name),
             # the standard scale 1/sqrt(D): the variant that carries the scale in Q
             "kernel": "prefill_kernel<%d, true>" % D if D != 256 else "prefill256_kernel<true>",
             "kernel_ms_per_launch": round(kms, 4),
             "algorithmic_flop_per_launch": flops,
             "timed": "attention kernel alone: HIP events recorded by the library on "
                      "its launch stream around every launch of the timed loop"},
            clk, PEAK_BF16_TFLOPS),
        "estimator": "value = 4*D*unmasked_pairs / ms_per_step, ms_per_step = events around "
                     "exactly `steps` back-to-back calls (main kernel + split merge) on the "
                     "launch stream, after `warmup` calls and the timing_protocol and roofline "
                     "passes, timing aid off; roofline.achieved = the same FLOP / the attention "
                     "kernel's own event time (aid on)",
        "timing_protocol": proto,
        # workgroups of the roofline pass, and those whose sums left
        # [2^-64, 2^64] after the fixed-reference pass and were redone exactly
        "fixed_reference_pass": {"workgroups": n_wg, "redone_exactly": n_redone},
        "tflops_mean_of_reps_3_to_7": round(flops / (proto["mean_of_reps_3_to_7_ms"] * 1e-3)
                                            / 1e12, 2),
    }
    if w.get("logits") == "rising":
        line["config"]["logits"] = ("K shifted so that logits rise by 150 nats over every "
                                    "4096-key block (without the periodic refresh of the "
                                    "fixed references every workgroup's sums would leave "
                                    "[2^-64, 2^64] and each would redo its range exactly)")
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_prefill(qc, kc, vc, w)
    return line


def bench_varlen(args, name):
    import causal_gqa_prefill_flash_amd as attn
    from causal_gqa_prefill_flash_amd import synth
    st = synth.VARLEN_STORE
    rows, cols, Hkv, D, Hq = st["rows"], st["cols"], st["Hkv"], st["D"], st["Hq"]
    if name == "varlen_pinned":
        info, attr, T = synth.pinned_varlen_table()
    else:  # short-query step: every segment decode-like over a full flat column
        qlens = [1, 4, 16, 1, 4, 16, 4, 1]
        rows_info, t = [], 0
        for s, ql in enumerate(qlens):
            rows_info.append((t, ql, s, rows))
            t += ql
        info = torch.tensor(rows_info, dtype=torch.int32)
        attr = torch.tensor([(1, 0, 0)] * len(qlens), dtype=torch.int32)
        T = t
    dev = torch.device("cuda:0")
    # rotate over several store copies so the 256 MB last-level cache cannot hold them
    ncopy = 8
    q = synth.varlen_inputs(T, 8, cols, Hkv, D, Hq, wid=60)[0].to(dev)
    stores = []
    for c in range(ncopy):
        ks = synth.randn_bf16((rows, cols, Hkv, D), 7000 + c).to(dev)
        vs = synth.randn_bf16((rows, cols, Hkv, D), 7100 + c).to(dev)
        stores.append((ks, vs))
    si, sa = info.to(dev), attr.to(dev)
    out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(attn.varlen_workspace_bytes(len(info), T, Hq, Hkv, D, rows, cols),
                     dtype=torch.uint8, device=dev)
    it = [0]

    def step():
        ks, vs = stores[it[0] % ncopy]
        it[0] += 1
        attn.sdpa_varlen(q, ks, vs, si, seg_attr=sa, out=out, workspace=ws)

    def launch(c):
        ks, vs = stores[c % ncopy]
        return lambda: attn.sdpa_varlen(q, ks, vs, si, seg_attr=sa, out=out, workspace=ws)

    # the step time: a captured graph of 10 back-to-back launches, each on
    # the next store copy; the kernel time and clock: an eager pass with the
    # library's events around the attention kernel
    ms = time_graph([launch(c) for c in range(10)], args.steps, args.warmup)
    eager_ms, kms, clk = time_calls(step, args.steps, args.warmup)
    pairs, kv_rows = varlen_pairs_and_bytes(info, attr, Hq, Hkv, D)
    nbytes = kv_rows * Hkv * D * 2 * 2 + T * Hq * D * 2 * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    kgbs = nbytes / (kms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_varlen(q.cpu(), stores[0][0].cpu(), stores[0][1].cpu(), info, attr,
                                  T, nbytes)
    line = {
        "metric": "varlen SDPA HBM GB/s (algorithmic bytes)", "value": round(gbs, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "timed": "graph replay: one captured graph of 10 back-to-back launches, each on the "
                 "next of %d store copies; ms_per_step = graph time / 10" % ncopy,
        "eager_ms_per_step": round(eager_ms, 4),
        "config": {"workload": name, "rows": rows, "cols": cols, "Hkv": Hkv, "D": D, "Hq": Hq,
                   "T": T, "S": int(info.shape[0]), "unmasked_pairs": pairs,
                   "store_copies_rotated": ncopy},
        "roofline": with_clock(
            {"bound": "hbm", "achieved": round(kgbs, 1), "peak": PEAK_HBM_GBS,
             "unit": "GB/s", "frac": round(kgbs / PEAK_HBM_GBS, 4),
             "traffic": traffic_from_profile(name), "algorithmic_bytes_per_launch": nbytes,
             "kernel": "varlen_kernel<%d>" % D, "kernel_ms_per_launch": round(kms, 4),
             "tflops_unmasked": round(4.0 * D * pairs / (ms * 1e-3) / 1e12, 3)},
            clk, None),
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    return line


def cpu_baseline_varlen(q, ks, vs, info, attr, T, nbytes):
    """The oracle, as it stands, on the whole varlen step (every segment,
    every head), rated in the same algorithmic bytes per second."""
    import oracle
    t0 = time.perf_counter()
    oracle.varlen(q, ks, vs, info, T=T, seg_attr=attr)
    dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "full run: all %d segments, all packed rows and heads, fp64, %.2f s"
                      % (int(info.shape[0]), dt)}


def bench_kv_write(args, name):
    """The step's K/V slot write (kv_write_pinned: the pinned table's step
    tokens into the column store), alone and followed by the varlen attention
    as one step (step_pinned); both replayed from captured graphs of 10
    launches rotating over 8 store copies."""
    import causal_gqa_prefill_flash_amd as attn
    from causal_gqa_prefill_flash_amd import synth
    st = synth.VARLEN_STORE
    rows, cols, Hkv, D, Hq = st["rows"], st["cols"], st["Hkv"], st["D"], st["Hq"]
    info, attr, T = synth.pinned_varlen_table()
    pos, col, srows = [], [], []
    for s_ in range(info.shape[0]):
        q_start, q_len, c, kv_end = (int(x) for x in info[s_])
        for j in range(q_len):
            pos.append(kv_end - q_len + j)
            col.append(c)
            srows.append(int(attr[s_][2]))
    n = len(pos)
    dev = torch.device("cuda:0")
    posd = torch.tensor(pos, dtype=torch.int64, device=dev)
    cold = torch.tensor(col, dtype=torch.int32, device=dev)
    srd = torch.tensor(srows, dtype=torch.int32, device=dev)
    kn = synth.randn_bf16((n, Hkv, D), 7200).to(dev)
    vn = synth.randn_bf16((n, Hkv, D), 7201).to(dev)
    q = synth.varlen_inputs(T, 8, cols, Hkv, D, Hq, wid=60)[0].to(dev)
    ncopy = 8
    stores = [(synth.randn_bf16((rows, cols, Hkv, D), 7000 + c).to(dev),
               synth.randn_bf16((rows, cols, Hkv, D), 7100 + c).to(dev)) for c in range(ncopy)]
    si, sa = info.to(dev), attr.to(dev)
    out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=dev)
    kws = torch.empty(attn.kv_write_workspace_bytes(n), dtype=torch.uint8, device=dev)
    vws = torch.empty(attn.varlen_workspace_bytes(len(info), T, Hq, Hkv, D, rows, cols),
                      dtype=torch.uint8, device=dev)
    with_attend = name == "step_pinned"

    def launch(c):
        ks, vs = stores[c % ncopy]

        def f():
            attn.kv_write(kn, vn, ks, vs, posd, cold, srd, workspace=kws)
            if with_attend:
                attn.sdpa_varlen(q, ks, vs, si, seg_attr=sa, out=out, workspace=vws)
        return f

    ms = time_graph([launch(c) for c in range(10)], args.steps, args.warmup)
    assert attn.kv_write_read_error(kws, n) == 0
    wbytes = n * Hkv * D * 2 * 2 * 2  # K and V rows: read once, written once
    if with_attend:
        pairs, kv_rows = varlen_pairs_and_bytes(info, attr, Hq, Hkv, D)
        abytes = kv_rows * Hkv * D * 2 * 2 + T * Hq * D * 2 * 2
        return {
            "metric": "decode/prefill step time (slot write + varlen SDPA)",
            "value": round(ms * 1e3, 2), "unit": "us", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": False,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "timed": "graph replay: one captured graph of 10 steps (slot write + attention), "
                     "each on the next of %d store copies; ms_per_step = graph time / 10" % ncopy,
            "config": {"workload": name, "rows": rows, "cols": cols, "Hkv": Hkv, "D": D,
                       "Hq": Hq, "T": T, "S": int(info.shape[0]), "step_tokens": n,
                       "store_copies_rotated": ncopy},
            "roofline": {"bound": "hbm", "achieved": round((wbytes + abytes) / (ms * 1e-3) / 1e9, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round((wbytes + abytes) / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         # counter bytes of the step's dominant kernel, the attention
                         "traffic": traffic_from_profile(name), "kernel": "varlen_kernel<%d>" % D,
                         "algorithmic_bytes_per_launch": wbytes + abytes},
        }
    gbs = wbytes / (ms * 1e-3) / 1e9
    return {
        "metric": "KV slot write HBM GB/s (algorithmic bytes)", "value": round(gbs, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "timed": "graph replay: one captured graph of 10 launches, each on the next of %d "
                 "store copies; ms_per_step = graph time / 10" % ncopy,
        "config": {"workload": name, "rows": rows, "cols": cols, "Hkv": Hkv, "D": D,
                   "step_tokens": n, "store_copies_rotated": ncopy},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic_from_profile(name),
                     "algorithmic_bytes_per_launch": wbytes,
                     "kernel": "kv_write_kernel"},
    }


def calibrate_copy():
    """A plain device copy of known size (256 MiB read, 256 MiB written),
    three times, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    n = 256 * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": n * 4, "bytes_written": n * 4,
                      "launches": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the engine clock ramps up over roughly the first 100 ms of sustained load:
    # the default warm-up covers that, so the timed steps see the steady clock
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="d128_lq1k_lkv128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bound", choices=("host", "device"), default="host",
                    help="prefill: q_pos0 and Lkv from the call, or read from device memory")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a 256 MiB copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.workload.startswith("varlen"):
        line = bench_varlen(args, args.workload)
    elif args.workload in ("kv_write_pinned", "step_pinned"):
        line = bench_kv_write(args, args.workload)
    else:
        line = bench_prefill(args, args.workload)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
