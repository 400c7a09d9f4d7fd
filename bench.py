"""Throughput of the fused PD-SSM forward pass (selection + chunked scan) on one
MI355X, in state-updates per second, with its HBM roofline fraction and the
fp64 CPU oracle timed beside it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload impulse]
                    [--no-cpu-baseline] [--copy-probe] [--pass fwd|bwd]
    python bench.py --pmc-summary FETCH_DIR WRITE_DIR [--workload impulse]

``--pass bwd`` times the gradient pass through the scan (pdssm_scan_bwd) on
the same workload instead, with its own roofline and oracle baseline;
``--pass fold`` times pdssm_fwd_wb (the drive term formed from u and W_b in
the same pass, so Bu is never read); ``--pass sens`` times the impulse
sensitivity dy_t/du_0 (pdssm_impulse_sens); ``--pass soft`` times the
soft-selection comparison path (pdssm_soft_select + pdssm_scan_fwd_pidx) with
the hard-selection forward pass beside it; ``--pass scan`` and ``--pass
select`` time the two stages of the forward pass alone (pdssm_scan_fwd given
the selections, pdssm_select); ``--pass multi [--n-out P]`` times
pdssm_fwd_wb_multi (the folded pass with P rows of C per head).
``timing`` in the JSON line gives the median, p10 and p90 of the per-call
event durations with a 1 GiB read sweep before each call ("cold", outside
the events: L2 and MALL hold nothing of the inputs; the headline ``value``,
``ms_per_step`` and ``roofline`` come from these) and back to back with warm
caches ("hot", the secondary line ``hot``).

Prints one JSON line.  A step is one pdssm_fwd call over the whole workload
(selection outputs not materialised), with every input already resident in
HBM.  The default workload is the 131072-step impulse-response shape
(B=1, H=32, L=131072, N=16, K=8, d=64, chunk=512, fp32).
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3        # MI355X fp32 (matrix / packed vector)
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
METRIC = "state-updates/sec (B·H·L·N) PD-SSM fwd select+scan; achieved HBM GB/s vs peak"
METRIC_FOLD = ("state-updates/sec (B·H·L·N) PD-SSM fwd select+scan with Bu = W_b u folded into the "
               "selection GEMM; achieved HBM GB/s vs peak")
CSRC = os.path.join(ROOT, "structured_sparse_state_pdssm_amd", "csrc")


# the sources each benchmarked kernel is built from
SOURCES = {
    "fwd": ("pdscan_device.h", "pdscan_plan.h", "pdscan_launch_general.h", "pdscan_launch_fused.hip",
            "pdscan_launch_fused16.hip", "pdscan_launch_fused_multi.hip", "pdscan_launch_fused_fold.hip"),
    "bwd": ("pdscan_device.h", "pdscan_plan.h", "pdscan_bwd_plan.h", "pdscan_bwd.h",
            "pdscan_launch_bwd.hip"),
}
SOURCES["fold"] = SOURCES["fwd"]
SOURCES["soft"] = ("pdscan_device.h", "pdscan_plan.h", "pdscan_soft_plan.h", "pdscan_soft.h",
                   "pdscan_launch_soft.hip", "pdscan_launch_scan.hip")
SOURCES["sens"] = ("pdscan_device.h", "pdscan_plan.h", "pdscan_sens_plan.h", "pdscan_sens.h",
                   "pdscan_launch_sens.hip")
SOURCES["scan"] = ("pdscan_device.h", "pdscan_plan.h", "pdscan_launch_scan.hip")
SOURCES["multi"] = SOURCES["fwd"]
SOURCES["select"] = ("pdscan_device.h", "pdscan_plan.h", "pdscan_launch_select.hip")
# u shared by the heads (bf16, N > 32 for the forward pass): the all-heads
# selection GEMM, and for the forward pass the chunked scan after it (the
# host code that picks the route is part of it)
SOURCES["select_gemm"] = ("pdscan_device.h", "pdscan_gemm_sel.h", "pdscan_gemm_sel_plan.h",
                          "pdscan_launch_gemm_sel.hip", "pdscan_api.cpp")
SOURCES["fwd_two_pass"] = SOURCES["select_gemm"] + ("pdscan_plan.h", "pdscan_launch_scan.hip")
# stem of the committed counter summary of each pass
TRAFFIC_STEM = {"fwd": "pdssm_fused", "bwd": "pdssm_bwd", "fold": "pdssm_fold", "sens": "pdssm_sens",
                "soft": "pdssm_soft", "scan": "pdssm_scan", "select": "pdssm_select", "multi": "pdssm_multi"}
EVICT_BYTES = 1 << 30           # read before each cold-cache rep (beyond L2 and MALL)


def source_key(which, workload=None):
    """Which source set a pass runs from on a workload: the forward passes
    (plain, drive folded, several outputs) and the selection on the LM-layer
    shape (u shared by the heads, bf16, N = 64) take the all-heads GEMMs (and,
    forward, the scan after them)."""
    if workload is not None and which in ("fwd", "fold", "multi", "select"):
        from pdssm_inputs import get_config
        cfg = get_config(workload)
        if cfg.u_shared and cfg.dtype == "bf16" and cfg.K <= 32 and cfg.N <= 64 and cfg.N % 4 == 0 \
                and cfg.d % 64 == 0 and (which == "select" or cfg.N > 32):
            return "select_gemm" if which == "select" else "fwd_two_pass"
    return which


def kernel_hash(which="fwd", workload=None) -> str:
    """Hash of a kernel's sources: ties a stored counter summary to the kernel
    it was measured on."""
    h = hashlib.sha256()
    for name in SOURCES[source_key(which, workload)]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic(cfg, fold=False):
    """Minimum traffic: every input read once, outputs written once; and the
    selection-GEMM flops 2 (K + N) d per (b, h, t).  fold: the drive term is
    formed from u and W_b (no Bu read; W_b read; 2 N d more flops)."""
    es = 2 if cfg.dtype == "bf16" else 4
    B, H, L, N, K, d = cfg.B, cfg.H, cfg.L, cfg.N, cfg.K, cfg.d
    u = B * (1 if cfg.u_shared else H) * L * d * es
    params = H * K * d * es + H * N * d * es + H * N * 4 + H * K * N * 4 + H * N * 4
    if fold:
        params += H * N * d * es
    drive = 0 if fold else B * H * L * N * 4
    total = u + drive + B * H * L * 4 + 2 * B * H * N * 4 + params
    flops = 2 * (K + (2 * N if fold else N)) * d * B * H * L
    return total, flops


def algorithmic_bwd(cfg):
    """Minimum traffic of the gradient pass: k*, D, dLoss/dy and the forward
    states read once, dBu and dD written once, plus parameters and the small
    per-sequence vectors."""
    B, H, L, N, K = cfg.B, cfg.H, cfg.L, cfg.N, cfg.K
    steps = B * H * L
    per_step = 4 + 4 * N + 4 + 4 * N + 4 * N + 4 * N
    small = H * K * N * 4 + 2 * H * N * 4 + 3 * B * H * N * 4
    return steps * per_step + small


def traffic_from_profile(workload, which="fwd"):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{TRAFFIC_STEM[which]}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_hash") != kernel_hash(which, workload):
        return None
    return rec.get("hbm_bytes_per_launch")


def _spin_cycles_per_us(torch, stream):
    """Cycles of torch's spin kernel per microsecond (it reads the shader
    clock, whose rate is not fixed), from one event-timed spin."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 2_000_000
    torch.cuda._sleep(1000)
    a.record(stream)
    torch.cuda._sleep(n)
    b.record(stream)
    torch.cuda.synchronize()
    return n / max(a.elapsed_time(b) * 1e3, 1.0)


def time_calls(torch, np, step, reps, stream, after=None):
    """Per-call durations (µs) from HIP events on the launch stream.

    Headline ("cold"): `reps` calls, each preceded (outside its events) by a
    read sweep over 1 GiB that evicts L2 and MALL without leaving dirty lines
    behind (a sum into one scalar), bracketed by synchronisations.  Secondary
    ("hot"): `reps` back-to-back calls with warm caches.

    The GPU is kept ahead of the host so that an event never waits on the
    host's argument marshalling (which would count host time as call time):
    a spin kernel that touches no memory runs before each cold rep's sweep
    (0.5 ms), and before the whole hot loop (long enough for the host to
    queue every hot call before the first one starts).

    `after` (optional) is enqueued after each call's end event, outside the
    timed region (the look-back status accumulation).

    Returns (seconds, durations, timing): the summed cold call durations
    (so seconds * 1e3 / reps is the per-step time in ms), the cold per-call
    durations, and median / p10 / p90 / mean of both sets."""
    def pct(v):
        return {"median_us": round(float(np.median(v)), 2), "p10_us": round(float(np.percentile(v, 10)), 2),
                "p90_us": round(float(np.percentile(v, 90)), 2), "mean_us": round(float(np.mean(v)), 2)}
    cyc_us = _spin_cycles_per_us(torch, stream)
    sweep = torch.ones(EVICT_BYTES // 4, device="cuda")
    sink = torch.empty((), device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        torch.cuda._sleep(int(500 * cyc_us))
        torch.sum(sweep, dim=0, out=sink)
        a.record(stream)
        step()
        b.record(stream)
        if after:
            after()
    torch.cuda.synchronize()
    wall_cold = time.perf_counter() - t0
    cold = [a.elapsed_time(b) * 1e3 for a, b in ev]
    del sweep
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    # host time per call (the cold loop's wall time less its GPU work is an
    # upper bound); the spin covers twice that for every hot call
    host_us = wall_cold * 1e6 / reps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    torch.cuda._sleep(int(min(2.0 * reps * host_us + 2000.0, 2e6) * cyc_us))
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
        if after:
            after()
    torch.cuda.synchronize()
    wall_hot = time.perf_counter() - t0
    hot = [a.elapsed_time(b) * 1e3 for a, b in ev]
    timing = {"reps": reps, "headline": "cold: each call after a 1 GiB read sweep (outside its events)",
              "cold": pct(cold), "hot": pct(hot),
              "cold_wall_ms_per_step_with_sweep": round(wall_cold * 1e3 / reps, 4),
              "hot_wall_ms_per_step_with_lead_spin": round(wall_hot * 1e3 / reps, 4)}
    return float(np.sum(cold)) / 1e6, cold, timing


COPY_PROBE_BYTES = 1 << 30      # the plain copy kernel's source (and destination) size


def copy_probe(torch):
    """A plain streaming kernel of known traffic (read 1 GiB, write 1 GiB):
    the scale of the HBM byte counters is read off it."""
    n = COPY_PROBE_BYTES // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(f"[bench] copy probe: 3 x neg over {COPY_PROBE_BYTES} B", file=sys.stderr, flush=True)


def add_box(rec, torch, np):
    """The box the line was measured on: device properties as the runtime
    reports them, and a same-box copy bandwidth (1 GiB read + 1 GiB written
    by a device-to-device copy, median of 10 event-timed reps), against which
    an HBM-bound line's achieved bandwidth is also given."""
    prop = torch.cuda.get_device_properties(0)
    n = COPY_PROBE_BYTES // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    ts = []
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / 1e3)
    del src, dst
    copy_gbps = 2 * COPY_PROBE_BYTES / float(np.median(ts)) / 1e9
    rec["box"] = {"device": prop.name, "arch": getattr(prop, "gcnArchName", ""),
                  "compute_units": prop.multi_processor_count,
                  "memory_GB": round(prop.total_memory / 1e9, 1), "copy_GBps": round(copy_gbps, 1)}
    roof = rec.get("roofline", {})
    if roof.get("unit") == "GB/s":
        roof["frac_of_copy"] = round(roof["achieved"] / copy_gbps, 4)


def _pmc_rows(d, counter):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            rows += [r for r in csv.DictReader(fh) if r["Counter_Name"] == counter]
    return rows


def _is_kernel(name, which):
    if which == "bwd":
        return "pdssm_bwd_kernel" in name
    if which == "sens":
        return "pdssm_sens_kernel" in name
    if which == "soft":
        return "pdssm_soft_kernel" in name or "pdssm_step16_kernel<1" in name
    if which == "scan":
        return "pdssm_step16_kernel" in name or ("pdssm_kernel<1," in name)
    if which == "select":
        return "pdssm_kernel<0," in name or "pdssm_kernel_wide<0," in name or "pdssm_gemm_sel_kernel" in name
    return "pdssm_" in name and "clear" not in name and "bwd" not in name and "fill" not in name.lower()


def pmc_summary(fetch_dir, write_dir, workload, which="fwd"):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch) of `bench.py --copy-probe` into HBM bytes per launch of the
    benchmarked kernel, each counter scaled by what it reads for the copy
    probe."""
    from statistics import mean
    out = {}
    for counter, d, probe_bytes in (("FETCH_SIZE", fetch_dir, COPY_PROBE_BYTES),
                                    ("WRITE_SIZE", write_dir, COPY_PROBE_BYTES)):
        rows = _pmc_rows(d, counter)
        # per kernel of the pass, the mean over its dispatches; a call that
        # launches several (the soft path: selection, then scan) sums them
        per = {}
        for r in rows:
            if _is_kernel(r["Kernel_Name"], which):
                per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        probe = [float(r["Counter_Value"]) for r in rows if "neg" in r["Kernel_Name"]]
        if not per or not probe:
            raise SystemExit(f"{counter}: no {which} kernel or copy-probe dispatches under {d}")
        kib = sum(mean(v) for v in per.values())
        scale = probe_bytes / (mean(probe) * 1024.0)
        out[counter] = {"kernel_kib": kib, "probe_kib": mean(probe),
                        "scale": scale, "bytes": kib * 1024.0 * scale,
                        "dispatches": sum(len(v) for v in per.values()), "kernels": sorted(per)}
    total = out["FETCH_SIZE"]["bytes"] + out["WRITE_SIZE"]["bytes"]
    rec = {"workload": workload, "pass": which, "kernel_hash": kernel_hash(which, workload),
           "hbm_bytes_per_launch": round(total), "counters": out,
           "copy_probe_bytes": COPY_PROBE_BYTES}
    path = os.path.join(ROOT, "profiles", f"{TRAFFIC_STEM[which]}_{workload}_traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def cpu_baseline(inp, fold=False):
    """The fp64 oracle, as it is, on the host cores: selection (and, with
    fold, the drive terms) plus the dense sequential scan over the whole
    workload (inputs already generated)."""
    import numpy as np  # noqa: F401
    import oracle
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(limits=cores)
    except Exception:                       # threadpoolctl missing: numpy defaults
        import contextlib
        ctx = contextlib.nullcontext()
    c = inp.cfg
    with ctx:
        t0 = time.perf_counter()
        if fold:
            oracle.forward_wb(inp.u, inp.W_sel, inp.dict_idx, inp.W_d, inp.b_d, inp.W_b, inp.C,
                              inp.h0, c.u_shared)
        else:
            oracle.forward_inputs(inp)
        dt = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": c.state_updates / dt, "unit": "state-updates/s", "cores": cores,
            "kind": "oracle", "seconds": round(dt, 3), "cpu": model,
            "sample": f"whole {c.name} workload ({c.B}x{c.H}x{c.L} steps, N={c.N}), one run; "
                      "BLAS threads = cores (the step loop itself is single-threaded)"}


def bench_bwd(args, torch, np, P):
    """Time pdssm_scan_bwd; selections and forward states come from the
    library's own forward calls, outside the timed region."""
    from pdssm_inputs import generate, get_config, upstream_grads
    cfg = get_config(args.workload)
    chunk = args.chunk or cfg.chunk
    t0 = time.time()
    inp = generate(cfg)
    print(f"[bench] generated {cfg.name} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    bf = cfg.dtype == "bf16"
    pdt = torch.bfloat16 if bf else torch.float32

    def dev(x, dt=None):
        return torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt)

    u, W_sel, W_d = dev(inp.u, pdt), dev(inp.W_sel, pdt), dev(inp.W_d, pdt)
    b_d, dic, Bu, C, h0 = dev(inp.b_d), dev(inp.dict_idx), dev(inp.Bu), dev(inp.C), dev(inp.h0)
    fw = P.pdssm_fwd(u, W_sel, dic, W_d, b_d, Bu, C, h0, chunk=chunk, want_k=True, want_D=True)
    k, D = fw["k_star"], fw["D"]
    del u
    _, _, Hs = P.pdssm_scan_states(k, dic, D, Bu, C, h0, chunk=chunk)
    g_y_h, g_hL_h = upstream_grads(cfg.B, cfg.H, cfg.L, cfg.N, cfg.seed)
    g_y, g_hL = dev(g_y_h), dev(g_hL_h)
    dims = P.make_dims(cfg.B, cfg.H, cfg.L, cfg.N, cfg.K, 8)
    ws = torch.zeros(P.scan_bwd_workspace_bytes(dims, chunk), dtype=torch.uint8, device="cuda")
    out = {"g_Bu": torch.empty_like(D), "g_D": torch.empty_like(D),
           "g_h0": torch.empty_like(h0), "g_C": torch.empty_like(C)}

    def step():
        P.pdssm_scan_bwd(k, dic, D, C, Hs, g_y, h0=h0, g_hL=g_hL, chunk=chunk, workspace=ws, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if P.workspace_error_flag(ws):
        raise RuntimeError("look-back wait gave up during warm-up")
    stream = torch.cuda.current_stream()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    wall, dur, timing = time_calls(torch, np, step, args.steps, stream,
                                   after=lambda: P.pdssm_workspace_status(ws, status))
    if int(status.item()):
        raise RuntimeError("a look-back wait gave up during timing")
    launch_s = float(np.mean(dur)) / 1e6
    ms_step = wall * 1e3 / args.steps
    alg = algorithmic_bwd(cfg)
    achieved = alg / launch_s / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic_from_profile(cfg.name, "bwd"),
            "algorithmic_bytes": alg, "launch_us": round(launch_s * 1e6, 2)}
    rec = {
        "metric": "state-updates/sec (B·H·L·N) PD-SSM gradient through the scan (fixed selections)",
        "value": cfg.state_updates / (ms_step / 1e3),
        "unit": "state-updates/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{cfg.name} gradient pass: B={cfg.B} H={cfg.H} L={cfg.L} N={cfg.N} "
                               f"K={cfg.K} chunk={chunk}",
                   "B": cfg.B, "H": cfg.H, "L": cfg.L, "N": cfg.N, "K": cfg.K, "chunk": chunk},
        "roofline": roof,
        "timing": timing,
        "kernel_hash": kernel_hash("bwd"),
    }
    add_box(rec, torch, np)
    if args.copy_probe:
        copy_probe(torch)
    if not args.no_cpu_baseline:
        import oracle
        cores = len(os.sched_getaffinity(0))
        Ls = cfg.L
        kh, Dh = k.cpu().numpy()[:, :, :Ls], D.cpu().numpy()[:, :, :Ls].astype(np.float64)
        t0 = time.perf_counter()
        oracle.scan_vjp(kh, inp.dict_idx, Dh, inp.Bu[:, :, :Ls], inp.C, inp.h0, g_y_h[:, :, :Ls], g_hL_h)
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": cfg.B * cfg.H * Ls * cfg.N / dt, "unit": "state-updates/s",
                               "cores": cores, "kind": "oracle", "seconds": round(dt, 3),
                               "sample": f"whole {cfg.name} workload ({cfg.B}x{cfg.H}x{Ls} steps) "
                                         "(oracle gradient: states plus the backward recurrence)"}
    print(json.dumps(rec), flush=True)


def algorithmic_sens(cfg):
    """Minimum traffic of the impulse sensitivity: k* and D read once, dY
    written once, plus the dictionary, C, W_d, W_b and h0."""
    B, H, L, N, K, d = cfg.B, cfg.H, cfg.L, cfg.N, cfg.K, cfg.d
    es = 2 if cfg.dtype == "bf16" else 4
    steps = B * H * L
    return steps * (4 + 4 * N + 4 * d) + H * K * N * 4 + H * N * 4 + 2 * H * N * d * es + B * H * N * 4


def bench_sens(args, torch, np, P):
    """Time pdssm_impulse_sens; the selections come from the library's own
    forward pass, outside the timed region."""
    from pdssm_inputs import generate, get_config
    cfg = get_config(args.workload)
    chunk = args.chunk or cfg.chunk
    t0 = time.time()
    inp = generate(cfg)
    print(f"[bench] generated {cfg.name} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    bf = cfg.dtype == "bf16"
    pdt = torch.bfloat16 if bf else torch.float32

    def dev(x, dt=None):
        return torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt)

    u, W_sel, W_d, W_b = dev(inp.u, pdt), dev(inp.W_sel, pdt), dev(inp.W_d, pdt), dev(inp.W_b, pdt)
    b_d, dic, Bu, C, h0 = dev(inp.b_d), dev(inp.dict_idx), dev(inp.Bu), dev(inp.C), dev(inp.h0)
    fw = P.pdssm_fwd(u, W_sel, dic, W_d, b_d, Bu, C, h0, chunk=chunk, want_k=True, want_D=True)
    k, D = fw["k_star"], fw["D"]
    del u, Bu
    dims = P.make_dims(cfg.B, cfg.H, cfg.L, cfg.N, cfg.K, cfg.d, 0, bf)
    ws = torch.zeros(P.impulse_sens_workspace_bytes(dims, chunk), dtype=torch.uint8, device="cuda")
    dY = torch.empty((cfg.B, cfg.H, cfg.L, cfg.d), device="cuda")

    def step():
        P.pdssm_impulse_sens(k, dic, D, W_d, W_b, C, h0, chunk=chunk, workspace=ws, out=dY)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if P.workspace_error_flag(ws):
        raise RuntimeError("look-back wait gave up during warm-up")
    stream = torch.cuda.current_stream()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    wall, dur, timing = time_calls(torch, np, step, args.steps, stream,
                                   after=lambda: P.pdssm_workspace_status(ws, status))
    if int(status.item()):
        raise RuntimeError("a look-back wait gave up during timing")
    launch_s = float(np.mean(dur)) / 1e6
    ms_step = wall * 1e3 / args.steps
    alg = algorithmic_sens(cfg)
    achieved = alg / launch_s / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic_from_profile(cfg.name, "sens"),
            "algorithmic_bytes": alg, "launch_us": round(launch_s * 1e6, 2)}
    rec = {
        "metric": "state-updates/sec (B·H·L·N) PD-SSM impulse sensitivity dy_t/du_0 (fixed selections)",
        "value": cfg.state_updates / (ms_step / 1e3),
        "unit": "state-updates/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{cfg.name} impulse sensitivity: B={cfg.B} H={cfg.H} L={cfg.L} N={cfg.N} "
                               f"K={cfg.K} d={cfg.d} chunk={chunk}",
                   "B": cfg.B, "H": cfg.H, "L": cfg.L, "N": cfg.N, "K": cfg.K, "d_in": cfg.d, "chunk": chunk},
        "roofline": roof,
        "timing": timing,
        "kernel_hash": kernel_hash("sens"),
    }
    add_box(rec, torch, np)
    if args.copy_probe:
        copy_probe(torch)
    if not args.no_cpu_baseline:
        import oracle
        cores = len(os.sched_getaffinity(0))
        Hs, Ls = min(cfg.H, 16), cfg.L
        kh = k.cpu().numpy()[:, :Hs, :Ls]
        Dh = D.cpu().numpy()[:, :Hs, :Ls].astype(np.float64)
        t0 = time.perf_counter()
        oracle.impulse_sensitivity(kh, inp.dict_idx[:Hs], Dh, inp.W_d[:Hs], inp.W_b[:Hs], inp.C[:Hs],
                                   inp.h0[:, :Hs])
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": cfg.B * Hs * Ls * cfg.N / dt, "unit": "state-updates/s",
                               "cores": cores, "kind": "oracle", "seconds": round(dt, 3),
                               "sample": f"all {Ls} steps of {Hs} of the {cfg.H} heads of {cfg.name} "
                                         "(dense forward-mode tangent, single-threaded step loop)"}
    print(json.dumps(rec), flush=True)


def algorithmic_soft(cfg):
    """Minimum traffic of the soft-selection pipeline as the original model
    runs it: u read, every dense mixture M_t written (the O(L N^2)
    materialisation), the per-step maps and diagonals written and read back
    by the scan together with Bu, y written, plus parameters."""
    B, H, L, N, K, d = cfg.B, cfg.H, cfg.L, cfg.N, cfg.K, cfg.d
    es = 2 if cfg.dtype == "bf16" else 4
    steps = B * H * L
    u = B * (1 if cfg.u_shared else H) * L * d * es
    per_step = 4 * N * N + 2 * (4 * N + 4 * N) + 4 * N + 4
    params = H * K * d * es + H * N * d * es + H * N * 4 + H * K * N * N * 4 + H * N * 4 + 2 * B * H * N * 4
    return u + steps * per_step + params


def bench_soft(args, torch, np, P):
    """Time the soft-selection comparison path (pdssm_soft_select, then
    pdssm_scan_fwd_pidx) and, in the same run, the hard-selection forward pass
    on the same inputs, for the ratio of the two."""
    from pdssm_inputs import dense_dictionary, generate, get_config
    cfg = get_config(args.workload)
    chunk = args.chunk or cfg.chunk
    t0 = time.time()
    inp = generate(cfg)
    print(f"[bench] generated {cfg.name} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    bf = cfg.dtype == "bf16"
    pdt = torch.bfloat16 if bf else torch.float32

    def dev(x, dt=None):
        return torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt)

    u, W_sel, W_d = dev(inp.u, pdt), dev(inp.W_sel, pdt), dev(inp.W_d, pdt)
    b_d, dic, Bu, C, h0 = dev(inp.b_d), dev(inp.dict_idx), dev(inp.Bu), dev(inp.C), dev(inp.h0)
    Mh = dense_dictionary(cfg.H, cfg.K, cfg.N, cfg.seed)
    M = dev(Mh)
    B, H, L, N = cfg.B, cfg.H, cfg.L, cfg.N
    sel = {"M_t": torch.empty((B, H, L, N, N), device="cuda"),
           "P_idx": torch.empty((B, H, L, N), dtype=torch.int32, device="cuda"),
           "D": torch.empty((B, H, L, N), device="cuda")}
    dims = P.make_dims(B, H, L, N, 1, 8, 0, False)
    ws = torch.zeros(P.scan_workspace_bytes(dims, chunk), dtype=torch.uint8, device="cuda")
    so = {"y": torch.empty((B, H, L), device="cuda"), "h_L": torch.empty((B, H, N), device="cuda")}

    def step():
        P.pdssm_soft_select(u, W_sel, M, W_d, b_d, out=sel)
        P.pdssm_scan_fwd_pidx(sel["P_idx"], sel["D"], Bu, C, h0, chunk=chunk, workspace=ws, out=so)

    dimsf = P.make_dims(B, H, L, N, cfg.K, cfg.d, cfg.u_shared, bf)
    wsf = torch.empty(P.fwd_workspace_bytes(dimsf, cfg.chunk), dtype=torch.uint8, device="cuda")
    fo = {"y": torch.empty((B, H, L), device="cuda"), "h_L": torch.empty((B, H, N), device="cuda")}

    def hard():
        P.pdssm_fwd(u, W_sel, dic, W_d, b_d, Bu, C, h0, chunk=cfg.chunk, workspace=wsf, out=fo)

    for _ in range(args.warmup):
        step()
        hard()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    wall, dur, timing = time_calls(torch, np, step, args.steps, stream,
                                   after=lambda: P.pdssm_workspace_status(ws, status))
    if int(status.item()):
        raise RuntimeError("a look-back wait gave up during timing")
    _, dur_h, _ = time_calls(torch, np, hard, args.steps, stream)
    launch_s = float(np.mean(dur)) / 1e6
    ms_step = wall * 1e3 / args.steps
    alg = algorithmic_soft(cfg)
    achieved = alg / launch_s / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic_from_profile(cfg.name, "soft"),
            "algorithmic_bytes": alg, "launch_us": round(launch_s * 1e6, 2)}
    hard_us = float(np.mean(dur_h))
    rec = {
        "metric": "state-updates/sec (B·H·L·N) original soft-selection PD-SSM forward (dense mixture "
                  "materialised, column hardmax, scan)",
        "value": cfg.state_updates / (ms_step / 1e3),
        "unit": "state-updates/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if bf else "f32", "data": "synthetic",
        "config": {"workload": f"{cfg.name} soft selection: B={B} H={H} L={L} N={N} K={cfg.K} d={cfg.d} "
                               f"scan chunk={chunk}",
                   "B": B, "H": H, "L": L, "N": N, "K": cfg.K, "d_in": cfg.d, "chunk": chunk},
        "roofline": roof,
        "timing": timing,
        "hard_selection_us": round(hard_us, 2),
        "soft_over_hard_time": round(launch_s * 1e6 / hard_us, 3),
        "kernel_hash": kernel_hash("soft"),
    }
    add_box(rec, torch, np)
    if args.copy_probe:
        copy_probe(torch)
    if not args.no_cpu_baseline:
        import oracle
        cores = len(os.sched_getaffinity(0))
        Hs, Ls = min(H, 8), L
        t0 = time.perf_counter()
        r = oracle.soft_select(inp.u[:, :Hs, :Ls], inp.W_sel[:Hs], Mh[:Hs], inp.W_d[:Hs], inp.b_d[:Hs])
        oracle.scan_pidx(r["P_idx"], r["D"], inp.Bu[:, :Hs, :Ls], inp.C[:Hs], inp.h0[:, :Hs])
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": B * Hs * Ls * N / dt, "unit": "state-updates/s", "cores": cores,
                               "kind": "oracle", "seconds": round(dt, 3),
                               "sample": f"all {Ls} steps of {Hs} of the {H} heads of {cfg.name} "
                                         "(soft selection plus the dense sequential scan)"}
    print(json.dumps(rec), flush=True)


def bench_part(args, torch, np, P):
    """Time one stage of the forward pass alone: ``select`` (pdssm_select:
    scores, argmax, diagonal; k* and D written) or ``scan`` (pdssm_scan_fwd
    given k* and D, which come from the library's own selection call outside
    the timed region)."""
    from pdssm_inputs import generate, get_config, launch_chunk
    cfg = get_config(args.workload)
    chunk = args.chunk or launch_chunk(args.which, cfg)
    t0 = time.time()
    inp = generate(cfg)
    print(f"[bench] generated {cfg.name} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    bf = cfg.dtype == "bf16"
    pdt = torch.bfloat16 if bf else torch.float32

    def dev(x, dt=None):
        return torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt)

    B, H, L, N, K, d = cfg.B, cfg.H, cfg.L, cfg.N, cfg.K, cfg.d
    u, W_sel, W_d = dev(inp.u, pdt), dev(inp.W_sel, pdt), dev(inp.W_d, pdt)
    b_d, dic, Bu, C, h0 = dev(inp.b_d), dev(inp.dict_idx), dev(inp.Bu), dev(inp.C), dev(inp.h0)
    so = {"k_star": torch.empty((B, H, L), dtype=torch.int32, device="cuda"),
          "D": torch.empty((B, H, L, N), device="cuda")}
    P.pdssm_select(u, W_sel, W_d, b_d, out=so)
    es = 2 if bf else 4
    steps = B * H * L
    if args.which == "select":
        def step():
            P.pdssm_select(u, W_sel, W_d, b_d, out=so)
        alg = (B * (1 if cfg.u_shared else H) * L * d * es + steps * (4 + 4 * N)
               + H * K * d * es + H * N * d * es + H * N * 4)
        flops = 2 * (K + N) * d * steps
        what = "selection alone (scores, argmax, diagonal; k* and D written)"
    else:
        dims = P.make_dims(B, H, L, N, K, 8, 0, False)
        ws = torch.zeros(P.scan_workspace_bytes(dims, chunk), dtype=torch.uint8, device="cuda")
        oo = {"y": torch.empty((B, H, L), device="cuda"), "h_L": torch.empty((B, H, N), device="cuda")}

        def step():
            P.pdssm_scan_fwd(so["k_star"], dic, so["D"], Bu, C, h0, chunk=chunk, workspace=ws, out=oo)
        alg = steps * (4 + 4 * N + 4 * N + 4) + H * K * N * 4 + H * N * 4 + 2 * B * H * N * 4
        flops = 0
        what = "scan alone given k* and D (chunked, look-back)"
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    after = (lambda: P.pdssm_workspace_status(ws, status)) if args.which == "scan" else None
    wall, dur, timing = time_calls(torch, np, step, args.steps, stream, after=after)
    if int(status.item()):
        raise RuntimeError("a look-back wait gave up during timing")
    launch_s = float(np.mean(dur)) / 1e6
    ms_step = wall * 1e3 / args.steps
    t_hbm = alg / (PEAK_HBM_GBPS * 1e9)
    peak_mma = PEAK_BF16_TFLOPS if (bf and d >= 128) else PEAK_FP32_TFLOPS
    if flops and flops / (peak_mma * 1e12) > t_hbm:
        roof = {"bound": "mfma", "achieved": round(flops / launch_s / 1e12, 2), "peak": peak_mma,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(alg / launch_s / 1e9, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = traffic_from_profile(cfg.name, args.which)
    roof["algorithmic_bytes"] = alg
    roof["launch_us"] = round(launch_s * 1e6, 2)
    rec = {
        "metric": f"state-updates/sec (B·H·L·N) PD-SSM {what}",
        "value": cfg.state_updates / (ms_step / 1e3),
        "unit": "state-updates/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if bf else "f32", "data": "synthetic",
        "config": {"workload": f"{cfg.name} {args.which}: B={B} H={H} L={L} N={N} K={K} d={d} chunk={chunk}",
                   "B": B, "H": H, "L": L, "N": N, "K": K, "d_in": d, "chunk": chunk},
        "roofline": roof,
        "timing": timing,
        "kernel_hash": kernel_hash(args.which, cfg.name),
    }
    add_box(rec, torch, np)
    if args.copy_probe:
        copy_probe(torch)
    if not args.no_cpu_baseline:
        import oracle
        cores = len(os.sched_getaffinity(0))
        Hs = H
        t0 = time.perf_counter()
        if args.which == "select":
            oracle.select(inp.u[:, :Hs] if not cfg.u_shared else inp.u, inp.W_sel[:Hs], inp.W_d[:Hs],
                          inp.b_d[:Hs], cfg.u_shared)
        else:
            k_h = so["k_star"][:, :Hs].cpu().numpy()
            D_h = so["D"][:, :Hs].cpu().numpy().astype(np.float64)
            t0 = time.perf_counter()
            oracle.scan(k_h, inp.dict_idx[:Hs], D_h, inp.Bu[:, :Hs], inp.C[:Hs], inp.h0[:, :Hs])
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": B * Hs * L * N / dt, "unit": "state-updates/s", "cores": cores,
                               "kind": "oracle", "seconds": round(dt, 3),
                               "sample": f"whole {cfg.name} workload ({B}x{H}x{L} steps, N={N}), one run"}
    print(json.dumps(rec), flush=True)


def bench_multi(args, torch, np, P):
    """Time pdssm_fwd_wb_multi: the folded forward pass with n_out rows of C
    per head (the layer call: u in, y [B,H,L,n_out] out), at the longest
    chunk its on-chip output rows allow unless --chunk is given."""
    from pdssm_inputs import generate, get_config, launch_chunk
    cfg = get_config(args.workload)
    P_out = args.n_out
    chunk = args.chunk or min(launch_chunk("multi", cfg), 256 if P_out <= 2 else 128)
    t0 = time.time()
    inp = generate(cfg)
    print(f"[bench] generated {cfg.name} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    bf = cfg.dtype == "bf16"
    pdt = torch.bfloat16 if bf else torch.float32

    def dev(x, dt=None):
        return torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt)

    B, H, L, N, K, d = cfg.B, cfg.H, cfg.L, cfg.N, cfg.K, cfg.d
    rng = np.random.default_rng(100 + P_out)
    Cm = (rng.standard_normal((H, P_out, N)) / np.sqrt(N)).astype(np.float32)
    u, W_sel, W_d, W_b = dev(inp.u, pdt), dev(inp.W_sel, pdt), dev(inp.W_d, pdt), dev(inp.W_b, pdt)
    b_d, dic, C, h0 = dev(inp.b_d), dev(inp.dict_idx), dev(Cm), dev(inp.h0)
    dims = P.make_dims(B, H, L, N, K, d, cfg.u_shared, bf)
    ws = torch.empty(P.fwd_workspace_bytes(dims, chunk), dtype=torch.uint8, device="cuda")
    out = {"y": torch.empty((B, H, L, P_out), device="cuda"), "h_L": torch.empty((B, H, N), device="cuda")}

    def step():
        P.pdssm_fwd_wb_multi(u, W_sel, dic, W_d, b_d, W_b, C, h0, chunk=chunk, workspace=ws, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    wall, dur, timing = time_calls(torch, np, step, args.steps, stream,
                                   after=lambda: P.pdssm_workspace_status(ws, status))
    if int(status.item()):
        raise RuntimeError("a look-back wait gave up during timing")
    launch_s = float(np.mean(dur)) / 1e6
    ms_step = wall * 1e3 / args.steps
    es = 2 if bf else 4
    steps = B * H * L
    alg = (B * (1 if cfg.u_shared else H) * L * d * es + steps * 4 * P_out + 2 * B * H * N * 4
           + H * K * d * es + 2 * H * N * d * es + H * N * 4 + H * K * N * 4 + H * P_out * N * 4)
    flops = 2 * (K + 2 * N) * d * steps
    peak_mma = PEAK_BF16_TFLOPS if (bf and d >= 128) else PEAK_FP32_TFLOPS
    if flops / (peak_mma * 1e12) > alg / (PEAK_HBM_GBPS * 1e9):
        roof = {"bound": "mfma", "achieved": round(flops / launch_s / 1e12, 2), "peak": peak_mma,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(alg / launch_s / 1e9, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = traffic_from_profile(cfg.name, "multi")
    roof["algorithmic_bytes"] = alg
    roof["launch_us"] = round(launch_s * 1e6, 2)
    rec = {
        "metric": f"state-updates/sec (B·H·L·N) PD-SSM fwd select+scan with Bu = W_b u folded and {P_out} "
                  "outputs per head (C [H,n_out,N])",
        "value": cfg.state_updates / (ms_step / 1e3),
        "unit": "state-updates/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if bf else "f32", "data": "synthetic",
        "config": {"workload": f"{cfg.name} multi-output: B={B} H={H} L={L} N={N} K={K} d={d} n_out={P_out} "
                               f"chunk={chunk}",
                   "B": B, "H": H, "L": L, "N": N, "K": K, "d_in": d, "n_out": P_out, "chunk": chunk},
        "roofline": roof,
        "timing": timing,
        "kernel_hash": kernel_hash("multi", cfg.name),
    }
    add_box(rec, torch, np)
    if args.copy_probe:
        copy_probe(torch)
    if not args.no_cpu_baseline:
        import oracle
        cores = len(os.sched_getaffinity(0))
        t0 = time.perf_counter()
        oracle.forward_wb_multi(inp.u, inp.W_sel, inp.dict_idx, inp.W_d, inp.b_d, inp.W_b, Cm, inp.h0,
                                cfg.u_shared)
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": steps * N / dt, "unit": "state-updates/s", "cores": cores,
                               "kind": "oracle", "seconds": round(dt, 3),
                               "sample": f"whole {cfg.name} workload ({B}x{H}x{L} steps, N={N}, n_out={P_out}), "
                                         "one run"}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="impulse")
    ap.add_argument("--chunk", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="which",
                    choices=("fwd", "bwd", "fold", "sens", "soft", "scan", "select", "multi"), default="fwd",
                    help="forward pass (default), the gradient pass through the scan, the "
                         "forward pass with the drive Bu = W_b u folded into the selection GEMM, "
                         "the impulse sensitivity dy_t/du_0, the soft-selection comparison path, "
                         "one stage of the forward pass alone (scan, select), or the folded pass "
                         "with several outputs per head (multi)")
    ap.add_argument("--n-out", type=int, default=2, help="rows of C per head for --pass multi (1..4)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain copy kernel of known size (counter calibration)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs into profiles/ and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, args.workload, args.which)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the forward pass shards over independent sequences with no exchange).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import structured_sparse_state_pdssm_amd as P
    from pdssm_inputs import generate, get_config, launch_chunk

    torch.cuda.set_device(0)
    if args.which == "bwd":
        return bench_bwd(args, torch, np, P)
    if args.which == "sens":
        return bench_sens(args, torch, np, P)
    if args.which == "soft":
        return bench_soft(args, torch, np, P)
    if args.which in ("scan", "select"):
        return bench_part(args, torch, np, P)
    if args.which == "multi":
        return bench_multi(args, torch, np, P)
    cfg = get_config(args.workload)
    chunk = args.chunk or launch_chunk(args.which, cfg)
    t0 = time.time()
    inp = generate(cfg)
    print(f"[bench] generated {cfg.name} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    bf = cfg.dtype == "bf16"
    pdt = torch.bfloat16 if bf else torch.float32

    def dev(x, dt=None):
        return torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt)

    fold = args.which == "fold"
    u, W_sel, W_d = dev(inp.u, pdt), dev(inp.W_sel, pdt), dev(inp.W_d, pdt)
    b_d, dic, C, h0 = dev(inp.b_d), dev(inp.dict_idx), dev(inp.C), dev(inp.h0)
    Bu = None if fold else dev(inp.Bu)
    W_b = dev(inp.W_b, pdt) if fold else None
    dims = P.make_dims(cfg.B, cfg.H, cfg.L, cfg.N, cfg.K, cfg.d, cfg.u_shared, bf)
    ws = torch.empty(P.fwd_workspace_bytes(dims, chunk), dtype=torch.uint8, device="cuda")
    out = {"y": torch.empty((cfg.B, cfg.H, cfg.L), device="cuda"),
           "h_L": torch.empty((cfg.B, cfg.H, cfg.N), device="cuda")}

    def step():
        if fold:
            P.pdssm_fwd_wb(u, W_sel, dic, W_d, b_d, W_b, C, h0, chunk=chunk, workspace=ws, out=out)
        else:
            P.pdssm_fwd(u, W_sel, dic, W_d, b_d, Bu, C, h0, chunk=chunk, workspace=ws, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if P.workspace_error_flag(ws):
        raise RuntimeError("look-back wait gave up during warm-up")
    # per-launch durations with events on the stream the kernels run on
    stream = torch.cuda.current_stream()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    wall, dur, timing = time_calls(torch, np, step, args.steps, stream,
                                   after=lambda: P.pdssm_workspace_status(ws, status))
    if int(status.item()):
        raise RuntimeError("a look-back wait gave up during timing")
    ms_step = wall * 1e3 / args.steps
    avg_launch_s = float(np.mean(dur)) / 1e6

    alg_bytes, flops = algorithmic(cfg, fold)
    # the dominant cost: HBM traffic, except where the score GEMM outweighs it
    t_hbm = alg_bytes / (PEAK_HBM_GBPS * 1e9)
    t_mma = flops / ((PEAK_BF16_TFLOPS if (bf and cfg.d >= 128) else PEAK_FP32_TFLOPS) * 1e12)
    if t_mma > t_hbm:
        peak = PEAK_BF16_TFLOPS if (bf and cfg.d >= 128) else PEAK_FP32_TFLOPS
        achieved = flops / avg_launch_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s"}
    else:
        achieved = alg_bytes / avg_launch_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = traffic_from_profile(cfg.name, args.which)
    roof["algorithmic_bytes"] = alg_bytes
    roof["launch_us"] = round(avg_launch_s * 1e6, 2)

    rec = {
        "metric": METRIC_FOLD if fold else METRIC,
        "value": cfg.state_updates / (ms_step / 1e3),
        "unit": "state-updates/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}{' (drive folded)' if fold else ''}: B={cfg.B} H={cfg.H} "
                               f"L={cfg.L} N={cfg.N} K={cfg.K} d={cfg.d} chunk={chunk} "
                               f"u={'shared' if cfg.u_shared else 'per-head'}",
                   "B": cfg.B, "H": cfg.H, "L": cfg.L, "N": cfg.N, "K": cfg.K, "d_in": cfg.d,
                   "chunk": chunk, "u_dtype": cfg.dtype, "state_dtype": "f32"},
        "hbm_GBps": round(alg_bytes / avg_launch_s / 1e9, 1),
        "roofline": roof,
        "timing": timing,
        "kernel_hash": kernel_hash(args.which, cfg.name),
    }
    # secondary line: the same calls back to back with warm caches
    hot_s = timing["hot"]["mean_us"] / 1e6
    hot_ach = (flops / hot_s / 1e12) if roof["bound"] == "mfma" else (alg_bytes / hot_s / 1e9)
    rec["hot"] = {"label": "back-to-back calls, warm L2 and MALL (secondary)",
                  "value": cfg.state_updates / hot_s, "ms_per_step": round(hot_s * 1e3, 4),
                  "roofline_achieved": round(hot_ach, 2), "roofline_frac": round(hot_ach / roof["peak"], 4)}
    add_box(rec, torch, np)
    if args.copy_probe:
        copy_probe(torch)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(inp, fold)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
