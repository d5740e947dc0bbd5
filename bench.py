#!/usr/bin/env python3
"""Benchmark of the routed, weight-quantized MoE expert FFN on one MI355X.

One step = one full forward (align -> gate_up GEMM + SiLU*up -> down GEMM + weighted
scatter-add -> bf16 output) on seeded synthetic inputs already resident in HBM. The timed
steps are plain calls without instrumentation (--launch graph: replays of one captured HIP
graph); the per-kernel times come from a separate pass of 10 K steps in which every tenth
step has HIP events recorded around every kernel on its launch stream.

  python bench.py [--gpus 1] [--steps K] [--warmup W]
                  [--workload decode|prefill|fp8|full384|tiny|router|grouped_prefill|grouped_decode|
                              decode_mxfp4|prefill_mxfp4|decode_nvfp4|prefill_nvfp4]

Prints one JSON line. The default workload is the decode layer (32 tokens, hidden 7168,
intermediate 2048, 48 local experts, top-8, INT4 group-32 weights); its value is the
expert-weight bytes the forward must read divided by the step time (GB/s). Prefill-type
workloads report TFLOP/s of the routed expert FLOPs. The grouped workloads take rows
already grouped by expert (contiguous: 48 experts x 128 rows; masked: 48 experts x 32
valid rows in a budget of 64), one pair of weight 1 per row. The "roofline" object covers the
dominant kernel (the gate_up GEMM), timed with HIP events recorded on the stream it runs
on, over the timed steps. "cpu_baseline" times the CPU oracle on a bounded sample, on every
CPU the process may use (and on one CPU for the decode-sized layers), with the host's CPU
model and core count.

The metric has two halves: decode GB/s and prefill TFLOP/s. The default run (workload
decode) therefore also times the 8192-token Zipf-routed prefill layer with the same K and W
and reports it as the "prefill" object of the same line (its own value, ms_per_step,
stage times, roofline against the bf16 matrix-core peak and CPU baseline).
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

METRIC = "MoE FFN decode weight GB/s and prefill TFLOP/s, % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}
# Kernel sources whose counters a traffic record covers (a change voids the record).
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "fp8", "full384", "tiny", "router",
                             "grouped_prefill", "grouped_decode", "decode_mxfp4",
                             "prefill_mxfp4", "decode_nvfp4", "prefill_nvfp4"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="with the default decode workload, skip the prefill leg (the metric's "
                         "TFLOP/s half, reported as the \"prefill\" object)")
    ap.add_argument("--launch", default="eager", choices=["eager", "graph"],
                    help="how the timed steps are issued: eager library calls (default), or "
                         "replays of one captured HIP graph of the forward (slower on this "
                         "ROCm for these few-kernel forwards)")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="token rows of the CPU-oracle sample (0 = workload default)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the MoE step, run a plain device-to-device copy of MIB "
                         "MiB (the known-size reference for HBM byte counters) and exit")
    return ap.parse_args()


def time_oracle(fn, min_s=10.0, max_reps=100):
    """Seconds per call of fn, repeated until about min_s of CPU work (at most max_reps
    calls), and the number of calls."""
    t0 = time.perf_counter()
    fn()
    first = time.perf_counter() - t0
    reps = min(max_reps, max(1, math.ceil(min_s / max(first, 1e-6))))
    t0 = time.perf_counter()
    for _ in range(reps - 1):
        fn()
    total = first + (time.perf_counter() - t0)
    return total / reps, reps


def weight_bytes_per_expert(cfg):
    H, I = cfg.H, cfg.I
    if cfg.fmt in ("w4a16", "mxfp4", "nvfp4"):
        sb = {"w4a16": 2, "mxfp4": 1, "nvfp4": 2}[cfg.fmt]  # scale bytes per 32 k
        w13 = 2 * I * H // 2 + 2 * I * (H // 32) * sb
        w2 = H * I // 2 + H * (I // 32) * sb
    else:
        w13 = 2 * I * H + (2 * I // 128) * (H // 128) * 4
        w2 = H * I + (H // 128) * (I // 128) * 4
    return w13, w2


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_record(kernel_key, launches_ok):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3 counters,
    or None when there is no record or the kernel source changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE) or not launches_ok:
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f).get(kernel_key)
    if not rec or rec.get("source_sha") != source_digest(rec["sources"]):
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def host_cpu_info():
    """The CPU the oracle baseline runs on: model name, logical CPUs of the host, and the
    CPUs this process may run on (its affinity mask, capped by OMP_NUM_THREADS when set:
    the share of the host that belongs to this GPU)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    import oracle
    return {"model": model, "nproc": os.cpu_count(), "usable": oracle.default_threads()}


WORKLOAD_NAMES = {
    "decode": "decode W4A16", "prefill": "prefill W4A16 (Zipf routing)",
    "fp8": "block-FP8 W8A8", "full384": "full 384-expert W4A16", "tiny": "tiny W4A16",
    "decode_mxfp4": "decode MXFP4 (E2M1 + E8M0 per 32, bf16 activations)",
    "prefill_mxfp4": "prefill MXFP4 (E2M1 + E8M0 per 32, bf16 activations; Zipf routing)",
    "decode_nvfp4": "decode NVFP4 (E2M1 + E4M3 per 16 + fp32 per expert, bf16 activations)",
    "prefill_nvfp4": "prefill NVFP4 (E2M1 + E4M3 per 16 + fp32 per expert, bf16 "
                     "activations; Zipf routing)"}
# Token rows of the CPU-oracle sample per workload: about 10 s of oracle work on 16 CPUs.
CPU_ROWS = {"full384": 192, "prefill": 192, "fp8": 32, "prefill_mxfp4": 48,
            "prefill_nvfp4": 48, "grouped_prefill": 1536, "grouped_decode": 1536}
# Workloads whose oracle also runs on one CPU (the latency-sized layers), and its sample.
ONE_CORE_ROWS = {"tiny": 16, "decode": 8, "decode_mxfp4": 2, "decode_nvfp4": 2}


# One forward in this many is recorded with per-stage HIP events in the instrumented pass.
SAMPLE_EVERY = 10


def measure(workload, steps, warmup, launch, cpu_rows, cpu, np, torch, binding, inputs, lib):
    """Times one workload: an instrumented pass (per-stage HIP events on the launch stream,
    for the per-kernel times and the roofline), then K plain steps (`value`,
    `ms_per_step`). Returns the result fields as a dict."""
    import ctypes

    grouped = inputs.GROUPED.get(workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.time()

    def to_dev(arrays):
        return {k: torch.from_numpy(np.ascontiguousarray(v.view(np.int16) if v.dtype == np.uint16 else v)).to(dev)
                for k, v in arrays.items()}

    if grouped:
        g = grouped
        case = inputs.grouped_case(workload)
        masked = g["layout"] == "masked"
        if masked:
            counts = np.clip(case["masked_m"], 0, g["max_m"])
            rows_total = g["E"] * g["max_m"]
            ids = np.where(np.arange(g["max_m"])[None, :] < counts[:, None],
                           np.arange(g["E"])[:, None], -1).reshape(-1, 1)
        else:
            rows_total = case["a"].shape[0]
            ids = case["m_indices"].reshape(-1, 1)
        # k = 1: every row is one pair of weight 1
        cfg = inputs.MoEConfig(workload, rows_total, g["H"], g["I"], g["E"], 1, "w4a16",
                               "grouped", 0)
    elif inputs.CONFIGS[workload].fmt == "w4a16":
        cfg = inputs.CONFIGS[workload]
        case = inputs.w4a16_case(cfg)
        ids = case["topk_ids"]
    elif inputs.CONFIGS[workload].fmt == "mxfp4":
        cfg = inputs.CONFIGS[workload]
        case = inputs.mxfp4_case(cfg)
        ids = case["topk_ids"]
    elif inputs.CONFIGS[workload].fmt == "nvfp4":
        cfg = inputs.CONFIGS[workload]
        case = inputs.nvfp4_case(cfg)
        ids = case["topk_ids"]
    else:
        cfg = inputs.CONFIGS[workload]

        def gpu_quant(v, br, bc):
            q, s = binding.fp8_quantize_blocks(torch.from_numpy(v).to(dev), br, bc)
            return q.cpu().numpy(), s.cpu().numpy()
        case = inputs.fp8_case(cfg, gpu_quant)
        ids = case["topk_ids"]
    d = to_dev(case)
    gen_s = time.time() - t_gen

    fmt = {"w4a16": binding.FORMAT_W4A16, "mxfp4": binding.FORMAT_MXFP4,
           "nvfp4": binding.FORMAT_NVFP4, "fp8": binding.FORMAT_FP8}[cfg.fmt]
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    if grouped:
        # The schedule AUTO picks from the expected rows per expert (k = 1).
        chosen = binding.plan(fmt, g["rows"] * cfg.E, cfg.H, cfg.I, cfg.E, 1)[0]
        ws_bytes = binding.grouped_workspace_bytes(masked, g["max_m"] if masked else cfg.T, cfg.H,
                                                   cfg.I, cfg.E, g["rows"])
    else:
        chosen, block_m, ws_bytes = binding.plan(fmt, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k)
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    if grouped and masked:
        a3 = d["a"]

        def step():
            binding.moe_w4a16_grouped_masked(a3, d["w13"], d["s13"], d["w2"], d["s2"],
                                             d["masked_m"], g["rows"], out=out,
                                             workspace=workspace)
    elif grouped:
        def step():
            binding.moe_w4a16_grouped_contiguous(d["a"], d["w13"], d["s13"], d["w2"], d["s2"],
                                                 d["m_indices"], g["rows"], out=out,
                                                 workspace=workspace)
    elif cfg.fmt == "w4a16":
        def step():
            binding.moe_w4a16_forward(d["x"], d["w13"], d["s13"], d["w2"], d["s2"], d["topk_ids"],
                                      d["topk_weights"], out=out, workspace=workspace)
    elif cfg.fmt == "mxfp4":
        def step():
            binding.moe_mxfp4_forward(d["x"], d["w13"], d["s13"], d["w2"], d["s2"], d["topk_ids"],
                                      d["topk_weights"], out=out, workspace=workspace)
    elif cfg.fmt == "nvfp4":
        def step():
            binding.moe_nvfp4_forward(d["x"], d["w13"], d["s13"], d["g13"], d["w2"], d["s2"],
                                      d["g2"], d["topk_ids"], d["topk_weights"], out=out,
                                      workspace=workspace)
    else:
        def step():
            binding.moe_fp8_block_forward(d["a_q"], d["a_s"], d["w13"], d["s13"], d["w2"], d["s2"],
                                          d["topk_ids"], d["topk_weights"], out=out,
                                          workspace=workspace)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # Instrumented pass: K * SAMPLE_EVERY eager steps, of which every SAMPLE_EVERY-th has
    # HIP events recorded by the library around every stage launch on the launch stream;
    # the per-kernel times (and the roofline) come from these K sampled forwards. When
    # every forward is bracketed, the pauses the events add between kernels move the GPU's
    # power state within a few steps and the HBM-bound kernels slow down by up to a fifth
    # (decode gate_up 152 -> 182 us in kernel traces); sampled forwards run amid unrecorded
    # ones, as the timed steps do. Room for every launch of a stage: align holds up to
    # three per forward (the grouped layouts' per-row routing, the sort, the row gather).
    if lib.qmoe_timing_begin(steps * 3) != 0 or lib.qmoe_timing_pause(1) != 0:
        raise RuntimeError(lib.qmoe_last_error())
    torch.cuda.synchronize()
    te0 = time.perf_counter()
    for i in range(steps * SAMPLE_EVERY):
        sampled = i % SAMPLE_EVERY == SAMPLE_EVERY - 1
        if sampled:
            lib.qmoe_timing_pause(0)
        step()
        if sampled:
            lib.qmoe_timing_pause(1)
    torch.cuda.synchronize()
    te1 = time.perf_counter()
    ms_sum = (ctypes.c_float * 6)()
    counts = (ctypes.c_int32 * 6)()
    if lib.qmoe_timing_end(ms_sum, counts) != 0:
        raise RuntimeError(lib.qmoe_last_error())
    stage_names = ["zero", "align", "gate_up", "requant", "down", "cast"]
    # Per forward: a stage can hold more than one launch (align = sort + row gather).
    stage_ms = {n: (ms_sum[i] / steps if counts[i] else None)
                for i, n in enumerate(stage_names)}
    instrumented_ms = (te1 - te0) * 1e3 / (steps * SAMPLE_EVERY)

    # Timed pass: K steps without instrumentation, as one captured graph replayed K times
    # (the forward's kernels are launched on the capturing stream; nothing in it allocates
    # or synchronizes) or as eager calls.
    if launch == "graph":
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step()
        run = graph.replay
    else:
        run = step
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    valid = (ids >= 0) & (ids < cfg.E)
    touched = int(np.unique(ids[valid]).size)
    pairs = int(valid.sum())  # routed (row, expert) pairs
    w13_b, w2_b = weight_bytes_per_expert(cfg)
    weight_bytes = touched * (w13_b + w2_b)
    flops = pairs * (2 * cfg.H * 2 * cfg.I + 2 * cfg.I * cfg.H)
    dtype = "fp8" if cfg.fmt == "fp8" else "bf16"
    hbm_bound = chosen == binding.SCHEDULE_DECODE
    if hbm_bound:
        value, unit = weight_bytes / (ms_per_step * 1e-3) / 1e9, "GB/s"
    else:
        value, unit = flops / (ms_per_step * 1e-3) / 1e12, "TFLOP/s"

    # Dominant kernel: gate_up (two thirds of the weight bytes, deep K = hidden size).
    gu_ms = ms_sum[2] / counts[2]  # per launch (one per forward)
    if hbm_bound:
        per_launch = touched * w13_b
        achieved = per_launch / (gu_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        per_launch = pairs * 2 * cfg.H * 2 * cfg.I
        achieved = per_launch / (gu_ms * 1e-3) / 1e12
        peak = MFMA_PEAK_TFLOPS[dtype]
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
    kernel_key = f"{workload}/gate_up"
    roof["kernel"] = kernel_key
    roof["kernel_ms"] = round(gu_ms, 4)
    roof["algorithmic_per_launch"] = per_launch
    roof["traffic"] = traffic_record(kernel_key, counts[2] > 0)

    cpu_base = None
    if cpu:
        import oracle
        host = host_cpu_info()
        nthreads = host["usable"]
        valid_rows = np.flatnonzero(valid.any(axis=1))

        def run_oracle(rows, nthreads):
            if grouped and masked:
                oracle.w4a16_grouped_masked(case["a"], case["w13"], case["s13"], case["w2"], case["s2"],
                                            case["masked_m"], rows=rows, nthreads=nthreads)
            elif grouped:
                oracle.w4a16_grouped_contiguous(case["a"], case["w13"], case["s13"], case["w2"],
                                                case["s2"], case["m_indices"], rows=rows,
                                                nthreads=nthreads)
            elif cfg.fmt == "nvfp4":
                oracle.nvfp4_moe(case["x"], case["w13"], case["s13"], case["g13"], case["w2"],
                                 case["s2"], case["g2"], case["topk_ids"], case["topk_weights"],
                                 rows=rows, nthreads=nthreads)
            elif cfg.fmt == "mxfp4":
                oracle.mxfp4_moe(case["x"], case["w13"], case["s13"], case["w2"], case["s2"],
                                 case["topk_ids"], case["topk_weights"], rows=rows, nthreads=nthreads)
            elif cfg.fmt == "w4a16":
                oracle.w4a16_moe(case["x"], case["w13"], case["s13"], case["w2"], case["s2"],
                                 case["topk_ids"], case["topk_weights"], rows=rows, nthreads=nthreads)
            else:
                oracle.fp8_moe(case["a_q"], case["a_s"], case["w13"], case["s13"], case["w2"],
                               case["s2"], case["topk_ids"], case["topk_weights"], rows=rows,
                               nthreads=nthreads)

        def timed(nrows, nthreads):
            rows = valid_rows[inputs.sample_rows(valid_rows.size, nrows, seed=cfg.seed)]
            cpu_s, reps = time_oracle(lambda: run_oracle(rows, nthreads))
            # The oracle loops per (row, slot) and re-reads the expert's weights for each,
            # so the full workload costs (rows holding a pair) / nrows times the sample.
            full_s = cpu_s * valid_rows.size / len(rows)
            v = (weight_bytes / full_s / 1e9) if hbm_bound else (flops / full_s / 1e12)
            sample = (f"{len(rows)} of {valid_rows.size} rows (all {cfg.k} slots each), "
                      f"{cpu_s:.2f} s per run (mean of {reps}) on {nthreads} threads, "
                      f"scaled by {valid_rows.size}/{len(rows)}")
            return round(v, 6), sample

        v, sample = timed(cpu_rows or CPU_ROWS.get(workload, cfg.T), nthreads)
        cpu_base = {"value": v, "unit": unit, "cores": nthreads, "kind": "oracle",
                    "sample": sample, "host": host}
        if workload in ONE_CORE_ROWS:
            v1, sample1 = timed(ONE_CORE_ROWS[workload], 1)
            cpu_base["one_core"] = {"value": v1, "unit": unit, "cores": 1, "sample": sample1}

    if grouped:
        layout = (f"masked, {g['rows']} valid rows per expert in a budget of {g['max_m']}"
                  if masked else f"contiguous, {g['rows']} rows per expert")
        name = (f"grouped W4A16 ({layout}): {cfg.T} rows, hidden {cfg.H}, intermediate "
                f"{cfg.I}, {cfg.E} experts, one pair of weight 1 per row")
    else:
        name = (f"{WORKLOAD_NAMES[workload]}: {cfg.T} tokens, hidden {cfg.H}, intermediate "
                f"{cfg.I}, {cfg.E} experts, top-{cfg.k}")
    return {
        "value": round(value, 3), "unit": unit, "ms_per_step": round(ms_per_step, 4),
        "dtype": dtype,
        "config": {"workload": name,
                   "tokens": cfg.T, "hidden": cfg.H, "intermediate": cfg.I, "experts": cfg.E,
                   "top_k": cfg.k, "schedule": ["auto", "decode", "prefill"][chosen],
                   "routed_pairs": pairs, "touched_experts": touched,
                   "weight_bytes": weight_bytes, "flops": flops},
        "launch": launch,
        "instrumented_ms_per_step": round(instrumented_ms, 4),
        "stage_ms": {k: (round(v, 4) if v is not None else None) for k, v in stage_ms.items()},
        "roofline": roof,
        "cpu_baseline": cpu_base,
        "input_gen_s": round(gen_s, 1),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the MoE "
              "path has no multi-GPU mode here", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": args.steps}))
        return

    from quantized_mixture_experts_amd import binding, inputs

    if not os.path.exists(binding.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    lib = binding.load()

    if args.workload == "router":
        bench_router(args, np, torch, binding, inputs)
        return

    cpu = not args.no_cpu_baseline
    res = measure(args.workload, args.steps, args.warmup, args.launch, args.cpu_rows, cpu,
                  np, torch, binding, inputs, lib)
    line = {
        "metric": METRIC, "value": res["value"], "unit": res["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": res["dtype"],
        "data": "synthetic (seeded; random-init quantized expert weights)",
        "config": res["config"],
    }
    for key in ("launch", "instrumented_ms_per_step", "stage_ms", "roofline", "cpu_baseline",
                "input_gen_s"):
        line[key] = res[key]
    # The metric's second half: the default run also times the 8192-token Zipf prefill
    # layer (TFLOP/s against the bf16 matrix-core peak), with the same K and W.
    if args.workload == "decode" and not args.no_prefill:
        torch.cuda.empty_cache()
        pre = measure("prefill", args.steps, args.warmup, args.launch, 0, cpu,
                      np, torch, binding, inputs, lib)
        line["prefill"] = {k: pre[k] for k in ("value", "unit", "ms_per_step", "dtype", "config",
                                                "instrumented_ms_per_step", "stage_ms",
                                                "roofline", "cpu_baseline", "input_gen_s")}
        line["prefill"]["steps"] = args.steps
        line["prefill"]["warmup"] = args.warmup
    line["device"] = torch.cuda.get_device_name(0)
    print(json.dumps(line), flush=True)


def bench_router(args, np, torch, binding, inputs):
    """Router step before align: softmax -> top-8 -> renormalization over the 384 experts of
    the full layer for a prefill batch of 8192 tokens, ids mapped to one GPU's share of
    48 experts (expert parallelism over 8). Bound: HBM (logits read, ids and weights
    written once); timed with HIP events on the launch stream."""
    T, E, k, share = 8192, 384, 8, 48
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rng = np.random.default_rng(97)
    logits_h = inputs.router_logits(rng, T, E, "zipf")
    emap_h = np.full(E, -1, np.int32)
    emap_h[share:2 * share] = np.arange(share, dtype=np.int32)
    logits = torch.from_numpy(logits_h).to(dev)
    emap = torch.from_numpy(emap_h).to(dev)
    stream = torch.cuda.current_stream()

    def step():
        return binding.moe_topk_softmax(logits, k, True, emap, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # One launch through the Python binding costs the host more than the kernel runs, so
    # the launches are queued behind a GPU spin long enough for the host to stay ahead:
    # the events then time the kernels back to back (launch gaps included).
    ev0.record(stream)
    torch.cuda._sleep(1_000_000)
    ev1.record(stream)
    torch.cuda.synchronize()
    cycles_per_ms = 1_000_000 / max(ev0.elapsed_time(ev1), 1e-3)
    t0 = time.perf_counter()
    spin_ms = 2.0 + 0.05 * args.steps
    torch.cuda._sleep(int(cycles_per_ms * spin_ms))
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    t_queued = time.perf_counter()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    host_ms = (t_queued - t0) * 1e3 / args.steps  # host time to issue one launch
    host_ahead = (t_queued - t0) * 1e3 < spin_ms
    nbytes = T * E * 4 + T * k * 8
    achieved = nbytes / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        rows = T
        cpu_s, reps = time_oracle(lambda: oracle.topk_softmax(logits_h[:rows], k, True, emap_h))
        full_s = cpu_s * T / rows
        cpu = {"value": round(nbytes / full_s / 1e9, 6), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"{rows} of {T} token rows, {cpu_s:.3f} s per run (mean of {reps}) "
                         f"on 1 thread"}
    line = {
        "metric": "router GB/s (logits read, ids and weights written), % of HBM roofline",
        "value": round(achieved, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "host_ms_per_launch": round(host_ms, 5),
        "timing": ("launches queued behind a GPU spin; events time the kernels back to back"
                   if host_ahead else "host-bound: the launches did not stay ahead of the GPU"),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded Zipf router logits)",
        "config": {"workload": f"router: {T} tokens, {E} experts, top-{k}, renormalized, "
                               f"ids mapped to {share} local experts",
                   "tokens": T, "experts": E, "top_k": k, "local_experts": share},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "kernel": "router/topk_softmax", "kernel_ms": round(ms, 5),
                     "algorithmic_per_launch": nbytes, "traffic": None},
        "cpu_baseline": cpu,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
