"""Measure the schedule configurations of a layer shape across routed rows per expert
(tok_e = T*k/E) on the current GPU, report the fastest per tok_e and how close the
library's automatic choice (qmoe_plan) comes to it. The thresholds the library uses (the
decode/prefill crossover, rows per decode pass, the prefill row tile, the down split-K
guard) were measured this way.

  python -m quantized_mixture_experts_amd.tune_schedule [--format w4a16|mxfp4|nvfp4|fp8]
        [--H 7168] [--I 2048] [--E 48] [--k 8] [--kind uniform|zipf] [--steps 10]
        [--tok-e 4,8,...]

Candidates (the 4-bit formats, forced through qmoe_set_tuning): decode with 16 or 32 rows
per weight pass, prefill with 128- or 256-row tiles (split-K and the persistent grid as
the library plans them), and each tile height also without split-K and with one
work-group per tile instead of the persistent grid; the report gives, for the faster tile
height, what each of the two buys. Block FP8: decode against prefill. Every configuration
is timed in two round-robin rounds (the faster counts). Seeded synthetic inputs of the
benchmark recipe; one JSON line per tok_e, then a markdown table.
"""
import argparse
import json
import time

import numpy as np
import torch

from . import binding, inputs


def _time(fn, steps):
    """Median over three blocks of `steps` calls, after at least 30 ms of the same calls
    (the shader clock ramps up under load; a short warm-up biases whichever candidate runs
    first)."""
    t0 = time.perf_counter()
    n = 0
    while n < 3 or time.perf_counter() - t0 < 0.03:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ms = []
    for _ in range(3):
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b) / steps)
    return sorted(ms)[1]


def _fp8_quant_host(v, br, bc):
    # Inputs only: the GPU quantizer on a host array (codes and scales back on the host).
    q, s = binding.fp8_quantize_blocks(torch.from_numpy(np.ascontiguousarray(v)).cuda(), br, bc)
    return q.cpu().numpy(), s.cpu().numpy()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--format", default="w4a16", choices=["w4a16", "mxfp4", "nvfp4", "fp8"])
    ap.add_argument("--H", type=int, default=7168)
    ap.add_argument("--I", type=int, default=2048)
    ap.add_argument("--E", type=int, default=48)
    ap.add_argument("--k", type=int, default=8)
    ap.add_argument("--kind", default="uniform", choices=["uniform", "zipf"])
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--tok-e", default="4,8,16,24,32,40,48,64,96,128,160,192,256")
    args = ap.parse_args()
    H, I, E, k = args.H, args.I, args.E, args.k
    fmt = {"w4a16": binding.FORMAT_W4A16, "mxfp4": binding.FORMAT_MXFP4,
           "nvfp4": binding.FORMAT_NVFP4, "fp8": binding.FORMAT_FP8}[args.format]
    four_bit = args.format != "fp8"
    # one set of weights for every T
    if args.format == "w4a16":
        base = inputs.custom_w4a16_case(16, H, I, E, k, seed=5)
    elif args.format == "mxfp4":
        base = inputs.custom_mxfp4_case(16, H, I, E, k, seed=5)
    elif args.format == "nvfp4":
        base = inputs.custom_nvfp4_case(16, H, I, E, k, seed=5)
    else:
        base = inputs.custom_fp8_case(16, H, I, E, k, seed=5, quantize=_fp8_quant_host)
    dev = {n: torch.from_numpy(np.ascontiguousarray(
        base[n].view(np.int16) if base[n].dtype == np.uint16 else base[n])).cuda()
        for n in ("w13", "s13", "w2", "s2", "g13", "g2") if n in base}

    def forward(x, tids, twts, **kw):
        if args.format == "fp8":
            return binding.moe_fp8_block_forward(x[0], x[1], dev["w13"], dev["s13"], dev["w2"],
                                                 dev["s2"], tids, twts, **kw)
        if args.format == "nvfp4":
            return binding.moe_nvfp4_forward(x, dev["w13"], dev["s13"], dev["g13"], dev["w2"],
                                             dev["s2"], dev["g2"], tids, twts, **kw)
        f = binding.moe_mxfp4_forward if args.format == "mxfp4" else binding.moe_w4a16_forward
        return f(x, dev["w13"], dev["s13"], dev["w2"], dev["s2"], tids, twts, **kw)

    def measure(x, tids, twts, T, sched, **tune):
        binding.set_tuning(**tune)
        try:
            _, _, ws = binding.plan(fmt, T, H, I, E, k, sched)
            work = torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda")
            out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
            return _time(lambda: forward(x, tids, twts, schedule=sched, out=out, workspace=work),
                         args.steps)
        finally:
            binding.set_tuning()

    D, PF = binding.SCHEDULE_DECODE, binding.SCHEDULE_PREFILL
    rows = []
    for te in [int(v) for v in args.tok_e.split(",")]:
        T = max(1, te * E // k)
        rng = np.random.default_rng(1000 + te)
        ids, wts = inputs.routing(rng, T, E, k, args.kind)
        tids, twts = torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda()
        xf = rng.standard_normal((T, H), dtype=np.float32)
        # every configuration, timed in two round-robin rounds (the faster of the two)
        if four_bit:
            x = torch.from_numpy(inputs.bf16_bits(xf).view(np.int16)).cuda()
            configs = {"decode/16": (D, {"rows_per_pass": 16}),
                       "decode/32": (D, {"rows_per_pass": 32}),
                       "prefill/128": (PF, {"tile_rows": 128}),
                       "prefill/256": (PF, {"tile_rows": 256})}
            for tr_ in (128, 256):
                configs[f"prefill/{tr_}/no_split_k"] = (PF, {"tile_rows": tr_, "kslices": 1})
                configs[f"prefill/{tr_}/one_wg_per_tile"] = (PF, {"tile_rows": tr_, "tile_grid": 1})
        else:
            x = binding.fp8_quantize_blocks(torch.from_numpy(xf).cuda(), 1, 128)
            configs = {"decode": (D, {}), "prefill": (PF, {})}
        configs["auto"] = (binding.SCHEDULE_AUTO, {})
        ms = {}
        for _ in range(2):
            for name, (sc, tune) in configs.items():
                v = measure(x, tids, twts, T, sc, **tune)
                ms[name] = min(ms.get(name, v), v)
        auto_ms = ms.pop("auto")
        cand = {n: v for n, v in ms.items() if n.count("/") < 2}
        sched, block_m, _ = binding.plan(fmt, T, H, I, E, k)
        if four_bit:
            tr = 128 if cand["prefill/128"] <= cand["prefill/256"] else 256
            extra = {"no_split_k": ms[f"prefill/{tr}/no_split_k"],
                     "one_wg_per_tile": ms[f"prefill/{tr}/one_wg_per_tile"]}
            binding.set_tuning(tile_rows=tr)
            try:
                slices = binding.workspace_regions(fmt, T, H, I, E, k, PF).get("y", (0, 0))[1] // (
                    4 * T * k * H) if T * k else 0
            finally:
                binding.set_tuning()
        best = min(cand, key=cand.get)
        row = {"format": args.format, "kind": args.kind, "tok_e": te, "T": T,
               "candidates_ms": {n: round(v, 4) for n, v in cand.items()},
               "best": best, "best_ms": round(cand[best], 4),
               "auto": {"schedule": "decode" if sched == D else "prefill", "block_m": block_m,
                        "ms": round(auto_ms, 4)},
               "auto_over_best": round(auto_ms / cand[best], 3)}
        if four_bit:
            pf = cand[f"prefill/{tr}"]
            row["prefill_tile_rows"] = tr
            row["prefill_down_slices"] = slices
            row["split_k_gain"] = round(extra["no_split_k"] / pf, 3)
            row["persistent_gain"] = round(extra["one_wg_per_tile"] / pf, 3)
        rows.append(row)
        print(json.dumps(row), flush=True)

    # markdown summary
    if four_bit:
        print(f"\n| tok_e | T | decode 16 / 32 rows (ms) | prefill 128 / 256 rows (ms) | best | "
              f"auto (ms, / best) | down slices | no split-K / split | one per tile / "
              f"persistent |")
        print("|---|---|---|---|---|---|---|---|---|")
        for r in rows:
            c = r["candidates_ms"]
            print(f"| {r['tok_e']} | {r['T']} | {c['decode/16']} / {c['decode/32']} | "
                  f"{c['prefill/128']} / {c['prefill/256']} | {r['best']} | "
                  f"{r['auto']['schedule']} {r['auto']['ms']} ({r['auto_over_best']}) | "
                  f"{r['prefill_down_slices']} | {r['split_k_gain']} | {r['persistent_gain']} |")
    else:
        print("\n| tok_e | T | decode (ms) | prefill (ms) | best | auto (ms, / best) |")
        print("|---|---|---|---|---|---|")
        for r in rows:
            c = r["candidates_ms"]
            print(f"| {r['tok_e']} | {r['T']} | {c['decode']} | {c['prefill']} | {r['best']} | "
                  f"{r['auto']['schedule']} {r['auto']['ms']} ({r['auto_over_best']}) |")
    print(json.dumps({"summary": "auto within 5% of best at tok_e " + str(
        [r["tok_e"] for r in rows if r["auto_over_best"] <= 1.05]),
        "auto_off_by_more": [(r["tok_e"], r["auto_over_best"]) for r in rows
                             if r["auto_over_best"] > 1.05]}), flush=True)


if __name__ == "__main__":
    main()
