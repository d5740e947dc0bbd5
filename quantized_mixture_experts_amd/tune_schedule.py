"""Measure the decode and prefill schedules of a layer shape across routed tokens per
expert (tok_e = T*k/E) on the current GPU and print where the prefill profile starts to
win. The library's automatic choice (qmoe_plan) uses the crossover measured this way.

  python -m quantized_mixture_experts_amd.tune_schedule [--format w4a16|mxfp4|nvfp4|fp8]
        [--H 7168] [--I 2048] [--E 48] [--k 8] [--steps 10]

Seeded synthetic inputs of the benchmark recipe; one JSON line per tok_e, then a summary.
"""
import argparse
import json

import numpy as np
import torch

from . import binding, inputs


def _time(fn, steps):
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


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
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--tok-e", default="4,8,16,24,32,40,48,64,96,128,192,256")
    args = ap.parse_args()
    H, I, E, k = args.H, args.I, args.E, args.k
    fmt = {"w4a16": binding.FORMAT_W4A16, "mxfp4": binding.FORMAT_MXFP4,
           "nvfp4": binding.FORMAT_NVFP4, "fp8": binding.FORMAT_FP8}[args.format]
    four_bit = args.format in ("w4a16", "mxfp4", "nvfp4")
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
        w = (dev["w13"], dev["s13"], dev["w2"], dev["s2"])
        if args.format == "nvfp4":
            return binding.moe_nvfp4_forward(x, dev["w13"], dev["s13"], dev["g13"], dev["w2"],
                                             dev["s2"], dev["g2"], tids, twts, **kw)
        f = binding.moe_mxfp4_forward if args.format == "mxfp4" else binding.moe_w4a16_forward
        return f(x, *w, tids, twts, **kw)
    rows = []
    for te in [int(v) for v in args.tok_e.split(",")]:
        T = max(1, te * E // k)
        rng = np.random.default_rng(1000 + te)
        ids, wts = inputs.routing(rng, T, E, k, "uniform")
        tids, twts = torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda()
        ms = {}
        for name, sched in (("decode", binding.SCHEDULE_DECODE), ("prefill", binding.SCHEDULE_PREFILL)):
            if four_bit:
                x = torch.from_numpy(inputs.bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
                                     .view(np.int16)).cuda()
                _, _, ws = binding.plan(fmt, T, H, I, E, k, sched)
                work = torch.empty(ws, dtype=torch.uint8, device="cuda")
                out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
                fn = lambda: forward(x, tids, twts, schedule=sched, out=out, workspace=work)
            else:
                xq, xs = binding.fp8_quantize_blocks(
                    torch.from_numpy(rng.standard_normal((T, H), dtype=np.float32)).cuda(), 1, 128)
                _, _, ws = binding.plan(fmt, T, H, I, E, k, sched)
                work = torch.empty(ws, dtype=torch.uint8, device="cuda")
                out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
                fn = lambda: binding.moe_fp8_block_forward(xq, xs, dev["w13"], dev["s13"], dev["w2"],
                                                           dev["s2"], tids, twts, schedule=sched,
                                                           out=out, workspace=work)
            ms[name] = _time(fn, args.steps)
        auto = binding.plan(fmt, T, H, I, E, k)[0]
        row = {"format": args.format, "tok_e": te, "T": T, "decode_ms": round(ms["decode"], 4),
               "prefill_ms": round(ms["prefill"], 4),
               "faster": "decode" if ms["decode"] <= ms["prefill"] else "prefill",
               "auto": "decode" if auto == binding.SCHEDULE_DECODE else "prefill"}
        rows.append(row)
        print(json.dumps(row), flush=True)
    first = next((r["tok_e"] for r in rows if r["faster"] == "prefill"), None)
    print(json.dumps({"summary": f"prefill first faster at tok_e = {first}",
                      "auto_mismatches": [r["tok_e"] for r in rows if r["faster"] != r["auto"]]}))


if __name__ == "__main__":
    main()
