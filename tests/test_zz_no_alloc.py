"""moe_w4a16_forward_noalloc (the forward on the library's static per-GPU scratch, for
callers that cannot allocate) through the C ABI, against moe_w4a16_forward with a
workspace: two calls in a row, the second with a smaller input, each held to the same
bar as the forwards (bit-identical on the deterministic prefill tiles, 1e-2 per token row
on the decode schedule, whose fp32 atomics add in any order)."""
import numpy as np
import pytest
import torch

from gpu_util import TOL, bf16_out_to_f64, report, to_dev
from quantized_mixture_experts_amd import binding, inputs

pytestmark = pytest.mark.gpu


def _both(case, schedule):
    d = to_dev(case)
    ref = binding.moe_w4a16_forward(d["x"], d["w13"], d["s13"], d["w2"], d["s2"], d["topk_ids"],
                                    d["topk_weights"], schedule=schedule)
    torch.cuda.synchronize()
    got = binding.moe_w4a16_forward_noalloc(d["x"], d["w13"], d["s13"], d["w2"], d["s2"],
                                            d["topk_ids"], d["topk_weights"], schedule=schedule)
    torch.cuda.synchronize()
    return bf16_out_to_f64(got), bf16_out_to_f64(ref)


def test_noalloc_matches_workspace_forward_twice_smaller_second():
    # first: prefill tiles (deterministic: bit-identical); second, smaller: decode schedule
    print("[noalloc] call 1: 600 tokens, prefill tiles", flush=True)
    big = inputs.custom_w4a16_case(600, 512, 256, 4, 2, seed=61)
    got, ref = _both(big, binding.SCHEDULE_PREFILL)
    assert np.array_equal(got, ref)
    print("[noalloc] call 2: 40 tokens, decode schedule", flush=True)
    small = inputs.custom_w4a16_case(40, 1024, 512, 8, 4, seed=62)
    got, ref = _both(small, binding.SCHEDULE_DECODE)
    assert report("noalloc decode", got, ref).max() <= TOL


def test_noalloc_decode_workload():
    # the 32-token decode layer (18 MB of scratch), then a smaller decode batch of it
    cfg = inputs.CONFIGS["decode"]
    print("[noalloc] decode workload", flush=True)
    case = inputs.w4a16_case(cfg)
    got, ref = _both(case, binding.SCHEDULE_AUTO)
    assert report("noalloc decode workload", got, ref).max() <= TOL
    sub = dict(case, x=case["x"][:8], topk_ids=case["topk_ids"][:8],
               topk_weights=case["topk_weights"][:8])
    got, ref = _both(sub, binding.SCHEDULE_AUTO)
    assert report("noalloc decode 8 tokens", got, ref).max() <= TOL
