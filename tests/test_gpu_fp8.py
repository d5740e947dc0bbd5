"""GPU block-FP8 path against the CPU oracle: the E4M3 block quantizer bit-exact, and the
W8A8 routed MoE forward within 1e-2 per token row (full-size workload on sampled rows,
ragged shapes in full)."""
import numpy as np
import pytest
import torch

from gpu_util import TOL, bf16_out_to_f64, report, to_dev
from quantized_mixture_experts_amd import binding, inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("R,C,br,bc", [(300, 520, 128, 128), (37, 1024, 1, 128), (5, 7, 2, 3),
                                       (128, 7168, 128, 128)])
def test_quantizer_bit_exact(oracle_mod, R, C, br, bc):
    print(f"[quant] R={R} C={C} block=[{br},{bc}]", flush=True)
    rng = np.random.default_rng(R + C)
    v = (rng.standard_normal((R, C)) * np.exp(rng.uniform(-8, 8, (R, 1)))).astype(np.float32)
    v[0, :3] = [0.0, -0.0, 1e-30]
    q, s = binding.fp8_quantize_blocks(torch.from_numpy(v).cuda(), br, bc)
    torch.cuda.synchronize()
    rq, rs = oracle_mod.fp8_quantize_blocks(v, br, bc)
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(q.cpu().numpy(), rq)


def _forward(case, schedule):
    d = to_dev(case)
    out = binding.moe_fp8_block_forward(d["a_q"], d["a_s"], d["w13"], d["s13"], d["w2"],
                                        d["s2"], d["topk_ids"], d["topk_weights"],
                                        schedule=schedule)
    torch.cuda.synchronize()
    return bf16_out_to_f64(out)


def _oracle(oracle_mod, case, rows):
    return oracle_mod.fp8_moe(case["a_q"], case["a_s"], case["w13"], case["s13"], case["w2"],
                              case["s2"], case["topk_ids"], case["topk_weights"], rows=rows)


_FP8_CASE = {}


@pytest.mark.parametrize("schedule", [binding.SCHEDULE_AUTO, binding.SCHEDULE_DECODE])
def test_fp8_workload(oracle_mod, schedule):
    cfg = inputs.CONFIGS["fp8"]
    print(f"[fp8] full workload schedule={schedule}", flush=True)
    if "case" not in _FP8_CASE:
        _FP8_CASE["case"] = inputs.fp8_case(cfg, oracle_mod.fp8_quantize_blocks)
    case = _FP8_CASE["case"]
    got = _forward(case, schedule)
    rows = inputs.sample_rows(cfg.T, 24, seed=cfg.seed)
    ref = _oracle(oracle_mod, case, rows)
    assert report(f"fp8/sched{schedule}", got[rows], ref).max() <= TOL


@pytest.mark.parametrize("T,H,I,E,k", [(40, 384, 256, 6, 3), (1, 128, 128, 1, 1), (80, 256, 384, 3, 2)])
@pytest.mark.parametrize("schedule", [binding.SCHEDULE_DECODE, binding.SCHEDULE_PREFILL])
def test_fp8_ragged(oracle_mod, T, H, I, E, k, schedule):
    print(f"[fp8] ragged T={T} H={H} I={I} E={E} k={k} schedule={schedule}", flush=True)
    case = inputs.custom_fp8_case(T, H, I, E, k, seed=T + H + I, quantize=oracle_mod.fp8_quantize_blocks)
    got = _forward(case, schedule)
    ref = _oracle(oracle_mod, case, None)
    assert report(f"fp8 ragged {T}x{H}x{I}", got, ref).max() <= TOL


def test_fp8_zero_routing_weights():
    import oracle
    case = inputs.custom_fp8_case(10, 256, 128, 4, 2, seed=3, quantize=oracle.fp8_quantize_blocks)
    case["topk_weights"][:] = 0
    assert np.all(_forward(case, binding.SCHEDULE_AUTO) == 0.0)
