"""GPU W4A16 forward on the grouped layouts (moe_w4a16_grouped_contiguous and
moe_w4a16_grouped_masked through the C ABI) against the CPU oracle, per row within 1e-2
relative error; padding rows and rows past a count exactly 0. Ragged per-expert counts
in both schedules, the grouped prefill (48 experts x 128 rows) and decode (48 experts x 32
rows in a budget of 64) workloads at full size on sampled rows, and empty inputs."""
import numpy as np
import pytest
import torch

from gpu_util import TOL, bf16_out_to_f64, report, tile_cover_rows, to_dev
from quantized_mixture_experts_amd import binding, inputs

pytestmark = pytest.mark.gpu

SCHEDULES = [binding.SCHEDULE_DECODE, binding.SCHEDULE_PREFILL]


def _contiguous(case, schedule, expected_m=0):
    d = to_dev(case)
    out = binding.moe_w4a16_grouped_contiguous(d["a"], d["w13"], d["s13"], d["w2"], d["s2"],
                                               d["m_indices"], expected_m, schedule)
    torch.cuda.synchronize()
    return bf16_out_to_f64(out)


def _masked(case, schedule, expected_m=0):
    d = to_dev(case)
    out = binding.moe_w4a16_grouped_masked(d["a"], d["w13"], d["s13"], d["w2"], d["s2"],
                                           d["masked_m"], expected_m, schedule)
    torch.cuda.synchronize()
    return bf16_out_to_f64(out)


@pytest.mark.parametrize("counts,H,I,pad", [
    ([0, 1, 37, 128, 200, 15], 512, 256, 128),  # empty, single-row and multi-tile experts
    ([5, 3, 0, 21], 800, 352, 16),              # ragged against tiles and column chunks
    ([64, 64], 256, 256, 64),                   # aligned, no padding
])
@pytest.mark.parametrize("schedule", SCHEDULES)
def test_contiguous_matches_oracle(oracle_mod, counts, H, I, pad, schedule):
    print(f"[grouped contiguous] counts={counts} H={H} I={I} schedule={schedule}", flush=True)
    case = inputs.grouped_contiguous_case(counts, H, I, pad, seed=sum(counts) + H)
    got = _contiguous(case, schedule)
    ref = oracle_mod.w4a16_grouped_contiguous(case["a"], case["w13"], case["s13"], case["w2"],
                                              case["s2"], case["m_indices"])
    valid = case["m_indices"] >= 0
    e = report(f"contiguous {counts} sched={schedule}", got[valid], ref[valid])
    assert e.max() <= TOL
    assert np.all(got[~valid] == 0.0)


@pytest.mark.parametrize("counts,max_m,H,I", [
    ([0, 1, 16, 17, 40, 70, -3], 40, 512, 256),  # 70 > max_m (all rows), -3 (none)
    ([2, 9, 0], 12, 288, 96),
])
@pytest.mark.parametrize("schedule", SCHEDULES)
def test_masked_matches_oracle(oracle_mod, counts, max_m, H, I, schedule):
    print(f"[grouped masked] counts={counts} max_m={max_m} H={H} I={I} schedule={schedule}",
          flush=True)
    case = inputs.grouped_masked_case(counts, max_m, H, I, seed=max_m + H)
    got = _masked(case, schedule)
    ref = oracle_mod.w4a16_grouped_masked(case["a"], case["w13"], case["s13"], case["w2"],
                                          case["s2"], case["masked_m"])
    n = np.clip(np.array(counts), 0, max_m)
    valid = (np.arange(max_m)[None, :] < n[:, None]).ravel()
    e = report(f"masked {counts} sched={schedule}", got[valid], ref[valid])
    assert e.max() <= TOL
    assert np.all(got[~valid] == 0.0)


@pytest.mark.parametrize("name", ["grouped_prefill", "grouped_decode"])
def test_grouped_workloads_full_size(oracle_mod, name):
    g = inputs.GROUPED[name]
    print(f"[grouped workload] {name}", flush=True)
    case = inputs.grouped_case(name)
    # At least 512 rows: the first and last row of every expert's run (and of each 128-row
    # piece of it) plus seeded random rows; the masked layout's sample also holds rows past
    # the counts, which must be exactly zero.
    if g["layout"] == "contiguous":
        got = _contiguous(case, binding.SCHEDULE_AUTO, g["rows"])
        rows = tile_cover_rows(case["m_indices"].reshape(-1, 1), g["E"], 512, seed=g["seed"])
        ref = oracle_mod.w4a16_grouped_contiguous(case["a"], case["w13"], case["s13"], case["w2"],
                                                  case["s2"], case["m_indices"], rows=rows)
        valid = case["m_indices"][rows] >= 0
    else:
        got = _masked(case, binding.SCHEDULE_AUTO, g["rows"])
        n = np.clip(case["masked_m"], 0, g["max_m"])
        flat_ids = np.where(np.arange(g["max_m"])[None, :] < n[:, None],
                            np.arange(g["E"])[:, None], -1).reshape(-1, 1)
        rows = tile_cover_rows(flat_ids, g["E"], 512, seed=g["seed"])
        ref = oracle_mod.w4a16_grouped_masked(case["a"], case["w13"], case["s13"], case["w2"],
                                              case["s2"], case["masked_m"], rows=rows)
        valid = rows % g["max_m"] < g["rows"]
    assert valid.any() and (g["layout"] == "contiguous" or (~valid).any())
    e = report(name, got[rows][valid], ref[valid])
    assert e.max() <= TOL
    assert np.all(got[rows][~valid] == 0.0)


def test_expected_m_only_picks_the_schedule(oracle_mod):
    # A hint on either side of the crossover gives the same result within tolerance.
    case = inputs.grouped_masked_case([30, 7, 64, 0], 64, 512, 256, seed=5)
    lo = _masked(case, binding.SCHEDULE_AUTO, 1)
    hi = _masked(case, binding.SCHEDULE_AUTO, 1000)
    ref = oracle_mod.w4a16_grouped_masked(case["a"], case["w13"], case["s13"], case["w2"],
                                          case["s2"], case["masked_m"])
    valid = ref.any(axis=1)
    for got in (lo, hi):
        assert report("masked hint", got[valid], ref[valid]).max() <= TOL
        assert np.all(got[~valid] == 0.0)


def test_grouped_empty_inputs():
    w = inputs.grouped_masked_case([0, 0], 1, 256, 128, seed=1)
    d = to_dev(w)
    a = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    out = binding.moe_w4a16_grouped_contiguous(a, d["w13"], d["s13"], d["w2"], d["s2"],
                                               torch.empty(0, dtype=torch.int32, device="cuda"))
    assert out.shape == (0, 256)
    a3 = torch.empty((2, 0, 256), dtype=torch.bfloat16, device="cuda")
    out = binding.moe_w4a16_grouped_masked(a3, d["w13"], d["s13"], d["w2"], d["s2"], d["masked_m"])
    assert out.shape == (0, 256)
    # all rows past their counts: the output is all zero
    out = binding.moe_w4a16_grouped_masked(d["a"], d["w13"], d["s13"], d["w2"], d["s2"],
                                           d["masked_m"])
    torch.cuda.synchronize()
    assert out.shape == (2, 256) and torch.all(out == 0)
