"""GPU W4A16 routed MoE forward (moe_w4a16_forward through the C ABI) against the CPU
oracle, per token row within 1e-2 relative error: every workload at full size (all rows of
the tiny, decode and 384-expert layers; for the 8192-token prefill layer the rows holding
the first and last pair of every 128-row piece of every expert's segment, so every row
tile is checked, topped up to at least 512), both schedules, ragged and degenerate shapes,
and exact special cases."""
import numpy as np
import pytest
import torch

from gpu_util import TOL, bf16_out_to_f64, report, tile_cover_rows, to_dev
from quantized_mixture_experts_amd import binding, inputs

pytestmark = pytest.mark.gpu

_CASES = {}


def _case(name):
    if name not in _CASES:
        _CASES.clear()
        _CASES[name] = inputs.w4a16_case(inputs.CONFIGS[name])
    return _CASES[name]


def _forward(case, schedule):
    d = to_dev(case)
    out = binding.moe_w4a16_forward(d["x"], d["w13"], d["s13"], d["w2"], d["s2"], d["topk_ids"],
                                    d["topk_weights"], schedule=schedule)
    torch.cuda.synchronize()
    return bf16_out_to_f64(out)


def _oracle(oracle_mod, case, rows):
    return oracle_mod.w4a16_moe(case["x"], case["w13"], case["s13"], case["w2"], case["s2"],
                                case["topk_ids"], case["topk_weights"], rows=rows)


def _rows(name, case):
    cfg = inputs.CONFIGS[name]
    if name == "prefill":
        return tile_cover_rows(case["topk_ids"], cfg.E, 512, seed=cfg.seed)
    return np.arange(cfg.T, dtype=np.int64)


_REF = {}


def _reference(oracle_mod, name, case):
    """The oracle's rows of a workload, computed once for all its schedules (expert by
    expert: bit-identical to the per-token oracle, and fast enough for full size)."""
    if _REF.get("name") != name:
        rows = _rows(name, case)
        ref = oracle_mod.w4a16_moe_experts(case["x"], case["w13"], case["s13"], case["w2"],
                                           case["s2"], case["topk_ids"], case["topk_weights"],
                                           rows=rows)
        _REF.clear()
        _REF.update(name=name, rows=rows, ref=ref)
    return _REF["rows"], _REF["ref"]


_WORKLOADS = [(n, s) for n in ("tiny", "decode", "prefill", "full384")
              for s in (binding.SCHEDULE_AUTO, binding.SCHEDULE_DECODE, binding.SCHEDULE_PREFILL)
              if not (n == "prefill" and s == binding.SCHEDULE_DECODE)]


@pytest.mark.parametrize("name,schedule", _WORKLOADS)
def test_w4a16_workloads(oracle_mod, name, schedule):
    print(f"[w4a16] {name} schedule={schedule}", flush=True)
    case = _case(name)
    got = _forward(case, schedule)
    rows, ref = _reference(oracle_mod, name, case)
    err = report(f"{name}/sched{schedule}", got[rows], ref)
    assert err.max() <= TOL


@pytest.mark.parametrize("T,H,I,E,k", [
    (50, 800, 352, 10, 3),   # ragged against the 256-deep k step and the column chunks
    (1, 256, 128, 1, 1),     # one token, one expert: a dense SwiGLU FFN
    (70, 288, 96, 4, 4),     # every expert active, > 16 rows per expert
    (9, 32, 32, 3, 2),       # smallest group-aligned sizes
])
@pytest.mark.parametrize("schedule", [binding.SCHEDULE_DECODE, binding.SCHEDULE_PREFILL])
def test_w4a16_ragged_shapes(oracle_mod, T, H, I, E, k, schedule):
    print(f"[w4a16] ragged T={T} H={H} I={I} E={E} k={k} schedule={schedule}", flush=True)
    case = inputs.custom_w4a16_case(T, H, I, E, k, seed=T * 31 + H)
    got = _forward(case, schedule)
    ref = _oracle(oracle_mod, case, None)
    assert report(f"ragged {T}x{H}x{I}", got, ref).max() <= TOL


# Decode profile shapes with K a multiple of 512 in one or both GEMMs, which run the
# persistent stream kernels: down ranges that split items between work-groups, several
# 16-row blocks per expert (zipf routing), fewer units than work-groups, and column tiles
# past the end of h (I = 96) or of the output (H = 800).
@pytest.mark.parametrize("T,H,I,E,k,kind", [
    (40, 1024, 512, 8, 4, "uniform"),
    (300, 1536, 1536, 16, 4, "zipf"),
    (3, 2560, 1024, 64, 2, "uniform"),
    (60, 800, 512, 12, 3, "uniform"),
    (25, 1024, 96, 5, 2, "uniform"),
    (200, 512, 512, 64, 8, "zipf"),
])
def test_w4a16_decode_persistent_shapes(oracle_mod, T, H, I, E, k, kind):
    print(f"[w4a16] persistent T={T} H={H} I={I} E={E} k={k} {kind}", flush=True)
    case = inputs.custom_w4a16_case(T, H, I, E, k, seed=T * 17 + I, kind=kind)
    got = _forward(case, binding.SCHEDULE_DECODE)
    ref = _oracle(oracle_mod, case, None)
    assert report(f"persistent {T}x{H}x{I}x{E}", got, ref).max() <= TOL


# The align arrays a decode forward leaves in its workspace (sorted rows, block experts,
# padded row count, offsets) against the oracle's align, with 512 pairs over 256 experts,
# past both, and with ids outside [0, E). The workspace starts as 0xFF bytes, so every
# array must have been written.
@pytest.mark.parametrize("T,H,I,E,k,drop", [
    (64, 512, 256, 256, 8, True),    # 512 pairs over 256 experts
    (65, 512, 256, 128, 8, False),   # 520 pairs
    (20, 1024, 512, 257, 4, False),  # 257 experts
    (9, 512, 256, 8, 3, True),       # a few pairs, some ids outside [0, E)
])
def test_w4a16_decode_align_arrays(oracle_mod, T, H, I, E, k, drop):
    print(f"[w4a16] align arrays T={T} H={H} I={I} E={E} k={k} drop={drop}", flush=True)
    case = inputs.custom_w4a16_case(T, H, I, E, k, seed=T * 3 + E)
    if drop:
        case["topk_ids"][::3, -1] = np.resize(np.array([-1, E, E + 7], np.int32),
                                               case["topk_ids"][::3, -1].shape)
    fmt, sch = binding.FORMAT_W4A16, binding.SCHEDULE_DECODE
    _, block_m, need = binding.plan(fmt, T, H, I, E, k, sch)
    assert block_m == 16
    regions = binding.workspace_regions(fmt, T, H, I, E, k, sch)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    d = to_dev(case)
    out = binding.moe_w4a16_forward(d["x"], d["w13"], d["s13"], d["w2"], d["s2"], d["topk_ids"],
                                    d["topk_weights"], schedule=sch, workspace=ws)
    torch.cuda.synchronize()
    ref = _oracle(oracle_mod, case, None)
    assert report(f"align arrays {T}x{E}", bf16_out_to_f64(out), ref).max() <= TOL
    sorted_ids, expert_ids, ntp, offsets = oracle_mod.moe_align(case["topk_ids"], E, 16)
    wsn = ws.cpu().numpy()

    def region(name):
        off, size = regions[name]
        return wsn[off:off + size].view(np.int32)

    got_sorted, got_eids = region("sorted_ids"), region("expert_ids")
    P = T * k
    n, nb = min(got_sorted.size, sorted_ids.size), min(got_eids.size, expert_ids.size)
    assert np.array_equal(got_sorted[:n], sorted_ids[:n]) and np.all(got_sorted[n:] == P)
    assert np.array_equal(got_eids[:nb], expert_ids[:nb]) and np.all(got_eids[nb:] == -1)
    assert int(region("num_tokens_padded")[0]) == ntp
    if "expert_offsets" in regions:
        assert np.array_equal(region("expert_offsets")[:E + 1], offsets)


def test_w4a16_zero_routing_weights_give_exact_zero():
    case = inputs.custom_w4a16_case(20, 256, 128, 8, 2, seed=5)
    case["topk_weights"][:] = 0.0
    assert np.all(_forward(case, binding.SCHEDULE_AUTO) == 0.0)


def test_w4a16_zero_point_weights_give_zero():
    case = inputs.custom_w4a16_case(20, 256, 128, 8, 2, seed=6)
    case["w13"][:] = 0x88
    got = _forward(case, binding.SCHEDULE_AUTO)
    assert np.abs(got).max() <= 1e-6


def test_w4a16_dropped_ids(oracle_mod):
    case = inputs.custom_w4a16_case(12, 256, 128, 8, 3, seed=7)
    case["topk_ids"][:, 2] = np.array([-1, 8, 100, -5] * 3, np.int32)
    got = _forward(case, binding.SCHEDULE_AUTO)
    ref = _oracle(oracle_mod, case, None)
    assert report("dropped ids", got, ref).max() <= TOL


def test_w4a16_empty_batch():
    case = inputs.custom_w4a16_case(4, 256, 128, 8, 2, seed=8)
    d = to_dev(case)
    out = binding.moe_w4a16_forward(d["x"][:0], d["w13"], d["s13"], d["w2"], d["s2"],
                                    d["topk_ids"][:0], d["topk_weights"][:0])
    torch.cuda.synchronize()
    assert out.shape == (0, 256)


def test_w4a16_repeat_calls_agree():
    case = inputs.custom_w4a16_case(33, 512, 256, 6, 2, seed=10)
    a = _forward(case, binding.SCHEDULE_AUTO)
    b = _forward(case, binding.SCHEDULE_AUTO)
    # fp32 atomics may add in a different order; the results stay within rounding
    assert np.max(np.abs(a - b)) <= 1e-2 * np.max(np.abs(a))


# Prefill schedule with H and I multiples of 256: the tile kernels (256-row tiles, or
# 128-row tiles up to 136 routed rows per expert) and the per-pair combine.
_TILE_CASES = [
    (600, 512, 256, 4, 2, "uniform"),    # two row tiles per expert, ragged second tile
    (1000, 768, 512, 3, 3, "uniform"),   # every token on every expert: 4 tiles, 232-row tail
    (256, 256, 256, 1, 1, "uniform"),    # exactly one full tile; K = 256 (one weight block)
    (300, 256, 256, 16, 4, "zipf"),      # skewed routing with empty experts (128-row tiles)
    (128, 256, 512, 2, 2, "uniform"),    # 128-row tiles: exactly one full tile per expert
    (520, 512, 256, 8, 2, "uniform"),    # 128-row tiles: ragged second tiles (130 rows per expert)
    (200, 768, 256, 5, 3, "zipf"),       # 128-row tiles, skewed counts
]


@pytest.mark.parametrize("T,H,I,E,k,kind", _TILE_CASES)
def test_w4a16_prefill_tiles(oracle_mod, T, H, I, E, k, kind):
    print(f"[w4a16] tiles T={T} H={H} I={I} E={E} k={k} {kind}", flush=True)
    case = inputs.custom_w4a16_case(T, H, I, E, k, seed=T * 7 + I, kind=kind)
    got = _forward(case, binding.SCHEDULE_PREFILL)
    ref = _oracle(oracle_mod, case, None)
    assert report(f"tiles {T}x{H}x{I} E{E}", got, ref).max() <= TOL


# Split-K of the down GEMM: few experts leave the down tiles far from filling the GPU, so
# the plan splits each tile's K (I / 256 blocks) into slices whose partial rows the combine
# pass sums (the slice count each shape gets is pinned in test_abi_cpu.py).
@pytest.mark.parametrize("T,H,I,E,k,kind", [
    (300, 1024, 1024, 2, 1, "uniform"),   # 4 slices
    (300, 1024, 2048, 2, 1, "uniform"),   # 8 slices
    (200, 1024, 1024, 3, 2, "zipf"),      # 4 slices, skewed, two pairs per token
    (160, 512, 512, 1, 1, "uniform"),     # 2 slices, one expert
])
def test_w4a16_prefill_split_k(oracle_mod, T, H, I, E, k, kind):
    print(f"[w4a16] split-K T={T} H={H} I={I} E={E} k={k} {kind}", flush=True)
    case = inputs.custom_w4a16_case(T, H, I, E, k, seed=T * 5 + I, kind=kind)
    case["topk_ids"][::9, -1] = -1  # dropped slots
    got = _forward(case, binding.SCHEDULE_PREFILL)
    ref = _oracle(oracle_mod, case, None)
    assert report(f"split-K {T}x{H}x{I} E{E}", got, ref).max() <= TOL
    assert np.array_equal(got, _forward(case, binding.SCHEDULE_PREFILL))  # deterministic


@pytest.mark.parametrize("T,H,I,E,k,kind", [(600, 1024, 1024, 3, 2, "zipf"),
                                            (200, 512, 768, 5, 3, "uniform")])
def test_w4a16_tuning_overrides(oracle_mod, T, H, I, E, k, kind):
    """Every forced schedule configuration (qmoe_set_tuning) matches the oracle, and the
    persistent grid and one work-group per tile compute each tile identically."""
    print(f"[w4a16] tuning overrides T={T} H={H} I={I} E={E} k={k} {kind}", flush=True)
    case = inputs.custom_w4a16_case(T, H, I, E, k, seed=T + 3 * I, kind=kind)
    case["topk_ids"][::7, 0] = -1  # dropped slots
    ref = _oracle(oracle_mod, case, None)
    try:
        for tr in (128, 256):
            for ks in (1, 2):
                binding.set_tuning(tile_rows=tr, kslices=ks)
                pers = _forward(case, binding.SCHEDULE_PREFILL)
                binding.set_tuning(tile_rows=tr, kslices=ks, tile_grid=1)
                one = _forward(case, binding.SCHEDULE_PREFILL)
                assert np.array_equal(pers, one)
                assert report(f"tuned prefill rows={tr} slices={ks}", pers, ref).max() <= TOL
        for rpp in (16, 32):
            binding.set_tuning(rows_per_pass=rpp)
            got = _forward(case, binding.SCHEDULE_DECODE)
            assert report(f"tuned decode rows/pass={rpp}", got, ref).max() <= TOL
    finally:
        binding.set_tuning()


def test_w4a16_prefill_tiles_deterministic():
    case = inputs.custom_w4a16_case(600, 512, 256, 4, 2, seed=11)
    a = _forward(case, binding.SCHEDULE_PREFILL)
    b = _forward(case, binding.SCHEDULE_PREFILL)
    # no atomics on this path: repeated calls agree bit for bit
    assert np.array_equal(a, b)


def test_w4a16_prefill_tiles_zero_weights_and_dropped_ids(oracle_mod):
    case = inputs.custom_w4a16_case(400, 512, 256, 6, 3, seed=12)
    case["topk_ids"][::3, 1] = -1
    case["topk_ids"][1::5, 2] = 6
    ref = _oracle(oracle_mod, case, None)
    got = _forward(case, binding.SCHEDULE_PREFILL)
    assert report("tiles dropped ids", got, ref).max() <= TOL
    case["topk_weights"][:] = 0.0
    assert np.all(_forward(case, binding.SCHEDULE_PREFILL) == 0.0)


@pytest.mark.parametrize("schedule", [binding.SCHEDULE_DECODE, binding.SCHEDULE_PREFILL])
def test_w4a16_max_expert_count(oracle_mod, schedule):
    # QMOE_MAX_EXPERTS experts, 512 routed pairs: most experts are empty, the routed
    # ones hold one or two rows (decode: the general kernel at K = 512 is persistent for
    # gate_up; prefill: 128-row tiles, one per active expert).
    T, H, I, E, k = 64, 512, 256, 4096, 8
    print(f"[w4a16] max experts E={E} schedule={schedule}", flush=True)
    case = inputs.custom_w4a16_case(T, H, I, E, k, seed=4096)
    got = _forward(case, schedule)
    e = report(f"E={E} sched={schedule}", got, _oracle(oracle_mod, case, None))
    assert e.max() <= TOL
