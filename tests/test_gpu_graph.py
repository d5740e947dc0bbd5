"""The forward captured once into a HIP graph (through torch.cuda.CUDAGraph on the
binding's launch stream) and replayed several times, with unrelated eager forwards and
synchronizations between the replays: every replay must reproduce the eager result. The
tile paths (prefill W4A16 and block FP8) are deterministic and must match bit for bit; the
decode path adds its rows with fp32 atomics, whose order may change between runs."""
import numpy as np
import pytest
import torch

from gpu_util import bf16_out_to_f64, row_rel_err, to_dev
from quantized_mixture_experts_amd import binding, inputs

pytestmark = pytest.mark.gpu


def _w4a16_runner(case, schedule):
    d = to_dev(case)
    T, H = case["x"].shape
    E, twoI, _ = case["w13"].shape
    k = case["topk_ids"].shape[1]
    _, _, ws = binding.plan(binding.FORMAT_W4A16, T, H, twoI // 2, E, k, schedule)
    work = torch.empty(ws, dtype=torch.uint8, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

    def run():
        binding.moe_w4a16_forward(d["x"], d["w13"], d["s13"], d["w2"], d["s2"], d["topk_ids"],
                                  d["topk_weights"], schedule=schedule, out=out, workspace=work)
    return run, out


def _fp8_runner(case, schedule):
    d = to_dev(case)
    T, H = case["a_q"].shape
    E, twoI, _ = case["w13"].shape
    k = case["topk_ids"].shape[1]
    _, _, ws = binding.plan(binding.FORMAT_FP8, T, H, twoI // 2, E, k, schedule)
    work = torch.empty(ws, dtype=torch.uint8, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

    def run():
        binding.moe_fp8_block_forward(d["a_q"], d["a_s"], d["w13"], d["s13"], d["w2"], d["s2"],
                                      d["topk_ids"], d["topk_weights"], schedule=schedule,
                                      out=out, workspace=work)
    return run, out


def _capture(run):
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        run()
    return graph


def _check_replays(run, out, other, exact):
    run()
    torch.cuda.synchronize()
    eager = bf16_out_to_f64(out)
    graph = _capture(run)
    for i in range(3):
        out.zero_()
        other()  # unrelated eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = bf16_out_to_f64(out)
        if exact:
            assert np.array_equal(got, eager), f"replay {i} differs"
        else:
            assert row_rel_err(got, eager).max() <= 1e-3, f"replay {i} differs"


@pytest.mark.parametrize("schedule,shape", [
    (binding.SCHEDULE_DECODE, (24, 512, 256, 8, 4)),
    (binding.SCHEDULE_PREFILL, (600, 512, 256, 4, 2)),
])
def test_w4a16_graph_replays(schedule, shape):
    print(f"[graph] w4a16 schedule={schedule} shape={shape}", flush=True)
    run, out = _w4a16_runner(inputs.custom_w4a16_case(*shape, seed=31), schedule)
    other, _ = _w4a16_runner(inputs.custom_w4a16_case(*shape, seed=32), schedule)
    _check_replays(run, out, other, exact=schedule == binding.SCHEDULE_PREFILL)


def test_fp8_graph_replays():
    import oracle
    print("[graph] fp8 prefill", flush=True)
    shape = (400, 512, 256, 4, 2)
    run, out = _fp8_runner(inputs.custom_fp8_case(*shape, seed=33,
                                                  quantize=oracle.fp8_quantize_blocks),
                           binding.SCHEDULE_PREFILL)
    other, _ = _fp8_runner(inputs.custom_fp8_case(*shape, seed=34,
                                                  quantize=oracle.fp8_quantize_blocks),
                           binding.SCHEDULE_PREFILL)
    _check_replays(run, out, other, exact=True)


def _mxfp4_runner(case, schedule):
    d = to_dev(case)
    T, H = case["x"].shape
    E, twoI, _ = case["w13"].shape
    k = case["topk_ids"].shape[1]
    _, _, ws = binding.plan(binding.FORMAT_MXFP4, T, H, twoI // 2, E, k, schedule)
    work = torch.empty(ws, dtype=torch.uint8, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

    def run():
        binding.moe_mxfp4_forward(d["x"], d["w13"], d["s13"], d["w2"], d["s2"], d["topk_ids"],
                                  d["topk_weights"], schedule=schedule, out=out, workspace=work)
    return run, out


@pytest.mark.parametrize("schedule,shape", [
    (binding.SCHEDULE_DECODE, (96, 1024, 512, 6, 2)),   # 32 rows per expert: two-block passes
    (binding.SCHEDULE_PREFILL, (300, 512, 256, 8, 2)),  # 75 rows per expert: 128-row tiles
    (binding.SCHEDULE_PREFILL, (600, 512, 256, 4, 2)),  # 300 rows per expert: 256-row tiles
])
def test_mxfp4_graph_replays(schedule, shape):
    print(f"[graph] mxfp4 schedule={schedule} shape={shape}", flush=True)
    run, out = _mxfp4_runner(inputs.custom_mxfp4_case(*shape, seed=35), schedule)
    other, _ = _mxfp4_runner(inputs.custom_mxfp4_case(*shape, seed=36), schedule)
    _check_replays(run, out, other, exact=schedule == binding.SCHEDULE_PREFILL)


def _nvfp4_runner(case, schedule):
    d = to_dev(case)
    T, H = case["x"].shape
    E, twoI, _ = case["w13"].shape
    k = case["topk_ids"].shape[1]
    _, _, ws = binding.plan(binding.FORMAT_NVFP4, T, H, twoI // 2, E, k, schedule)
    work = torch.empty(ws, dtype=torch.uint8, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

    def run():
        binding.moe_nvfp4_forward(d["x"], d["w13"], d["s13"], d["g13"], d["w2"], d["s2"], d["g2"],
                                  d["topk_ids"], d["topk_weights"], schedule=schedule, out=out,
                                  workspace=work)
    return run, out


@pytest.mark.parametrize("schedule,shape", [
    (binding.SCHEDULE_DECODE, (96, 1024, 512, 6, 2)),   # 32 rows per expert: two-block passes
    (binding.SCHEDULE_PREFILL, (300, 512, 256, 8, 2)),  # 75 rows per expert: 128-row tiles
])
def test_nvfp4_graph_replays(schedule, shape):
    print(f"[graph] nvfp4 schedule={schedule} shape={shape}", flush=True)
    run, out = _nvfp4_runner(inputs.custom_nvfp4_case(*shape, seed=38), schedule)
    other, _ = _nvfp4_runner(inputs.custom_nvfp4_case(*shape, seed=39), schedule)
    _check_replays(run, out, other, exact=schedule == binding.SCHEDULE_PREFILL)


def test_grouped_masked_graph_follows_device_counts():
    # masked_m is read on the device at replay time: rewriting it between replays (an
    # expert-parallel dispatch would) changes which rows the captured forward computes.
    print("[graph] grouped masked", flush=True)
    case = inputs.grouped_masked_case([5, 20, 0, 33], 40, 512, 256, seed=37)
    d = to_dev(case)
    ws = binding.grouped_workspace_bytes(True, 40, 512, 256, 4, 16)
    work = torch.empty(ws, dtype=torch.uint8, device="cuda")
    out = torch.empty((160, 512), dtype=torch.bfloat16, device="cuda")
    counts = d["masked_m"]

    def run():
        binding.moe_w4a16_grouped_masked(d["a"], d["w13"], d["s13"], d["w2"], d["s2"], counts, 16,
                                         out=out, workspace=work)
    graph = _capture(run)
    for i, new in enumerate(([5, 20, 0, 33], [40, 0, 7, 1], [0, 0, 0, 0], [12, 40, 40, 3])):
        counts.copy_(torch.tensor(new, dtype=torch.int32))
        run()
        torch.cuda.synchronize()
        eager = bf16_out_to_f64(out)
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = bf16_out_to_f64(out)
        valid = (np.arange(40)[None, :] < np.array(new)[:, None]).ravel()
        assert np.all(got[~valid] == 0.0), f"replay {i}: rows past the counts"
        if valid.any():
            assert row_rel_err(got[valid], eager[valid]).max() <= 1e-3, f"replay {i} differs"
