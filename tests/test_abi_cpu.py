"""The C-ABI library without a GPU: it loads, exports every function include/qmoe.h
declares, and rejects bad arguments with status codes before any GPU work."""
import ctypes

import pytest

from quantized_mixture_experts_amd import binding

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 0x10000  # an aligned non-NULL address; never dereferenced by the checks


@pytest.fixture(scope="module")
def lib():
    return binding.load()


def test_exports_every_declared_function(lib):
    names = binding.declared_functions()
    assert {"moe_topk_softmax", "moe_align", "moe_w4a16_forward", "moe_fp8_block_forward",
            "moe_w4a16_grouped_contiguous", "moe_w4a16_grouped_masked", "moe_mxfp4_forward", "moe_nvfp4_forward",
            "qmoe_plan", "qmoe_fp8_quantize_blocks", "qmoe_fp8_quantize_blocks_bf16",
            "qmoe_status_string", "qmoe_last_error", "qmoe_abi_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.qmoe_abi_version() == 1
    assert lib.qmoe_status_string(3) == b"workspace too small"


def test_timing_pause_outside_begin_end(lib):
    # pausing or resuming stage timing needs a begun timing (host-only check)
    assert lib.qmoe_timing_pause(1) == INVALID
    assert lib.qmoe_timing_pause(0) == INVALID
    assert b"timing not begun" in lib.qmoe_last_error()


def _w4(lib, T=32, H=7168, I=2048, E=48, k=8, sched=0, ptr=FAKE, ws=None, size=1 << 40, out=FAKE):
    sz = ctypes.c_size_t(size)
    st = lib.moe_w4a16_forward(ptr, ptr, ptr, ptr, ptr, ptr, ptr, T, H, I, E, k, sched, out, ws,
                               ctypes.byref(sz), None)
    return st, sz.value


def test_workspace_query_and_plan(lib):
    st, need = _w4(lib, ws=None)
    assert st == OK and need > 0
    chosen, bm, ws = binding.plan(binding.FORMAT_W4A16, 32, 7168, 2048, 48, 8)
    assert chosen == binding.SCHEDULE_DECODE and ws == need and bm == 16
    assert binding.plan(binding.FORMAT_W4A16, 8192, 7168, 2048, 48, 8)[0] == binding.SCHEDULE_PREFILL
    # the workspace holds at least the combine buffer and h
    assert need >= 32 * 7168 * 4 + 32 * 8 * 2048 * 2
    assert binding.plan(binding.FORMAT_W4A16, 32, 7168, 2048, 48, 8, binding.SCHEDULE_PREFILL)[0] == 2


@pytest.mark.parametrize("kw,status", [
    (dict(H=7169), UNSUPPORTED), (dict(H=7200 - 16), UNSUPPORTED), (dict(I=2040), UNSUPPORTED),
    (dict(k=49), INVALID), (dict(E=0), INVALID), (dict(E=5000, k=8), UNSUPPORTED),
    (dict(sched=7), INVALID), (dict(T=-1), INVALID),
])
def test_w4a16_rejects_bad_shapes(lib, kw, status):
    st, _ = _w4(lib, ws=FAKE, **kw)
    assert st == status, binding.load().qmoe_last_error()
    assert lib.qmoe_last_error()


def test_w4a16_rejects_small_workspace_null_and_misaligned(lib):
    st, need = _w4(lib, ws=None)
    assert _w4(lib, ws=FAKE, size=need - 1)[0] == WORKSPACE
    assert _w4(lib, ws=FAKE, size=need, ptr=None)[0] == INVALID
    assert _w4(lib, ws=FAKE, size=need, out=None)[0] == INVALID
    assert _w4(lib, ws=FAKE, size=need, ptr=FAKE + 4)[0] == INVALID
    assert _w4(lib, ws=FAKE + 16, size=need)[0] == INVALID  # workspace not 256-aligned
    assert _w4(lib, T=0, ws=FAKE, size=need)[0] == OK  # nothing to do, nothing launched


def test_fp8_rejects_bad_shapes(lib):
    sz = ctypes.c_size_t(1 << 40)
    f = lib.moe_fp8_block_forward
    args = [FAKE] * 8
    assert f(*args, 16, 7168 + 32, 2048, 32, 8, 0, FAKE, FAKE, ctypes.byref(sz), None) == UNSUPPORTED
    assert f(*args, 16, 7168, 2048 + 64, 32, 8, 0, FAKE, FAKE, ctypes.byref(sz), None) == UNSUPPORTED
    assert f(*args, 16, 7168, 2048, 32, 33, 0, FAKE, FAKE, ctypes.byref(sz), None) == INVALID
    sz = ctypes.c_size_t(0)
    assert f(*args, 16, 7168, 2048, 32, 8, 0, FAKE, None, ctypes.byref(sz), None) == OK
    assert sz.value > 16 * 7168 * 4
    need = sz.value
    sz = ctypes.c_size_t(need - 1)
    assert f(*args, 16, 7168, 2048, 32, 8, 0, FAKE, FAKE, ctypes.byref(sz), None) == WORKSPACE


def test_align_and_quantizer_reject_bad_arguments(lib):
    for bm in (0, 3, 512, -16):
        assert lib.moe_align(FAKE, 4, 2, 8, bm, FAKE, FAKE, FAKE, FAKE, None) == INVALID
    assert lib.moe_align(FAKE, 4, 2, 0, 16, FAKE, FAKE, FAKE, FAKE, None) == INVALID
    assert lib.moe_align(FAKE, 4, 2, 8, 16, None, FAKE, FAKE, FAKE, None) == INVALID
    assert lib.moe_align(FAKE, 4, 2, 8, 16, FAKE + 2, FAKE, FAKE, FAKE, None) == INVALID
    assert lib.moe_align(FAKE, 4, 2, 9000, 16, FAKE, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    q = lib.qmoe_fp8_quantize_blocks
    assert q(FAKE, 4, 4, 0, 128, FAKE, FAKE, None) == UNSUPPORTED
    assert q(FAKE, 4, 4, 129, 128, FAKE, FAKE, None) == UNSUPPORTED
    assert q(FAKE, 4, 4, 128, 2048, FAKE, FAKE, None) == UNSUPPORTED
    assert q(FAKE, -1, 4, 1, 128, FAKE, FAKE, None) == INVALID
    assert q(None, 4, 4, 1, 128, FAKE, FAKE, None) == INVALID
    assert q(FAKE, 0, 4, 1, 128, FAKE, FAKE, None) == OK  # empty: nothing launched
    qb = lib.qmoe_fp8_quantize_blocks_bf16
    assert qb(FAKE + 1, 4, 4, 1, 128, FAKE, FAKE, None) == INVALID
    assert qb(FAKE, 4, 4, 0, 128, FAKE, FAKE, None) == UNSUPPORTED
    assert qb(None, 4, 4, 1, 128, FAKE, FAKE, None) == INVALID


def test_router_rejects_bad_arguments(lib):
    r = lib.moe_topk_softmax
    assert r(FAKE, 4, 8, 0, 1, None, FAKE, FAKE, None) == INVALID   # k = 0
    assert r(FAKE, 4, 8, 9, 1, None, FAKE, FAKE, None) == INVALID   # k > E
    assert r(FAKE, -1, 8, 2, 1, None, FAKE, FAKE, None) == INVALID  # T < 0
    assert r(FAKE, 4, 0, 1, 1, None, FAKE, FAKE, None) == INVALID   # E = 0
    assert r(FAKE, 4, 5000, 2, 1, None, FAKE, FAKE, None) == UNSUPPORTED
    assert r(None, 4, 8, 2, 1, None, FAKE, FAKE, None) == INVALID
    assert r(FAKE, 4, 8, 2, 1, None, None, FAKE, None) == INVALID
    assert r(FAKE + 2, 4, 8, 2, 1, None, FAKE, FAKE, None) == INVALID
    assert r(FAKE, 4, 8, 2, 1, FAKE + 1, FAKE, FAKE, None) == INVALID  # misaligned map
    assert r(None, 0, 8, 2, 1, None, None, None, None) == OK  # empty: nothing launched


def _grouped(lib, masked, M=128, H=7168, I=2048, E=48, em=0, sched=0, ptr=FAKE, route=FAKE,
             ws=None, size=1 << 40, out=FAKE):
    fn = lib.moe_w4a16_grouped_masked if masked else lib.moe_w4a16_grouped_contiguous
    sz = ctypes.c_size_t(size)
    st = fn(ptr, ptr, ptr, ptr, ptr, route, M, H, I, E, em, sched, out, ws, ctypes.byref(sz), None)
    return st, sz.value


@pytest.mark.parametrize("masked", [False, True])
def test_grouped_layouts_check_arguments(lib, masked):
    st, need = _grouped(lib, masked)
    assert st == OK
    rows = 48 * 128 if masked else 128
    # the indexed forward's regions at k = 1 without the per-pair fp32 rows (the grouped
    # layouts write their output rows directly), plus the weights of 1
    regions = binding.workspace_regions(binding.FORMAT_W4A16, rows, 7168, 2048, 48, 1)
    end = max(o + n for name, (o, n) in regions.items() if name != "y")
    base = (end + 255) // 256 * 256
    assert need == base + (4 * rows + 255) // 256 * 256
    assert _grouped(lib, masked, ws=FAKE, size=need - 1)[0] == WORKSPACE
    assert _grouped(lib, masked, ws=FAKE, size=need, route=None)[0] == INVALID
    assert _grouped(lib, masked, ws=FAKE, size=need, route=FAKE + 2)[0] == INVALID
    assert _grouped(lib, masked, ws=FAKE, size=need, ptr=FAKE + 8)[0] == INVALID
    assert _grouped(lib, masked, ws=FAKE, size=need, out=None)[0] == INVALID
    assert _grouped(lib, masked, M=-1, ws=FAKE)[0] == INVALID
    assert _grouped(lib, masked, em=-1, ws=FAKE)[0] == INVALID
    assert _grouped(lib, masked, H=7168 + 16, ws=FAKE)[0] == UNSUPPORTED
    assert _grouped(lib, masked, E=0, ws=FAKE)[0] == INVALID
    assert _grouped(lib, masked, sched=9, ws=FAKE)[0] == INVALID
    assert _grouped(lib, masked, M=0, ws=FAKE, size=need)[0] == OK  # no rows: nothing launched


def test_mxfp4_checks_arguments_like_w4a16(lib):
    f = lib.moe_mxfp4_forward
    sz = ctypes.c_size_t(0)
    assert f(*([FAKE] * 7), 32, 7168, 2048, 48, 8, 0, FAKE, None, ctypes.byref(sz), None) == OK
    assert sz.value == _w4(lib, ws=None)[1]  # the same plan and workspace as W4A16
    need = sz.value
    big = ctypes.c_size_t(need)
    assert f(*([FAKE] * 7), 32, 7168 + 16, 2048, 48, 8, 0, FAKE, FAKE, ctypes.byref(big), None) == UNSUPPORTED
    assert f(*([FAKE] * 7), 32, 7168, 2048, 48, 49, 0, FAKE, FAKE, ctypes.byref(big), None) == INVALID
    assert f(FAKE, FAKE, None, *([FAKE] * 4), 32, 7168, 2048, 48, 8, 0, FAKE, FAKE,
             ctypes.byref(big), None) == INVALID
    small = ctypes.c_size_t(need - 1)
    assert f(*([FAKE] * 7), 32, 7168, 2048, 48, 8, 0, FAKE, FAKE, ctypes.byref(small), None) == WORKSPACE
    assert binding.plan(binding.FORMAT_MXFP4, 8192, 7168, 2048, 48, 8)[0] == binding.SCHEDULE_PREFILL


def test_nvfp4_checks_arguments(lib):
    f = lib.moe_nvfp4_forward
    sz = ctypes.c_size_t(0)
    assert f(*([FAKE] * 9), 32, 7168, 2048, 48, 8, 0, FAKE, None, ctypes.byref(sz), None) == OK
    assert sz.value == _w4(lib, ws=None)[1]
    big = ctypes.c_size_t(sz.value)
    # a missing per-expert global scale (g13 or g2) is rejected
    for i in (3, 6):
        p = [FAKE] * 9
        p[i] = None
        assert f(*p, 32, 7168, 2048, 48, 8, 0, FAKE, FAKE, ctypes.byref(big), None) == INVALID
    # K must hold whole 32-column groups (the E4M3 scales come in pairs)
    assert f(*([FAKE] * 9), 32, 7168 + 16, 2048, 48, 8, 0, FAKE, FAKE, ctypes.byref(big), None) == UNSUPPORTED
    small = ctypes.c_size_t(sz.value - 1)
    assert f(*([FAKE] * 9), 32, 7168, 2048, 48, 8, 0, FAKE, FAKE, ctypes.byref(small), None) == WORKSPACE
    # NVFP4's measured crossover (36 rows per expert) sits below INT4's (44)
    assert binding.plan(binding.FORMAT_NVFP4, 240, 7168, 2048, 48, 8)[0] == binding.SCHEDULE_PREFILL
    assert binding.plan(binding.FORMAT_W4A16, 240, 7168, 2048, 48, 8)[0] == binding.SCHEDULE_DECODE
    assert binding.plan(binding.FORMAT_NVFP4, 192, 7168, 2048, 48, 8)[0] == binding.SCHEDULE_DECODE


def test_binding_functions_reference_only_defined_names():
    # The GPU entry points cannot run here; at least every global name their code loads
    # must exist in the module or the builtins.
    import builtins
    import dis
    import types
    missing = []
    for name, fn in vars(binding).items():
        if not isinstance(fn, types.FunctionType) or fn.__module__ != binding.__name__:
            continue
        for ins in dis.get_instructions(fn):
            if ins.opname in ("LOAD_GLOBAL", "LOAD_NAME"):
                g = ins.argval
                if g not in fn.__globals__ and not hasattr(builtins, g):
                    missing.append((name, g))
    assert not missing, missing


def test_plan_two_block_passes_above_sixteen_rows_per_expert():
    D = binding.SCHEDULE_DECODE
    # 32 tokens x top-8 / 48 experts = 5.3 rows per expert: one 16-row block per pass
    assert binding.plan(binding.FORMAT_W4A16, 32, 7168, 2048, 48, 8)[1] == 16
    # 72 tokens: 12 rows per expert, one block for W4A16, two for MXFP4 (cheaper per MFMA)
    assert binding.plan(binding.FORMAT_W4A16, 72, 7168, 2048, 48, 8)[1] == 16
    assert binding.plan(binding.FORMAT_MXFP4, 72, 7168, 2048, 48, 8)[1] == 32
    # 192 tokens: 32 rows per expert, passes of two blocks (align pads to 32 rows)
    for fmt in (binding.FORMAT_W4A16, binding.FORMAT_MXFP4):
        chosen, bm, ws = binding.plan(fmt, 192, 7168, 2048, 48, 8)
        assert chosen == D and bm == 32
    # the tile path keeps 16-row align blocks; FP8 always does
    assert binding.plan(binding.FORMAT_W4A16, 8192, 7168, 2048, 48, 8)[1] == 16
    assert binding.plan(binding.FORMAT_FP8, 192, 7168, 2048, 48, 8, D)[1] == 16


def test_plan_schedule_with_few_experts():
    W, D, PF = binding.FORMAT_W4A16, binding.SCHEDULE_DECODE, binding.SCHEDULE_PREFILL
    # 48 experts, top-8: decode up to 44 rows per expert, prefill from 48
    assert binding.plan(W, 240, 7168, 2048, 48, 8)[0] == D
    assert binding.plan(W, 288, 7168, 2048, 48, 8)[0] == PF
    # few experts: decode while the routed pairs stay under ~450, at any rows per expert
    assert binding.plan(W, 192, 7168, 2048, 8, 2)[0] == D       # 48 rows, 384 pairs
    assert binding.plan(W, 256, 7168, 2048, 8, 2)[0] == PF      # 64 rows, 512 pairs
    assert binding.plan(W, 384, 7168, 2048, 4, 1)[0] == D       # 96 rows
    assert binding.plan(W, 512, 7168, 2048, 4, 1)[0] == PF      # 128 rows
    # two-block passes need more than ~225 routed pairs as well as 16 rows per expert
    assert binding.plan(W, 96, 7168, 2048, 8, 2)[1] == 16       # 24 rows, 192 pairs
    assert binding.plan(W, 128, 7168, 2048, 8, 2)[1] == 32      # 32 rows, 256 pairs
    assert binding.plan(W, 192, 7168, 2048, 4, 1)[1] == 16      # 48 rows, 192 pairs
    # block FP8 keeps its rows-per-expert crossover
    assert binding.plan(binding.FORMAT_FP8, 96, 7168, 2048, 4, 1)[0] == PF


@pytest.mark.parametrize("fmt,T,E,sched", [(binding.FORMAT_W4A16, 32, 48, 0),
                                           (binding.FORMAT_W4A16, 8192, 48, 0),
                                           (binding.FORMAT_FP8, 1024, 32, 1),
                                           (binding.FORMAT_FP8, 1024, 32, 2),
                                           (binding.FORMAT_MXFP4, 200, 8, 1)])
def test_workspace_regions_tile_the_workspace(fmt, T, E, sched):
    # regions are 256-byte aligned, disjoint, in increasing order and end within the plan's
    # workspace size; each schedule has exactly the regions its launches use
    H, I, k = 7168, 2048, 8
    regions = binding.workspace_regions(fmt, T, H, I, E, k, sched)
    chosen, bm, total = binding.plan(fmt, T, H, I, E, k, sched)
    spans = sorted(regions.values())
    for (o, n), (o2, _) in zip(spans, spans[1:]):
        assert o % 256 == 0 and o + n <= o2
    assert spans[-1][0] + spans[-1][1] <= total
    L = T * k + E * (bm - 1)
    assert regions["sorted_ids"][1] == 4 * L
    four_bit = fmt != binding.FORMAT_FP8
    assert ("xs" in regions) == four_bit and ("h" in regions) == four_bit
    assert ("hq" in regions) == (not four_bit)
    tiled = chosen == binding.SCHEDULE_PREFILL
    assert ("y" in regions) == tiled and ("out32" in regions) == (not tiled)
    if not four_bit:
        assert ("h32" in regions) == (not tiled)
        assert regions["hq"][1] == L * I and regions["hs"][1] == 4 * L * (I // 128)


def test_noalloc_forward_rejects_plans_beyond_its_scratch(lib):
    # The 8192-token prefill layer needs about 2.9 GB: rejected before any GPU work (the
    # fake pointers are never read); the 32-token decode layer fits in the 64 MiB.
    T, H, I, E, k = 8192, 7168, 2048, 48, 8
    assert binding.plan(binding.FORMAT_W4A16, T, H, I, E, k)[2] > (64 << 20)
    assert binding.plan(binding.FORMAT_W4A16, 32, H, I, E, k)[2] <= (64 << 20)
    st = lib.moe_w4a16_forward_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, T, H, I, E, k, 0,
                                       FAKE, None)
    assert st == UNSUPPORTED
    assert b"scratch" in lib.qmoe_last_error()
    st = lib.moe_w4a16_forward_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 32, 7169, I, E,
                                       k, 0, FAKE, None)
    assert st == UNSUPPORTED


@pytest.mark.parametrize("T,H,I,E,k,slices", [
    (8192, 7168, 2048, 48, 8, 1),   # the prefill layer fills the GPU: no split
    (1024, 7168, 2048, 4, 2, 1),    # 224 down tiles: no split
    (1024, 7168, 2048, 2, 1, 1),    # 2 x 512 rows, counted high: 5 tiles of 128 each, 280 tiles
    (512, 7168, 2048, 2, 2, 1),     # 128-row tiles (256-row ones fill a quarter wave): 224 tiles, one wave
    (128, 7168, 2048, 1, 1, 8),     # 28 down tiles: 8 slices
    (96, 7168, 2048, 4, 2, 2),      # 48 rows per expert, 128-row tiles: 112 tiles, 2 slices
    (300, 1024, 1024, 2, 1, 4),     # 8 down tiles, K = 1024 (4 blocks): 4 slices
    (300, 1024, 2048, 2, 1, 8),     # 8 slices
    (200, 1024, 1024, 3, 2, 4),
    (160, 512, 512, 1, 1, 2),
    (600, 512, 256, 4, 2, 1),       # K = 256: one block, nothing to split
])
def test_split_k_plan(T, H, I, E, k, slices):
    regions = binding.workspace_regions(binding.FORMAT_W4A16, T, H, I, E, k,
                                        binding.SCHEDULE_PREFILL)
    assert regions["y"][1] == slices * 4 * T * k * H


def test_tile_kernels_limited_to_32_bit_weight_offsets():
    # one expert's weights must stay below 2^31 bytes of codes for the tile kernels' buffer
    # resources; at I * H = 2^31 the prefill schedule runs on the stream kernels instead
    big = binding.workspace_regions(binding.FORMAT_W4A16, 64, 65536, 32768, 4, 2,
                                    binding.SCHEDULE_PREFILL)
    assert "out32" in big and "y" not in big
    ok = binding.workspace_regions(binding.FORMAT_W4A16, 64, 65536, 16384, 4, 2,
                                   binding.SCHEDULE_PREFILL)
    assert "y" in ok


def test_tuning_overrides_validate_and_reach_the_plan():
    S = binding
    W, F, M = S.FORMAT_W4A16, S.FORMAT_FP8, S.FORMAT_MXFP4

    def y_slices(fmt, T, H, I, E, k):
        return S.workspace_regions(fmt, T, H, I, E, k, S.SCHEDULE_PREFILL)["y"][1] // (4 * T * k * H)

    base_block = S.plan(W, 32, 7168, 2048, 48, 8, S.SCHEDULE_DECODE)[1]
    base_fp8 = S.plan(F, 32, 7168, 2048, 48, 8, S.SCHEDULE_DECODE)
    base_slices = y_slices(W, 300, 1024, 1024, 2, 1)
    try:
        for bad in ({"tile_rows": 64}, {"rows_per_pass": 8}, {"kslices": 3}, {"kslices": 128},
                    {"tile_grid": 2}, {"kslices": -1}):
            S.set_tuning(rows_per_pass=32)
            with pytest.raises(S.QMoEError):
                S.set_tuning(**bad)
            # a rejected call changes nothing
            assert S.plan(W, 32, 7168, 2048, 48, 8, S.SCHEDULE_DECODE)[1] == 32
        S.set_tuning(rows_per_pass=32)
        assert S.plan(W, 32, 7168, 2048, 48, 8, S.SCHEDULE_DECODE)[1] == 32
        assert S.plan(M, 8, 7168, 2048, 48, 8, S.SCHEDULE_DECODE)[1] == 32
        assert S.plan(F, 32, 7168, 2048, 48, 8, S.SCHEDULE_DECODE) == base_fp8
        S.set_tuning(rows_per_pass=16)
        assert S.plan(W, 400, 7168, 2048, 48, 8, S.SCHEDULE_DECODE)[1] == 16
        for ks in (1, 2, 4):
            S.set_tuning(kslices=ks)
            assert y_slices(W, 300, 1024, 1024, 2, 1) == ks
        S.set_tuning(kslices=8)  # does not divide I / 256 = 4: no split
        assert y_slices(W, 300, 1024, 1024, 2, 1) == 1
        S.set_tuning(tile_rows=128, tile_grid=1)
        assert y_slices(W, 300, 1024, 1024, 2, 1) >= 1
    finally:
        S.set_tuning()
    assert S.plan(W, 32, 7168, 2048, 48, 8, S.SCHEDULE_DECODE)[1] == base_block
    assert y_slices(W, 300, 1024, 1024, 2, 1) == base_slices
