"""GPU router (moe_topk_softmax) against the oracle: expert ids bit-exact, weights within
1e-5 relative. The GPU forms the weights in fp32: exp(x) for x = l - m <= 0 as 2^(x log2 e)
(relative error about |x| * 2^-24 from the product's rounding plus an ulp: 1.3e-6 at
x = -20), a sum of at most E/64 + 6 terms per lane and across the wave (at most
(E/64 + 6) * 2^-24 relative, 4.2e-6 at E = 4096) and one division; the oracle in fp64."""
import numpy as np
import pytest
import torch

from quantized_mixture_experts_amd import binding, inputs

pytestmark = pytest.mark.gpu

RTOL = 1e-5


def _check(oracle_mod, logits, k, renormalize=True, expert_map=None):
    T, E = logits.shape
    print(f"[route] T={T} E={E} k={k} renormalize={renormalize} "
          f"map={expert_map is not None}", flush=True)
    lg = torch.from_numpy(logits).cuda()
    mp = None if expert_map is None else torch.from_numpy(expert_map).cuda()
    ids, w = binding.moe_topk_softmax(lg, k, renormalize, mp)
    torch.cuda.synchronize()
    rids, rw = oracle_mod.topk_softmax(logits, k, renormalize, expert_map)
    np.testing.assert_array_equal(ids.cpu().numpy(), rids)
    got = w.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - rw) <= RTOL * np.abs(rw) + 1e-30), np.max(np.abs(got - rw) / rw)
    return ids, w


@pytest.mark.parametrize("T,E,k,kind,renorm", [
    (1, 8, 1, "uniform", True),
    (2, 1, 1, "uniform", False),       # one expert: weight 1 (renormalized or not)
    (4, 2, 2, "uniform", True),        # k = E = 2, one lane
    (1, 384, 1, "zipf", False),        # one token, one slot
    (7, 8, 2, "uniform", True),
    (256, 48, 8, "uniform", True),
    (8192, 48, 8, "zipf", True),
    (256, 384, 8, "uniform", True),
    (33, 65, 8, "uniform", False),     # 2 per lane: lane 32 holds one, the lanes past it none
    (5, 600, 4, "zipf", True),         # more than 512 experts: rescanned from memory
    (4, 4096, 8, "uniform", False),    # the largest expert count
    (3, 200, 100, "uniform", True),    # k > 64: slots written in two batches
    (16, 384, 384, "uniform", False),  # k = E
    (64, 151, 8, "uniform", True),     # 3 experts per lane (each count 1..8 has its own kernel)
    (64, 298, 8, "zipf", False),       # 5 per lane, the last used lane partly filled
    (32, 420, 70, "uniform", True),    # 7 per lane, k > 64
    (64, 512, 8, "zipf", True),        # the largest count held in registers (8 per lane)
    (16, 513, 16, "uniform", False),   # the smallest count scanned from memory
])
def test_router_matches_oracle(oracle_mod, T, E, k, kind, renorm):
    rng = np.random.default_rng(T * 131 + E * 7 + k)
    _check(oracle_mod, inputs.router_logits(rng, T, E, kind), k, renorm)


@pytest.mark.parametrize("E", [48, 151, 298, 384, 420, 600])
def test_router_ties_and_signed_zeros(oracle_mod, E):
    rng = np.random.default_rng(3 + E)
    # logits on a coarse grid: many exact ties, within a lane's experts and across lanes,
    # which keep the lower id first
    logits = (np.round(rng.standard_normal((300, E)) * 2.0) / 2.0).astype(np.float32)
    logits[:5, :] = 0.0
    logits[:5, ::2] = -0.0
    _check(oracle_mod, logits, 8)
    _check(oracle_mod, logits, 8, renormalize=False)
    _check(oracle_mod, logits[:40], min(70, E))


def test_router_expert_map_and_empty(oracle_mod):
    rng = np.random.default_rng(9)
    E, k = 384, 8
    emap = np.full(E, -1, np.int32)
    emap[48:96] = np.arange(48, dtype=np.int32)  # one GPU's share of 8: experts 48..95
    logits = inputs.router_logits(rng, 512, E, "uniform")
    ids, w = _check(oracle_mod, logits, k, expert_map=emap)
    local = ids.cpu().numpy()
    assert np.all((local == -1) | ((local >= 0) & (local < 48)))
    ids0, w0 = binding.moe_topk_softmax(torch.empty((0, E), device="cuda"), k)
    assert ids0.shape == (0, k) and w0.shape == (0, k)


def test_router_is_deterministic():
    rng = np.random.default_rng(21)
    lg = torch.from_numpy(inputs.router_logits(rng, 4096, 48, "zipf")).cuda()
    a = binding.moe_topk_softmax(lg, 8)
    b = binding.moe_topk_softmax(lg, 8)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("schedule", [binding.SCHEDULE_DECODE, binding.SCHEDULE_PREFILL])
def test_router_to_w4a16_forward_under_expert_parallelism(oracle_mod, schedule):
    # The GPU's share: global experts 4..11 of 16 as local experts 0..7. Router on the
    # GPU (global top-4, renormalized, ids mapped, remote slots -1), then the forward on
    # the local experts; the oracle takes the same path from the same logits.
    from gpu_util import TOL, bf16_out_to_f64, report, to_dev
    T, H, I, E_glob, E_loc, k = 300, 512, 256, 16, 8, 4
    print(f"[route->w4a16] schedule={schedule}", flush=True)
    case = inputs.custom_w4a16_case(T, H, I, E_loc, k, seed=77)
    emap = np.full(E_glob, -1, np.int32)
    emap[4:12] = np.arange(E_loc, dtype=np.int32)
    logits = inputs.router_logits(np.random.default_rng(78), T, E_glob, "zipf")
    ids, wts = binding.moe_topk_softmax(torch.from_numpy(logits).cuda(), k, True,
                                        torch.from_numpy(emap).cuda())
    d = to_dev(case)
    out = binding.moe_w4a16_forward(d["x"], d["w13"], d["s13"], d["w2"], d["s2"], ids, wts,
                                    schedule=schedule)
    torch.cuda.synchronize()
    rids, rw = oracle_mod.topk_softmax(logits, k, True, emap)
    np.testing.assert_array_equal(ids.cpu().numpy(), rids)
    ref = oracle_mod.w4a16_moe(case["x"], case["w13"], case["s13"], case["w2"], case["s2"], rids,
                               rw.astype(np.float32))
    e = report(f"router->w4a16 EP share sched={schedule}", bf16_out_to_f64(out), ref)
    assert e.max() <= TOL
    remote = np.all(rids < 0, axis=1)  # tokens whose top-4 are all held elsewhere
    assert np.all(bf16_out_to_f64(out)[remote] == 0.0)


def test_router_and_bf16_quantizer_to_fp8_forward(oracle_mod):
    # bf16 activations quantized on the GPU (E4M3 per token and 128 columns) and routed
    # on the GPU, then the block-FP8 forward; the oracle quantizes and routes the same way,
    # and the forward is held to the W8A8 rule (fp8_rule.py) on the oracle's routing.
    import fp8_rule
    from gpu_util import bf16_out_to_f64
    T, H, I, E, k = 400, 512, 256, 8, 2
    print("[route+quant->fp8]", flush=True)
    case = inputs.custom_fp8_case(T, H, I, E, k, seed=55, quantize=oracle_mod.fp8_quantize_blocks)
    x = inputs.bf16_bits(np.random.default_rng(56).standard_normal((T, H), dtype=np.float32))
    logits = inputs.router_logits(np.random.default_rng(57), T, E, "uniform")
    a_q, a_s = binding.fp8_quantize_blocks(torch.from_numpy(x.view(np.int16)).cuda(), 1, 128)
    ids, wts = binding.moe_topk_softmax(torch.from_numpy(logits).cuda(), k)
    dev = {n: torch.from_numpy(case[n]).cuda() for n in ("w13", "s13", "w2", "s2")}
    need = binding.plan(binding.FORMAT_FP8, T, H, I, E, k)[2]
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    out = binding.moe_fp8_block_forward(a_q, a_s, dev["w13"], dev["s13"], dev["w2"], dev["s2"],
                                        ids, wts, workspace=ws)
    torch.cuda.synchronize()
    rq, rs = oracle_mod.fp8_quantize_blocks(inputs.bf16_value(x), 1, 128)
    rids, rw = oracle_mod.topk_softmax(logits, k)
    assert np.array_equal(a_q.cpu().numpy(), rq) and np.array_equal(a_s.cpu().numpy(), rs)
    assert np.array_equal(ids.cpu().numpy(), rids)
    chain = dict(case, a_q=rq, a_s=rs, topk_ids=rids, topk_weights=rw.astype(np.float32))
    regions = binding.workspace_regions(binding.FORMAT_FP8, T, H, I, E, k)
    fp8_rule.check(oracle_mod, "router+quantizer->fp8", chain, E, bf16_out_to_f64(out),
                   ws.cpu().numpy(), regions)


def test_router_bench_configuration(oracle_mod):
    # The benchmark's router workload at full size: 8192 tokens, 384 experts, top-8,
    # renormalized, Zipf logits, ids mapped to the share of experts 48..95.
    T, E, k, share = 8192, 384, 8, 48
    logits = inputs.router_logits(np.random.default_rng(97), T, E, "zipf")
    emap = np.full(E, -1, np.int32)
    emap[share:2 * share] = np.arange(share, dtype=np.int32)
    ids, _ = _check(oracle_mod, logits, k, True, emap)
    local = ids.cpu().numpy()
    assert np.all((local == -1) | ((local >= 0) & (local < share)))
    assert (local >= 0).any() and (local == -1).any()
