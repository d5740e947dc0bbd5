"""GPU router (moe_topk_softmax) against the oracle: expert ids bit-exact, weights within
1e-5 relative. The GPU forms the weights in fp32: exp (about 2 ulp), a sum of at most
E/64 + 6 terms per lane and across the wave (at most (E/64 + 6) * 2^-24 relative, 4.4e-6
at E = 4096) and one division; the oracle in fp64."""
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
    (7, 8, 2, "uniform", True),
    (256, 48, 8, "uniform", True),
    (8192, 48, 8, "zipf", True),
    (256, 384, 8, "uniform", True),
    (33, 65, 8, "uniform", False),     # a lane holds one more expert than the rest
    (5, 600, 4, "zipf", True),         # experts past the register chunks
    (4, 4096, 8, "uniform", False),    # the largest expert count
    (3, 200, 100, "uniform", True),    # k > 64: slots written in two batches
    (16, 384, 384, "uniform", False),  # k = E
])
def test_router_matches_oracle(oracle_mod, T, E, k, kind, renorm):
    rng = np.random.default_rng(T * 131 + E * 7 + k)
    _check(oracle_mod, inputs.router_logits(rng, T, E, kind), k, renorm)


def test_router_ties_and_signed_zeros(oracle_mod):
    rng = np.random.default_rng(3)
    # logits on a coarse grid: many exact ties, which keep the lower id first
    logits = (np.round(rng.standard_normal((300, 48)) * 2.0) / 2.0).astype(np.float32)
    logits[:5, :] = 0.0
    logits[:5, ::2] = -0.0
    _check(oracle_mod, logits, 8)
    _check(oracle_mod, logits, 8, renormalize=False)


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
