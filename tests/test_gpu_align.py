"""GPU align (moe_align through the C ABI) against the CPU oracle: bit-exact on every
output, for every workload's routing and a range of block sizes and edge cases."""
import numpy as np
import pytest
import torch

from quantized_mixture_experts_amd import binding, inputs

pytestmark = pytest.mark.gpu


def _run(oracle_mod, ids, E, B):
    print(f"[align] T={ids.shape[0]} k={ids.shape[1]} E={E} block_m={B}", flush=True)
    s, eids, ntp, offs = binding.moe_align(torch.from_numpy(ids).cuda(), E, B)
    torch.cuda.synchronize()
    rs, reids, rntp, roffs = oracle_mod.moe_align(ids, E, B)
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(eids.cpu().numpy(), reids)
    assert int(ntp.item()) == rntp
    assert np.array_equal(offs.cpu().numpy(), roffs)


@pytest.mark.parametrize("name", list(inputs.CONFIGS))
@pytest.mark.parametrize("B", [1, 16, 64, 128, 256])
def test_align_workloads(oracle_mod, name, B):
    cfg = inputs.CONFIGS[name]
    rng = np.random.default_rng(cfg.seed)
    rng.standard_normal((cfg.T, cfg.H), dtype=np.float32)  # keep the generator's draw order
    ids, _ = inputs.routing(rng, cfg.T, cfg.E, cfg.k, cfg.routing)
    _run(oracle_mod, ids, cfg.E, B)


@pytest.mark.parametrize("T,k,E,B", [(1, 1, 1, 16), (37, 3, 5, 4), (1000, 7, 7, 256),
                                     (3, 2, 4000, 16), (513, 4, 64, 32), (0, 4, 8, 16)])
def test_align_ragged_and_edge(oracle_mod, T, k, E, B):
    rng = np.random.default_rng(T + E)
    ids = np.zeros((T, k), np.int32)
    for t in range(T):
        ids[t] = rng.permutation(E)[:k]
    _run(oracle_mod, ids, E, B)


def test_align_invalid_and_skewed_ids(oracle_mod):
    rng = np.random.default_rng(9)
    ids = rng.integers(-3, 12, size=(700, 4)).astype(np.int32)
    ids[:300] = 2
    _run(oracle_mod, ids, 10, 16)
