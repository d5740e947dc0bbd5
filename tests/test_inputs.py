"""The seeded input generator: determinism, routing invariants (weights sum to one,
distinct ids, descending probability), Zipf skew, and storage conversions against
torch's bf16 conversion."""
import numpy as np
import torch

from quantized_mixture_experts_amd import inputs


def test_routing_invariants_uniform_and_zipf():
    rng = np.random.default_rng(0)
    for kind in ("uniform", "zipf"):
        ids, w = inputs.routing(rng, 512, 48, 8, kind)
        assert ids.dtype == np.int32 and w.dtype == np.float32 and ids.shape == (512, 8)
        assert np.all((ids >= 0) & (ids < 48))
        assert all(len(set(r)) == 8 for r in ids.tolist())
        assert np.abs(w.sum(axis=1) - 1).max() <= 1e-6
        assert np.all(np.diff(w, axis=1) <= 0)


def test_zipf_skew_matches_prefill_shape():
    cfg = inputs.CONFIGS["prefill"]
    rng = np.random.default_rng(cfg.seed)
    rng.standard_normal((cfg.T, cfg.H), dtype=np.float32)  # same draw order as the case
    ids, _ = inputs.routing(rng, cfg.T, cfg.E, cfg.k, "zipf")
    c = np.bincount(ids.reshape(-1), minlength=cfg.E)
    assert c.sum() == cfg.P and c.argmax() == 0
    assert c[0] > 4 * c[-1]  # skewed, every expert still used
    assert c.min() > 0


def test_bf16_bits_matches_torch():
    x = np.random.default_rng(1).standard_normal(100000).astype(np.float32) * 37
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(inputs.bf16_bits(x), ref)
    assert np.array_equal(inputs.bf16_value(ref), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_cases_are_deterministic_and_shaped():
    cfg = inputs.CONFIGS["tiny"]
    a, b = inputs.w4a16_case(cfg), inputs.w4a16_case(cfg)
    for key in a:
        assert np.array_equal(a[key], b[key])
    assert a["w13"].shape == (8, 256, 128) and a["s13"].shape == (8, 256, 8)
    assert a["w2"].shape == (8, 256, 64) and a["s2"].shape == (8, 256, 4)
    s = inputs.bf16_value(a["s13"])
    assert np.all(s >= 0) and 0.01 < s.mean() < 0.02  # |N(0,1)|*0.02 has mean 0.016
