"""Pins for the oracle's NVFP4 MoE FFN (E2M1 codes, E4M3 scales per 16 columns, an fp32
scale per expert and projection), independent of the oracle's own code:

- brute-force dense evaluation with numpy, decoding the E2M1 codes through their E4M3
  embedding and the E4M3 scales with torch's float8_e4m3fn;
- a scale-block probe (16 columns per scale, not 32);
- the down projection's global scale acts linearly on the output, and the gate/up
  global scale equals scaling every block scale of w13.
"""
import math

import numpy as np
import pytest
import torch

from quantized_mixture_experts_amd import inputs


def e2m1_via_e4m3(codes):
    codes = np.asarray(codes, dtype=np.int64)
    s, e, m = (codes >> 3) & 1, (codes >> 1) & 3, codes & 1
    exp = np.where(e > 0, e + 6, np.where(m == 1, 6, 0))
    man = np.where(e > 0, m << 2, 0)
    byte = ((s << 7) | (exp << 3) | man).astype(np.uint8)
    return torch.from_numpy(byte).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def dequant(w, s, g):
    codes = np.empty((w.shape[0], w.shape[1] * 2), np.int64)
    codes[:, 0::2] = w & 0x0F
    codes[:, 1::2] = w >> 4
    return e2m1_via_e4m3(codes) * np.repeat(e4m3(s), 16, axis=1) * np.float64(g)


def brute_dense(c):
    x = inputs.bf16_value(c["x"]).astype(np.float64)
    ids, wts = c["topk_ids"], c["topk_weights"]
    E, I, T = c["w13"].shape[0], c["w13"].shape[1] // 2, x.shape[0]
    out = np.zeros((T, x.shape[1]))
    for e in range(E):
        r = np.array([sum(float(wts[t, s]) for s in range(ids.shape[1]) if ids[t, s] == e)
                      for t in range(T)])
        gu = x @ dequant(c["w13"][e], c["s13"][e], c["g13"][e]).T
        g, u = gu[:, :I], gu[:, I:]
        out += r[:, None] * ((g / (1.0 + np.exp(-g)) * u) @ dequant(c["w2"][e], c["s2"][e], c["g2"][e]).T)
    return out


def run(oracle_mod, c, rows=None):
    return oracle_mod.nvfp4_moe(c["x"], c["w13"], c["s13"], c["g13"], c["w2"], c["s2"], c["g2"],
                                c["topk_ids"], c["topk_weights"], rows=rows, nthreads=4)


def rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


@pytest.mark.parametrize("T,H,I,E,k", [(16, 256, 128, 8, 2), (7, 64, 96, 5, 3), (4, 32, 32, 1, 1)])
def test_matches_brute_force_dense(oracle_mod, T, H, I, E, k):
    c = inputs.custom_nvfp4_case(T, H, I, E, k, seed=300 + T)
    assert rel(run(oracle_mod, c), brute_dense(c)) < 1e-12


def test_scale_block_is_sixteen_columns(oracle_mod):
    """Gate row 0 all +1 (code 2) with scale 1.0, except block 1 (columns 16..31) at
    scale 2.0; up rows and down weights +1; x = 1, H = 64: g0 = 48 + 16 * 2 = 80."""
    H, I = 64, 32
    one = 0x38  # E4M3 1.0
    c = dict(x=np.full((1, H), 0x3F80, np.uint16), topk_ids=np.zeros((1, 1), np.int32),
             topk_weights=np.ones((1, 1), np.float32),
             w13=np.zeros((1, 2 * I, H // 2), np.uint8), s13=np.full((1, 2 * I, H // 16), one, np.uint8),
             g13=np.ones(1, np.float32), w2=np.full((1, H, I // 2), 0x22, np.uint8),
             s2=np.full((1, H, I // 16), one, np.uint8), g2=np.ones(1, np.float32))
    c["w13"][0, 0, :] = 0x22
    c["w13"][0, I:, :] = 0x22
    c["s13"][0, 0, 1] = 0x40  # E4M3 2.0
    got = run(oracle_mod, c)[0]
    g0 = 48.0 + 16.0 * 2.0
    assert np.allclose(got, g0 / (1 + math.exp(-g0)) * 64.0, rtol=1e-14, atol=0)


def test_global_scales(oracle_mod):
    c = inputs.custom_nvfp4_case(6, 64, 64, 3, 2, seed=8)
    base = run(oracle_mod, c)
    d = dict(c)
    d["g2"] = (c["g2"] * np.float32(4.0)).astype(np.float32)
    np.testing.assert_allclose(run(oracle_mod, d), 4.0 * base, rtol=1e-13)
    # doubling g13 equals doubling every E4M3 block scale of w13 (exponent field + 1)
    e = dict(c)
    e["g13"] = (c["g13"] * np.float32(2.0)).astype(np.float32)
    f = dict(c)
    f["s13"] = (c["s13"] + np.uint8(8)).astype(np.uint8)
    assert np.all(e4m3(f["s13"]) == 2.0 * e4m3(c["s13"]))
    np.testing.assert_allclose(run(oracle_mod, e), run(oracle_mod, f), rtol=1e-13)
