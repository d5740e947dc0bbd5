"""Pins for the oracle's W4A16 routed MoE FFN.

- brute-force dense fp64 evaluation written independently with numpy (dense routing
  matrix, every expert evaluated on every token);
- the E=1, k=1, w=1 special case equals the textbook SwiGLU FFN computed with
  torch's own silu and matmul;
- closed forms on constructed weights, invariants of the combine (zero weights,
  linearity, slot permutation, duplicate split, dropped ids), and row subsets.
"""
import math

import numpy as np
import pytest
import torch

from quantized_mixture_experts_amd import inputs


def dequant(w, s):
    """[..., N, K/2] codes + [..., N, K/32] bf16 scales -> fp64 [..., N, K]."""
    lo = (w & 0x0F).astype(np.float64)
    hi = (w >> 4).astype(np.float64)
    codes = np.stack([lo, hi], axis=-1).reshape(*w.shape[:-1], w.shape[-1] * 2)
    scales = inputs.bf16_value(s).astype(np.float64)
    return (codes - 8.0) * np.repeat(scales, 32, axis=-1)


def brute_dense(case):
    x = inputs.bf16_value(case["x"]).astype(np.float64)
    ids, wts = case["topk_ids"], case["topk_weights"]
    E = case["w13"].shape[0]
    I = case["w13"].shape[1] // 2
    T = x.shape[0]
    R = np.zeros((T, E))
    for t in range(T):
        for s in range(ids.shape[1]):
            if 0 <= ids[t, s] < E:
                R[t, ids[t, s]] += wts[t, s]
    out = np.zeros((T, x.shape[1]))
    for e in range(E):
        w13 = dequant(case["w13"][e], case["s13"][e])
        w2 = dequant(case["w2"][e], case["s2"][e])
        gu = x @ w13.T
        g, u = gu[:, :I], gu[:, I:]
        h = g / (1.0 + np.exp(-g)) * u
        out += R[:, e:e + 1] * (h @ w2.T)
    return out


def run_oracle(oracle_mod, case, rows=None):
    return oracle_mod.w4a16_moe(case["x"], case["w13"], case["s13"], case["w2"], case["s2"],
                                case["topk_ids"], case["topk_weights"], rows=rows, nthreads=4)


def rel_row_err(a, b):
    return np.max(np.abs(a - b), axis=1) / np.maximum(np.max(np.abs(b), axis=1), 1e-300)


@pytest.mark.parametrize("T,H,I,E,k", [(16, 256, 128, 8, 2), (7, 64, 96, 5, 3), (4, 32, 32, 1, 1)])
def test_oracle_matches_brute_force_dense(oracle_mod, T, H, I, E, k):
    case = inputs.custom_w4a16_case(T, H, I, E, k, seed=100 + T)
    got = run_oracle(oracle_mod, case)
    exp = brute_dense(case)
    assert rel_row_err(got, exp).max() < 1e-12


def test_tiny_config_matches_brute_force(oracle_mod):
    case = inputs.w4a16_case(inputs.CONFIGS["tiny"])
    assert rel_row_err(run_oracle(oracle_mod, case), brute_dense(case)).max() < 1e-12


def test_single_expert_is_textbook_swiglu(oracle_mod):
    case = inputs.custom_w4a16_case(5, 64, 64, 1, 1, seed=9)
    case["topk_weights"][:] = 1.0
    x = torch.from_numpy(inputs.bf16_value(case["x"]).astype(np.float64))
    w13 = torch.from_numpy(dequant(case["w13"][0], case["s13"][0]))
    w2 = torch.from_numpy(dequant(case["w2"][0], case["s2"][0]))
    gate = torch.nn.functional.linear(x, w13[:64])
    up = torch.nn.functional.linear(x, w13[64:])
    ref = torch.nn.functional.linear(torch.nn.functional.silu(gate) * up, w2).numpy()
    assert rel_row_err(run_oracle(oracle_mod, case), ref).max() < 1e-12


def _const_case(T, H, I, E, k):
    return dict(
        x=np.full((T, H), 0x3F80, np.uint16),  # 1.0
        topk_ids=np.zeros((T, k), np.int32), topk_weights=np.zeros((T, k), np.float32),
        w13=np.full((E, 2 * I, H // 2), 0x88, np.uint8), s13=np.full((E, 2 * I, H // 32), 0x3F80, np.uint16),
        w2=np.full((E, H, I // 2), 0x88, np.uint8), s2=np.full((E, H, I // 32), 0x3F80, np.uint16))


def test_closed_form_two_experts(oracle_mod):
    """x = 1; expert 0: gate weight 1/16, up 1/8; expert 1: gate -1/16, up 1/8;
    down weight (n mod 4 + 1)/32. With H = I = 32: g = +-2, u = 4, y_n = h (n mod 4 + 1),
    out_n = (0.75 * 8 / (1 + e^-2) - 0.25 * 8 / (1 + e^2)) (n mod 4 + 1)."""
    H = I = 32
    c = _const_case(1, H, I, 2, 2)
    c["s13"][:] = 0x3D80  # 1/16
    c["w13"][0, :I] = 0x99  # codes 9 -> +1
    c["w13"][0, I:] = 0xAA  # codes 10 -> +2
    c["w13"][1, :I] = 0x77  # codes 7 -> -1
    c["w13"][1, I:] = 0xAA
    c["s2"][:] = 0x3D00  # 1/32
    for n in range(H):
        code = 8 + n % 4 + 1
        c["w2"][:, n, :] = code | (code << 4)
    c["topk_ids"][0] = [0, 1]
    c["topk_weights"][0] = [0.75, 0.25]
    got = run_oracle(oracle_mod, c)[0]
    base = 0.75 * 8 / (1 + math.exp(-2)) - 0.25 * 8 / (1 + math.exp(2))
    exp = np.array([base * (n % 4 + 1) for n in range(H)])
    assert np.allclose(got, exp, rtol=1e-14, atol=0)


def test_nibble_order_low_is_even_column(oracle_mod):
    """Only byte 0 of gate row 0 differs from zero-point: low nibble 9 -> column 0 = +s,
    high nibble 6 -> column 1 = -2s. With x_0 = 3, x_1 = 5: g_0 = 3s - 10s = -7s."""
    H = I = 32
    c = _const_case(1, H, I, 1, 1)
    c["x"][0, 0] = 0x4040  # 3.0
    c["x"][0, 1] = 0x40A0  # 5.0
    c["w13"][0, 0, 0] = 0x69
    c["w13"][0, I:, :] = 0x99  # up weights = +1 -> u = sum(x) = 30 + 8
    c["w2"][0, :, :] = 0x99  # down weights = +1 -> y_n = sum_j h_j = h_0 + 31*0
    c["topk_weights"][0] = 1.0
    got = run_oracle(oracle_mod, c)[0]
    g0 = -7.0
    u = 3.0 + 5.0 + 30.0
    h0 = g0 / (1 + math.exp(-g0)) * u
    # other gate columns have g = 0 -> silu(0) = 0
    assert np.allclose(got, h0, rtol=1e-14, atol=0)


def test_group_scale_index(oracle_mod):
    """Scale of group 1 of gate row 0 set to 2: only columns 32..63 are scaled."""
    H, I = 64, 32
    c = _const_case(1, H, I, 1, 1)
    c["w13"][0, 0, :] = 0x99  # gate row 0: all +1
    c["s13"][0, 0, 1] = 0x4000  # 2.0 for columns 32..63
    c["w13"][0, I:, :] = 0x99
    c["w2"][0] = 0x99
    c["topk_weights"][0] = 1.0
    got = run_oracle(oracle_mod, c)[0]
    g0 = 32 * 1.0 + 32 * 2.0
    u = 64.0
    assert np.allclose(got, g0 / (1 + math.exp(-g0)) * u, rtol=1e-14, atol=0)


def test_zero_weights_and_zero_routing_give_exact_zero(oracle_mod):
    case = inputs.custom_w4a16_case(6, 64, 64, 4, 2, seed=21)
    z = dict(case)
    z["topk_weights"] = np.zeros_like(case["topk_weights"])
    assert np.all(run_oracle(oracle_mod, z) == 0.0)
    z = dict(case)
    z["w13"] = np.full_like(case["w13"], 0x88)
    assert np.all(run_oracle(oracle_mod, z) == 0.0)
    z = dict(case)
    z["w2"] = np.full_like(case["w2"], 0x88)
    assert np.all(run_oracle(oracle_mod, z) == 0.0)


def test_combine_linearity_permutation_and_split(oracle_mod):
    case = inputs.custom_w4a16_case(6, 64, 64, 4, 3, seed=22)
    base = run_oracle(oracle_mod, case)
    c2 = dict(case)
    c2["topk_weights"] = (case["topk_weights"] * np.float32(4.0)).astype(np.float32)
    assert rel_row_err(run_oracle(oracle_mod, c2), 4.0 * base).max() < 1e-14
    perm = [2, 0, 1]
    c3 = dict(case)
    c3["topk_ids"] = np.ascontiguousarray(case["topk_ids"][:, perm])
    c3["topk_weights"] = np.ascontiguousarray(case["topk_weights"][:, perm])
    assert rel_row_err(run_oracle(oracle_mod, c3), base).max() < 1e-13
    # one slot with weight w == two slots on that expert with w/2 each (w/2 exact in fp32)
    c4 = dict(case)
    c4["topk_ids"] = np.concatenate([case["topk_ids"], case["topk_ids"][:, :1]], axis=1)
    w = case["topk_weights"].copy()
    w4 = np.concatenate([w, w[:, :1] / 2], axis=1)
    w4[:, 0] /= 2
    c4["topk_weights"] = np.ascontiguousarray(w4.astype(np.float32))
    assert rel_row_err(run_oracle(oracle_mod, c4), base).max() < 1e-13


def test_out_of_range_ids_are_dropped(oracle_mod):
    case = inputs.custom_w4a16_case(4, 64, 64, 4, 2, seed=23)
    base_ids = case["topk_ids"].copy()
    c = dict(case)
    ids = base_ids.copy()
    ids[:, 1] = np.array([-1, 4, 100, -7])
    c["topk_ids"] = ids
    only0 = dict(case)
    only0["topk_ids"] = base_ids[:, :1].copy()
    only0["topk_weights"] = case["topk_weights"][:, :1].copy()
    assert np.array_equal(run_oracle(oracle_mod, c), run_oracle(oracle_mod, only0))


def test_row_subset_equals_full(oracle_mod):
    case = inputs.custom_w4a16_case(9, 64, 64, 4, 2, seed=24)
    full = run_oracle(oracle_mod, case)
    rows = np.array([8, 0, 3])
    assert np.array_equal(run_oracle(oracle_mod, case, rows=rows), full[rows])
