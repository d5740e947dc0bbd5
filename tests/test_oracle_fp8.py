"""Pins for the oracle's W8A8 block-FP8 routed MoE FFN.

Brute-force dense fp64 evaluation written independently: numpy matmuls over every
expert, E4M3 decoding and the h requantization done with torch's float8_e4m3fn
conversion (a library routine) after clamping; plus the single-expert special case,
zero routing, and the block-scale indexing on constructed inputs."""
import math

import numpy as np
import pytest
import torch

from quantized_mixture_experts_amd import inputs


def e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_quant_rows(h32):
    """Per-row, per-128-column E4M3 quantization with torch's conversion (fp32)."""
    T, I = h32.shape
    g = h32.reshape(T, I // 128, 128)
    amax = np.abs(g).max(axis=2)
    s = (np.maximum(amax, np.float32(1e-10)) / np.float32(448.0)).astype(np.float32)
    t = np.clip(g / s[:, :, None], np.float32(-448), np.float32(448)).astype(np.float32)
    q = torch.from_numpy(t).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    return (q * s[:, :, None].astype(np.float64)).reshape(T, I)


def brute_dense(case):
    aq, As = case["a_q"], case["a_s"]
    T, H = aq.shape
    E, twoI, _ = case["w13"].shape
    I = twoI // 2
    x = e4m3(aq) * np.repeat(As.astype(np.float64), 128, axis=1)
    out = np.zeros((T, H))
    for e in range(E):
        w13 = e4m3(case["w13"][e]) * np.repeat(np.repeat(case["s13"][e].astype(np.float64), 128, 0), 128, 1)
        w2 = e4m3(case["w2"][e]) * np.repeat(np.repeat(case["s2"][e].astype(np.float64), 128, 0), 128, 1)
        gu = x @ w13.T
        g, u = gu[:, :I], gu[:, I:]
        h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
        hd = torch_quant_rows(h)
        y = hd @ w2.T
        for t in range(T):
            for s in range(case["topk_ids"].shape[1]):
                if case["topk_ids"][t, s] == e:
                    out[t] += float(case["topk_weights"][t, s]) * y[t]
    return out


def run_oracle(oracle_mod, case, rows=None):
    return oracle_mod.fp8_moe(case["a_q"], case["a_s"], case["w13"], case["s13"], case["w2"],
                              case["s2"], case["topk_ids"], case["topk_weights"], rows=rows,
                              nthreads=4)


def rel_row_err(a, b):
    return np.max(np.abs(a - b), axis=1) / np.maximum(np.max(np.abs(b), axis=1), 1e-300)


@pytest.mark.parametrize("T,H,I,E,k", [(6, 256, 128, 4, 2), (3, 128, 256, 3, 3)])
def test_fp8_oracle_matches_brute_force(oracle_mod, T, H, I, E, k):
    case = inputs.custom_fp8_case(T, H, I, E, k, seed=200 + T, quantize=oracle_mod.fp8_quantize_blocks)
    assert rel_row_err(run_oracle(oracle_mod, case), brute_dense(case)).max() < 1e-12


def test_fp8_single_expert_with_torch_ops(oracle_mod):
    case = inputs.custom_fp8_case(4, 128, 128, 1, 1, seed=31, quantize=oracle_mod.fp8_quantize_blocks)
    case["topk_weights"][:] = 1.0
    x = torch.from_numpy(e4m3(case["a_q"]) * float(1)) * torch.from_numpy(
        np.repeat(case["a_s"].astype(np.float64), 128, 1))
    w13 = torch.from_numpy(e4m3(case["w13"][0])) * float(case["s13"][0].reshape(-1)[0])
    assert case["s13"].shape[1:] == (2, 1)
    w13[128:] *= float(case["s13"][0, 1, 0]) / float(case["s13"][0, 0, 0])
    w2 = torch.from_numpy(e4m3(case["w2"][0])) * float(case["s2"][0, 0, 0])
    gate = torch.nn.functional.linear(x, w13[:128])
    up = torch.nn.functional.linear(x, w13[128:])
    h = (torch.nn.functional.silu(gate) * up).to(torch.float32).numpy()
    ref = torch.nn.functional.linear(torch.from_numpy(torch_quant_rows(h)), w2).numpy()
    assert rel_row_err(run_oracle(oracle_mod, case), ref).max() < 1e-12


def test_fp8_zero_routing_and_dropped_ids(oracle_mod):
    case = inputs.custom_fp8_case(3, 128, 128, 2, 2, seed=32, quantize=oracle_mod.fp8_quantize_blocks)
    z = dict(case)
    z["topk_weights"] = np.zeros_like(case["topk_weights"])
    assert np.all(run_oracle(oracle_mod, z) == 0.0)
    d = dict(case)
    ids = case["topk_ids"].copy()
    ids[:, :] = -1
    d["topk_ids"] = ids
    assert np.all(run_oracle(oracle_mod, d) == 0.0)


def test_fp8_block_scale_indexing_closed_form(oracle_mod):
    """All codes 1.0 (0x38); activation scales 1; gate weight block scale 2^-7 for
    n-block 0, up 2^-6 for n-block 1; K = 256 -> two K-blocks with As = (1, 0.5).
    g = 128*2^-7 + 128*0.5*2^-7 = 1.5, u = 3, h = silu(1.5)*3 (requantized: 448 code,
    scale h/448), down weights 1 with scale 2^-8: y_n = 128*h/256 = h/2."""
    H, I = 256, 128
    c = dict(a_q=np.full((1, H), 0x38, np.uint8), a_s=np.array([[1.0, 0.5]], np.float32),
             w13=np.full((1, 2 * I, H), 0x38, np.uint8),
             s13=np.array([[[2.0 ** -7, 2.0 ** -7], [2.0 ** -6, 2.0 ** -6]]], np.float32),
             w2=np.full((1, H, I), 0x38, np.uint8), s2=np.full((1, 2, 1), 2.0 ** -8, np.float32),
             topk_ids=np.zeros((1, 1), np.int32), topk_weights=np.ones((1, 1), np.float32))
    got = run_oracle(oracle_mod, c)[0]
    h = np.float32(1.5 / (1 + math.exp(-1.5)) * 3.0)
    s = np.float32(h / np.float32(448.0))
    hq = 448.0 * float(s)  # the group's absmax lands on code 448
    assert np.allclose(got, hq * 128 * 2.0 ** -8, rtol=1e-15, atol=0)
