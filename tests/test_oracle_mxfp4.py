"""Pins for the oracle's MXFP4 (E2M1 codes, E8M0 scales per 32 columns) MoE FFN,
independent of the oracle's own code:

- E8M0 decode equals torch's float8_e8m0fnu for all 256 codes (NaN at 255);
- E2M1 decode: every E2M1 value is an E4M3 value (one more exponent bit, two more
  mantissa bits), so each code is re-encoded bit-wise as an E4M3 byte and decoded by
  torch's float8_e4m3fn; plus sign symmetry and strictly increasing magnitudes;
- brute-force dense evaluation with numpy from that independent decode, the single
  expert as torch's SwiGLU, a nibble-order probe and a scale-block index probe.
"""
import math

import numpy as np
import pytest
import torch

from quantized_mixture_experts_amd import inputs


def e2m1_via_e4m3(codes):
    """E2M1 code -> value by re-encoding as E4M3 (bias 7 instead of 1, mantissa bit at
    the top of E4M3's three) and decoding with torch."""
    codes = np.asarray(codes, dtype=np.int64)
    s, e, m = (codes >> 3) & 1, (codes >> 1) & 3, codes & 1
    # E2M1 subnormal 0.5 * m is the E4M3 normal 2^-1 (exponent field 6) when m = 1
    exp = np.where(e > 0, e + 6, np.where(m == 1, 6, 0))
    man = np.where(e > 0, m << 2, 0)
    byte = (s << 7) | (exp << 3) | man
    t = torch.from_numpy(byte.astype(np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_e8m0_matches_torch(oracle_mod):
    codes = np.arange(256, dtype=np.uint8)
    got = oracle_mod.e8m0_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(got[255]) and np.isnan(ref[255])
    np.testing.assert_array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127


def test_e2m1_matches_e4m3_embedding_and_invariants(oracle_mod):
    codes = np.arange(16, dtype=np.uint8)
    got = oracle_mod.e2m1_to_f64(codes)
    np.testing.assert_array_equal(got, e2m1_via_e4m3(codes))
    mag = got[:8]
    assert np.all(np.diff(mag) > 0) and mag[0] == 0.0
    np.testing.assert_array_equal(got[8:], -mag)
    assert math.copysign(1.0, got[8]) == -1.0  # code 8 is -0
    # only the low nibble of a byte is a code
    np.testing.assert_array_equal(oracle_mod.e2m1_to_f64(codes | 0xF0), got)


def dequant(w, s):
    """[N, K/2] E2M1 pairs + [N, K/32] E8M0 -> fp64 [N, K], independent decode."""
    codes = np.empty((w.shape[0], w.shape[1] * 2), np.int64)
    codes[:, 0::2] = w & 0x0F
    codes[:, 1::2] = w >> 4
    scale = np.ldexp(1.0, s.astype(np.int64) - 127)
    return e2m1_via_e4m3(codes) * np.repeat(scale, 32, axis=1)


def brute_dense(case):
    x = inputs.bf16_value(case["x"]).astype(np.float64)
    ids, wts = case["topk_ids"], case["topk_weights"]
    E, I, T = case["w13"].shape[0], case["w13"].shape[1] // 2, x.shape[0]
    R = np.zeros((T, E))
    for t in range(T):
        for s in range(ids.shape[1]):
            if 0 <= ids[t, s] < E:
                R[t, ids[t, s]] += wts[t, s]
    out = np.zeros((T, x.shape[1]))
    for e in range(E):
        gu = x @ dequant(case["w13"][e], case["s13"][e]).T
        g, u = gu[:, :I], gu[:, I:]
        out += R[:, e:e + 1] * ((g / (1.0 + np.exp(-g)) * u) @ dequant(case["w2"][e], case["s2"][e]).T)
    return out


def run(oracle_mod, case, rows=None):
    return oracle_mod.mxfp4_moe(case["x"], case["w13"], case["s13"], case["w2"], case["s2"],
                                case["topk_ids"], case["topk_weights"], rows=rows, nthreads=4)


def rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


@pytest.mark.parametrize("T,H,I,E,k", [(16, 256, 128, 8, 2), (7, 64, 96, 5, 3), (4, 32, 32, 1, 1)])
def test_matches_brute_force_dense(oracle_mod, T, H, I, E, k):
    case = inputs.custom_mxfp4_case(T, H, I, E, k, seed=200 + T)
    assert rel(run(oracle_mod, case), brute_dense(case)) < 1e-12


def test_single_expert_is_textbook_swiglu(oracle_mod):
    case = inputs.custom_mxfp4_case(5, 64, 64, 1, 1, seed=19)
    case["topk_weights"][:] = 1.0
    x = torch.from_numpy(inputs.bf16_value(case["x"]).astype(np.float64))
    w13 = torch.from_numpy(dequant(case["w13"][0], case["s13"][0]))
    w2 = torch.from_numpy(dequant(case["w2"][0], case["s2"][0]))
    F = torch.nn.functional
    ref = F.linear(F.silu(F.linear(x, w13[:64])) * F.linear(x, w13[64:]), w2).numpy()
    assert rel(run(oracle_mod, case), ref) < 1e-12


def _probe_case(H, I):
    c = dict(x=np.zeros((1, H), np.uint16), topk_ids=np.zeros((1, 1), np.int32),
             topk_weights=np.ones((1, 1), np.float32),
             w13=np.zeros((1, 2 * I, H // 2), np.uint8), s13=np.full((1, 2 * I, H // 32), 127, np.uint8),
             w2=np.full((1, H, I // 2), 0x22, np.uint8), s2=np.full((1, H, I // 32), 127, np.uint8))
    c["w13"][0, I:, :] = 0x22  # up weights all +1 (code 2)
    return c


def test_nibble_order_low_is_even_column(oracle_mod):
    """Byte 0 of gate row 0 = 0xB3: low nibble 3 (+1.5) is column 0, high nibble 11 (-1.5)
    column 1. x_0 = 2, x_1 = 1: g_0 = 3 - 1.5 = 1.5; u = 3; out_n = silu(1.5) * 3."""
    H = I = 32
    c = _probe_case(H, I)
    c["x"][0, 0] = 0x4000  # 2.0
    c["x"][0, 1] = 0x3F80  # 1.0
    c["w13"][0, 0, 0] = 0xB3
    got = run(oracle_mod, c)[0]
    assert np.allclose(got, 1.5 / (1 + math.exp(-1.5)) * 3.0, rtol=1e-14, atol=0)


def test_scale_block_index(oracle_mod):
    """Gate row 0 all +1 with scale code 129 (x4) on columns 32..63 only; x = 1."""
    H, I = 64, 32
    c = _probe_case(H, I)
    c["x"][:] = 0x3F80
    c["w13"][0, 0, :] = 0x22
    c["s13"][0, 0, 1] = 129
    got = run(oracle_mod, c)[0]
    g0 = 32 * 1.0 + 32 * 4.0
    assert np.allclose(got, g0 / (1 + math.exp(-g0)) * 64.0, rtol=1e-14, atol=0)


def test_zero_codes_and_row_subset(oracle_mod):
    case = inputs.custom_mxfp4_case(9, 64, 64, 4, 2, seed=25)
    z = dict(case)
    z["w2"] = np.full_like(case["w2"], 0x80)  # +0 and -0
    assert np.all(run(oracle_mod, z) == 0.0)
    full = run(oracle_mod, case)
    rows = np.array([8, 0, 3])
    np.testing.assert_array_equal(run(oracle_mod, case, rows=rows), full[rows])
