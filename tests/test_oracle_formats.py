"""Pins for the oracle's scalar formats: bf16 rounding, E4M3 decode/encode and the
block E4M3 quantizer. Checked against the pages' stated format facts (golden files),
torch's float8_e4m3fn / bfloat16 conversions (library special cases), exact brute
force, and invariants of block quantization."""
import json
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_e4m3_decode_matches_page_facts(oracle_mod):
    g = _golden("e4m3_format.json")
    codes = np.arange(256, dtype=np.uint8)
    v = oracle_mod.e4m3_to_f64(codes)
    finite = v[np.isfinite(v)]
    assert finite.max() == g["max_finite"] and finite.min() == -g["max_finite"]
    # 3 mantissa bits: the step just above 1.0 is 2^-3; 4 exponent bits, bias 7
    assert oracle_mod.e4m3_to_f64(np.uint8(0x39)) - 1.0 == 2.0 ** -g["mantissa_bits"]
    assert oracle_mod.e4m3_to_f64(np.uint8(0x38)) == 1.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isfinite(v).sum() == 254


def test_e4m3_decode_matches_torch(oracle_mod):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle_mod.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


def test_e4m3_encode_matches_torch(oracle_mod):
    rng = np.random.default_rng(7)
    parts = [
        rng.uniform(-448, 448, 200000),
        rng.standard_normal(200000) * 0.01,  # subnormal range (< 2^-6)
        rng.standard_normal(200000),
        np.array([0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11, 9.5, 11.5,
                  1.0625, 1.1875, 240.0, 232.0, 248.0, 440.0, 447.99]),
    ]
    # every midpoint between adjacent finite codes: exercises ties-to-even
    vals = np.sort(oracle_mod.e4m3_to_f64(np.arange(0, 0x7F, dtype=np.uint8)))
    mids = (vals[:-1] + vals[1:]) / 2
    parts += [mids, -mids]
    x = np.concatenate(parts).astype(np.float32)
    x = np.clip(x, -448, 448)
    ours = oracle_mod.f32_to_e4m3(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_bf16_rounding_is_nearest_even_brute_force(oracle_mod):
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0])])
    b = oracle_mod.f64_to_bf16(x)
    v = oracle_mod.bf16_to_f64(b)
    # neighbours of the chosen bf16 value
    up = oracle_mod.bf16_to_f64((b.astype(np.int32) + 1).astype(np.uint16))
    dn = oracle_mod.bf16_to_f64((b.astype(np.int32) - 1).astype(np.uint16))
    err = np.abs(v - x)
    ok_nonzero = x != 0
    assert np.all(err[ok_nonzero] <= np.abs(up - x)[ok_nonzero])
    assert np.all(err[ok_nonzero] <= np.abs(dn - x)[ok_nonzero])
    # exact ties go to the even significand
    assert b[-4] == 0x3F80 and b[-3] == 0x3F82 and b[-2] == 0xBF80
    # agrees with torch's fp32 -> bf16 conversion where the value is exactly an fp32
    xf = x.astype(np.float32)
    ref = torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle_mod.f64_to_bf16(xf.astype(np.float64)), ref)


def test_block_quantizer_invariants(oracle_mod):
    rng = np.random.default_rng(11)
    R, C = 300, 520  # ragged against [128, 128]
    v = rng.standard_normal((R, C)).astype(np.float32)
    q, s = oracle_mod.fp8_quantize_blocks(v, 128, 128)
    assert s.shape == (3, 5)
    deq = oracle_mod.e4m3_to_f64(q) * np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)[:R, :C]
    for bi in range(3):
        for bj in range(5):
            blk = np.abs(v[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128])
            qb = q[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            # the block's absmax element lands on the largest code, +-448
            i = np.unravel_index(np.argmax(blk), blk.shape)
            assert (qb[i] & 0x7F) == 0x7E
            # scale is absmax/448 to fp32 rounding
            assert math.isclose(float(s[bi, bj]) * 448.0, float(blk.max()), rel_tol=2 ** -22)
    # 3 mantissa bits: relative error at most 2^-4 for normal codes
    normal = np.abs(oracle_mod.e4m3_to_f64(q)) >= 2.0 ** -6
    rel = np.abs(deq - v)[normal] / np.abs(v)[normal]
    assert rel.max() <= 2.0 ** -4 + 1e-7


def test_block_quantizer_blocks_are_independent_and_scale_equivariant(oracle_mod):
    rng = np.random.default_rng(12)
    v = rng.standard_normal((256, 256)).astype(np.float32)
    q, s = oracle_mod.fp8_quantize_blocks(v, 128, 128)
    v2 = v.copy()
    v2[:128, :128] *= np.float32(8.0)  # power of two: codes unchanged, scale x8
    v2[128:, 128:] = 0.0  # an all-zero block
    q2, s2 = oracle_mod.fp8_quantize_blocks(v2, 128, 128)
    assert np.array_equal(q2[:128, :128], q[:128, :128]) and s2[0, 0] == s[0, 0] * 8
    assert np.array_equal(q2[:128, 128:], q[:128, 128:]) and s2[0, 1] == s[0, 1]
    assert np.array_equal(q2[128:, :128], q[128:, :128]) and s2[1, 0] == s[1, 0]
    assert np.all((q2[128:, 128:] & 0x7F) == 0)
    assert s2[1, 1] == np.float32(np.float32(1e-10) / np.float32(448.0))


def test_block_quantizer_token_groups_and_exact_values(oracle_mod):
    # per-token-group [1,128]: every row and 128-column group is its own block
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    vals = oracle_mod.e4m3_to_f64(codes)
    row = np.zeros(128, np.float32)
    row[:127] = vals.astype(np.float32)
    row[127] = 448.0
    v = np.stack([row, -row * np.float32(0.5)])
    q, s = oracle_mod.fp8_quantize_blocks(v, 1, 128)
    assert s.shape == (2, 1) and s[0, 0] == np.float32(1.0) and s[1, 0] == np.float32(0.5)
    assert np.array_equal(q[0, :127], codes)  # representable values survive exactly


def test_fp8_scale_shapes_follow_cdiv_rule(oracle_mod):
    g = _golden("fp8_scale_shapes.json")
    for case in g["cases"]:
        bn, bk = case["block"]
        v = np.zeros((case["N"], 8), np.float32)  # rows only: the block count along N
        _, s = oracle_mod.fp8_quantize_blocks(v, bn, bk)
        assert s.shape[0] == case["Bs_shape"][0]
        assert -(-case["K"] // bk) == case["Bs_shape"][1]
