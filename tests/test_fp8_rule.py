"""Pins of the block-FP8 parity rule (fp8_rule.py) on the CPU.

code_intervals: every code that a perturbed h can produce, with the block scale formed
from the perturbed values exactly as the GPU forms it, decodes (torch's float8_e4m3fn
cast after clamping, independent of the oracle's encoder) to a value inside [vlo, vhi];
checked on random perturbations within the error bound, on the bound's extremes, and on a
constructed block in which only the shift of the block scale moves an element across a
rounding midpoint (a rule that ignored the scale's uncertainty fails there).
flip_bound: any choice of codes inside the intervals changes each output element by at
most the bound."""
import numpy as np
import torch

import fp8_rule
from quantized_mixture_experts_amd import inputs


def _e4m3_value(t):
    t = np.clip(t, -448, 448).astype(np.float32)
    return torch.from_numpy(t).to(torch.float8_e4m3fn).double().numpy()


def _gpu_codes(h, I):
    """Decoded E4M3 values of h quantized per 128 columns the way the GPU does it: scale
    max(absmax, 1e-10) / 448 from the values themselves, fp32 division, clamp, RNE."""
    hf = h.astype(np.float32).reshape(h.shape[0], I // 128, 128)
    s = (np.maximum(np.abs(hf).max(axis=2), np.float32(1e-10)) / np.float32(448)).astype(np.float32)
    return _e4m3_value(hf / s[..., None]).reshape(h.shape[0], I)


def _brute_force_inside(det, dh, vlo, vhi, rng, samples=48):
    h = det["h32"].astype(np.float64)
    n, I = h.shape
    for i in range(samples):
        if i % 2:
            z = rng.uniform(-1.0, 1.0, h.shape)
        else:
            z = rng.choice([-1.0, 1.0], h.shape)  # the bound's extremes
        v = _gpu_codes(h + z * dh * (1 - 1e-9), I)
        if not np.all((v >= vlo) & (v <= vhi)):
            return False
    return True


def _detail(oracle_mod, T=40, H=384, I=256, E=5, k=2, seed=3):
    c = inputs.custom_fp8_case(T, H, I, E, k, seed=seed, quantize=oracle_mod.fp8_quantize_blocks)
    ref, det = oracle_mod.fp8_moe_experts(c["a_q"], c["a_s"], c["w13"], c["s13"], c["w2"],
                                          c["s2"], c["topk_ids"], c["topk_weights"], detail=True)
    return c, ref, det


def test_code_intervals_contain_every_reachable_code(oracle_mod):
    c, _, det = _detail(oracle_mod)
    dh = fp8_rule.h_error_bound(det)
    vlo, vhi, _, _ = fp8_rule.code_intervals(oracle_mod, det, dh)
    assert np.all(vlo <= vhi)
    # unflagged elements: the interval is the oracle's own code value
    lut = fp8_rule.e4m3_lut(oracle_mod)
    v = lut[det["hq"]]
    assert np.all((vlo <= v) & (v <= vhi))
    flagged = vlo != vhi
    assert 0 < flagged.mean() < 0.2
    assert _brute_force_inside(det, dh, vlo, vhi, np.random.default_rng(1))
    # a bound ten times wider still holds every code (the rule is monotone in the bound)
    vlo10, vhi10, _, _ = fp8_rule.code_intervals(oracle_mod, det, 10 * dh)
    assert np.all((vlo10 <= vlo) & (vhi10 >= vhi))


def _scale_shift_block():
    """One pair, one 128-column block: element 0 is the block maximum with a large error
    bound, element 1 has none and lies just above a rounding midpoint, so only a larger
    block scale can move it to the code below."""
    I = 128
    h = np.zeros((1, I), np.float64)
    dh = np.zeros((1, I), np.float64)
    h[0, 0], dh[0, 0] = 448.0, 4.0               # scale 1.0, may grow to 452 / 448
    h[0, 1] = 100.0 * (1 + 1e-3)                 # midpoint of 96 and 104 is 100
    h[0, 2:] = np.linspace(-50, 50, I - 2)
    det = {"h32": h.astype(np.float32)}
    return det, dh


def test_scale_uncertainty_is_part_of_the_interval(oracle_mod):
    det, dh = _scale_shift_block()
    vlo, vhi, _, _ = fp8_rule.code_intervals(oracle_mod, det, dh)
    assert vlo[0, 1] == 96.0 and vhi[0, 1] == 104.0
    assert _brute_force_inside(det, dh, vlo, vhi, np.random.default_rng(2))

    def fixed_scale_intervals(det, dh):
        # a plausible mistake: the element's own bound only, the scale taken as exact
        h = det["h32"].astype(np.float64)
        s = np.repeat(np.abs(h).reshape(h.shape[0], -1, 128).max(axis=2), 128, axis=1) / 448
        lut = fp8_rule.e4m3_lut(oracle_mod)
        lo = lut[oracle_mod.f32_to_e4m3(np.clip((h - dh) / s, -448, 448).astype(np.float32))]
        hi = lut[oracle_mod.f32_to_e4m3(np.clip((h + dh) / s, -448, 448).astype(np.float32))]
        return lo, hi

    lo, hi = fixed_scale_intervals(det, dh)
    assert lo[0, 1] == hi[0, 1] == 104.0
    assert not _brute_force_inside(det, dh, lo, hi, np.random.default_rng(2))


def test_flip_bound_covers_any_codes_inside_the_intervals(oracle_mod):
    T, H, I, E, k = 30, 256, 256, 4, 3
    c, ref, det = _detail(oracle_mod, T, H, I, E, k, seed=9)
    dh = fp8_rule.h_error_bound(det) * 30  # wide intervals: many flagged elements
    vlo, vhi, _, _ = fp8_rule.code_intervals(oracle_mod, det, dh)
    B = fp8_rule.flip_bound(oracle_mod, c, det, vlo, vhi, E, k)
    lut = fp8_rule.e4m3_lut(oracle_mod)
    hs = np.repeat(det["hs"].astype(np.float64), 128, axis=1)
    v0 = lut[det["hq"]]
    ids, wts = c["topk_ids"], c["topk_weights"].astype(np.float64)
    w2d = [_e4m3_w(c["w2"][e]) * np.repeat(np.repeat(c["s2"][e].astype(np.float64), 128, 0), 128, 1)
           for e in range(E)]

    def output(v):
        y = np.zeros((T, H))
        for t in range(T):
            for s in range(k):
                e = ids[t, s]
                y[t] += wts[t, s] * (w2d[e] @ (v[t * k + s] * hs[t * k + s]))
        return y

    y0 = output(v0)
    np.testing.assert_allclose(y0, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())
    rng = np.random.default_rng(5)
    assert (vlo != vhi).mean() > 0.05
    for _ in range(4):
        v = np.where(rng.random(v0.shape) < 0.5, vlo, vhi)
        assert np.all(np.abs(output(v) - y0) <= B * (1 + 1e-9) + 1e-9)
    # the extreme choice reaches the bound where every flagged term has one sign: the
    # bound is not loose by more than the cancellation between terms
    assert np.abs(output(vhi) - output(vlo)).max() > 0.1 * B.max()


def _e4m3_w(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()
