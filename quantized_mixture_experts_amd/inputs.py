"""Seeded synthetic inputs for the routed MoE expert FFN.

This module only draws random numbers and converts them to the storage dtypes the
library takes (bf16 bits, packed bytes). It holds none of the FFN's arithmetic: the
E4M3 block quantizer is passed in by the caller, so tests can use the CPU oracle's
and the benchmark can use the library's.

Workloads (Kimi K2.x-style serving shapes from "vLLM x Novita AI: Chord W4A16 INT4
MoE Kernel for Kimi K2.x", summary and Figure 2; block-FP8 format from "SGLang W8A8
Block FP8 quantization kernel config guide", background section):

  tiny      16 tokens, H 256,  I 128,  8 experts, top-2,  W4A16
  decode    32 tokens, H 7168, I 2048, 48 experts, top-8, W4A16, uniform routing
  prefill   8192 tokens, H 7168, I 2048, 48 experts, top-8, W4A16, Zipf(1.0) routing
  fp8       1024 tokens, H 7168, I 2048, 32 experts, top-8, W8A8 block FP8
  full384   256 tokens, H 7168, I 2048, 384 experts, top-8, W4A16, uniform routing

MXFP4 weights (weight-only, bf16 activations; "xiaotu-moe" project page, overview: the
MoE engine's weight formats include MXFP4 (E2M1)), at the decode and prefill shapes:

  decode_mxfp4   32 tokens, H 7168, I 2048, 48 experts, top-8, uniform routing
  prefill_mxfp4  8192 tokens, H 7168, I 2048, 48 experts, top-8, Zipf(1.0) routing

NVFP4 weights (weight-only, same page's list; "NVFP4-W4A16" checkpoints in the
"guqiong96/Lsglang" README), at the same shapes: decode_nvfp4, prefill_nvfp4.

Grouped layouts (same page, SM90 grouped kernels, Figure 3 and the grouped rows of the
measurements; rows already grouped by expert, one pair of weight 1 per row):

  grouped_prefill  contiguous, 48 experts x 128 rows (no padding), H 7168, I 2048
  grouped_decode   masked, 48 experts x 32 valid rows in a budget of max_m = 64

Recipe (per case, numpy default_rng(seed), draws in this order):
  x       bf16(N(0,1)) [T,H]                      (FP8: fp32 N(0,1) source)
  router  logits N(0,1) [T,E]; Zipf: log(1/(e+1)) + Gumbel(0,1)
          softmax (fp32, max-subtracted) -> top-k (ties to the lower id) -> renormalize
  W4A16   w13 uniform bytes [E,2I,H/2]; s13 bf16(|N(0,1)|*0.02) [E,2I,H/32];
          w2 uniform bytes [E,H,I/2];  s2 bf16(|N(0,1)|*0.02) [E,H,I/32]
  FP8     per expert: w13 source N(0,1) [2I,H], then w2 source N(0,1) [H,I],
          each quantized in [128,128] blocks by the caller's quantizer
  NVFP4   w13 uniform bytes; s13 E4M3 codes with exponent field 4..6 and any mantissa
          (0.125 .. 0.9375) [E,2I,H/16]; g13 fp32 |N(0,1)|*0.02+0.01 [E]; w2, s2, g2 likewise
  MXFP4   w13 uniform bytes [E,2I,H/2] (every E2M1 code, -0 included);
          s13 E8M0 codes uniform in {119, 120, 121} (2^-8 .. 2^-6) [E,2I,H/32];
          w2 uniform bytes [E,H,I/2]; s2 likewise [E,H,I/32]
"""
from dataclasses import dataclass

import numpy as np

SEED_BASE = 20260


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    fmt: str  # "w4a16", "mxfp4", "nvfp4" or "fp8"
    routing: str  # "uniform" or "zipf"
    index: int  # 1-based position in the workload list; seeds are SEED_BASE + index

    @property
    def P(self) -> int:
        return self.T * self.k

    @property
    def seed(self) -> int:
        return SEED_BASE + self.index


CONFIGS = {
    "tiny": MoEConfig("tiny", 16, 256, 128, 8, 2, "w4a16", "uniform", 1),
    "decode": MoEConfig("decode", 32, 7168, 2048, 48, 8, "w4a16", "uniform", 2),
    "prefill": MoEConfig("prefill", 8192, 7168, 2048, 48, 8, "w4a16", "zipf", 3),
    "fp8": MoEConfig("fp8", 1024, 7168, 2048, 32, 8, "fp8", "uniform", 4),
    "full384": MoEConfig("full384", 256, 7168, 2048, 384, 8, "w4a16", "uniform", 5),
    "decode_mxfp4": MoEConfig("decode_mxfp4", 32, 7168, 2048, 48, 8, "mxfp4", "uniform", 8),
    "prefill_mxfp4": MoEConfig("prefill_mxfp4", 8192, 7168, 2048, 48, 8, "mxfp4", "zipf", 9),
    "decode_nvfp4": MoEConfig("decode_nvfp4", 32, 7168, 2048, 48, 8, "nvfp4", "uniform", 10),
    "prefill_nvfp4": MoEConfig("prefill_nvfp4", 8192, 7168, 2048, 48, 8, "nvfp4", "zipf", 11),
}


def bf16_bits(a) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (storage conversion)."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_value(b) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def router_logits(rng: np.random.Generator, T: int, E: int, kind: str = "uniform"):
    """Router logits fp32 [T,E].

    uniform: i.i.d. N(0,1), so every k-subset of experts is equally likely to be the top k.
    zipf: log(p_e) + Gumbel(0,1) with p_e proportional to 1/(e+1); the top-k of
    Gumbel-perturbed log-probabilities samples k distinct experts without replacement
    in proportion to p (expert 0 the most popular).
    """
    if kind == "uniform":
        return rng.standard_normal((T, E), dtype=np.float32)
    if kind == "zipf":
        logp = -np.log(np.arange(1, E + 1, dtype=np.float64))
        logp -= np.log(np.exp(logp).sum())
        g = rng.gumbel(0.0, 1.0, size=(T, E))
        return (logp[None, :] + g).astype(np.float32)
    raise ValueError(kind)


def routing(rng: np.random.Generator, T: int, E: int, k: int, kind: str = "uniform"):
    """Routed FFN inputs: topk_ids int32 [T,k] (descending probability), topk_weights fp32
    [T,k], from router_logits by a host softmax (fp32) -> top-k -> renormalization. This
    only draws inputs for the expert FFN; the router step itself is tested separately
    against the oracle on the logits alone."""
    logits = router_logits(rng, T, E, kind)
    z = logits - logits.max(axis=1, keepdims=True)
    ez = np.exp(z, dtype=np.float32)
    p = ez / ez.sum(axis=1, keepdims=True, dtype=np.float32)
    order = np.argsort(-p, axis=1, kind="stable")  # equal values keep the lower id first
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(p, ids, axis=1).astype(np.float32)
    w = (sel / sel.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    return np.ascontiguousarray(ids), np.ascontiguousarray(w)


def _scales(rng, shape):
    return bf16_bits(np.abs(rng.standard_normal(shape, dtype=np.float32)) * np.float32(0.02))


def _bytes(rng, shape):
    n = int(np.prod(shape))
    return np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(shape).copy()


def w4a16_case(cfg: MoEConfig, seed=None) -> dict:
    """All host arrays of one W4A16 case (see the module recipe)."""
    if cfg.fmt != "w4a16":
        raise ValueError(cfg.fmt)
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    x = bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    ids, wts = routing(rng, T, E, k, cfg.routing)
    w13 = _bytes(rng, (E, 2 * I, H // 2))
    s13 = _scales(rng, (E, 2 * I, H // 32))
    w2 = _bytes(rng, (E, H, I // 2))
    s2 = _scales(rng, (E, H, I // 32))
    return dict(x=x, topk_ids=ids, topk_weights=wts, w13=w13, s13=s13, w2=w2, s2=s2)


def _e8m0(rng, shape):
    return rng.integers(119, 122, size=shape, dtype=np.uint8)


def mxfp4_case(cfg: MoEConfig, seed=None) -> dict:
    """All host arrays of one MXFP4 case (see the module recipe)."""
    if cfg.fmt != "mxfp4":
        raise ValueError(cfg.fmt)
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    x = bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    ids, wts = routing(rng, T, E, k, cfg.routing)
    w13 = _bytes(rng, (E, 2 * I, H // 2))
    s13 = _e8m0(rng, (E, 2 * I, H // 32))
    w2 = _bytes(rng, (E, H, I // 2))
    s2 = _e8m0(rng, (E, H, I // 32))
    return dict(x=x, topk_ids=ids, topk_weights=wts, w13=w13, s13=s13, w2=w2, s2=s2)


def _e4m3_scales(rng, shape):
    # positive E4M3 codes: exponent field 4..6, any mantissa
    return (rng.integers(4, 7, size=shape, dtype=np.uint8) << 3) | rng.integers(0, 8, size=shape, dtype=np.uint8)


def nvfp4_case(cfg: MoEConfig, seed=None) -> dict:
    """All host arrays of one NVFP4 case (see the module recipe)."""
    if cfg.fmt != "nvfp4":
        raise ValueError(cfg.fmt)
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    x = bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    ids, wts = routing(rng, T, E, k, cfg.routing)
    w13 = _bytes(rng, (E, 2 * I, H // 2))
    s13 = _e4m3_scales(rng, (E, 2 * I, H // 16))
    g13 = (np.abs(rng.standard_normal(E, dtype=np.float32)) * np.float32(0.02) + np.float32(0.01))
    w2 = _bytes(rng, (E, H, I // 2))
    s2 = _e4m3_scales(rng, (E, H, I // 16))
    g2 = (np.abs(rng.standard_normal(E, dtype=np.float32)) * np.float32(0.02) + np.float32(0.01))
    return dict(x=x, topk_ids=ids, topk_weights=wts, w13=w13, s13=s13, g13=g13, w2=w2, s2=s2,
                g2=g2)


def custom_nvfp4_case(T, H, I, E, k, seed, kind="uniform") -> dict:
    return nvfp4_case(MoEConfig("custom", T, H, I, E, k, "nvfp4", kind, 0), seed=seed)


def custom_mxfp4_case(T, H, I, E, k, seed, kind="uniform") -> dict:
    return mxfp4_case(MoEConfig("custom", T, H, I, E, k, "mxfp4", kind, 0), seed=seed)


def fp8_case(cfg: MoEConfig, quantize, seed=None) -> dict:
    """All host arrays of one W8A8 block-FP8 case.

    quantize(v_fp32_2d, br, bc) -> (codes uint8, scales fp32) is the caller's block
    quantizer; activations use [1,128] blocks, weights [128,128].
    """
    if cfg.fmt != "fp8":
        raise ValueError(cfg.fmt)
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    x_src = rng.standard_normal((T, H), dtype=np.float32)
    ids, wts = routing(rng, T, E, k, cfg.routing)
    a_q, a_s = quantize(x_src, 1, 128)
    w13 = np.empty((E, 2 * I, H), np.uint8)
    s13 = np.empty((E, 2 * I // 128, H // 128), np.float32)
    w2 = np.empty((E, H, I), np.uint8)
    s2 = np.empty((E, H // 128, I // 128), np.float32)
    for e in range(E):
        w13[e], s13[e] = quantize(rng.standard_normal((2 * I, H), dtype=np.float32), 128, 128)
        w2[e], s2[e] = quantize(rng.standard_normal((H, I), dtype=np.float32), 128, 128)
    return dict(a_q=a_q, a_s=a_s, topk_ids=ids, topk_weights=wts, w13=w13, s13=s13, w2=w2, s2=s2)


def custom_w4a16_case(T, H, I, E, k, seed, kind="uniform") -> dict:
    """A W4A16 case of any shape with the same recipe (for ragged and edge shapes)."""
    return w4a16_case(MoEConfig("custom", T, H, I, E, k, "w4a16", kind, 0), seed=seed)


def custom_fp8_case(T, H, I, E, k, seed, quantize, kind="uniform") -> dict:
    return fp8_case(MoEConfig("custom", T, H, I, E, k, "fp8", kind, 0), quantize, seed=seed)


def _w4a16_weights(rng, H, I, E):
    w13 = _bytes(rng, (E, 2 * I, H // 2))
    s13 = _scales(rng, (E, 2 * I, H // 32))
    w2 = _bytes(rng, (E, H, I // 2))
    s2 = _scales(rng, (E, H, I // 32))
    return dict(w13=w13, s13=s13, w2=w2, s2=s2)


def grouped_contiguous_case(counts, H, I, pad, seed) -> dict:
    """Contiguous grouped layout: expert g's counts[g] rows, then padding rows (index -1)
    up to a multiple of `pad` rows, expert after expert. Draws: a bf16(N(0,1)) [M,H]
    (padding rows too), then the W4A16 weights of len(counts) experts."""
    rng = np.random.default_rng(seed)
    counts = [int(c) for c in counts]
    padded = [-(-c // pad) * pad for c in counts]
    M = sum(padded)
    a = bf16_bits(rng.standard_normal((M, H), dtype=np.float32))
    m_indices = np.full(M, -1, np.int32)
    at = 0
    for g, (c, p) in enumerate(zip(counts, padded)):
        m_indices[at:at + c] = g
        at += p
    return dict(a=a, m_indices=m_indices, **_w4a16_weights(rng, H, I, len(counts)))


def grouped_masked_case(counts, max_m, H, I, seed) -> dict:
    """Masked grouped layout: a [E, max_m, H] bf16(N(0,1)) (every budget row drawn),
    masked_m = counts as int32, then the W4A16 weights of len(counts) experts."""
    rng = np.random.default_rng(seed)
    E = len(counts)
    a = bf16_bits(rng.standard_normal((E, max_m, H), dtype=np.float32))
    masked_m = np.asarray(counts, dtype=np.int32)
    return dict(a=a, masked_m=masked_m, **_w4a16_weights(rng, H, I, E))


GROUPED = {
    "grouped_prefill": dict(layout="contiguous", E=48, rows=128, H=7168, I=2048, seed=SEED_BASE + 6),
    "grouped_decode": dict(layout="masked", E=48, rows=32, max_m=64, H=7168, I=2048,
                           seed=SEED_BASE + 7),
}


def grouped_case(name: str) -> dict:
    """One of the GROUPED workloads: every expert holds the same number of valid rows."""
    g = GROUPED[name]
    counts = [g["rows"]] * g["E"]
    if g["layout"] == "contiguous":
        return grouped_contiguous_case(counts, g["H"], g["I"], 128, g["seed"])
    return grouped_masked_case(counts, g["max_m"], g["H"], g["I"], g["seed"])


def sample_rows(T: int, n: int, seed: int) -> np.ndarray:
    """A sorted seeded subset of n token rows (all rows if n >= T)."""
    if n >= T:
        return np.arange(T, dtype=np.int64)
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(T, size=n, replace=False)).astype(np.int64)
