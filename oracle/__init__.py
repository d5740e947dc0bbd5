"""CPU oracle for the routed, weight-quantized MoE expert FFN (ctypes front end).

TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the benchmark's CPU
baseline may import this package; the product package never does, and the HIP
library shares no code with it. The arithmetic lives in oracle.c (plain loops,
fp64); this module only marshals numpy arrays.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_moe_align.argtypes = [_P, _I64, _I32, _I32, _P, _I64, _P, _I64, _P, _P]
    lib.oracle_moe_align.restype = ctypes.c_int
    lib.oracle_topk_softmax.argtypes = [_P, _I64, _I32, _I32, _I32, _P, _P, _P]
    lib.oracle_topk_softmax.restype = ctypes.c_int
    lib.oracle_w4a16_moe.argtypes = [_P] * 7 + [_I64] * 5 + [_P, _I64, _P, ctypes.c_int]
    lib.oracle_w4a16_moe.restype = ctypes.c_int
    lib.oracle_mxfp4_moe.argtypes = [_P] * 7 + [_I64] * 5 + [_P, _I64, _P, ctypes.c_int]
    lib.oracle_mxfp4_moe.restype = ctypes.c_int
    lib.oracle_nvfp4_moe.argtypes = [_P] * 9 + [_I64] * 5 + [_P, _I64, _P, ctypes.c_int]
    lib.oracle_nvfp4_moe.restype = ctypes.c_int
    lib.oracle_fp8_moe.argtypes = [_P] * 8 + [_I64] * 5 + [_P, _I64, _P, ctypes.c_int]
    lib.oracle_fp8_moe.restype = ctypes.c_int
    for fn in ("oracle_w4a16_moe_experts", "oracle_mxfp4_moe_experts"):
        getattr(lib, fn).argtypes = [_P] * 7 + [_I64] * 5 + [_P, _I64, _P, ctypes.c_int]
        getattr(lib, fn).restype = ctypes.c_int
    lib.oracle_nvfp4_moe_experts.argtypes = [_P] * 9 + [_I64] * 5 + [_P, _I64, _P, ctypes.c_int]
    lib.oracle_nvfp4_moe_experts.restype = ctypes.c_int
    lib.oracle_fp8_moe_experts.argtypes = ([_P] * 8 + [_I64] * 5 + [_P, _I64, _P, ctypes.c_int]
                                           + [_P] * 7)
    lib.oracle_fp8_moe_experts.restype = ctypes.c_int
    lib.oracle_fp8_quantize_blocks.argtypes = [_P, _I64, _I64, _I64, _I64, _P, _P]
    lib.oracle_fp8_quantize_blocks.restype = ctypes.c_int
    lib.oracle_f64_to_bf16_array.argtypes = [_P, _I64, _P]
    lib.oracle_e4m3_to_f64_array.argtypes = [_P, _I64, _P]
    lib.oracle_e2m1_to_f64_array.argtypes = [_P, _I64, _P]
    lib.oracle_e8m0_to_f64_array.argtypes = [_P, _I64, _P]
    lib.oracle_f32_to_e4m3_array.argtypes = [_P, _I64, _P]
    _lib = lib
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def default_threads() -> int:
    """Every CPU this process may run on (its affinity mask), capped by OMP_NUM_THREADS
    when that is set (the host's share for one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def align_capacity(P: int, E: int, B: int):
    """Sorted-id capacity L = P + E*(B-1) and block capacity NB = ceil(L/B)."""
    L = P + E * (B - 1)
    return L, (L + B - 1) // B


def topk_softmax(logits, k: int, renormalize: bool = True, expert_map=None):
    """Router: softmax over each token's fp32 logits [T,E], its k largest (equal logits:
    lower id first), weights renormalized over the k or not; ids mapped through
    expert_map [E] when given. Returns (ids int32 [T,k], weights float64 [T,k])."""
    lg = _c(logits, np.float32)
    T, E = lg.shape
    mp = None if expert_map is None else _c(expert_map, np.int32)
    ids = np.empty((T, k), np.int32)
    wts = np.empty((T, k), np.float64)
    rc = _load().oracle_topk_softmax(_ptr(lg), T, E, k, 1 if renormalize else 0,
                                     None if mp is None else _ptr(mp), _ptr(ids), _ptr(wts))
    if rc != 0:
        raise ValueError("oracle_topk_softmax: bad arguments")
    return ids, wts


def moe_align(topk_ids, E: int, B: int):
    """Stable counting sort of flat pair indices by expert, padded per expert to B.

    Returns (sorted_ids [L], expert_ids [NB], num_tokens_padded, expert_offsets [E+1]).
    """
    ids = _c(np.asarray(topk_ids).reshape(-1), np.int32)
    P = ids.size
    L, NB = align_capacity(P, E, B)
    sorted_ids = np.empty(L, np.int32)
    expert_ids = np.empty(NB, np.int32)
    ntp = np.zeros(1, np.int32)
    offs = np.empty(E + 1, np.int32)
    rc = _load().oracle_moe_align(_ptr(ids), P, E, B, _ptr(sorted_ids), L, _ptr(expert_ids), NB,
                                  _ptr(ntp), _ptr(offs))
    if rc != 0:
        raise ValueError("oracle_moe_align: bad arguments")
    return sorted_ids, expert_ids, int(ntp[0]), offs


def _w4_moe(fn, sdtype, x, w13, s13, w2, s2, topk_ids, topk_weights, rows, nthreads):
    x = _c(x, np.uint16)
    w13 = _c(w13, np.uint8)
    s13 = _c(s13, sdtype)
    w2 = _c(w2, np.uint8)
    s2 = _c(s2, sdtype)
    ids = _c(topk_ids, np.int32)
    wts = _c(topk_weights, np.float32)
    T, H = x.shape
    E, twoI, _ = w13.shape
    I = twoI // 2
    k = ids.shape[1]
    if rows is None:
        rows_arr, nrows, rp = None, T, None
    else:
        rows_arr = _c(np.asarray(rows, dtype=np.int64), np.int64)
        nrows, rp = rows_arr.size, _ptr(rows_arr)
    out = np.zeros((nrows, H), np.float64)
    rc = getattr(_load(), fn)(_ptr(x), _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2), _ptr(ids),
                              _ptr(wts), T, H, I, E, k, rp, nrows, _ptr(out),
                              nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"{fn}: bad arguments")
    return out


def w4a16_moe(x, w13, s13, w2, s2, topk_ids, topk_weights, rows=None, nthreads=None):
    """Routed W4A16 MoE FFN in fp64 for the given token rows (all rows if None).

    x [T,H] uint16 (bf16 bits); w13 [E,2I,H/2] uint8; s13 [E,2I,H/32] uint16;
    w2 [E,H,I/2] uint8; s2 [E,H,I/32] uint16; topk_ids int32 [T,k];
    topk_weights float32 [T,k]. Returns float64 [nrows, H] (before bf16 rounding).
    """
    return _w4_moe("oracle_w4a16_moe", np.uint16, x, w13, s13, w2, s2, topk_ids, topk_weights,
                   rows, nthreads)


def mxfp4_moe(x, w13, s13, w2, s2, topk_ids, topk_weights, rows=None, nthreads=None):
    """Routed MoE FFN with MXFP4 weights (E2M1 codes packed like the INT4 codes, E8M0
    scales per row and 32 columns: s13 [E,2I,H/32] uint8, s2 [E,H,I/32] uint8) and bf16
    activations, in fp64. Returns float64 [nrows, H] (before bf16 rounding)."""
    return _w4_moe("oracle_mxfp4_moe", np.uint8, x, w13, s13, w2, s2, topk_ids, topk_weights,
                   rows, nthreads)

def nvfp4_moe(x, w13, s13, g13, w2, s2, g2, topk_ids, topk_weights, rows=None, nthreads=None):
    """Routed MoE FFN with NVFP4 weights (E2M1 codes packed like the INT4 codes, E4M3
    scales per row and 16 columns: s13 [E,2I,H/16] uint8, s2 [E,H,I/16] uint8, fp32
    global scales g13 [E], g2 [E]) and bf16 activations, in fp64. Returns float64
    [nrows, H] (before bf16 rounding)."""
    x = _c(x, np.uint16)
    w13, s13, w2, s2 = (_c(a, np.uint8) for a in (w13, s13, w2, s2))
    g13, g2 = _c(g13, np.float32), _c(g2, np.float32)
    ids = _c(topk_ids, np.int32)
    wts = _c(topk_weights, np.float32)
    T, H = x.shape
    E, twoI, _ = w13.shape
    k = ids.shape[1]
    if rows is None:
        nrows, rp = T, None
    else:
        rows_arr = _c(np.asarray(rows, dtype=np.int64), np.int64)
        nrows, rp = rows_arr.size, _ptr(rows_arr)
    out = np.zeros((nrows, H), np.float64)
    rc = _load().oracle_nvfp4_moe(_ptr(x), _ptr(w13), _ptr(s13), _ptr(g13), _ptr(w2), _ptr(s2),
                                  _ptr(g2), _ptr(ids), _ptr(wts), T, H, twoI // 2, E, k, rp,
                                  nrows, _ptr(out), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_nvfp4_moe: bad arguments")
    return out


def w4a16_grouped_contiguous(a, w13, s13, w2, s2, m_indices, rows=None, nthreads=None):
    """The W4A16 expert FFN on the contiguous grouped layout ("vLLM x Novita AI: Chord W4A16
    INT4 MoE Kernel for Kimi K2.x", SM90 grouped kernels and Figure 3): row r is the single
    pair (r, m_indices[r]) of weight 1; an index outside [0, E) marks padding, whose output
    row is 0. a [M,H] bf16 bits, m_indices int32 [M]. Returns float64 [nrows, H]."""
    ids = np.ascontiguousarray(np.asarray(m_indices, dtype=np.int32).reshape(-1, 1))
    return w4a16_moe(a, w13, s13, w2, s2, ids, np.ones(ids.shape, np.float32), rows, nthreads)


def w4a16_grouped_masked(a, w13, s13, w2, s2, masked_m, rows=None, nthreads=None):
    """The W4A16 expert FFN on the masked grouped layout (same page and section): a
    [E, max_m, H] bf16 bits; row r of expert g (flat row g * max_m + r) is the pair (row,
    g) of weight 1 when r < masked_m[g] (counts taken within [0, max_m]) and 0 otherwise.
    Returns float64 [nrows, H] over the flat rows."""
    E, max_m, H = a.shape
    counts = np.clip(np.asarray(masked_m, dtype=np.int64), 0, max_m)
    valid = np.arange(max_m)[None, :] < counts[:, None]
    ids = np.where(valid, np.arange(E)[:, None], -1).astype(np.int32).reshape(-1, 1)
    return w4a16_moe(np.ascontiguousarray(a).reshape(E * max_m, H), w13, s13, w2, s2, ids,
                     np.ones(ids.shape, np.float32), rows, nthreads)


def fp8_moe(a_q, a_s, w13, s13, w2, s2, topk_ids, topk_weights, rows=None, nthreads=None):
    """Routed W8A8 block-FP8 MoE FFN in fp64 (h requantized per 128 in fp32)."""
    a_q = _c(a_q, np.uint8)
    a_s = _c(a_s, np.float32)
    w13 = _c(w13, np.uint8)
    s13 = _c(s13, np.float32)
    w2 = _c(w2, np.uint8)
    s2 = _c(s2, np.float32)
    ids = _c(topk_ids, np.int32)
    wts = _c(topk_weights, np.float32)
    T, H = a_q.shape
    E, twoI, _ = w13.shape
    I = twoI // 2
    k = ids.shape[1]
    if rows is None:
        rows_arr, nrows, rp = None, T, None
    else:
        rows_arr = _c(np.asarray(rows, dtype=np.int64), np.int64)
        nrows, rp = rows_arr.size, _ptr(rows_arr)
    out = np.zeros((nrows, H), np.float64)
    rc = _load().oracle_fp8_moe(_ptr(a_q), _ptr(a_s), _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2),
                                _ptr(ids), _ptr(wts), T, H, I, E, k, rp, nrows, _ptr(out),
                                nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_fp8_moe: bad arguments")
    return out


def _rows(rows, T):
    if rows is None:
        return None, T, None
    rows_arr = _c(np.asarray(rows, dtype=np.int64), np.int64)
    return rows_arr, rows_arr.size, _ptr(rows_arr)


def w4a16_moe_experts(x, w13, s13, w2, s2, topk_ids, topk_weights, rows=None, nthreads=None):
    """oracle_w4a16_moe's result, computed expert by expert (each weight row dequantized
    once for all the expert's routed pairs; every sum in the same order, so the result is
    bit-identical). For checking full-size workloads."""
    return _w4_moe("oracle_w4a16_moe_experts", np.uint16, x, w13, s13, w2, s2, topk_ids,
                   topk_weights, rows, nthreads)


def mxfp4_moe_experts(x, w13, s13, w2, s2, topk_ids, topk_weights, rows=None, nthreads=None):
    """mxfp4_moe's result, computed expert by expert (bit-identical)."""
    return _w4_moe("oracle_mxfp4_moe_experts", np.uint8, x, w13, s13, w2, s2, topk_ids,
                   topk_weights, rows, nthreads)


def nvfp4_moe_experts(x, w13, s13, g13, w2, s2, g2, topk_ids, topk_weights, rows=None,
                      nthreads=None):
    """nvfp4_moe's result, computed expert by expert (bit-identical)."""
    x = _c(x, np.uint16)
    w13, s13, w2, s2 = (_c(a, np.uint8) for a in (w13, s13, w2, s2))
    g13, g2 = _c(g13, np.float32), _c(g2, np.float32)
    ids = _c(topk_ids, np.int32)
    wts = _c(topk_weights, np.float32)
    T, H = x.shape
    E, twoI, _ = w13.shape
    k = ids.shape[1]
    _, nrows, rp = _rows(rows, T)
    out = np.zeros((nrows, H), np.float64)
    rc = _load().oracle_nvfp4_moe_experts(_ptr(x), _ptr(w13), _ptr(s13), _ptr(g13), _ptr(w2),
                                          _ptr(s2), _ptr(g2), _ptr(ids), _ptr(wts), T, H,
                                          twoI // 2, E, k, rp, nrows, _ptr(out),
                                          nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_nvfp4_moe_experts: bad arguments")
    return out


def fp8_moe_experts(a_q, a_s, w13, s13, w2, s2, topk_ids, topk_weights, rows=None,
                    nthreads=None, detail=False):
    """fp8_moe's result, computed expert by expert (bit-identical). With detail=True also
    returns a dict of per-pair arrays indexed [r * k + s] for the listed rows (r = position
    in `rows`; dropped slots are left zero): g, u (fp64 gate and up sums), gmag, umag
    (sum over c of |x_c W13(j, c)|, the magnitudes an accumulation error scales with), h32
    (fp32 SiLU(g) * u before quantization), hq (its E4M3 codes), hs (fp32 scale per 128)."""
    a_q = _c(a_q, np.uint8)
    a_s = _c(a_s, np.float32)
    w13 = _c(w13, np.uint8)
    s13 = _c(s13, np.float32)
    w2 = _c(w2, np.uint8)
    s2 = _c(s2, np.float32)
    ids = _c(topk_ids, np.int32)
    wts = _c(topk_weights, np.float32)
    T, H = a_q.shape
    E, twoI, _ = w13.shape
    I = twoI // 2
    k = ids.shape[1]
    _, nrows, rp = _rows(rows, T)
    out = np.zeros((nrows, H), np.float64)
    d = None
    dp = [None] * 7
    if detail:
        n = nrows * k
        d = dict(g=np.zeros((n, I)), u=np.zeros((n, I)), gmag=np.zeros((n, I)),
                 umag=np.zeros((n, I)), h32=np.zeros((n, I), np.float32),
                 hq=np.zeros((n, I), np.uint8), hs=np.zeros((n, I // 128), np.float32))
        dp = [_ptr(d[key]) for key in ("g", "u", "gmag", "umag", "h32", "hq", "hs")]
    rc = _load().oracle_fp8_moe_experts(_ptr(a_q), _ptr(a_s), _ptr(w13), _ptr(s13), _ptr(w2),
                                        _ptr(s2), _ptr(ids), _ptr(wts), T, H, I, E, k, rp, nrows,
                                        _ptr(out), nthreads or default_threads(), *dp)
    if rc != 0:
        raise ValueError("oracle_fp8_moe_experts: bad arguments")
    return (out, d) if detail else out


def fp8_quantize_blocks(v, br: int, bc: int):
    """Block E4M3 quantizer on a 2-D fp32 array: returns (codes uint8, scales fp32)."""
    v = _c(v, np.float32)
    R, C = v.shape
    q = np.empty((R, C), np.uint8)
    s = np.empty(((R + br - 1) // br, (C + bc - 1) // bc), np.float32)
    rc = _load().oracle_fp8_quantize_blocks(_ptr(v), R, C, br, bc, _ptr(q), _ptr(s))
    if rc != 0:
        raise ValueError("oracle_fp8_quantize_blocks: bad arguments")
    return q, s


def e2m1_to_f64(codes):
    """E2M1 codes (low 4 bits of each uint8) -> float64."""
    c = _c(np.asarray(codes, dtype=np.uint8), np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().oracle_e2m1_to_f64_array(_ptr(c), c.size, _ptr(out))
    return out


def e8m0_to_f64(codes):
    """E8M0 scale codes (uint8) -> float64 2^(code - 127); 255 -> NaN."""
    c = _c(np.asarray(codes, dtype=np.uint8), np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().oracle_e8m0_to_f64_array(_ptr(c), c.size, _ptr(out))
    return out


def f64_to_bf16(x):
    """fp64 -> bf16 bits (uint16), round to nearest even from the exact value."""
    x = _c(np.asarray(x, dtype=np.float64), np.float64)
    out = np.empty(x.shape, np.uint16)
    _load().oracle_f64_to_bf16_array(_ptr(x), x.size, _ptr(out))
    return out


def bf16_to_f64(b):
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3_to_f64(codes):
    c = _c(np.asarray(codes, dtype=np.uint8), np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().oracle_e4m3_to_f64_array(_ptr(c), c.size, _ptr(out))
    return out


def f32_to_e4m3(x):
    x = _c(np.asarray(x, dtype=np.float32), np.float32)
    out = np.empty(x.shape, np.uint8)
    _load().oracle_f32_to_e4m3_array(_ptr(x), x.size, _ptr(out))
    return out
