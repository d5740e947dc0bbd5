/*
 * CPU oracle for the routed, weight-quantized MoE expert FFN.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or load
 * this file or the library built from it: only the tests, the smoke check and the
 * benchmark's CPU-baseline leg use it. It shares no code, header, table or helper
 * with the HIP library; the two meet only through the seeded inputs both are given.
 *
 * Every step is written out plainly, in the order the method states it, in fp64
 * unless a step fixes a narrower precision (the E4M3 quantizer decides integer
 * codes, so it runs in fp32, the precision a GPU kernel takes that decision in).
 *
 * Sources (web pages, cited by title and section):
 *  [CHORD]  "vLLM x Novita AI: Chord W4A16 INT4 MoE Kernel for Kimi K2.x"
 *           (Novita AI blog): summary (BF16 activations, INT4 weights, group-32
 *           scales); section "Two kernel families" (indexed routing tensors
 *           sorted_ids / expert_ids / num_tokens_padded); section "vLLM
 *           integration" (uint4, group-32, BF16 scales; over-allocated align
 *           buffers); section "H200 and Blackwell indexed decode" (dequantize as
 *           subtract-then-scale on the extracted nibble); Figure 3 (padding guards
 *           in the routing indices; -1 marks padding rows).
 *  [SGL]    "SGLang W8A8 Block FP8 quantization kernel config guide" (xdnf.cn):
 *           section "Background of the W8A8 Block FP8 kernel" (E4M3, 4-bit
 *           exponent, 3-bit mantissa, max about 448; per-[BLOCK_N, BLOCK_K] weight
 *           scales from the block absmax; per-token-group activation scales As).
 *  [LSG]    "guqiong96/Lsglang" README (SkillsMP page), section "Super Mix
 *           Prefill": the fp32-activation engine matches the CPU reference.
 *  [XT]     "xiaotu-moe" (PyPI project page), overview: the weight-only formats the
 *           MoE engine supports include MXFP4 (E2M1) beside BF16, FP8 and NVFP4.
 *
 * Readings where the pages are silent (each stated again in the design notes):
 *  - fused w13 rows [0, I) are gate, rows [I, 2I) are up;
 *  - activation is silu(gate) * up with silu(z) = z / (1 + exp(-z));
 *  - INT4 byte c/2 holds code c, low nibble = even c; weight = (code - 8) * scale;
 *  - align order inside an expert's segment is ascending flat pair index;
 *    padding and tail slots hold P = T*k, unused block entries hold -1;
 *  - MXFP4 weights (weight-only, bf16 activations, [XT] overview): E2M1 codes packed
 *    like the INT4 codes (byte c/2, low nibble = even c), one E8M0 scale per row and
 *    32 consecutive columns (the OCP microscaling block of 32); weight = e2m1(code) *
 *    2^(scale - 127), with E2M1 = sign bit 3, exponent bits 2..1 (bias 1), mantissa
 *    bit 0, exponent 0 subnormal (0.5 * mantissa); E8M0 code 255 is NaN;
 *  - NVFP4 weights (weight-only, [XT] overview; the "NVFP4-W4A16" checkpoints of [LSG]):
 *    the same E2M1 codes and packing, one E4M3 scale per row and 16 consecutive columns,
 *    and one fp32 scale per expert and projection; weight = e2m1(code) * e4m3(scale) *
 *    global;
 *  - routed ids outside [0, E) are dropped;
 *  - E4M3 is OCP E4M3FN, round-to-nearest-even after clamping to +-448;
 *    block scale = max(absmax, 1e-10) / 448;
 *  - in the W8A8 variant the SiLU*up output is requantized per token and per
 *    128-column group before the down projection;
 *  - the router that feeds the path (the pages give the kernels top-k ids and
 *    weights, [CHORD] "Two kernel families") is softmax over the token's logits,
 *    the k largest, optionally renormalized over the k; equal logits keep the lower
 *    expert id first; an expert-parallel map sends global ids to local ones (-1: held
 *    by another GPU, [CHORD] "vLLM integration", EP8 profiles).
 *
 * Parity pins for every function live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1

/* ------------------------------------------------------------------------- */
/* Scalar formats                                                             */
/* ------------------------------------------------------------------------- */

/* bf16 bit pattern -> value: bf16 is the top half of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round half to even, written out (no reliance on the FP environment). */
static double rne_int(double x) {
  double r = floor(x + 0.5);
  if (r - x == 0.5 && fmod(r, 2.0) != 0.0) r -= 1.0;
  return r;
}

/* fp64 -> bf16, round to nearest even, directly from the exact value.
 * bf16 keeps 8 significant bits and binary32's exponent range. */
uint16_t oracle_f64_to_bf16(double x) {
  if (isnan(x)) return 0x7FC0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
  /* binary32 normal range starts at 2^-126 (e = -125); below it the step is fixed */
  int ee = e < -125 ? -125 : e;
  double scaled = ldexp(a, 8 - ee); /* significand with 8 bits before the point */
  double r = rne_int(scaled);
  double v = ldexp(r, ee - 8);
  if (v >= ldexp(1.0, 128)) return sign | 0x7F80; /* overflow to inf */
  float f = (float)v;                              /* exact: v has <= 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return sign | (uint16_t)((u >> 16) & 0x7FFF);
}

/* OCP E4M3FN decode: sign, 4-bit exponent (bias 7), 3-bit mantissa; exponent 0
 * is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there are no infinities. */
double oracle_e4m3_to_f64(uint8_t c) {
  int s = (c >> 7) & 1, ex = (c >> 3) & 0xF, m = c & 7;
  double v;
  if (ex == 0xF && m == 7) return NAN;
  if (ex == 0)
    v = ldexp((double)m, -9); /* (m/8) * 2^-6 */
  else
    v = ldexp(1.0 + m / 8.0, ex - 7);
  return s ? -v : v;
}

/* fp32 value already clamped to [-448, 448] -> E4M3FN code, round to nearest
 * even. Codes are monotone in magnitude, so subnormals and the first normal
 * binade share one rule below 2^-6 (step 2^-9). */
uint8_t oracle_f32_to_e4m3(float f) {
  double a = fabs((double)f);
  uint8_t sign = (f < 0.0f || (f == 0.0f && signbit(f))) ? 0x80 : 0;
  if (isnan(f)) return 0x7F;
  if (a > 448.0) a = 448.0;
  if (a < ldexp(1.0, -6)) {
    int q = (int)rne_int(a * 512.0); /* 0..8; 8 is the smallest normal */
    return sign | (uint8_t)q;
  }
  int e;
  double m = frexp(a, &e); /* a = m 2^e, m in [0.5,1) -> a = (2m) 2^(e-1) */
  int ex = e - 1;          /* unbiased exponent, -6..8 */
  double frac = 2.0 * m - 1.0;
  int mant = (int)rne_int(frac * 8.0);
  if (mant == 8) {
    mant = 0;
    ex += 1;
  }
  int code = ((ex + 7) << 3) | mant;
  if (code > 0x7E) code = 0x7E; /* cannot happen after the clamp; keep 448 */
  return sign | (uint8_t)code;
}

/* F0: quantize an [R, C] fp32 matrix in [br, bc] blocks. Each block gets
 * scale = max(absmax, 1e-10) / 448 (fp32), and each element becomes
 * e4m3(clamp(v / scale, -448, 448)), all in fp32. scale is [ceil(R/br), ceil(C/bc)]
 * row-major. Per-token-group activations use br = 1, bc = 128; weights use
 * br = bc = 128. */
int oracle_fp8_quantize_blocks(const float* v, int64_t R, int64_t C, int64_t br, int64_t bc,
                               uint8_t* q, float* scale) {
  if (!v || !q || !scale || R < 0 || C < 0 || br <= 0 || bc <= 0) return ORACLE_BAD_ARG;
  int64_t nbr = (R + br - 1) / br, nbc = (C + bc - 1) / bc;
  for (int64_t bi = 0; bi < nbr; ++bi) {
    for (int64_t bj = 0; bj < nbc; ++bj) {
      int64_t r0 = bi * br, r1 = r0 + br < R ? r0 + br : R;
      int64_t c0 = bj * bc, c1 = c0 + bc < C ? c0 + bc : C;
      float amax = 0.0f;
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = c0; c < c1; ++c) {
          float a = fabsf(v[r * C + c]);
          if (a > amax) amax = a;
        }
      float s = (amax > 1e-10f ? amax : 1e-10f) / 448.0f;
      scale[bi * nbc + bj] = s;
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = c0; c < c1; ++c) {
          float t = v[r * C + c] / s;
          if (t > 448.0f) t = 448.0f;
          if (t < -448.0f) t = -448.0f;
          q[r * C + c] = oracle_f32_to_e4m3(t);
        }
    }
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------- */
/* Router (softmax over a token's logits, its top k, optional renormalization) */
/* ------------------------------------------------------------------------- */

/* logits [T, E] fp32. For each token t, in order of decreasing probability:
 *   p_e = exp(l_e) / sum_j exp(l_j)   (softmax),
 *   the k experts with the largest p (= the largest logits; equal logits: lower id),
 *   weight_s = p_s / sum over the k selected p   (renormalize != 0), else p_s.
 * ids[t*k + s] = map ? map[id] : id. Probabilities in fp64 (max-subtracted exponents,
 * which leaves each ratio unchanged). */
int oracle_topk_softmax(const float* logits, int64_t T, int32_t E, int32_t k, int32_t renormalize,
                        const int32_t* map, int32_t* ids, double* weights) {
  if (T < 0 || E <= 0 || k <= 0 || k > E || (T > 0 && (!logits || !ids || !weights)))
    return ORACLE_BAD_ARG;
  double* p = (double*)malloc((size_t)E * sizeof(double));
  unsigned char* used = (unsigned char*)malloc((size_t)E);
  if (!p || !used) {
    free(p);
    free(used);
    return ORACLE_BAD_ARG;
  }
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * E;
    double m = (double)l[0];
    for (int32_t e = 1; e < E; ++e)
      if ((double)l[e] > m) m = (double)l[e];
    double total = 0.0;
    for (int32_t e = 0; e < E; ++e) {
      p[e] = exp((double)l[e] - m);
      total += p[e];
    }
    for (int32_t e = 0; e < E; ++e) p[e] /= total;
    memset(used, 0, (size_t)E);
    double sel = 0.0;
    for (int32_t s = 0; s < k; ++s) {
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e) /* strict '>' keeps the lower id among equals */
        if (!used[e] && (best < 0 || (double)l[e] > (double)l[best])) best = e;
      used[best] = 1;
      ids[t * k + s] = map ? map[best] : best;
      weights[t * k + s] = p[best];
      sel += p[best];
    }
    if (renormalize)
      for (int32_t s = 0; s < k; ++s) weights[t * k + s] /= sel;
  }
  free(p);
  free(used);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------- */
/* Align (sort tokens to experts, pad each expert to a multiple of B)         */
/* ------------------------------------------------------------------------- */

/* Inputs: topk_ids [P] (P = T*k, flat pair index i = t*k + s), E experts, block B.
 * Outputs (capacities given by the caller):
 *   sorted_ids [L]: each expert e owns segment [off_e, off_e + ceil(c_e/B)*B);
 *     its first c_e entries are its pair indices in ascending order, the rest
 *     of the segment and everything past off_E hold the sentinel P;
 *   expert_ids [NB]: expert of each B-row block, -1 past the used blocks;
 *   num_tokens_padded [1] = off_E;  expert_offsets [E+1] = off (may be NULL).
 * Requires L >= P + E*(B-1) and NB >= ceil(L/B). Ids outside [0, E) are dropped. */
int oracle_moe_align(const int32_t* topk_ids, int64_t P, int32_t E, int32_t B, int32_t* sorted_ids,
                     int64_t L, int32_t* expert_ids, int64_t NB, int32_t* num_tokens_padded,
                     int32_t* expert_offsets) {
  if (!topk_ids || !sorted_ids || !expert_ids || !num_tokens_padded || P < 0 || E <= 0 || B <= 0)
    return ORACLE_BAD_ARG;
  if (L < P + (int64_t)E * (B - 1) || NB * B < L) return ORACLE_BAD_ARG;
  int64_t* cnt = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  int64_t* off = (int64_t*)calloc((size_t)E + 1, sizeof(int64_t));
  int64_t* fill = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  if (!cnt || !off || !fill) {
    free(cnt);
    free(off);
    free(fill);
    return ORACLE_BAD_ARG;
  }
  for (int64_t i = 0; i < P; ++i) {
    int32_t e = topk_ids[i];
    if (e >= 0 && e < E) cnt[e] += 1;
  }
  for (int32_t e = 0; e < E; ++e) off[e + 1] = off[e] + (cnt[e] + B - 1) / B * B;
  for (int64_t r = 0; r < L; ++r) sorted_ids[r] = (int32_t)P;
  for (int64_t i = 0; i < P; ++i) { /* ascending i: stable within each expert */
    int32_t e = topk_ids[i];
    if (e < 0 || e >= E) continue;
    sorted_ids[off[e] + fill[e]] = (int32_t)i;
    fill[e] += 1;
  }
  for (int64_t b = 0; b < NB; ++b) expert_ids[b] = -1;
  for (int32_t e = 0; e < E; ++e)
    for (int64_t b = off[e] / B; b < off[e + 1] / B; ++b) expert_ids[b] = e;
  num_tokens_padded[0] = (int32_t)off[E];
  if (expert_offsets)
    for (int32_t e = 0; e <= E; ++e) expert_offsets[e] = (int32_t)off[e];
  free(cnt);
  free(off);
  free(fill);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------- */
/* W4A16 expert FFN                                                           */
/* ------------------------------------------------------------------------- */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* E2M1 code (low 4 bits) -> value: sign bit 3, exponent bits 2..1 with bias 1,
 * mantissa bit 0; exponent 0 is subnormal, 0.5 * mantissa. */
double oracle_e4m3_to_f64(uint8_t c);

double oracle_e2m1_to_f64(uint8_t c) {
  int sign = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return sign ? -mag : mag;
}

/* E8M0 scale code -> 2^(code - 127); code 255 is NaN. */
double oracle_e8m0_to_f64(uint8_t c) { return c == 255 ? NAN : ldexp(1.0, (int)c - 127); }

enum { FMT_INT4 = 0, FMT_MXFP4 = 1, FMT_NVFP4 = 2 };

/* Dequantized 4-bit weight of row n, column c of a [N, K] matrix stored as packed
 * codes [N, K/2] (low nibble = even column) with one scale per row and 32 columns
 * ([N, K/32]). INT4: bf16 scales, (code - 8) * scale, subtract then scale. MXFP4:
 * E8M0 scales, e2m1(code) * 2^(scale - 127). Exact in fp64. */
static double w4_weight(int fmt, const uint8_t* w, const void* s, int64_t K, int64_t n,
                        int64_t c) {
  uint8_t byte = w[n * (K / 2) + c / 2];
  int code = (c & 1) ? (byte >> 4) & 0xF : byte & 0xF;
  if (fmt == FMT_NVFP4) /* the expert's global scale is applied by the caller */
    return oracle_e2m1_to_f64((uint8_t)code) *
           oracle_e4m3_to_f64(((const uint8_t*)s)[n * (K / 16) + c / 16]);
  int64_t si = n * (K / 32) + c / 32;
  if (fmt == FMT_MXFP4)
    return oracle_e2m1_to_f64((uint8_t)code) * oracle_e8m0_to_f64(((const uint8_t*)s)[si]);
  return ((double)code - 8.0) * oracle_bf16_to_f64(((const uint16_t*)s)[si]);
}

/* One token row of the routed MoE FFN with W4A16 experts:
 *   out[n] = sum_s w_s * sum_j h_j W2_e(n, j),  h_j = silu(g_j) * u_j,
 *   g_j = sum_c x_c W13_e(j, c),  u_j = sum_c x_c W13_e(I + j, c),
 * slots in s order, every sum sequential, all in fp64. h is kept in fp64. */
static void w4a16_token(int fmt, const uint16_t* x, const uint8_t* w13, const void* s13,
                        const float* g13, const uint8_t* w2, const void* s2, const float* g2,
                        const int32_t* ids, const float* wts, int64_t t, int64_t H, int64_t I,
                        int64_t E, int64_t k, double* xrow, double* h, double* out) {
  const int64_t ssz = fmt == FMT_INT4 ? 2 : 1;   /* bytes per scale */
  const int64_t blk = fmt == FMT_NVFP4 ? 16 : 32; /* columns per scale */
  for (int64_t c = 0; c < H; ++c) xrow[c] = oracle_bf16_to_f64(x[t * H + c]);
  for (int64_t n = 0; n < H; ++n) out[n] = 0.0;
  const int64_t w13_expert = 2 * I * (H / 2), s13_expert = 2 * I * (H / blk);
  const int64_t w2_expert = H * (I / 2), s2_expert = H * (I / blk);
  for (int64_t s = 0; s < k; ++s) {
    int32_t e = ids[t * k + s];
    if (e < 0 || e >= E) continue;
    double wt = (double)wts[t * k + s];
    const uint8_t* we13 = w13 + e * w13_expert;
    const uint8_t* se13 = (const uint8_t*)s13 + e * s13_expert * ssz;
    const uint8_t* we2 = w2 + e * w2_expert;
    const uint8_t* se2 = (const uint8_t*)s2 + e * s2_expert * ssz;
    /* NVFP4: every weight of the expert's projection times its global scale */
    const double gg13 = fmt == FMT_NVFP4 ? (double)g13[e] : 1.0;
    const double gg2 = fmt == FMT_NVFP4 ? (double)g2[e] : 1.0;
    for (int64_t j = 0; j < I; ++j) {
      double g = 0.0, u = 0.0;
      for (int64_t c = 0; c < H; ++c)
        g += xrow[c] * (w4_weight(fmt, we13, se13, H, j, c) * gg13);
      for (int64_t c = 0; c < H; ++c)
        u += xrow[c] * (w4_weight(fmt, we13, se13, H, I + j, c) * gg13);
      h[j] = silu(g) * u;
    }
    for (int64_t n = 0; n < H; ++n) {
      double y = 0.0;
      for (int64_t j = 0; j < I; ++j) y += h[j] * (w4_weight(fmt, we2, se2, I, n, j) * gg2);
      out[n] += wt * y;
    }
  }
}

/* Routed W4A16 MoE FFN for the token rows listed in rows[0..nrows) (all rows if
 * rows == NULL, nrows = T). x [T,H] bf16 bits; w13 [E,2I,H/2] u8; s13 [E,2I,H/32]
 * bf16 bits; w2 [E,H,I/2] u8; s2 [E,H,I/32] bf16 bits; ids/wts [T,k].
 * out [nrows, H] fp64 before the final bf16 rounding. Rows are independent and
 * are spread over nthreads OpenMP threads; each row is computed as written. */
static int w4_moe(int fmt, const uint16_t* x, const uint8_t* w13, const void* s13,
                  const float* g13, const uint8_t* w2, const void* s2, const float* g2,
                  const int32_t* ids, const float* wts, int64_t T, int64_t H, int64_t I,
                  int64_t E, int64_t k, const int64_t* rows, int64_t nrows, double* out,
                  int nthreads) {
  if (fmt == FMT_NVFP4 && (!g13 || !g2)) return ORACLE_BAD_ARG;
  if (!x || !w13 || !s13 || !w2 || !s2 || !ids || !wts || !out) return ORACLE_BAD_ARG;
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0 || H % 32 || I % 32) return ORACLE_BAD_ARG;
  if (!rows) nrows = T;
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t t = rows ? rows[r] : r;
    if (t < 0 || t >= T) return ORACLE_BAD_ARG;
  }
  int bad = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
  {
    double* xrow = (double*)malloc(sizeof(double) * (size_t)H);
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    if (!xrow || !h) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < nrows; ++r) {
        int64_t t = rows ? rows[r] : r;
        w4a16_token(fmt, x, w13, s13, g13, w2, s2, g2, ids, wts, t, H, I, E, k, xrow, h,
                    out + r * H);
      }
    }
    free(xrow);
    free(h);
  }
  return bad ? ORACLE_BAD_ARG : ORACLE_OK;
}

int oracle_w4a16_moe(const uint16_t* x, const uint8_t* w13, const uint16_t* s13, const uint8_t* w2,
                     const uint16_t* s2, const int32_t* ids, const float* wts, int64_t T, int64_t H,
                     int64_t I, int64_t E, int64_t k, const int64_t* rows, int64_t nrows,
                     double* out, int nthreads) {
  return w4_moe(FMT_INT4, x, w13, s13, NULL, w2, s2, NULL, ids, wts, T, H, I, E, k, rows, nrows,
                out, nthreads);
}

/* Routed MXFP4 MoE FFN (weight-only, [XT] overview): as oracle_w4a16_moe with E2M1
 * codes and E8M0 scales s13 [E,2I,H/32] u8, s2 [E,H,I/32] u8. */
int oracle_mxfp4_moe(const uint16_t* x, const uint8_t* w13, const uint8_t* s13, const uint8_t* w2,
                     const uint8_t* s2, const int32_t* ids, const float* wts, int64_t T, int64_t H,
                     int64_t I, int64_t E, int64_t k, const int64_t* rows, int64_t nrows,
                     double* out, int nthreads) {
  return w4_moe(FMT_MXFP4, x, w13, s13, NULL, w2, s2, NULL, ids, wts, T, H, I, E, k, rows,
                nrows, out, nthreads);
}

/* Routed NVFP4 MoE FFN (weight-only): E2M1 codes, E4M3 scales s13 [E,2I,H/16] and
 * s2 [E,H,I/16] (u8), fp32 global scales g13 [E] and g2 [E]. */
int oracle_nvfp4_moe(const uint16_t* x, const uint8_t* w13, const uint8_t* s13, const float* g13,
                     const uint8_t* w2, const uint8_t* s2, const float* g2, const int32_t* ids,
                     const float* wts, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                     const int64_t* rows, int64_t nrows, double* out, int nthreads) {
  return w4_moe(FMT_NVFP4, x, w13, s13, g13, w2, s2, g2, ids, wts, T, H, I, E, k, rows, nrows,
                out, nthreads);
}

/* ------------------------------------------------------------------------- */
/* Block-FP8 W8A8 expert FFN                                                  */
/* ------------------------------------------------------------------------- */

/* One token row of the W8A8 block-FP8 MoE FFN:
 *   x_c = e4m3(a_q[t,c]) * As[t, c/128]
 *   W13(n,c) = e4m3(w13[e,n,c]) * Bs13[e, n/128, c/128]  (likewise W2)
 *   g, u, silu(g)*u as in the W4A16 path (fp64);
 *   h is rounded to fp32 and requantized per 128 consecutive j with the block
 *   quantizer (fp32 decision), then y_n = sum_j e4m3(hq_j) * hs_{j/128} * W2(n,j). */
static void fp8_token(const uint8_t* aq, const float* as, const uint8_t* w13, const float* s13,
                      const uint8_t* w2, const float* s2, const int32_t* ids, const float* wts,
                      int64_t t, int64_t H, int64_t I, int64_t E, int64_t k, double* xrow,
                      float* h32, uint8_t* hq, float* hs, double* out) {
  const int64_t HB = H / 128, IB = I / 128;
  for (int64_t c = 0; c < H; ++c)
    xrow[c] = oracle_e4m3_to_f64(aq[t * H + c]) * (double)as[t * HB + c / 128];
  for (int64_t n = 0; n < H; ++n) out[n] = 0.0;
  for (int64_t s = 0; s < k; ++s) {
    int32_t e = ids[t * k + s];
    if (e < 0 || e >= E) continue;
    double wt = (double)wts[t * k + s];
    const uint8_t* we13 = w13 + e * (2 * I * H);
    const float* se13 = s13 + e * (2 * IB * HB);
    const uint8_t* we2 = w2 + e * (H * I);
    const float* se2 = s2 + e * (HB * IB);
    for (int64_t j = 0; j < I; ++j) {
      double g = 0.0, u = 0.0;
      for (int64_t c = 0; c < H; ++c)
        g += xrow[c] * (oracle_e4m3_to_f64(we13[j * H + c]) * (double)se13[(j / 128) * HB + c / 128]);
      for (int64_t c = 0; c < H; ++c)
        u += xrow[c] * (oracle_e4m3_to_f64(we13[(I + j) * H + c]) *
                        (double)se13[((I + j) / 128) * HB + c / 128]);
      h32[j] = (float)(silu(g) * u);
    }
    oracle_fp8_quantize_blocks(h32, 1, I, 1, 128, hq, hs);
    for (int64_t n = 0; n < H; ++n) {
      double y = 0.0;
      for (int64_t j = 0; j < I; ++j)
        y += (oracle_e4m3_to_f64(hq[j]) * (double)hs[j / 128]) *
             (oracle_e4m3_to_f64(we2[n * I + j]) * (double)se2[(n / 128) * IB + j / 128]);
      out[n] += wt * y;
    }
  }
}

/* Routed W8A8 block-FP8 MoE FFN for the listed token rows (all if rows == NULL).
 * a_q [T,H] e4m3; as [T,H/128] f32; w13 [E,2I,H] e4m3; s13 [E,2I/128,H/128] f32;
 * w2 [E,H,I] e4m3; s2 [E,H/128,I/128] f32; out [nrows,H] fp64 before bf16 rounding. */
int oracle_fp8_moe(const uint8_t* aq, const float* as, const uint8_t* w13, const float* s13,
                   const uint8_t* w2, const float* s2, const int32_t* ids, const float* wts, int64_t T,
                   int64_t H, int64_t I, int64_t E, int64_t k, const int64_t* rows, int64_t nrows,
                   double* out, int nthreads) {
  if (!aq || !as || !w13 || !s13 || !w2 || !s2 || !ids || !wts || !out) return ORACLE_BAD_ARG;
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0 || H % 128 || I % 128) return ORACLE_BAD_ARG;
  if (!rows) nrows = T;
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t t = rows ? rows[r] : r;
    if (t < 0 || t >= T) return ORACLE_BAD_ARG;
  }
  int bad = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
  {
    double* xrow = (double*)malloc(sizeof(double) * (size_t)H);
    float* h32 = (float*)malloc(sizeof(float) * (size_t)I);
    uint8_t* hq = (uint8_t*)malloc((size_t)I);
    float* hs = (float*)malloc(sizeof(float) * (size_t)(I / 128));
    if (!xrow || !h32 || !hq || !hs) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < nrows; ++r) {
        int64_t t = rows ? rows[r] : r;
        fp8_token(aq, as, w13, s13, w2, s2, ids, wts, t, H, I, E, k, xrow, h32, hq, hs,
                  out + r * H);
      }
    }
    free(xrow);
    free(h32);
    free(hq);
    free(hs);
  }
  return bad ? ORACLE_BAD_ARG : ORACLE_OK;
}

/* ------------------------------------------------------------------------- */
/* Array forms of the scalar conversions (for the Python side)               */
/* ------------------------------------------------------------------------- */

void oracle_f64_to_bf16_array(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_bf16(x[i]);
}

void oracle_e4m3_to_f64_array(const uint8_t* c, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_to_f64(c[i]);
}

void oracle_e2m1_to_f64_array(const uint8_t* c, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e2m1_to_f64(c[i]);
}

void oracle_e8m0_to_f64_array(const uint8_t* c, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e8m0_to_f64(c[i]);
}

void oracle_f32_to_e4m3_array(const float* x, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_e4m3(x[i]);
}

/* ------------------------------------------------------------------------- */
/* Expert-major evaluation: the same arithmetic in another loop order        */
/* ------------------------------------------------------------------------- */

/* The functions above walk token by token and dequantize every weight again for each
 * routed pair. The functions below compute exactly the same numbers expert by expert:
 * the routed pairs of the listed rows are grouped by expert, each weight row is
 * dequantized once into a buffer, and every pair's dot product with it is summed
 * sequentially over the column index, as in the per-token functions. Several pairs'
 * sums run side by side (they are independent); no sum is split or reordered. Each
 * pair's down output y is kept, and a token row's output is then summed over its slots in
 * slot order. Products are formed with the same expressions, so the results are
 * bit-identical to oracle_w4a16_moe / _mxfp4_ / _nvfp4_ / oracle_fp8_moe (pinned in
 * tests/test_oracle_experts.py); they exist so that full-size workloads can be checked. */

#define PB 8 /* pairs whose sums run side by side */

typedef struct {
  int64_t npairs;  /* routed pairs of the listed rows */
  int64_t* start;  /* [E + 1]: expert e owns pair slots [start[e], start[e+1]) */
  int64_t* pair;   /* [npairs]: r * k + s, r = position in the row list */
} pair_lists;

static void free_pair_lists(pair_lists* pl) {
  free(pl->start);
  free(pl->pair);
}

/* Groups the valid (row, slot) pairs of the listed rows by expert, ascending r*k+s. */
static int make_pair_lists(const int32_t* ids, int64_t k, int64_t E, const int64_t* rows,
                           int64_t nrows, pair_lists* pl) {
  pl->start = (int64_t*)calloc((size_t)E + 1, sizeof(int64_t));
  pl->pair = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nrows * k + 1));
  if (!pl->start || !pl->pair) return ORACLE_BAD_ARG;
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t t = rows ? rows[r] : r;
    for (int64_t s = 0; s < k; ++s) {
      int32_t e = ids[t * k + s];
      if (e >= 0 && e < E) pl->start[e + 1] += 1;
    }
  }
  for (int64_t e = 0; e < E; ++e) pl->start[e + 1] += pl->start[e];
  pl->npairs = pl->start[E];
  int64_t* fill = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  if (!fill) return ORACLE_BAD_ARG;
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t t = rows ? rows[r] : r;
    for (int64_t s = 0; s < k; ++s) {
      int32_t e = ids[t * k + s];
      if (e < 0 || e >= E) continue;
      pl->pair[pl->start[e] + fill[e]] = r * k + s;
      fill[e] += 1;
    }
  }
  free(fill);
  return ORACLE_OK;
}

/* acc[q] = sum over c (sequential) of xt[c * np + q] * w[c], for the PB = 8 pairs q of a
 * block (xt holds the pairs' activation rows transposed, np a multiple of PB). The eight
 * sums are written out as separate variables so that they stay in registers. */
static void dot_block(const double* xt, int64_t np, const double* w, int64_t K, double* acc) {
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0, a4 = 0.0, a5 = 0.0, a6 = 0.0, a7 = 0.0;
  for (int64_t c = 0; c < K; ++c) {
    const double wc = w[c];
    const double* xc = xt + c * np;
    a0 += xc[0] * wc;
    a1 += xc[1] * wc;
    a2 += xc[2] * wc;
    a3 += xc[3] * wc;
    a4 += xc[4] * wc;
    a5 += xc[5] * wc;
    a6 += xc[6] * wc;
    a7 += xc[7] * wc;
  }
  acc[0] = a0;
  acc[1] = a1;
  acc[2] = a2;
  acc[3] = a3;
  acc[4] = a4;
  acc[5] = a5;
  acc[6] = a6;
  acc[7] = a7;
}

/* The same with the magnitude sums mag[q] = sum_c |x_c * w_c| beside it. */
static void dot_block_abs(const double* xt, int64_t np, const double* w, int64_t K, double* acc,
                          double* mag) {
  double a[PB], m[PB];
  for (int q = 0; q < PB; ++q) a[q] = m[q] = 0.0;
  for (int64_t c = 0; c < K; ++c) {
    const double wc = w[c];
    const double* xc = xt + c * np;
    for (int q = 0; q < PB; ++q) {
      double p = xc[q] * wc;
      a[q] += p;
      m[q] += fabs(p);
    }
  }
  for (int q = 0; q < PB; ++q) {
    acc[q] = a[q];
    mag[q] = m[q];
  }
}

enum { FMT_FP8 = 3 };

/* Weight row n of expert e's [N, K] matrix, dequantized into w[0..K) exactly as the
 * per-token functions form it. */
static void weight_row(int fmt, const uint8_t* w, const void* s, const float* gsc, int64_t e,
                       int64_t N, int64_t K, int64_t n, double* out) {
  if (fmt == FMT_FP8) {
    const uint8_t* we = w + e * N * K;
    const float* se = (const float*)s + e * (N / 128) * (K / 128);
    for (int64_t c = 0; c < K; ++c)
      out[c] = oracle_e4m3_to_f64(we[n * K + c]) * (double)se[(n / 128) * (K / 128) + c / 128];
    return;
  }
  const int64_t ssz = fmt == FMT_INT4 ? 2 : 1, blk = fmt == FMT_NVFP4 ? 16 : 32;
  const uint8_t* we = w + e * N * (K / 2);
  const uint8_t* se = (const uint8_t*)s + e * N * (K / blk) * ssz;
  const double g = fmt == FMT_NVFP4 ? (double)gsc[e] : 1.0;
  for (int64_t c = 0; c < K; ++c) out[c] = w4_weight(fmt, we, se, K, n, c) * g;
}

/* The routed FFN for the listed rows, expert by expert. fmt: FMT_INT4 / FMT_MXFP4 /
 * FMT_NVFP4 (x = bf16 bits [T,H]) or FMT_FP8 (x = E4M3 a_q [T,H] with fp32 scales as
 * [T,H/128]). out [nrows, H] fp64. The optional FP8 detail arrays (NULL to skip) receive,
 * per pair slot r*k+s of the listed rows (untouched for dropped slots), per h column j:
 * g, u (fp64), gmag / umag = sum_c |x_c W13(j, c)| / |x_c W13(I + j, c)|, the fp32 h
 * before quantization, its E4M3 codes, and the fp32 scale per 128 columns. */
static int experts_moe(int fmt, const void* xin, const float* as, const uint8_t* w13,
                       const void* s13, const float* g13, const uint8_t* w2, const void* s2,
                       const float* g2, const int32_t* ids, const float* wts, int64_t T,
                       int64_t H, int64_t I, int64_t E, int64_t k, const int64_t* rows,
                       int64_t nrows, double* out, int nthreads, double* d_g, double* d_u,
                       double* d_gmag, double* d_umag, float* d_h32, uint8_t* d_hq,
                       float* d_hs) {
  const int fp8 = fmt == FMT_FP8;
  const int q = fp8 ? 128 : 32;
  if (!xin || !w13 || !s13 || !w2 || !s2 || !ids || !wts || !out) return ORACLE_BAD_ARG;
  if (fp8 && !as) return ORACLE_BAD_ARG;
  if (fmt == FMT_NVFP4 && (!g13 || !g2)) return ORACLE_BAD_ARG;
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0 || H % q || I % q) return ORACLE_BAD_ARG;
  if (!rows) nrows = T;
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t t = rows ? rows[r] : r;
    if (t < 0 || t >= T) return ORACLE_BAD_ARG;
  }
  const int detail = fp8 && d_h32;
  pair_lists pl;
  if (make_pair_lists(ids, k, E, rows, nrows, &pl) != ORACLE_OK) {
    free_pair_lists(&pl);
    return ORACLE_BAD_ARG;
  }
  double* y = (double*)calloc((size_t)(nrows * k) * (size_t)H, sizeof(double));
  int bad = y == NULL;
  const int nt = nthreads > 0 ? nthreads : 1;
  for (int64_t e = 0; e < E && !bad; ++e) {
    const int64_t ne = pl.start[e + 1] - pl.start[e];
    if (ne == 0) continue;
    const int64_t np = (ne + PB - 1) / PB * PB; /* padded with zero rows, results unused */
    const int64_t* pe = pl.pair + pl.start[e];
    double* xt = (double*)calloc((size_t)(H * np), sizeof(double));
    double* gg = (double*)malloc(sizeof(double) * (size_t)(np * I));
    double* uu = (double*)malloc(sizeof(double) * (size_t)(np * I));
    double* gm = detail ? (double*)malloc(sizeof(double) * (size_t)(np * I)) : NULL;
    double* um = detail ? (double*)malloc(sizeof(double) * (size_t)(np * I)) : NULL;
    double* hh = (double*)malloc(sizeof(double) * (size_t)(np * I));
    if (!xt || !gg || !uu || !hh || (detail && (!gm || !um))) {
      bad = 1;
    } else {
      /* the pairs' activation rows, transposed: xt[c * np + p] */
      for (int64_t p = 0; p < ne; ++p) {
        int64_t t = rows ? rows[pe[p] / k] : pe[p] / k;
        for (int64_t c = 0; c < H; ++c)
          xt[c * np + p] = fp8 ? oracle_e4m3_to_f64(((const uint8_t*)xin)[t * H + c]) *
                                     (double)as[t * (H / 128) + c / 128]
                               : oracle_bf16_to_f64(((const uint16_t*)xin)[t * H + c]);
      }
#pragma omp parallel num_threads(nt)
      {
        double* wg = (double*)malloc(sizeof(double) * (size_t)H);
        double* wu = (double*)malloc(sizeof(double) * (size_t)H);
        if (!wg || !wu) {
#pragma omp atomic write
          bad = 1;
        } else {
          /* g_j = sum_c x_c W13(j, c), u_j = sum_c x_c W13(I + j, c) */
#pragma omp for schedule(dynamic, 4)
          for (int64_t j = 0; j < I; ++j) {
            weight_row(fmt, w13, s13, g13, e, 2 * I, H, j, wg);
            weight_row(fmt, w13, s13, g13, e, 2 * I, H, I + j, wu);
            for (int64_t p0 = 0; p0 < np; p0 += PB) {
              double ag[PB], au[PB], mg[PB], mu[PB];
              if (detail) {
                dot_block_abs(xt + p0, np, wg, H, ag, mg);
                dot_block_abs(xt + p0, np, wu, H, au, mu);
              } else {
                dot_block(xt + p0, np, wg, H, ag);
                dot_block(xt + p0, np, wu, H, au);
              }
              for (int qq = 0; qq < PB; ++qq) {
                gg[(p0 + qq) * I + j] = ag[qq];
                uu[(p0 + qq) * I + j] = au[qq];
                if (detail) {
                  gm[(p0 + qq) * I + j] = mg[qq];
                  um[(p0 + qq) * I + j] = mu[qq];
                }
              }
            }
          }
        }
        free(wg);
        free(wu);
      }
    }
    if (!bad) {
      /* h = silu(g) * u; block FP8 requantizes it per 128 columns (F0 on its fp32 value) */
      for (int64_t p = 0; p < np; ++p) {
        double* hp = hh + p * I;
        for (int64_t j = 0; j < I; ++j) hp[j] = silu(gg[p * I + j]) * uu[p * I + j];
        if (fp8 && p < ne) {
          float* h32 = (float*)malloc(sizeof(float) * (size_t)I);
          uint8_t* hq = (uint8_t*)malloc((size_t)I);
          float* hs = (float*)malloc(sizeof(float) * (size_t)(I / 128));
          if (!h32 || !hq || !hs) {
            bad = 1;
          } else {
            for (int64_t j = 0; j < I; ++j) h32[j] = (float)hp[j];
            oracle_fp8_quantize_blocks(h32, 1, I, 1, 128, hq, hs);
            for (int64_t j = 0; j < I; ++j)
              hp[j] = oracle_e4m3_to_f64(hq[j]) * (double)hs[j / 128];
            if (detail) {
              const int64_t slot = pe[p];
              memcpy(d_g + slot * I, gg + p * I, sizeof(double) * (size_t)I);
              memcpy(d_u + slot * I, uu + p * I, sizeof(double) * (size_t)I);
              memcpy(d_gmag + slot * I, gm + p * I, sizeof(double) * (size_t)I);
              memcpy(d_umag + slot * I, um + p * I, sizeof(double) * (size_t)I);
              memcpy(d_h32 + slot * I, h32, sizeof(float) * (size_t)I);
              memcpy(d_hq + slot * I, hq, (size_t)I);
              memcpy(d_hs + slot * (I / 128), hs, sizeof(float) * (size_t)(I / 128));
            }
          }
          free(h32);
          free(hq);
          free(hs);
        }
      }
    }
    if (!bad) {
      /* y_n = sum_j h_j W2(n, j), transposed h for the side-by-side sums */
      double* ht = (double*)malloc(sizeof(double) * (size_t)(I * np));
      if (!ht) {
        bad = 1;
      } else {
        for (int64_t p = 0; p < np; ++p)
          for (int64_t j = 0; j < I; ++j) ht[j * np + p] = hh[p * I + j];
#pragma omp parallel num_threads(nt)
        {
          double* wr = (double*)malloc(sizeof(double) * (size_t)I);
          if (!wr) {
#pragma omp atomic write
            bad = 1;
          } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t n = 0; n < H; ++n) {
              weight_row(fmt, w2, s2, g2, e, H, I, n, wr);
              for (int64_t p0 = 0; p0 < np; p0 += PB) {
                double ay[PB];
                dot_block(ht + p0, np, wr, I, ay);
                for (int qq = 0; qq < PB && p0 + qq < ne; ++qq) y[pe[p0 + qq] * H + n] = ay[qq];
              }
            }
          }
          free(wr);
        }
      }
      free(ht);
    }
    free(xt);
    free(gg);
    free(uu);
    free(gm);
    free(um);
    free(hh);
  }
  if (!bad) {
    /* out[r] = sum over the row's valid slots, in slot order, of w_s * y_s */
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
      int64_t t = rows ? rows[r] : r;
      double* o = out + r * H;
      for (int64_t n = 0; n < H; ++n) o[n] = 0.0;
      for (int64_t s = 0; s < k; ++s) {
        int32_t e = ids[t * k + s];
        if (e < 0 || e >= E) continue;
        double wt = (double)wts[t * k + s];
        const double* ys = y + (r * k + s) * H;
        for (int64_t n = 0; n < H; ++n) o[n] += wt * ys[n];
      }
    }
  }
  free(y);
  free_pair_lists(&pl);
  return bad ? ORACLE_BAD_ARG : ORACLE_OK;
}

int oracle_w4a16_moe_experts(const uint16_t* x, const uint8_t* w13, const uint16_t* s13,
                             const uint8_t* w2, const uint16_t* s2, const int32_t* ids,
                             const float* wts, int64_t T, int64_t H, int64_t I, int64_t E,
                             int64_t k, const int64_t* rows, int64_t nrows, double* out,
                             int nthreads) {
  return experts_moe(FMT_INT4, x, NULL, w13, s13, NULL, w2, s2, NULL, ids, wts, T, H, I, E, k,
                     rows, nrows, out, nthreads, NULL, NULL, NULL, NULL, NULL, NULL, NULL);
}

int oracle_mxfp4_moe_experts(const uint16_t* x, const uint8_t* w13, const uint8_t* s13,
                             const uint8_t* w2, const uint8_t* s2, const int32_t* ids,
                             const float* wts, int64_t T, int64_t H, int64_t I, int64_t E,
                             int64_t k, const int64_t* rows, int64_t nrows, double* out,
                             int nthreads) {
  return experts_moe(FMT_MXFP4, x, NULL, w13, s13, NULL, w2, s2, NULL, ids, wts, T, H, I, E, k,
                     rows, nrows, out, nthreads, NULL, NULL, NULL, NULL, NULL, NULL, NULL);
}

int oracle_nvfp4_moe_experts(const uint16_t* x, const uint8_t* w13, const uint8_t* s13,
                             const float* g13, const uint8_t* w2, const uint8_t* s2,
                             const float* g2, const int32_t* ids, const float* wts, int64_t T,
                             int64_t H, int64_t I, int64_t E, int64_t k, const int64_t* rows,
                             int64_t nrows, double* out, int nthreads) {
  return experts_moe(FMT_NVFP4, x, NULL, w13, s13, g13, w2, s2, g2, ids, wts, T, H, I, E, k,
                     rows, nrows, out, nthreads, NULL, NULL, NULL, NULL, NULL, NULL, NULL);
}

/* Block FP8, expert by expert; the detail arrays may be NULL (see experts_moe). */
int oracle_fp8_moe_experts(const uint8_t* aq, const float* as, const uint8_t* w13,
                           const float* s13, const uint8_t* w2, const float* s2,
                           const int32_t* ids, const float* wts, int64_t T, int64_t H, int64_t I,
                           int64_t E, int64_t k, const int64_t* rows, int64_t nrows, double* out,
                           int nthreads, double* d_g, double* d_u, double* d_gmag, double* d_umag,
                           float* d_h32, uint8_t* d_hq, float* d_hs) {
  if (d_h32 && (!d_g || !d_u || !d_gmag || !d_umag || !d_hq || !d_hs)) return ORACLE_BAD_ARG;
  return experts_moe(FMT_FP8, aq, as, w13, s13, NULL, w2, s2, NULL, ids, wts, T, H, I, E, k,
                     rows, nrows, out, nthreads, d_g, d_u, d_gmag, d_umag, d_h32, d_hq, d_hs);
}
