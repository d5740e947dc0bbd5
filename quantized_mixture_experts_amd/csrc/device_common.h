// Device-side helpers shared by the gfx950 kernels of the MoE expert FFN library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short bf16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef int i32x8 __attribute__((__vector_size__(8 * sizeof(int))));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

// ---------------------------------------------------------------------------
// MFMA wrappers (one wave, 16x16 output tile; lane l holds rows 4*(l/16)+r, r=0..3,
// of column l%16). A operand: lane l supplies row l%16, k-slice (l/16); B operand:
// lane l supplies column l%16, the same k-slice.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(const uint32_t (&a)[4], const uint32_t (&b)[4],
                                                    f32x4 c) {
  bf16x8 av, bv;
  __builtin_memcpy(&av, a, 16);
  __builtin_memcpy(&bv, b, 16);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
}

// E4M3 x E4M3, K = 128 per instruction (lane supplies 32 consecutive k values).
// The block-scale operands are fixed at E8M0 127 (= 1.0): the block scales of this
// format are general fp32 values and are applied to the fp32 accumulator instead.
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(const u32x4 (&a)[2], const u32x4 (&b)[2],
                                                    f32x4 c) {
  i32x8 av, bv;
  __builtin_memcpy(&av, a, 32);
  __builtin_memcpy(&bv, b, 32);
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, 127, 0, 127);
}

// ---------------------------------------------------------------------------
// Cross-lane 4x4 transpose of 32-bit words among the four 16-lane rows of a wave:
// on entry register j of row q holds M[q][j]; on exit register g of row q holds M[g][q].
// Two permlane32 swaps exchange the off-diagonal 2x2 blocks of rows {0,1} x {2,3},
// two permlane16 swaps finish inside each half.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void transpose4_rows(uint32_t (&m)[4]) {
  auto s02 = __builtin_amdgcn_permlane32_swap(m[0], m[2], false, false);
  auto s13 = __builtin_amdgcn_permlane32_swap(m[1], m[3], false, false);
  m[0] = s02[0];
  m[2] = s02[1];
  m[1] = s13[0];
  m[3] = s13[1];
  auto s01 = __builtin_amdgcn_permlane16_swap(m[0], m[1], false, false);
  auto s23 = __builtin_amdgcn_permlane16_swap(m[2], m[3], false, false);
  m[0] = s01[0];
  m[1] = s01[1];
  m[2] = s23[0];
  m[3] = s23[1];
}

// ---------------------------------------------------------------------------
// INT4 codes -> bf16 operand registers.
// A 32-bit word holds 8 codes n0..n7 (nibble j = bits 4j..4j+3). OR-ing a nibble into
// the mantissa of bf16 128.0 (0x4300) gives exactly 128 + code, so
//   b[0] = (n0, n4), b[1] = (n1, n5), b[2] = (n2, n6), b[3] = (n3, n7)
// as bf16 pairs (low half first). The zero point (128 + 8) is removed on the fp32
// accumulator (see the kernels), and the activation operand is permuted to the same
// k order with perm_act8.
// ---------------------------------------------------------------------------
constexpr uint32_t kNibbleMask = 0x000F000Fu;
constexpr uint32_t kBf16Bias128 = 0x43004300u;

// `mask` must hold kNibbleMask (in an SGPR) and `one28` kBf16Bias128 (in a VGPR), see
// opaque_sgpr / opaque_vgpr: with register operands the compiler selects one
// v_and_or_b32 per pair (a VOP3 encoding reads at most one SGPR);
// with two literal operands it would emit v_and_b32 + v_or_b32, since gfx9 VOP3
// encodings take no literal.
__device__ __forceinline__ void int4_to_bf16_biased(uint32_t w, uint32_t mask, uint32_t one28,
                                                    uint32_t (&b)[4]) {
  b[0] = (w & mask) | one28;
  b[1] = ((w >> 4) & mask) | one28;
  b[2] = ((w >> 8) & mask) | one28;
  b[3] = ((w >> 12) & mask) | one28;
}

// Values the compiler must keep in a register and cannot fold (the empty asm emits no
// instruction).
__device__ __forceinline__ uint32_t opaque_vgpr(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}
__device__ __forceinline__ uint32_t opaque_sgpr(uint32_t v) {
  asm volatile("" : "+s"(v));
  return v;
}

// 8 consecutive bf16 activations x0..x7 (dwords d0..d3) -> operand order
// (x0,x4), (x1,x5), (x2,x6), (x3,x7), matching int4_to_bf16_biased.
__device__ __forceinline__ void perm_act8(const u32x4 d, uint32_t (&a)[4]) {
  a[0] = __builtin_amdgcn_perm(d[2], d[0], 0x05040100u);
  a[1] = __builtin_amdgcn_perm(d[2], d[0], 0x07060302u);
  a[2] = __builtin_amdgcn_perm(d[3], d[1], 0x05040100u);
  a[3] = __builtin_amdgcn_perm(d[3], d[1], 0x07060302u);
}

// Position of element e (0..7) of an 8-element k slice in the operand k order
// (0, 4, 1, 5, 2, 6, 3, 7): element e sits at ((e & 3) << 1) | (e >> 2).
__device__ __forceinline__ int operand_pos8(int e) { return ((e & 3) << 1) | (e >> 2); }

// Element offset of (row r, k index k) of an [rows, K] activation matrix in the tiled
// operand layout used for the GEMMs' activation side: the operand of one (16-row block,
// 32-deep k group) is 64 lanes x 16 B contiguous, lane (k slice q = (k % 32) / 8) * 16 +
// (row r % 16) holding that slice's 8 values in operand k order, or in natural order
// when kNatural (the order the FP4 converts produce). Rows must come in whole 16-row
// blocks; the footprint equals the row-major one.
template <bool kNatural = false>
__device__ __forceinline__ size_t tiled_offset(int r, int k, int K) {
  const int m = r & 15, q = (k >> 3) & 3;
  const int pos = kNatural ? (k & 7) : operand_pos8(k & 7);
  return (((size_t)(r >> 4) * (K >> 5) + (k >> 5)) * 64 + q * 16 + m) * 8 + pos;
}

// ---------------------------------------------------------------------------
// MXFP4 codes -> bf16 operand registers.
// A 32-bit word holds 8 E2M1 codes, code j in bits 4j..4j+3 (byte j/2, low nibble for
// even j). v_cvt_scalef32_pk_bf16_fp4 turns byte `sel` into the bf16 pair (code 2 sel,
// code 2 sel + 1) times 2^(exponent of the fp32 scale operand): with a power-of-two
// scale every result is exact (E2M1 has one mantissa bit), so the four pairs are the
// dequantized weights in natural k order.
template <int SEL>
__device__ __forceinline__ uint32_t fp4_pair_sel(uint32_t w, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, SEL));
}

// Pair `sel` (a constant after unrolling) of fp4_to_bf16.
__device__ __forceinline__ uint32_t fp4_pair(uint32_t w, float scale, int sel) {
  switch (sel) {
    case 0: return fp4_pair_sel<0>(w, scale);
    case 1: return fp4_pair_sel<1>(w, scale);
    case 2: return fp4_pair_sel<2>(w, scale);
    default: return fp4_pair_sel<3>(w, scale);
  }
}

__device__ __forceinline__ void fp4_to_bf16(uint32_t w, float scale, uint32_t (&b)[4]) {
  b[0] = fp4_pair_sel<0>(w, scale);
  b[1] = fp4_pair_sel<1>(w, scale);
  b[2] = fp4_pair_sel<2>(w, scale);
  b[3] = fp4_pair_sel<3>(w, scale);
}

// NVFP4: the pair `sel` of a code word (codes 2 sel, 2 sel + 1) times the fp32 block
// scale sc (the E4M3 scale of the codes' 16-column block times the expert's global
// scale), rounded once to a bf16 pair. The FP4 convert is exact in fp32 (scale 1.0).
typedef float qf32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 qbf16x2 __attribute__((ext_vector_type(2)));
template <int SEL>
__device__ __forceinline__ uint32_t nvfp4_pair_sel(uint32_t w, float sc) {
  const auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  const qf32x2 p = {f[0] * sc, f[1] * sc};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(p, qbf16x2));
}
__device__ __forceinline__ uint32_t nvfp4_pair(uint32_t w, float sc, int sel) {
  switch (sel) {
    case 0: return nvfp4_pair_sel<0>(w, sc);
    case 1: return nvfp4_pair_sel<1>(w, sc);
    case 2: return nvfp4_pair_sel<2>(w, sc);
    default: return nvfp4_pair_sel<3>(w, sc);
  }
}
__device__ __forceinline__ void nvfp4_to_bf16(uint32_t w, float sc, uint32_t (&b)[4]) {
  b[0] = nvfp4_pair_sel<0>(w, sc);
  b[1] = nvfp4_pair_sel<1>(w, sc);
  b[2] = nvfp4_pair_sel<2>(w, sc);
  b[3] = nvfp4_pair_sel<3>(w, sc);
}
// E4M3 code in the low byte of v -> fp32 (gfx950's OCP E4M3FN convert).
__device__ __forceinline__ float e4m3_low(uint32_t v) {
  return __builtin_amdgcn_cvt_f32_fp8((int)v, 0);
}

// E8M0 scale code -> an fp32 whose exponent field is the code (2^(code - 127) for codes
// 1..254), the form the FP4 converts take their scale in.
__device__ __forceinline__ float e8m0_scale(uint32_t code) {
  return __builtin_bit_cast(float, (code & 0xFFu) << 23);
}

// ---------------------------------------------------------------------------
// XCD-aware work distribution. MI355X has 8 XCDs, each with its own L2, and the
// dispatcher deals work-groups to them round-robin by launch index. With a 1-D grid of
// xcd_major_grid(items) work-groups, xcd_major_item() hands XCD x the contiguous item
// range [x * per, (x + 1) * per): items that share data (the same expert) stay on one
// L2. Returns -1 for the padding work-groups.
// ---------------------------------------------------------------------------
constexpr int kNumXcd = 8;

__host__ __device__ inline int xcd_major_grid(int items) {
  return (items + kNumXcd - 1) / kNumXcd * kNumXcd;
}

__device__ __forceinline__ int xcd_major_item(int block, int grid, int items) {
  const int per = grid / kNumXcd;
  const int item = (block % kNumXcd) * per + block / kNumXcd;
  return item < items ? item : -1;
}

// A read of data that no launch in flight writes, through the constant address space so
// that a uniform index becomes a scalar load: a vector load would enter the in-order
// vector memory counter, and waiting for it would also wait for outstanding prefetches.
__device__ __forceinline__ int32_t ld_invariant(const int32_t* p, int i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }
// With the accurate exponential: for h that is requantized to E4M3 (a step function),
// where the fast exponential's ~1e-6 relative error flips codes measurably often.
__device__ __forceinline__ float silu_f32_accurate(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

}  // namespace qmoe
