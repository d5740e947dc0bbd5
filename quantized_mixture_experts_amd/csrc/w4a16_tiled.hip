// W4A16 grouped expert GEMMs, prefill profile (row tiles of 256, MFMA-bound).
//
// Method: BF16 activations times INT4 group-32 weights with BF16 scales, fp32
// accumulation ("vLLM x Novita AI: Chord W4A16 INT4 MoE Kernel for Kimi K2.x": summary;
// "vLLM integration"). With hundreds of routed rows per expert the product is a grouped
// GEMM over the expert segments of the sorted row list ("SGLang fused_moe_triton":
// moe_align_block_size and the fused kernel's expert blocks), so the cost is the
// contraction and the kernel is laid out for the matrix cores.
//
// gfx950 mapping. A work-group owns one (256-row tile of an expert segment, 256 weight
// rows) output tile; its four waves each own all 256 rows and 64 weight rows (four
// 16-column MFMA tiles), so every weight element is dequantized exactly once per tile
// and reused for 16 row blocks:
//   * activation rows (bf16, tiled layout: the operand of one 16-row block and k group
//     is 1 KB contiguous) go global -> LDS through global_load_lds_dwordx4 into a ring of
//     four 16 KB stages, three k groups ahead; each wave copies four of the sixteen
//     blocks of a stage and waits on its own copies with vmcnt before the stage's
//     barrier (the compiler does not track these asynchronous LDS writes);
//   * each lane loads 2 x 16 B of its weight row per 256 k (a whole 128 B line per row)
//     plus the 16 B of that row's eight group scales, one block ahead in registers; a
//     4x4 permlane transpose regroups the words so that every lane quarter holds its
//     k slice of each group (the B operand layout of v_mfma_f32_16x16x32_bf16);
//   * dequantization folds the scale into the operand: OR-ing a code into fp16 1024.0
//     gives 1024 + code exactly, v_fma_mix_f32 forms (1024 + code) * s - 1032 * s =
//     (code - 8) * s exactly in fp32 (1032 * s is exact for a bf16 s), and
//     v_cvt_pk_bf16_f32 rounds it to the bf16 operand; 16 M tiles share each operand;
//   * 64 accumulator tiles (256 fp32 per lane) per wave.
// gate_up stores h = SiLU(gate) * up (bf16, tiled layout); down stores the routing-
// weighted rows per (token, slot) pair in fp32 and a combine kernel sums the top-k rows
// of every token, so the prefill output does not depend on atomic ordering.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace qmoe {

namespace {

constexpr int kTileRows = 256;                    // rows per work-group tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kRowBlocks = kTileRows / 16;        // 16-row MFMA tiles per wave
constexpr int kColTiles = 4;                      // 16-column MFMA tiles per wave
constexpr int kStages = 4;                        // LDS ring of activation k groups
constexpr int kAhead = kStages - 1;               // groups copied ahead of use
constexpr int kCopiesPerWave = kRowBlocks / kWaves;  // 1 KB copies per wave and group
constexpr int kGroupsPerBlock = 8;                // k groups per 256-deep weight block

enum class TEpi { GateUp, Down };

struct TiledArgs {
  const uint16_t* act;          // [L, K] activation rows, tiled layout
  const uint8_t* w;             // [E, N, K/2]
  const uint16_t* s;            // [E, N, K/32]
  const int32_t* sorted_ids;    // [L]
  const int32_t* offsets;       // [E + 1] segment starts (multiples of 16)
  const int32_t* tile_offsets;  // [E + 1] 256-row tiles per expert, exclusive scan
  const float* topk_weights;    // [P]
  uint16_t* h;                  // gate_up output [L, I], tiled layout
  float* y;                     // down output [P, N] per routed pair
  int32_t P, E, K, N, I;
  int32_t col_tiles;            // output column tiles per row tile
};

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Largest e with toff[e] <= m, for 0 <= m < toff[E] (skips empty experts).
__device__ __forceinline__ int expert_of_tile(const int32_t* toff, int E, int m) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (toff[mid] <= m) lo = mid;
    else hi = mid;
  }
  return lo;
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding: vmcnt bits
// [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Four MFMAs of one row block (A operand `a`) against the wave's four column tiles,
// accumulating in place. Written as assembly so that the 256 accumulator values stay
// pinned in AGPRs (the register allocator otherwise shuffles them through VGPRs);
// `s_nop 1` gives the two wait states a VALU write of an operand register needs before
// an MFMA reads it.
__device__ __forceinline__ void mfma4_acc(f32x4 (&acc)[4], const u32x4& a, const u32x4 (&b)[4]) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %5, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %4, %6, %1\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %4, %7, %2\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %4, %8, %3"
      : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3])
      : "v"(a), "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]));
}

// Orders every later read of the accumulators after at least 24 wait states following
// the last MFMA (more than an MFMA-write to VALU-read dependency requires). The
// accumulators pass through volatile statements, which keep their program order.
__device__ __forceinline__ void drain_acc(f32x4 (&acc)[kRowBlocks][kColTiles]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int m = 0; m < kRowBlocks; ++m)
    asm volatile("" : "+a"(acc[m][0]), "+a"(acc[m][1]), "+a"(acc[m][2]), "+a"(acc[m][3]));
}

template <TEpi EPI>
__global__ void __launch_bounds__(kThreads) w4a16_tiled_kernel(TiledArgs a) {
  __shared__ u32x4 a_lds[kStages][kRowBlocks][kWave];  // 64 KB

  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int col = lane & 15, quad = lane >> 4;

  // XCD-aware item order over the real tile count: XCD x takes a contiguous range.
  const int total = a.tile_offsets[a.E] * a.col_tiles;
  const int per = (total + kNumXcd - 1) / kNumXcd;
  const int xi = blockIdx.x / kNumXcd;
  const int item = (blockIdx.x % kNumXcd) * per + xi;
  if (xi >= per || item >= total) return;
  const int rtile = item / a.col_tiles, ctile = item % a.col_tiles;
  const int e = expert_of_tile(a.tile_offsets, a.E, rtile);
  const int seg1 = a.offsets[e + 1];
  const int row0 = a.offsets[e] + (rtile - a.tile_offsets[e]) * kTileRows;
  const int rb0 = row0 >> 4;
  const int rb_last = (seg1 >> 4) - 1;
  const int K = a.K, KG = K >> 5;
  const int nsteps = KG, nblocks = K >> 8;

  // Weight rows of this wave's four column tiles; per-lane byte offsets stay 32-bit
  // (host-checked) on top of the expert's uniform base.
  int wrow[kColTiles];
#pragma unroll
  for (int t = 0; t < kColTiles; ++t) {
    if constexpr (EPI == TEpi::GateUp) {
      const int j = ctile * 128 + wave * 32 + (t & 1) * 16 + col;
      wrow[t] = (t < 2) ? j : a.I + j;
    } else {
      wrow[t] = ctile * 256 + wave * 64 + t * 16 + col;
    }
  }
  const uint8_t* wbase = a.w + (size_t)e * a.N * (size_t)(K >> 1);
  const uint8_t* sbase = reinterpret_cast<const uint8_t*>(a.s + (size_t)e * a.N * (size_t)KG);
  uint32_t woff[kColTiles], soff[kColTiles];
#pragma unroll
  for (int t = 0; t < kColTiles; ++t) {
    woff[t] = (uint32_t)wrow[t] * (uint32_t)(K >> 1) + 16u * quad;
    soff[t] = (uint32_t)wrow[t] * (uint32_t)(KG * 2);
  }

  // Activation copies of this wave: row blocks wave*4 .. wave*4+3 of the tile.
  const uint8_t* abase = reinterpret_cast<const uint8_t*>(a.act);
  uint32_t aoff[kCopiesPerWave];
#pragma unroll
  for (int i = 0; i < kCopiesPerWave; ++i) {
    const int rb = min(rb0 + wave * kCopiesPerWave + i, rb_last);
    aoff[i] = (uint32_t)rb * (uint32_t)(KG * 1024) + lane * 16u;
  }
  // Copies group min(g, last) into stage g % kStages. Past the end the copy repeats the
  // last group into a free stage, so that every k step issues the same number of vector
  // memory instructions and the vmcnt thresholds below hold at the tail too.
  auto copy_group = [&](int g) {
    const int st = g & (kStages - 1);
    const uint32_t src = (uint32_t)min(g, nsteps - 1) * 1024u;
#pragma unroll
    for (int i = 0; i < kCopiesPerWave; ++i)
      __builtin_amdgcn_global_load_lds(
          (const void*)(abase + (aoff[i] + src)),
          (__attribute__((address_space(3))) void*)&a_lds[st][wave * kCopiesPerWave + i][0], 16,
          0, 0);
  };
  // Weight words of half `hf` (groups 4*hf .. 4*hf+3) of block min(kb, last): 16 B per
  // tile; the scales of a block are one 16 B load per tile. Clamped, never skipped, for
  // the same reason as copy_group.
  auto load_half = [&](int kb, int hf, u32x4 (&dst)[kColTiles]) {
    const uint32_t o = (uint32_t)min(kb, nblocks - 1) * 128u + 64u * hf;
#pragma unroll
    for (int t = 0; t < kColTiles; ++t) dst[t] = ld16(wbase + (woff[t] + o));
  };
  auto load_scales = [&](int kb, u32x4 (&dst)[kColTiles]) {
    const uint32_t o = (uint32_t)min(kb, nblocks - 1) * 16u;
#pragma unroll
    for (int t = 0; t < kColTiles; ++t) dst[t] = ld16(sbase + (soff[t] + o));
  };

  f32x4 acc[kRowBlocks][kColTiles];
#pragma unroll
  for (int m = 0; m < kRowBlocks; ++m)
#pragma unroll
    for (int t = 0; t < kColTiles; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint32_t mask = opaque_sgpr(0x000F000Fu);
  const uint32_t magic = opaque_vgpr(0x64006400u);

  // Weight words of the next half block (`pend`) are loaded four groups ahead of their
  // first use; `spend` holds the next block's scales. Step g runs the MFMAs of group g
  // on operands dequantized during step g-1 (buffer g % 2) and dequantizes group g+1
  // into the other buffer, one (tile, pair) piece after each row block's MFMAs, so the
  // VALU work overlaps the matrix core.
  u32x4 pend[kColTiles], spend[kColTiles], scur[kColTiles];
  uint32_t tw[kColTiles][4];
  u32x4 bq[2][kColTiles];
  auto transpose_pend = [&]() {
#pragma unroll
    for (int t = 0; t < kColTiles; ++t) {
      tw[t][0] = pend[t].x;
      tw[t][1] = pend[t].y;
      tw[t][2] = pend[t].z;
      tw[t][3] = pend[t].w;
      transpose4_rows(tw[t]);
    }
  };
  // Piece p (0..15) of group j's operands: tile p / 4, bf16 pair p % 4.
  auto dequant_piece = [&](int j, int p, u32x4 (&dst)[kColTiles]) {
    const int t = p >> 2, i = p & 3;
    const uint32_t sw = scur[t][j >> 1];
    const float sc = (j & 1) ? bf16_hi(sw) : bf16_lo(sw);
    const uint32_t pr = ((tw[t][j & 3] >> (4 * i)) & mask) | magic;
    const f16x2 hv = __builtin_bit_cast(f16x2, pr);
    const float c = -1032.0f * sc;
    const f32x2 f = {__builtin_fmaf((float)hv.x, sc, c), __builtin_fmaf((float)hv.y, sc, c)};
    dst[t][i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
  };

  // Prologue: block 0's first half and scales, the first kAhead activation groups, then
  // (as at the end of a block) the operands of group 0 and the load of the second half.
  load_half(0, 0, pend);
  load_scales(0, spend);
#pragma unroll
  for (int g = 0; g < kAhead; ++g) copy_group(g);
  transpose_pend();
#pragma unroll
  for (int t = 0; t < kColTiles; ++t) scur[t] = spend[t];
#pragma unroll
  for (int p = 0; p < 16; ++p) dequant_piece(0, p, bq[0]);
  load_half(0, 1, pend);

  for (int kb = 0; kb < nblocks; ++kb) {
#pragma unroll
    for (int j = 0; j < kGroupsPerBlock; ++j) {
      const int g = kb * kGroupsPerBlock + j;
      // This wave's copies of group g are complete once no more than what it issued
      // after them is pending: the copies of groups g+1 and g+2 plus the weight loads
      // of the three previous steps (8 issued at j = 3, 4 at j = 7). Vector memory
      // loads complete in issue order.
      if (j == 3 || j == 7) wait_vmcnt<2 * kCopiesPerWave>();
      else if (j < 3) wait_vmcnt<2 * kCopiesPerWave + kColTiles>();
      else wait_vmcnt<2 * kCopiesPerWave + 2 * kColTiles>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      copy_group(g + kAhead);
      // The vmcnt thresholds assume the weight loads below issue after this step's
      // copies; keep the scheduler from swapping them.
      __builtin_amdgcn_sched_barrier(0);
      // The next half's words are transposed at j = 3 and 7 (the current half is no
      // longer needed: group j's operands already exist), then the following half is
      // requested.
      if (j == 3 || j == 7) {
        transpose_pend();
        if (j == 7) {
#pragma unroll
          for (int t = 0; t < kColTiles; ++t) scur[t] = spend[t];
          load_half(kb + 1, 1, pend);
        } else {
          load_half(kb + 1, 0, pend);
          load_scales(kb + 1, spend);
        }
      }
      const int st = g & (kStages - 1);
      const int jn = (j + 1) & 7;
      u32x4 a0 = a_lds[st][0][lane];
      u32x4 a1 = a_lds[st][1][lane];
#pragma unroll
      for (int m = 0; m < kRowBlocks; ++m) {
        u32x4 a2 = a1;
        if (m + 2 < kRowBlocks) a2 = a_lds[st][m + 2][lane];
        mfma4_acc(acc[m], a0, bq[j & 1]);
        dequant_piece(jn, m, bq[(j + 1) & 1]);
        a0 = a1;
        a1 = a2;
      }
    }
  }
  // The matrix-core results must be settled before ordinary instructions read them.
  drain_acc(acc);

  // Epilogue. Lane (col, quad) holds rows 4*quad + r of each 16-row block, column col.
  if constexpr (EPI == TEpi::GateUp) {
#pragma unroll
    for (int m = 0; m < kRowBlocks; ++m) {
      const int rb = rb0 + m;
      if (rb > rb_last) break;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        const int j = ctile * 128 + wave * 32 + tp * 16 + col;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gv = acc[m][tp][r], uv = acc[m][tp + 2][r];
          a.h[tiled_offset(rb * 16 + 4 * quad + r, j, a.I)] = f32_to_bf16(silu_f32(gv) * uv);
        }
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < kRowBlocks; ++m) {
      const int rb = rb0 + m;
      if (rb > rb_last) break;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pair = a.sorted_ids[rb * 16 + 4 * quad + r];
        if (pair >= a.P) continue;
        const float wt = a.topk_weights[pair];
        float* yrow = a.y + (size_t)pair * a.N;
#pragma unroll
        for (int t = 0; t < kColTiles; ++t) yrow[wrow[t]] = wt * acc[m][t][r];
      }
    }
  }
}

// out[t, :] = bf16(sum of y[t*k + s, :] over the valid slots s of token t).
constexpr int kCombineThreads = 256;

__global__ void __launch_bounds__(kCombineThreads)
    combine_rows_kernel(const float* __restrict__ y, const int32_t* __restrict__ ids,
                        int32_t T, int32_t k, int32_t E, int32_t H, uint16_t* __restrict__ out) {
  const int64_t quads = (int64_t)T * (H >> 2);
  for (int64_t i = (int64_t)blockIdx.x * kCombineThreads + threadIdx.x; i < quads;
       i += (int64_t)gridDim.x * kCombineThreads) {
    const int64_t t = i / (H >> 2);
    const int c = (int)(i - t * (H >> 2)) * 4;
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < k; ++s) {
      const int64_t pair = t * k + s;
      const int id = ids[pair];
      if (id < 0 || id >= E) continue;
      sum += *reinterpret_cast<const f32x4*>(y + pair * H + c);
    }
    const uint32_t lo = (uint32_t)f32_to_bf16(sum.x) | ((uint32_t)f32_to_bf16(sum.y) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(sum.z) | ((uint32_t)f32_to_bf16(sum.w) << 16);
    *reinterpret_cast<uint2*>(out + t * H + c) = make_uint2(lo, hi);
  }
}

template <TEpi EPI>
hipError_t launch_tiled(const TiledArgs& a, int64_t max_row_tiles, hipStream_t stream) {
  const int64_t items = max_row_tiles * a.col_tiles;
  if (items <= 0) return hipSuccess;
  if (items > (int64_t(1) << 30)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((w4a16_tiled_kernel<EPI>), dim3(xcd_major_grid((int)items)),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

bool w4a16_tiled_supported(int32_t H, int32_t I) { return H % 256 == 0 && I % 256 == 0; }

int32_t w4a16_tiled_rows() { return kTileRows; }

hipError_t launch_w4a16_gateup_tiled(const W4A16Problem& p, const Routing& r, hipStream_t stream) {
  TiledArgs a{p.xs, p.w13, p.s13, r.sorted_ids, r.offsets, r.tile_offsets, r.topk_weights,
              p.h, nullptr, r.P, r.E, p.H, 2 * p.I, p.I, p.I / 128};
  return launch_tiled<TEpi::GateUp>(a, (int64_t)r.P / kTileRows + r.E, stream);
}

hipError_t launch_w4a16_down_tiled(const W4A16Problem& p, const Routing& r, float* y,
                                   hipStream_t stream) {
  TiledArgs a{p.h, p.w2, p.s2, r.sorted_ids, r.offsets, r.tile_offsets, r.topk_weights,
              nullptr, y, r.P, r.E, p.I, p.H, p.I, p.H / 256};
  return launch_tiled<TEpi::Down>(a, (int64_t)r.P / kTileRows + r.E, stream);
}

hipError_t launch_combine_rows(const float* y, const int32_t* topk_ids, int32_t T, int32_t k,
                               int32_t E, int32_t H, uint16_t* out, hipStream_t stream) {
  const int64_t quads = (int64_t)T * (H / 4);
  if (quads <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((quads + kCombineThreads - 1) / kCombineThreads, 8192);
  hipLaunchKernelGGL(combine_rows_kernel, dim3((unsigned)blocks), dim3(kCombineThreads), 0,
                     stream, y, topk_ids, T, k, E, H, out);
  return hipGetLastError();
}

}  // namespace qmoe
