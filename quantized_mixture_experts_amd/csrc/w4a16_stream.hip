// W4A16 grouped expert GEMMs, decode profile (weights streamed once per pass).
//
// Method: BF16 activations times INT4 group-32 weights with BF16 scales, fp32
// accumulation ("vLLM x Novita AI: Chord W4A16 INT4 MoE Kernel for Kimi K2.x": summary;
// "vLLM integration"). At a few routed rows per expert the work is a weight stream, so
// the decode profile puts the dequantized weights on the MFMA column side and the
// expert's rows (padded to 16) on the row side (the page's decode profile swaps the MMA
// operands the same way, section "H200 and Blackwell indexed decode"), and one wave owns
// (expert, two column tiles) so each weight byte is read once per pass.
//
// gfx950 mapping, per wave and per 256-deep k step:
//   * each lane loads 2 x 16 B of one weight row, so one step consumes a whole 128 B
//     cache line per row; lane quarter q holds whole groups q and 4+q; a 4x4 permlane
//     transpose regroups them so that for every group the four quarters hold its four
//     words, the k layout of one v_mfma_f32_16x16x32_bf16 (one MFMA = one scale group);
//   * codes become bf16 (128 + code) with one AND-OR per pair; the zero point is removed
//     through the MFMA's C operand: C = x . (-136) for the group, computed once per
//     work-group and group (one MFMA on the activation operand) and kept in LDS beside
//     the operand, so the weight MFMAs of a group do not wait on each other;
//   * the group scale multiplies the fp32 MFMA result (one FMA per output element);
//   * weights are prefetched three k steps ahead through a ring of four register
//     stages: under full load HBM latency is a few microseconds, so each wave keeps
//     ~12 KB in flight; scales (one 128 B line per row covers 8 steps) are loaded once
//     per 8 steps into the wave's LDS slice, since per-step reads would re-fetch lines
//     the weight stream has already evicted from L2;
//   * the activation operand (the expert's 16 rows) is shared by the work-group's eight
//     waves: 512-deep chunks are copied once into LDS (double-buffered, one barrier per
//     chunk) and read with ds_read_b128. Every byte loaded besides the weight stream
//     costs the stream bandwidth, so the eight waves share one copy. Activation rows live
//     in a tiled layout in which the operand of one (16-row block, k group) is 1 KB
//     contiguous.
// gate_up fuses SiLU(gate) * up and stores h (bf16, tiled by sorted row); down scales by
// the routing weight and scatter-adds into the fp32 output with hardware atomics.
//
// MXFP4 weights (E2M1 codes, E8M0 scales per 32 k; the weight-only MXFP4 format of the
// "xiaotu-moe" project page, overview) run through the same kernels with MX = true: one
// v_cvt_scalef32_pk_bf16_fp4 per code pair gives the exact scaled bf16 weight (the scale
// is a power of two), so there is no zero-point term and no scale multiply after the
// MFMA, which accumulates in place. The FP4 converts produce natural k order, so the
// activation rows and h use the natural-order tiled layout. NVFP4 (NV = true; E4M3
// scales per 16 k and an fp32 scale per expert, the same page's list) converts each code
// pair to fp32, multiplies by the block scale times the expert's scale and rounds once
// to bf16; each lane's 8 codes of a group lie in one 16-k half, so one scale per lane.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace qmoe {

namespace {

constexpr int kThreads = 512;
constexpr int kWavesPerGroup = kThreads / kWave;
constexpr int kChunkPieces = 1024 / kThreads;  // 16 B chunk pieces per thread and block
constexpr uint32_t kNeg136Pair = 0xC308C308u;  // bf16 -136, twice
constexpr int kChunkGroups = 16;               // k groups per LDS activation chunk

enum class Epi { GateUp, Down };

struct StreamArgs {
  const uint16_t* act;        // [L, K] activation rows, tiled layout (tiled_offset)
  const uint8_t* w;           // [E, N, K/2]
  const uint16_t* s;          // [E, N, K/32] bf16 (INT4) or E8M0 bytes (MXFP4)
  const int32_t* sorted_ids;  // [L]
  const int32_t* offsets;     // [E + 1]
  const int32_t* expert_ids;  // [L / block_m], expert of each align block (16 MB rows)
  const int32_t* ntp;         // rows in use (a multiple of 16)
  const float* topk_weights;  // [P]
  uint16_t* h;                // gate_up output [L, I], tiled layout
  float* out32;               // down output [T, N]
  int32_t P, k, K, N, I;
  int32_t chunks, items;      // column chunks per expert; E * chunks
  float* zero_out;            // persistent gate_up: fp32 buffer it clears first (or null)
  int64_t zero_n;             // its length in floats, a multiple of 4
  const float* g = nullptr;   // NVFP4: [E] fp32 scale per expert of this projection
  // Persistent gate_up: the activation rows [T, K] in their natural layout, read by token
  // through sorted_ids (then `act` is unused and no gathered copy is needed).
  const uint16_t* x = nullptr;
  // Persistent gate_up with one pair per row (k = 1): clear only the rows of zero_out
  // (K floats each) that a sorted row routes, not all of it.
  bool zero_routed = false;
};

struct Stage {
  u32x4 w[2][2];  // two 16 B chunks of each column tile's row (groups q and 4+q)
};

constexpr int kScaleBlockSteps = 8;  // one 128 B line of bf16 scales = 64 groups = 8 steps
constexpr int kStages = 4;           // weight register stages (loads run kStages-1 ahead)

template <Epi EPI, int MB, bool MX, bool NV>
__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(2)))
    w4a16_stream_kernel(StreamArgs a) {
  // Activation chunks: [buffer][M-block][group in chunk][lane], 16 B each, and the
  // zero-point term of each group in the MFMA result layout (4 fp32 per lane).
  __shared__ u32x4 a_lds[2][MB][kChunkGroups][kWave];
  __shared__ f32x4 c_lds[2][MB][kChunkGroups][kWave];
  // Group scales of each wave's tiles for one 8-step block: [wave][tile][row][piece],
  // piece p = the 8 scales of step p.
  __shared__ u32x4 s_lds[kWavesPerGroup][2][16][kScaleBlockSteps];

  // Work-groups are dealt to the 8 XCDs round-robin by launch index; give each XCD a
  // contiguous range of (expert, column chunk) items in expert-major order so that an
  // expert's activation rows are read into one XCD's L2, not all eight.
  const int item = xcd_major_item(blockIdx.x, gridDim.x, a.items);
  if (item < 0) return;
  const int e = item / a.chunks, chunk = item % a.chunks;
  const int seg0 = a.offsets[e], seg1 = a.offsets[e + 1];
  if (seg0 == seg1) return;
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int col = lane & 15, quad = lane >> 4;

  // Two column tiles of 16 weight rows per wave: gate and up rows of the same 16 h
  // columns for gate_up, 32 consecutive output columns for down. Waves past the end
  // keep running (with a clamped tile) to take part in the work-group's barriers.
  int row[2];
  bool tile_ok[2];
  int j0 = 0;
  if constexpr (EPI == Epi::GateUp) {
    j0 = (chunk * kWavesPerGroup + wave) * 16;
    const bool ok = j0 < a.I;
    const int jc = ok ? j0 : 0;
    row[0] = jc + col;
    row[1] = a.I + jc + col;
    tile_ok[0] = tile_ok[1] = ok;
  } else {
    j0 = (chunk * kWavesPerGroup + wave) * 32;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      tile_ok[t] = j0 + 16 * t < a.N;
      row[t] = tile_ok[t] ? j0 + 16 * t + col : col;
    }
  }

  const int K = a.K, G = K / 32, KB = K / 2;
  const uint8_t* wrow[2];
  const uint16_t* srow[2];
  const uint8_t* mrow[2];  // FP4: the row's scale bytes (E8M0 per 32 k, E4M3 per 16 k)
  constexpr int kScalesPerGroup = NV ? 2 : 1;
  const float gsc = NV ? a.g[e] : 1.f;
  const int hsel = NV ? quad >> 1 : 0;  // this lane's 16-k half of a group
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    wrow[t] = a.w + ((size_t)e * a.N + row[t]) * KB;
    srow[t] = a.s + ((size_t)e * a.N + row[t]) * G;
    mrow[t] = reinterpret_cast<const uint8_t*>(a.s) +
              ((size_t)e * a.N + row[t]) * G * kScalesPerGroup;
  }
  // FP4 scale of group gg of tile t for this lane, in the form the dequantization takes.
  auto fp4_scale = [&](int t, int gg) {
    if constexpr (NV) return e4m3_low(mrow[t][2 * gg + hsel]) * gsc;
    else return e8m0_scale(mrow[t][gg]);
  };
  const int nstep = G / 8;  // full 256-deep steps
  const int nchunk = (G + kChunkGroups - 1) / kChunkGroups;
  const uint32_t neg136[4] = {kNeg136Pair, kNeg136Pair, kNeg136Pair, kNeg136Pair};
  const uint32_t one28 = opaque_vgpr(kBf16Bias128), nib = opaque_sgpr(kNibbleMask);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  const int nmb_total = (seg1 - seg0) / kSegRows;
  for (int mb0 = 0; mb0 < nmb_total; mb0 += MB) {
    const int nmb = min(MB, nmb_total - mb0);
    // Tiled activation blocks of this pass. Blocks past the pass's last one re-read
    // the first (results unused); padding rows inside a block hold zeros.
    const u32x4* ablk[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const int blk = seg0 / kSegRows + (b < nmb ? mb0 + b : mb0);
      ablk[b] = reinterpret_cast<const u32x4*>(a.act) + (size_t)blk * G * kWave;
    }

    // Chunk c of every block: 16 groups x 64 lanes x 16 B, four 16 B pieces per thread
    // and block. Loads are never predicated (chunks past the end re-read the last);
    // a predicated load would make the compiler's wait-count insertion wait for every
    // outstanding load.
    u32x4 creg[MB][kChunkPieces];
    auto chunk_load = [&](int c) {
      c = min(c, nchunk - 1);
#pragma unroll
      for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int i = 0; i < kChunkPieces; ++i) {
          const int idx = threadIdx.x + kThreads * i;  // group-in-chunk * 64 + lane
          const int g = min(c * kChunkGroups + idx / kWave, G - 1);
          creg[b][i] = ablk[b][(size_t)g * kWave + (idx % kWave)];
        }
    };
    // Piece i of this thread is the MFMA activation operand of group wave + 8i for this
    // lane, so each wave also derives the zero-point term x . (-136) of those groups (one
    // MFMA each) and parks it next to the operands: the weight MFMAs then take it as
    // their accumulator input without waiting on another MFMA.
    auto chunk_store = [&](int buf) {
#pragma unroll
      for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int i = 0; i < kChunkPieces; ++i) {
          const int g = wave + kWavesPerGroup * i;
          a_lds[buf][b][g][lane] = creg[b][i];
          if constexpr (!MX) {
            const uint32_t av[4] = {creg[b][i][0], creg[b][i][1], creg[b][i][2],
                                    creg[b][i][3]};
            c_lds[buf][b][g][lane] = mfma_bf16_16x16x32(av, neg136, zero4);
          }
        }
    };

    f32x4 acc[2][MB];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int b = 0; b < MB; ++b) acc[t][b] = zero4;

    auto load = [&](Stage& st, int it) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint8_t* p = wrow[t] + it * 128 + 16 * quad;
        st.w[t][0] = ld16(p);
        st.w[t][1] = ld16(p + 64);
      }
      // Keep the prefetch ahead of the compute that follows it.
      __builtin_amdgcn_sched_barrier(0);
    };

    // Scales: one 128 B line per weight row covers 8 steps. Reading them per step from
    // global memory re-fetches the line up to eight times (the weight stream evicts it
    // from L2 between steps), so each block of 8 steps is loaded once (lane quarter q
    // takes pieces 2q and 2q+1 of its row), parked in this wave's LDS slice, and read
    // back per step. Pieces past the end of a row are clamped into it (never used).
    u32x4 sreg[2][2];
    const int row_bytes = G * 2;
    auto scale_load = [&](int blk) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int off = min(blk * 128 + 16 * (2 * quad + i), row_bytes - 16);
          sreg[t][i] = ld16(reinterpret_cast<const uint8_t*>(srow[t]) + max(off, 0));
        }
    };
    auto scale_store = [&]() {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 2; ++i) s_lds[wave][t][col][2 * quad + i] = sreg[t][i];
    };

    // One group: activation operand and zero-point term from LDS, then each tile.
    auto group = [&](int buf, int gl, uint32_t w0, uint32_t w1, float sc0, float sc1) {
      uint32_t av[MB][4];
      f32x4 corr[MB];
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        const u32x4 v = a_lds[buf][b][gl][lane];
        av[b][0] = v[0];
        av[b][1] = v[1];
        av[b][2] = v[2];
        av[b][3] = v[3];
        if constexpr (!MX) corr[b] = c_lds[buf][b][gl][lane];
      }
      uint32_t bw0[4], bw1[4];
      if constexpr (MX) {
        // sc0, sc1: the scales in the form fp4_to_bf16 / nvfp4_to_bf16 take
        if constexpr (NV) {
          nvfp4_to_bf16(w0, sc0, bw0);
          nvfp4_to_bf16(w1, sc1, bw1);
        } else {
          fp4_to_bf16(w0, sc0, bw0);
          fp4_to_bf16(w1, sc1, bw1);
        }
#pragma unroll
        for (int b = 0; b < MB; ++b) {
          if (b < nmb) {
            acc[0][b] = mfma_bf16_16x16x32(av[b], bw0, acc[0][b]);
            acc[1][b] = mfma_bf16_16x16x32(av[b], bw1, acc[1][b]);
          }
        }
        return;
      }
      int4_to_bf16_biased(w0, nib, one28, bw0);
      int4_to_bf16_biased(w1, nib, one28, bw1);
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        if (b < nmb) {
          const f32x4 d0 = mfma_bf16_16x16x32(av[b], bw0, corr[b]);
          const f32x4 d1 = mfma_bf16_16x16x32(av[b], bw1, corr[b]);
          acc[0][b] += sc0 * d0;
          acc[1][b] += sc1 * d1;
        }
      }
    };

    // A full step (eight groups) from the staged weights; gl0 = first group in chunk,
    // sp = the step's scale piece within the current scale block, it = the step. MXFP4
    // reads its scale bytes directly (this kernel serves only K not a multiple of 512).
    auto compute = [&](Stage& st, int buf, int gl0, int sp, int it) {
      const u32x4 sv[2] = {s_lds[wave][0][col][sp], s_lds[wave][1][col][sp]};
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t wt[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int i = 0; i < 4; ++i) wt[t][i] = st.w[t][half][i];
          transpose4_rows(wt[t]);
        }
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int g = 4 * half + g4;
          float sc0, sc1;
          if constexpr (MX) {
            sc0 = fp4_scale(0, it * 8 + g);
            sc1 = fp4_scale(1, it * 8 + g);
          } else {
            const uint32_t s0w = sv[0][g >> 1], s1w = sv[1][g >> 1];
            sc0 = (g & 1) ? bf16_hi(s0w) : bf16_lo(s0w);
            sc1 = (g & 1) ? bf16_hi(s1w) : bf16_lo(s1w);
          }
          group(buf, gl0 + g, wt[0][g4], wt[1][g4], sc0, sc1);
        }
      }
    };

    chunk_load(0);
    chunk_store(0);
    chunk_load(1);
    __syncthreads();
    if (nstep > 0) {
      // Steps 2c and 2c+1 use chunk c; steps 8b..8b+7 use scale block b. Loads are
      // never predicated (a step or block past the end re-reads the last one, which the
      // cache serves): a predicated load would make the compiler's wait-count insertion
      // wait for every outstanding load. Scales run one block ahead.
      const int last = nstep - 1;
      const int nblk = (nstep + kScaleBlockSteps - 1) / kScaleBlockSteps;
      const int nscale_blk = (G + 63) / 64;
      // Four register stages in a ring, weights loaded three steps ahead.
      Stage st[kStages];
      scale_load(0);
#pragma unroll
      for (int i = 0; i < kStages - 1; ++i) load(st[i], min(i, last));
      for (int blk = 0; blk < nblk; ++blk) {
        scale_store();
        scale_load(min(blk + 1, nscale_blk - 1));
#pragma unroll
        for (int j = 0; j < kScaleBlockSteps; ++j) {
          const int it = blk * kScaleBlockSteps + j;
          const int c = it / 2, buf = c & 1;
          load(st[(j + kStages - 1) % kStages], min(it + kStages - 1, last));
          if (it < nstep) compute(st[j % kStages], buf, 8 * (j & 1), j, it);
          if (j & 1) {
            // Chunk boundary: chunk c+1 goes to the other buffer (whose readers, chunk
            // c-1, all passed the previous barrier), then the next chunk is requested.
            chunk_store(buf ^ 1);
            chunk_load(c + 2);
            __syncthreads();
          }
        }
      }
    }
    // Groups past the last full step (K not a multiple of 256): lane quarter q reads word
    // q of the group directly; the activation comes from the chunk holding the group.
    for (int g = nstep * 8; g < G; ++g) {
      const int c = g / kChunkGroups;
      const uint32_t w0 = *reinterpret_cast<const uint32_t*>(wrow[0] + g * 16 + 4 * quad);
      const uint32_t w1 = *reinterpret_cast<const uint32_t*>(wrow[1] + g * 16 + 4 * quad);
      if constexpr (MX)
        group(c & 1, g % kChunkGroups, w0, w1, fp4_scale(0, g), fp4_scale(1, g));
      else
        group(c & 1, g % kChunkGroups, w0, w1, bf16_to_f32(srow[0][g]), bf16_to_f32(srow[1][g]));
    }

    // Epilogue.
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      if (b >= nmb) continue;
      const int rbase = seg0 + (mb0 + b) * kSegRows + 4 * quad;
      if constexpr (EPI == Epi::GateUp) {
        if (tile_ok[0]) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            a.h[tiled_offset<MX>(rbase + r, j0 + col, a.I)] =
                f32_to_bf16(silu_f32(acc[0][b][r]) * acc[1][b][r]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int sid = a.sorted_ids[rbase + r];
          if (sid >= a.P) continue;
          const float wt = a.topk_weights[sid];
          float* orow = a.out32 + (size_t)(sid / a.k) * a.N + j0 + col;
#pragma unroll
          for (int t = 0; t < 2; ++t)
            if (tile_ok[t]) unsafeAtomicAdd(orow + 16 * t, wt * acc[t][b][r]);
        }
      }
    }
    if (mb0 + MB < nmb_total) __syncthreads();  // LDS chunks are reused by the next pass
  }
}

// Persistent variant for K a multiple of 512. The grid is one work-group per compute
// unit; work-group w takes a contiguous range of units, a unit being 512 of one item's K
// (two 256-deep steps, i.e. one activation chunk), in (row block of 16 MB rows, column
// chunk, k) order. The weight ring, the activation chunk double buffer and the scale pieces run on
// across item boundaries, so a work-group never waits for a pipeline refill after the
// first, and every work-group gets the same number of units up to one. down ranges may
// start or end inside an item: each piece adds its partial sum into the fp32 output with
// the same atomics as whole items. gate_up ranges hold whole items, since SiLU needs the
// complete sums.
constexpr int kUnitGroups = 16;  // k groups per unit (= kChunkGroups)
// Work-group shape of the persistent kernel: kPWaves waves, kPGroupsPerCu work-groups
// per compute unit (kPWavesPerEu waves per SIMD).
constexpr int kPWaves = 8;
constexpr int kPGroupsPerCu = 1;
constexpr int kPThreads = kPWaves * kWave;
constexpr int kPWavesPerEu = kPWaves * kPGroupsPerCu / 4;
constexpr int kPPieces = 1024 / kPThreads;  // 16 B chunk pieces per thread
static_assert(1024 % kPThreads == 0, "chunk pieces per thread");
// Groups per batch of a half step: their activation operands and zero-point terms are
// read from LDS at once and their MFMAs issued back to back before the scale FMAs.
constexpr int kPBatch = 4;
// Weight ring depth in 256-deep steps (loads run kRing - 1 steps ahead). Under full load
// HBM latency is a few microseconds; each step holds 4 KB per wave.
constexpr int kRing = 4;
static_assert(kRing % 2 == 0 && kRing >= 4, "ring of whole units, at least two");
// Group scales are staged per block of kScaleUnits units: 128 B (one cache line) of
// each weight row, loaded a block ahead with whole lines per row.
constexpr int kScaleUnits = 4;
// f32x4 entries per staged scale piece: its two half steps of 16 rows, plus two of pad.
constexpr int kPieceStride = 2 * 16 + 2;
constexpr int kBodyUnits = (kRing / 2) % 2 == 0 ? kRing / 2 : kRing;
constexpr int kWin = kRing / 2 + 1;  // unit descriptors kept ahead (the farthest load)

template <typename F, int... U>
__device__ __forceinline__ void unroll_units(F& f, int u, std::integer_sequence<int, U...>) {
  (f(std::integral_constant<int, U>{}, u + U), ...);
}

struct Unit {
  int rb, cc, kc, e;  // row block (16 MB rows), column chunk, unit within the item's K, expert
};

// MB: 16-row MFMA blocks per row block (align pads every expert's segment to 16 MB
// rows, so a row block never spans two experts). Each dequantized weight operand feeds
// the MFMAs of all MB blocks, so a pass over the weights serves 16 MB rows.
// DX: the activation chunks come straight from the rows of x (gate_up), found through the
// pair ids, instead of from a gathered copy in the operand layout.
template <Epi EPI, bool MX, bool NV, int MB, bool DX>
__global__ void __launch_bounds__(kPThreads)
    __attribute__((amdgpu_waves_per_eu(kPWavesPerEu)))
    w4a16_persist_kernel(StreamArgs a) {
  static_assert(MB == 1 || MB == 2, "LDS holds the activation chunks of at most two blocks");
  __shared__ u32x4 a_lds[2][MB][kChunkGroups][kWave];
  // Zero-point term of each group per activation row: the same for every column, so one
  // float per row (read by the four lanes of a row quarter at once).
  __shared__ float c_lds[2][MB][kChunkGroups][16];
  // Scales of the current block as fp32, converted once when the block is staged:
  // [wave][tile][step in block][half step * 16 + row], four groups each (rows innermost,
  // so the sixteen rows a wave reads at once are 16 B apart). Each piece's 2 x 16 entries
  // are padded to kPieceStride: the block store writes eight rows of eight pieces at
  // once, and without the pad the pieces (512 B apart) would all land on the same LDS
  // banks.
  __shared__ f32x4 s_lds[kPWaves][2][2 * kScaleUnits][kPieceStride];

  // gate_up clears the fp32 output that down accumulates into (down starts after the
  // last gate_up work-group has ended).
  if constexpr (EPI == Epi::GateUp) {
    if (a.zero_out && a.zero_routed) {
      const int row4 = a.K / 4;
      const int64_t n4 = (int64_t)ld_invariant(a.ntp, 0) * row4;
      for (int64_t i = (int64_t)blockIdx.x * kPThreads + threadIdx.x; i < n4;
           i += (int64_t)gridDim.x * kPThreads) {
        const int r = (int)(i / row4);
        const int sid = a.sorted_ids[r];
        if (sid < a.P)
          reinterpret_cast<f32x4*>(a.zero_out + (size_t)sid * a.K)[i - (int64_t)r * row4] =
              f32x4{0.f, 0.f, 0.f, 0.f};
      }
    } else if (a.zero_out) {
      const int64_t n4 = a.zero_n / 4;
      for (int64_t i = (int64_t)blockIdx.x * kPThreads + threadIdx.x; i < n4;
           i += (int64_t)gridDim.x * kPThreads)
        reinterpret_cast<f32x4*>(a.zero_out)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  const int K = a.K, G = K / 32, KB = K / 2, N = a.N;
  const int upi = K / 512;  // units per item
  const int items = (ld_invariant(a.ntp, 0) / (kSegRows * MB)) * a.chunks;
  const int nwg = gridDim.x;  // a multiple of the XCD count
  // XCD-major numbering: the work-groups of one XCD hold consecutive ranges, so the
  // column chunks of one expert (which share its activation rows) meet in one L2.
  const int wg = (blockIdx.x % kNumXcd) * (nwg / kNumXcd) + blockIdx.x / kNumXcd;
  // gate_up: work-group k of an XCD (of wpx) takes items xbase + k, xbase + k + wpx,
  // xbase + k + 2 wpx, ... of its XCD's range: at any time the XCD's work-groups work on
  // the column chunks of the same one or two row blocks, so each activation chunk is
  // read once into the XCD's L2 and shared, instead of being read again by one
  // work-group item after item (by then the weight stream has evicted it). Its units are
  // numbered locally: unit u is unit u % upi of its item u / upi. down: a contiguous
  // range of global units.
  const int wpx = nwg / kNumXcd, kk = wg % wpx;
  int per_items = 0, xbase = 0;
  int u0, u1;
  if constexpr (EPI == Epi::GateUp) {
    per_items = (items + nwg - 1) / nwg;
    xbase = (wg / wpx) * wpx * per_items;
    // items of this work-group: the j with xbase + j * wpx + kk < items (a prefix)
    const int left = items - xbase - kk;
    const int mine = left <= 0 ? 0 : min(per_items, (left + wpx - 1) / wpx);
    u0 = 0;
    u1 = mine * upi;
  } else {
    const int total = items * upi;
    const int per = (total + nwg - 1) / nwg;
    u0 = min(total, wg * per);
    u1 = min(total, wg * per + per);
  }
  if (u0 >= u1) return;
  const int ulast = u1 - 1;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = lane_id();
  const int col = lane & 15, quad = lane >> 4;
  const uint32_t neg136[4] = {kNeg136Pair, kNeg136Pair, kNeg136Pair, kNeg136Pair};
  const uint32_t one28 = opaque_vgpr(kBf16Bias128), nib = opaque_sgpr(kNibbleMask);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  auto desc = [&](int u) {
    Unit d;
    int item;
    if constexpr (EPI == Epi::GateUp) {
      const int j = u / upi;
      d.kc = u - j * upi;
      item = xbase + j * wpx + kk;
    } else {
      item = u / upi;
      d.kc = u - item * upi;
    }
    d.rb = item / a.chunks;
    d.cc = item - d.rb * a.chunks;
    d.e = ld_invariant(a.expert_ids, d.rb);
    return d;
  };
  // First weight row of tile t of this wave in column chunk cc, and whether the tile
  // exists (tiles past the end read rows 0..15 of the expert; results unused).
  auto tile_row0 = [&](int cc, int t) {
    if constexpr (EPI == Epi::GateUp) {
      const int j0 = (cc * kPWaves + wave) * 16;
      return (j0 < a.I ? j0 : 0) + (t ? a.I : 0);
    } else {
      const int j0 = (cc * kPWaves + wave) * 32 + 16 * t;
      return j0 < N ? j0 : 0;
    }
  };
  // Per-lane parts of the weight and scale addresses, the same for every unit.
  const uint32_t lane_w = col * KB + 16 * quad;

  auto load = [&](Stage& s, const Unit& d, int p) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint8_t* base = a.w + ((size_t)d.e * N + tile_row0(d.cc, t)) * KB + d.kc * 256;
      const uint8_t* q = base + lane_w + p * 128;
      s.w[t][0] = ld16(q);
      s.w[t][1] = ld16(q + 64);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // A block's scales: load i covers tile i / 2, rows 8 (i % 2) .. + 7, one 128 B line
  // per row (lane l: row + l / 8, 16 B piece l % 8, i.e. step l % 8 of the block). Pieces
  // past the end of a row are clamped into it (never used).
  // MXFP4: the block is 64 B per row (one E8M0 byte per group), lane piece l % 8 is the
  // step's 8 B.
  u32x4 snext[4];
  const int s_row = lane >> 3, s_piece = lane & 7;
  auto scale_block_load = [&](u32x4 (&dst)[4], const Unit& d) {
    if constexpr (MX && !NV) {
      const int off = min((d.kc & ~(kScaleUnits - 1)) * 16 + s_piece * 8, G - 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = tile_row0(d.cc, i >> 1) + 8 * (i & 1) + s_row;
        const uint32_t* p = reinterpret_cast<const uint32_t*>(
            reinterpret_cast<const uint8_t*>(a.s) + ((size_t)d.e * N + row) * G + off);
        dst[i] = u32x4{p[0], p[1], 0u, 0u};
      }
    } else {
      const int off = min((d.kc & ~(kScaleUnits - 1)) * 32 + s_piece * 16, G * 2 - 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = tile_row0(d.cc, i >> 1) + 8 * (i & 1) + s_row;
        dst[i] = ld16(reinterpret_cast<const uint8_t*>(a.s) + ((size_t)d.e * N + row) * G * 2 + off);
      }
    }
  };
  auto scale_block_store = [&](const u32x4 (&src)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 v = src[i];
      if constexpr (NV) {
        // the step's 16 E4M3 bytes of this row (two per group), kept raw
        s_lds[wave][i >> 1][s_piece][8 * (i & 1) + s_row] = __builtin_bit_cast(f32x4, v);
      } else if constexpr (MX) {
        s_lds[wave][i >> 1][s_piece][8 * (i & 1) + s_row] =
            f32x4{e8m0_scale(v[0]), e8m0_scale(v[0] >> 8), e8m0_scale(v[0] >> 16),
                  e8m0_scale(v[0] >> 24)};
        s_lds[wave][i >> 1][s_piece][16 + 8 * (i & 1) + s_row] =
            f32x4{e8m0_scale(v[1]), e8m0_scale(v[1] >> 8), e8m0_scale(v[1] >> 16),
                  e8m0_scale(v[1] >> 24)};
      } else {
        s_lds[wave][i >> 1][s_piece][8 * (i & 1) + s_row] =
            f32x4{bf16_lo(v[0]), bf16_hi(v[0]), bf16_lo(v[1]), bf16_hi(v[1])};
        s_lds[wave][i >> 1][s_piece][16 + 8 * (i & 1) + s_row] =
            f32x4{bf16_lo(v[2]), bf16_hi(v[2]), bf16_lo(v[3]), bf16_hi(v[3])};
      }
    }
  };
  // First unit of the block after unit u's (the next item's first unit at an item end).
  auto next_block = [&](int u, int kc) {
    return min(u + min(kScaleUnits - (kc & (kScaleUnits - 1)), upi - kc), ulast);
  };

  u32x4 creg[MB][kPPieces];
  bool creal[MB];  // DX: the lane's row of each block holds a routed pair (else padding)
  // DX: the row block whose tokens tok_cache holds (a row block lasts a whole item, K / 512
  // units, so the pair ids are looked up once per item).
  int rb_cache = -1;
  int tok_cache[MB];
  // DX: token of this lane's activation row (row `col` of the 16-row block rb16), or -1 for
  // a padding row. The block's sixteen pair ids come through scalar loads (the block index
  // is made wave-uniform explicitly; from a per-lane address they would be vector loads),
  // which do not enter the vector memory counter: waiting for them does not wait for the
  // weight loads in flight.
  auto row_token = [&](int rb16) {
    const int32_t* ids = a.sorted_ids + __builtin_amdgcn_readfirstlane(rb16) * 16;
    int sid = 0;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int v = ld_invariant(ids, m);
      sid = (col == m) ? v : sid;
    }
    return sid < a.P ? sid / a.k : -1;
  };
  // Piece i of this thread is the operand slice of group wave + 8 i for this lane: row
  // `col`, k slice `quad`, i.e. 8 activations at k = 32 (16 kc + wave + 8 i) + 8 quad.
  auto chunk_load = [&](const Unit& d) {
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      if constexpr (DX) {
        if (d.rb != rb_cache) tok_cache[b] = row_token(d.rb * MB + b);
        const int tok = tok_cache[b];
        creal[b] = tok >= 0;
        const uint16_t* src =
            a.x + (size_t)max(tok, 0) * K + d.kc * (kUnitGroups * 32) + 8 * quad;
#pragma unroll
        for (int i = 0; i < kPPieces; ++i) creg[b][i] = ld16(src + (wave + kPWaves * i) * 32);
        if (b == MB - 1) rb_cache = d.rb;
      } else {
        const u32x4* ablk =
            reinterpret_cast<const u32x4*>(a.act) + (size_t)(d.rb * MB + b) * G * kWave;
#pragma unroll
        for (int i = 0; i < kPPieces; ++i) {
          const int idx = threadIdx.x + kPThreads * i;  // group-in-chunk * 64 + lane
          creg[b][i] = ablk[(size_t)(d.kc * kUnitGroups + idx / kWave) * kWave + idx % kWave];
        }
      }
    }
  };
  auto chunk_store = [&](int buf) {
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int i = 0; i < kPPieces; ++i) {
        const int g = wave + kPWaves * i;
        u32x4 v = creg[b][i];
        if constexpr (DX) {
          // natural k order -> the operand order of the INT4 dequantization; padding
          // rows are zero
          if constexpr (!MX) {
            uint32_t pv[4];
            perm_act8(v, pv);
            v = u32x4{pv[0], pv[1], pv[2], pv[3]};
          }
          if (!creal[b]) v = u32x4{0u, 0u, 0u, 0u};
        }
        a_lds[buf][b][g][lane] = v;
        if constexpr (!MX) {
          const uint32_t av[4] = {v[0], v[1], v[2], v[3]};
          const f32x4 c = mfma_bf16_16x16x32(av, neg136, zero4);
          if (col == 0) *reinterpret_cast<f32x4*>(&c_lds[buf][b][g][4 * quad]) = c;
        }
      }
  };

  // Groups per batch of the INT4 path: fewer with two blocks, whose products would
  // otherwise not fit the registers.
  constexpr int kBatch = kPBatch / MB;
  f32x4 acc[2][MB];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[t][b] = zero4;
  // One 256-deep step: groups 8p..8p+7 of the unit's chunk, scale piece p, in batches of
  // kPBatch groups whose LDS reads and MFMAs are issued together, so neither the LDS
  // latency nor the MFMA latency is paid once per group.
  const int hsel = NV ? quad >> 1 : 0;  // this lane's 16-k half of a group (NVFP4)
  auto compute = [&](Stage& s, int buf, int p, int sp, float gs) {
    f32x4 sv[2][2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      sv[0][half] = s_lds[wave][0][sp][16 * half + col];
      sv[1][half] = s_lds[wave][1][sp][16 * half + col];
      uint32_t wt[2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) wt[t][i] = s.w[t][half][i];
        transpose4_rows(wt[t]);
      }
      if constexpr (MX) {
        // Exact scaled weights from the converts; the MFMAs accumulate in place.
#pragma unroll
        for (int gb = 0; gb < 4; ++gb) {
          uint32_t a4[MB][4];
#pragma unroll
          for (int b = 0; b < MB; ++b) {
            const u32x4 v = a_lds[buf][b][8 * p + 4 * half + gb][lane];
            a4[b][0] = v[0];
            a4[b][1] = v[1];
            a4[b][2] = v[2];
            a4[b][3] = v[3];
          }
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            uint32_t bw[4];
            if constexpr (NV) {
              // byte 2 g + hsel of the step's raw scales (entry 0 holds them)
              const int g = 4 * half + gb;
              const u32x4 raw = __builtin_bit_cast(u32x4, sv[t][0]);
              nvfp4_to_bf16(wt[t][gb], e4m3_low(raw[g >> 1] >> (16 * (g & 1) + 8 * hsel)) * gs,
                            bw);
            } else {
              fp4_to_bf16(wt[t][gb], sv[t][half][gb], bw);
            }
#pragma unroll
            for (int b = 0; b < MB; ++b) acc[t][b] = mfma_bf16_16x16x32(a4[b], bw, acc[t][b]);
          }
        }
        continue;
      }
#pragma unroll
      for (int b0 = 0; b0 < 4; b0 += kBatch) {
        u32x4 av[MB][kBatch];
        f32x4 cv[MB][kBatch];
#pragma unroll
        for (int b = 0; b < MB; ++b)
#pragma unroll
          for (int gb = 0; gb < kBatch; ++gb) {
            const int gl = 8 * p + 4 * half + b0 + gb;
            av[b][gb] = a_lds[buf][b][gl][lane];
            cv[b][gb] = *reinterpret_cast<const f32x4*>(&c_lds[buf][b][gl][4 * quad]);
          }
        f32x4 d[2][MB][kBatch];
#pragma unroll
        for (int gb = 0; gb < kBatch; ++gb) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            uint32_t bw[4];
            int4_to_bf16_biased(wt[t][b0 + gb], nib, one28, bw);
#pragma unroll
            for (int b = 0; b < MB; ++b) {
              const uint32_t a4[4] = {av[b][gb][0], av[b][gb][1], av[b][gb][2], av[b][gb][3]};
              d[t][b][gb] = mfma_bf16_16x16x32(a4, bw, cv[b][gb]);
            }
          }
        }
#pragma unroll
        for (int gb = 0; gb < kBatch; ++gb) {
          const int g = 4 * half + b0 + gb;
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int b = 0; b < MB; ++b) acc[t][b] += sv[t][half][g & 3] * d[t][b][gb];
        }
      }
    }
  };
  // down: pair ids of this lane's four rows for the current and the next unit, and the
  // routing weights of the current unit's rows, loaded a unit ahead of their use.
  int sid_c[MB][4], sid_n[MB][4];
  float wt_c[MB][4];
  auto sid_load = [&](int (&sid)[MB][4], const Unit& d) {
    if constexpr (EPI == Epi::Down) {
#pragma unroll
      for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sid[b][r] = a.sorted_ids[(d.rb * MB + b) * kSegRows + 4 * quad + r];
    }
  };
  auto wt_load = [&]() {
    if constexpr (EPI == Epi::Down) {
#pragma unroll
      for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) wt_c[b][r] = a.topk_weights[min(sid_c[b][r], a.P - 1)];
    }
  };
  auto epilogue = [&](const Unit& d) {
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const int rbase = (d.rb * MB + b) * kSegRows + 4 * quad;
      if constexpr (EPI == Epi::GateUp) {
        const int j0 = (d.cc * kPWaves + wave) * 16;
        if (j0 < a.I) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            a.h[tiled_offset<MX>(rbase + r, j0 + col, a.I)] =
                f32_to_bf16(silu_f32(acc[0][b][r]) * acc[1][b][r]);
        }
      } else {
        const int j0 = (d.cc * kPWaves + wave) * 32;
        (void)rbase;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int sid = sid_c[b][r];
          if (sid >= a.P) continue;
          float* orow = a.out32 + (size_t)(sid / a.k) * N + j0 + col;
#pragma unroll
          for (int t = 0; t < 2; ++t)
            if (j0 + 16 * t < N) unsafeAtomicAdd(orow + 16 * t, wt_c[b][r] * acc[t][b][r]);
        }
      }
      acc[0][b] = zero4;
      acc[1][b] = zero4;
    }
  };

  // Descriptors of units u .. u + kWin - 1, clamped to the range (loads past its end
  // re-read the last unit, which the cache serves, and are never used).
  Unit dq[kWin];
#pragma unroll
  for (int i = 0; i < kWin; ++i) dq[i] = desc(min(u0 + i, ulast));
  // The scales of the first two blocks are loaded ahead of the weight ring: the loop
  // waits for the prefetched block's scales at the next block start, and the compiler
  // counts that wait over every path into the loop, this one included. Loaded after the
  // ring, they would be the youngest loads on this path, and the wait would drain the
  // ring at every block start.
  sid_load(sid_c, dq[0]);
  u32x4 sfirst[4];
  scale_block_load(sfirst, dq[0]);
  scale_block_load(snext, desc(next_block(u0, dq[0].kc)));
  chunk_load(dq[0]);
  Stage st[kRing];
#pragma unroll
  for (int j = 0; j < kRing - 1; ++j) load(st[j], dq[j / 2], j & 1);
  chunk_store(0);
  chunk_load(dq[1]);
  scale_block_store(sfirst);
  __syncthreads();

  // Unit u at position U of the unrolled body uses activation buffer and scale registers
  // U & 1 and ring slots (2U + p) % kRing for its steps p = 0, 1; the loads of local step
  // s + kRing - 1 are issued at step s.
  auto unit = [&](auto U_, int u) {
    constexpr int U = decltype(U_)::value;
    constexpr int P = U & 1;
    constexpr int a0 = kRing - 1, a1 = kRing;  // steps ahead of the loads, from step 0
    const bool live = u < u1;
    wt_load();
    sid_load(sid_n, dq[1]);
    const int kc = dq[0].kc;
    if (live && u != u0 && (kc & (kScaleUnits - 1)) == 0) {
      scale_block_store(snext);
      scale_block_load(snext, desc(next_block(u, kc)));
    }
    const int sp = 2 * (kc & (kScaleUnits - 1));
    // NVFP4: the expert's global scale (a scalar load; 1 otherwise)
    const float gs =
        NV ? __builtin_bit_cast(float, ld_invariant(reinterpret_cast<const int32_t*>(a.g), dq[0].e))
           : 1.f;
    load(st[(2 * U + a0) % kRing], dq[a0 / 2], a0 & 1);
    if (live) compute(st[(2 * U) % kRing], P, 0, sp, gs);
    load(st[(2 * U + 1 + a0) % kRing], dq[a1 / 2], a1 & 1);
    if (live) compute(st[(2 * U + 1) % kRing], P, 1, sp + 1, gs);
    if (live && (dq[0].kc == upi - 1 || u == ulast)) epilogue(dq[0]);
    chunk_store(P ^ 1);
    chunk_load(dq[2]);
    __syncthreads();
#pragma unroll
    for (int i = 0; i + 1 < kWin; ++i) dq[i] = dq[i + 1];
    dq[kWin - 1] = desc(min(u + kWin, ulast));
    if constexpr (EPI == Epi::Down) {
#pragma unroll
      for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) sid_c[b][r] = sid_n[b][r];
    }
  };
  for (int u = u0; u < u1; u += kBodyUnits)
    unroll_units(unit, u, std::make_integer_sequence<int, kBodyUnits>{});
}

// xs = x gathered by sorted row in the tiled operand layout, for rows below
// num_tokens_padded; padding rows are zero so the GEMMs load them unmasked.
// One work-group per (16-row block, range of kGatherGroups k groups), so that a few
// hundred rows still fill the chip; each wave writes whole 1 KB operands (one k group of
// the block): lane (q, m) reads 16 B of row m at k slice q and stores them, permuted to
// the operand k order, at its place in the operand, so every store is a full line.
constexpr int kGatherThreads = 256;
constexpr int kGatherWaves = kGatherThreads / kWave;
constexpr int kGatherGroups = 32;  // 1024 columns per work-group

template <bool kNatural>
__global__ void __launch_bounds__(kGatherThreads)
    gather_rows_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ sorted_ids,
                       const int32_t* __restrict__ ntp, int32_t P, int32_t k, int32_t H,
                       uint16_t* __restrict__ xs) {
  const int rb = blockIdx.x;
  if (rb * 16 >= ntp[0]) return;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int q = lane >> 4, m = lane & 15;
  const int sid = sorted_ids[rb * 16 + m];
  const bool real = sid < P;
  const uint16_t* src = x + (size_t)(real ? sid / k : 0) * H + 8 * q;
  const int KG = H >> 5;
  const int kg_end = min(KG, (int)(blockIdx.y + 1) * kGatherGroups);
  uint16_t* dst = xs + ((size_t)rb * KG * 64 + lane) * 8;
  int kg = blockIdx.y * kGatherGroups + wave;
  // A whole range: all of this wave's loads are issued before the first store.
  constexpr int kPer = kGatherGroups / kGatherWaves;
  if (kg + (kPer - 1) * kGatherWaves < kg_end) {
    u32x4 v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) v[i] = ld16(src + (kg + i * kGatherWaves) * 32);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      uint32_t p0[4] = {v[i][0], v[i][1], v[i][2], v[i][3]};
      if constexpr (!kNatural) perm_act8(v[i], p0);
      *reinterpret_cast<u32x4*>(dst + (size_t)(kg + i * kGatherWaves) * 512) =
          real ? u32x4{p0[0], p0[1], p0[2], p0[3]} : u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }
  for (; kg < kg_end; kg += kGatherWaves) {
    const u32x4 v0 = ld16(src + kg * 32);
    uint32_t p0[4] = {v0[0], v0[1], v0[2], v0[3]};
    if constexpr (!kNatural) perm_act8(v0, p0);
    *reinterpret_cast<u32x4*>(dst + (size_t)kg * 512) =
        real ? u32x4{p0[0], p0[1], p0[2], p0[3]} : u32x4{0u, 0u, 0u, 0u};
  }
}

}  // namespace

// One work-group per compute unit (the persistent kernels' resources allow no second),
// rounded down to a multiple of the XCD count; queried once per device.
int persistent_grid() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cu = 0;
    n = std::max(kNumXcd, cu / kNumXcd * kNumXcd);
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

namespace {

template <Epi EPI, bool MX, bool NV, int MB, bool DX>
void launch_persist(const StreamArgs& args, hipStream_t stream) {
  hipLaunchKernelGGL((w4a16_persist_kernel<EPI, MX, NV, MB, DX>),
                     dim3(persistent_grid() * kPGroupsPerCu), dim3(kPThreads), 0, stream, args);
}

template <Epi EPI, bool MX, bool NV>
hipError_t launch_stream(const StreamArgs& a, int E, int mb, hipStream_t stream) {
  const bool persist = a.K % 512 == 0;
  const int waves = persist ? kPWaves : kWavesPerGroup;
  const int cols_per_group = (EPI == Epi::GateUp) ? 16 * waves : 32 * waves;
  const int extent = (EPI == Epi::GateUp) ? a.I : a.N;
  StreamArgs args = a;
  args.chunks = (extent + cols_per_group - 1) / cols_per_group;
  args.items = E * args.chunks;
  // The persistent kernel serves mb 16-row blocks per weight pass (align made segments
  // of 16 mb rows); the general kernel one 16-row block at a time of any segments.
  if (persist) {
    // gate_up with one block per pass reads the rows of x directly (no gathered copy)
    if constexpr (EPI == Epi::GateUp) {
      if (mb == 1)
        launch_persist<EPI, MX, NV, 1, true>(args, stream);
      else
        launch_persist<EPI, MX, NV, 2, false>(args, stream);
    } else {
      if (mb == 2)
        launch_persist<EPI, MX, NV, 2, false>(args, stream);
      else
        launch_persist<EPI, MX, NV, 1, false>(args, stream);
    }
  } else {
    hipLaunchKernelGGL((w4a16_stream_kernel<EPI, 1, MX, NV>), dim3(xcd_major_grid(args.items)),
                       dim3(kThreads), 0, stream, args);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gather_rows(const uint16_t* x, const Routing& r, const int32_t* ntp, int32_t H,
                              uint16_t* xs, hipStream_t stream, bool natural) {
  if (r.L <= 0) return hipSuccess;
  // L is at least num_tokens_padded, a multiple of 16
  const int kchunks = (H / 32 + kGatherGroups - 1) / kGatherGroups;
  const dim3 grid((r.L + 15) / 16, kchunks);
  if (natural)
    hipLaunchKernelGGL(gather_rows_kernel<true>, grid, dim3(kGatherThreads), 0, stream, x,
                       r.sorted_ids, ntp, r.P, r.k, H, xs);
  else
    hipLaunchKernelGGL(gather_rows_kernel<false>, grid, dim3(kGatherThreads), 0, stream, x,
                       r.sorted_ids, ntp, r.P, r.k, H, xs);
  return hipGetLastError();
}

bool w4a16_stream_zeroes_output(int32_t H) { return H % 512 == 0; }

// One 16-row block per pass holds few routed rows (the padding rows need no loads), so
// reading the token rows directly beats a gathered copy; with two blocks per pass the rows
// are dense and the gathered operands (1 KB contiguous each) load faster (measured on
// MI355X: grouped decode, 48 experts x 32 rows, gate_up 220 us gathered, 232 us direct).
bool w4a16_stream_reads_rows(int32_t H, int mb) { return H % 512 == 0 && mb == 1; }

hipError_t launch_w4a16_gateup_stream(const W4A16Problem& p, const Routing& r, int mb,
                                      hipStream_t stream) {
  const bool zero = w4a16_stream_zeroes_output(p.H);
  StreamArgs a{p.xs, p.w13, p.s13, r.sorted_ids, r.offsets, r.expert_ids, r.ntp, r.topk_weights,
               p.h, nullptr,
               r.P, r.k, p.H, 2 * p.I, p.I, 0, 0,
               zero ? p.out32 : nullptr, zero ? (int64_t)p.T * p.H : 0};
  a.g = p.g13;
  a.x = p.x;
  a.zero_routed = p.routed_rows_only;
  return p.nv   ? launch_stream<Epi::GateUp, true, true>(a, r.E, mb, stream)
         : p.mx ? launch_stream<Epi::GateUp, true, false>(a, r.E, mb, stream)
                : launch_stream<Epi::GateUp, false, false>(a, r.E, mb, stream);
}

hipError_t launch_w4a16_down_stream(const W4A16Problem& p, const Routing& r, int mb,
                                    hipStream_t stream) {
  StreamArgs a{p.h, p.w2, p.s2, r.sorted_ids, r.offsets, r.expert_ids, r.ntp, r.topk_weights,
               nullptr, p.out32,
               r.P, r.k, p.I, p.H, p.I, 0, 0, nullptr, 0};
  a.g = p.g2;
  return p.nv   ? launch_stream<Epi::Down, true, true>(a, r.E, mb, stream)
         : p.mx ? launch_stream<Epi::Down, true, false>(a, r.E, mb, stream)
                : launch_stream<Epi::Down, false, false>(a, r.E, mb, stream);
}

}  // namespace qmoe
