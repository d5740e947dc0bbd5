// W4A16 grouped expert GEMMs, decode profile (weights streamed once per pass).
//
// Method: BF16 activations times INT4 group-32 weights with BF16 scales, fp32
// accumulation ("vLLM x Novita AI: Chord W4A16 INT4 MoE Kernel for Kimi K2.x": summary;
// "vLLM integration"). At a few routed rows per expert the work is a weight stream, so
// the decode profile puts the dequantized weights on the MFMA column side and the
// expert's rows (padded to 16) on the row side (the page's decode profile swaps the MMA
// operands the same way, section "H200 and Blackwell indexed decode"), and one
// work-group owns (expert, column chunk) so each weight byte is read once per pass.
//
// gfx950 mapping, per wave and per 256-deep k step:
//   * each lane loads 2 x 16 B of one weight row (128 B per row, full cache lines);
//     lane quarter q holds whole groups q and 4+q; a 4x4 permlane transpose regroups
//     them so that for every group the four quarters hold its four words, which is the
//     k layout of one v_mfma_f32_16x16x32_bf16 (one MFMA = one scale group);
//   * codes become bf16 (128 + code) with one AND-OR per pair; the zero point is removed
//     through the MFMA's C operand: C = x . (-136) for the group, computed by one extra
//     MFMA per group shared by all column tiles;
//   * the group scale multiplies the fp32 MFMA result (one FMA per output element);
//   * gate_up fuses SiLU(gate) * up and stores h (bf16, by sorted row); down scales by
//     the routing weight and scatter-adds into the fp32 output with hardware atomics.
#include "device_common.h"
#include "internal.h"

namespace qmoe {

namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerGroup = kThreads / kWave;
constexpr uint32_t kNeg136Pair = 0xC308C308u;  // bf16 -136, twice

enum class Epi { GateUp, Down };

struct StreamArgs {
  const uint16_t* act;        // gate_up: x [T, K] (rows gathered by token); down: h [L, K]
  const uint8_t* w;           // [E, N, K/2]
  const uint16_t* s;          // [E, N, K/32]
  const int32_t* sorted_ids;  // [L]
  const int32_t* offsets;     // [E + 1]
  const float* topk_weights;  // [P]
  uint16_t* h;                // gate_up output [L, I]
  float* out32;               // down output [T, N]
  int32_t P, k, K, N, I;
};

struct WBuf {
  u32x4 w[4][2];
  u32x4 s[4];
};

template <Epi EPI, int MB>
__global__ void __launch_bounds__(kThreads) w4a16_stream_kernel(StreamArgs a) {
  const int e = blockIdx.y;
  const int seg0 = a.offsets[e], seg1 = a.offsets[e + 1];
  if (seg0 == seg1) return;
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int col = lane & 15, quad = lane >> 4;

  // Column tiles of this wave (4 x 16 weight rows).
  int row[4];
  bool tile_ok[4];
  int j0 = 0;
  if constexpr (EPI == Epi::GateUp) {
    j0 = (blockIdx.x * kWavesPerGroup + wave) * 32;
    if (j0 >= a.I) return;
    row[0] = j0 + col;
    row[1] = j0 + 16 + col;
    row[2] = a.I + j0 + col;
    row[3] = a.I + j0 + 16 + col;
#pragma unroll
    for (int t = 0; t < 4; ++t) tile_ok[t] = true;
  } else {
    j0 = (blockIdx.x * kWavesPerGroup + wave) * 64;
    if (j0 >= a.N) return;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      tile_ok[t] = j0 + 16 * t < a.N;
      row[t] = tile_ok[t] ? j0 + 16 * t + col : col;
    }
  }

  const int K = a.K, G = K / 32, KB = K / 2;
  const uint8_t* wrow[4];
  const uint16_t* srow[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    wrow[t] = a.w + ((size_t)e * a.N + row[t]) * KB;
    srow[t] = a.s + ((size_t)e * a.N + row[t]) * G;
  }
  const int nfull = K / 256;
  uint32_t neg136[4] = {kNeg136Pair, kNeg136Pair, kNeg136Pair, kNeg136Pair};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  const int nmb_total = (seg1 - seg0) / kSegRows;
  for (int mb0 = 0; mb0 < nmb_total; mb0 += MB) {
    const int nmb = min(MB, nmb_total - mb0);
    const uint16_t* arow[MB];
    bool aok[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const int r = seg0 + (mb0 + b) * kSegRows + col;
      int sid = a.P;
      if (b < nmb) sid = a.sorted_ids[r];
      aok[b] = sid < a.P;
      if constexpr (EPI == Epi::GateUp)
        arow[b] = a.act + (size_t)(aok[b] ? sid / a.k : 0) * K + 8 * quad;
      else
        arow[b] = a.act + (size_t)(aok[b] ? r : 0) * K + 8 * quad;
    }

    f32x4 acc[4][MB];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int b = 0; b < MB; ++b) acc[t][b] = zero4;

    auto load = [&](WBuf& buf, int it) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint8_t* p = wrow[t] + it * 128 + 16 * quad;
        buf.w[t][0] = ld16(p);
        buf.w[t][1] = ld16(p + 64);
        buf.s[t] = ld16(srow[t] + it * 8);
      }
    };

    auto compute = [&](const WBuf& buf, int it) {
      uint32_t wt[4][8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint32_t lo[4] = {buf.w[t][0][0], buf.w[t][0][1], buf.w[t][0][2], buf.w[t][0][3]};
        uint32_t hi[4] = {buf.w[t][1][0], buf.w[t][1][1], buf.w[t][1][2], buf.w[t][1][3]};
        transpose4_rows(lo);
        transpose4_rows(hi);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          wt[t][g] = lo[g];
          wt[t][4 + g] = hi[g];
        }
      }
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        uint32_t av[MB][4];
        f32x4 corr[MB];
#pragma unroll
        for (int b = 0; b < MB; ++b) {
          u32x4 xv = {0u, 0u, 0u, 0u};
          if (aok[b]) xv = ld16(arow[b] + it * 256 + 32 * g);
          perm_act8(xv, av[b]);
          corr[b] = mfma_bf16_16x16x32(av[b], neg136, zero4);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          uint32_t bw[4];
          int4_to_bf16_biased(wt[t][g], bw);
          const uint32_t sw = buf.s[t][g >> 1];
          const float sc = (g & 1) ? bf16_hi(sw) : bf16_lo(sw);
#pragma unroll
          for (int b = 0; b < MB; ++b) {
            if (b < nmb) {
              f32x4 d = mfma_bf16_16x16x32(av[b], bw, corr[b]);
              acc[t][b] += sc * d;
            }
          }
        }
      }
    };

    if (nfull > 0) {
      WBuf b0, b1;
      load(b0, 0);
      for (int it = 0; it < nfull; it += 2) {
        if (it + 1 < nfull) load(b1, it + 1);
        compute(b0, it);
        if (it + 1 < nfull) {
          if (it + 2 < nfull) load(b0, it + 2);
          compute(b1, it + 1);
        }
      }
    }
    // Remaining groups (K not a multiple of 256): one group at a time, lane quarter q
    // reads word q of the group directly.
    for (int g = nfull * 8; g < G; ++g) {
      uint32_t av[MB][4];
      f32x4 corr[MB];
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        u32x4 xv = {0u, 0u, 0u, 0u};
        if (aok[b]) xv = ld16(arow[b] + 32 * g);
        perm_act8(xv, av[b]);
        corr[b] = mfma_bf16_16x16x32(av[b], neg136, zero4);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t word = *reinterpret_cast<const uint32_t*>(wrow[t] + g * 16 + 4 * quad);
        uint32_t bw[4];
        int4_to_bf16_biased(word, bw);
        const float sc = bf16_to_f32(srow[t][g]);
#pragma unroll
        for (int b = 0; b < MB; ++b) {
          if (b < nmb) {
            f32x4 d = mfma_bf16_16x16x32(av[b], bw, corr[b]);
            acc[t][b] += sc * d;
          }
        }
      }
    }

    // Epilogue.
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      if (b >= nmb) continue;
      const int rbase = seg0 + (mb0 + b) * kSegRows + 4 * quad;
      if constexpr (EPI == Epi::GateUp) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          uint16_t* hrow = a.h + (size_t)(rbase + r) * a.I + j0 + col;
          hrow[0] = f32_to_bf16(silu_f32(acc[0][b][r]) * acc[2][b][r]);
          hrow[16] = f32_to_bf16(silu_f32(acc[1][b][r]) * acc[3][b][r]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int sid = a.sorted_ids[rbase + r];
          if (sid >= a.P) continue;
          const float wt = a.topk_weights[sid];
          float* orow = a.out32 + (size_t)(sid / a.k) * a.N + j0 + col;
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (tile_ok[t]) unsafeAtomicAdd(orow + 16 * t, wt * acc[t][b][r]);
        }
      }
    }
  }
}

template <Epi EPI>
hipError_t launch_stream(const StreamArgs& a, int E, int mb, hipStream_t stream) {
  const int cols_per_group = (EPI == Epi::GateUp) ? 32 * kWavesPerGroup : 64 * kWavesPerGroup;
  const int extent = (EPI == Epi::GateUp) ? a.I : a.N;
  dim3 grid((extent + cols_per_group - 1) / cols_per_group, E);
  switch (mb) {
    case 1:
      hipLaunchKernelGGL((w4a16_stream_kernel<EPI, 1>), grid, dim3(kThreads), 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL((w4a16_stream_kernel<EPI, 2>), grid, dim3(kThreads), 0, stream, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_w4a16_gateup_stream(const W4A16Problem& p, const Routing& r, int mb,
                                      hipStream_t stream) {
  StreamArgs a{p.x, p.w13, p.s13, r.sorted_ids, r.offsets, r.topk_weights, p.h, nullptr,
               r.P, r.k, p.H, 2 * p.I, p.I};
  return launch_stream<Epi::GateUp>(a, r.E, mb, stream);
}

hipError_t launch_w4a16_down_stream(const W4A16Problem& p, const Routing& r, int mb,
                                    hipStream_t stream) {
  StreamArgs a{p.h, p.w2, p.s2, r.sorted_ids, r.offsets, r.topk_weights, nullptr, p.out32,
               r.P, r.k, p.I, p.H, p.I};
  return launch_stream<Epi::Down>(a, r.E, mb, stream);
}

}  // namespace qmoe
