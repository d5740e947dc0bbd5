// W8A8 block-FP8 grouped expert GEMMs, stream profile.
//
// Method ("SGLang W8A8 Block FP8 quantization kernel config guide", background
// section): E4M3 activations with one fp32 scale per token and 128-column group (As),
// E4M3 weights with one fp32 scale per [128, 128] block (Bs); the per-expert
// contraction is C = sum over 128-deep k blocks of (A_q B_q^T)_block * As * Bs.
//
// gfx950 mapping: one v_mfma_scale_f32_16x16x128_f8f6f4 (scales pinned to 1.0) covers
// exactly one 128-deep k block, so its fp32 result is multiplied by As[token, kb] *
// Bs[n/128, kb] and accumulated in fp32. As in the W4A16 decode profile, weights sit on
// the MFMA column side, the expert's rows (16 per block) on the row side, and one
// work-group owns (expert, column chunk). gate_up writes SiLU(gate) * up in fp32 by
// sorted row (requantized to E4M3 per 128 columns by the quantizer kernel); down
// scatter-adds routing-weighted rows into the fp32 output.
#include "device_common.h"
#include "internal.h"

namespace qmoe {

namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerGroup = kThreads / kWave;

enum class Epi { GateUp, Down };

struct Fp8StreamArgs {
  const uint8_t* act;         // gate_up: a_q [T, K]; down: hq [L, K]
  const float* act_scale;     // gate_up: a_scale [T, K/128]; down: hs [L, K/128]
  const uint8_t* w;           // [E, N, K]
  const float* ws;            // [E, N/128, K/128]
  const int32_t* sorted_ids;  // [L]
  const int32_t* offsets;     // [E + 1]
  const float* topk_weights;  // [P]
  float* h32;                 // gate_up output [L, I]
  float* out32;               // down output [T, N]
  int32_t P, k, K, N, I;
};

template <Epi EPI, int MB>
__global__ void __launch_bounds__(kThreads) fp8_stream_kernel(Fp8StreamArgs a) {
  const int e = blockIdx.y;
  const int seg0 = a.offsets[e], seg1 = a.offsets[e + 1];
  if (seg0 == seg1) return;
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int col = lane & 15, quad = lane >> 4;

  int base[4];
  bool tile_ok[4];
  int j0 = 0;
  if constexpr (EPI == Epi::GateUp) {
    j0 = (blockIdx.x * kWavesPerGroup + wave) * 32;
    if (j0 >= a.I) return;
    base[0] = j0;
    base[1] = j0 + 16;
    base[2] = a.I + j0;
    base[3] = a.I + j0 + 16;
#pragma unroll
    for (int t = 0; t < 4; ++t) tile_ok[t] = true;
  } else {
    j0 = (blockIdx.x * kWavesPerGroup + wave) * 64;
    if (j0 >= a.N) return;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      tile_ok[t] = j0 + 16 * t < a.N;
      base[t] = tile_ok[t] ? j0 + 16 * t : 0;
    }
  }
  const int K = a.K, KBLK = K / 128;
  const uint8_t* wrow[4];
  const float* wsrow[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    wrow[t] = a.w + ((size_t)e * a.N + base[t] + col) * K + 32 * quad;
    wsrow[t] = a.ws + ((size_t)e * (a.N / 128) + base[t] / 128) * KBLK;
  }
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  const int nmb_total = (seg1 - seg0) / kSegRows;
  for (int mb0 = 0; mb0 < nmb_total; mb0 += MB) {
    const int nmb = min(MB, nmb_total - mb0);
    const uint8_t* arow[MB];
    bool aok[MB];
    const float* asrow[MB][4];  // scale rows of this lane's four output rows
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const int r = seg0 + (mb0 + b) * kSegRows + col;
      int sid = a.P;
      if (b < nmb) sid = a.sorted_ids[r];
      aok[b] = sid < a.P;
      const size_t arow_idx = (EPI == Epi::GateUp) ? (size_t)(aok[b] ? sid / a.k : 0) : (size_t)(aok[b] ? r : 0);
      arow[b] = a.act + arow_idx * K + 32 * quad;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int ro = seg0 + (mb0 + b) * kSegRows + 4 * quad + rr;
        int s2 = a.P;
        if (b < nmb) s2 = a.sorted_ids[ro];
        size_t idx = 0;
        if (s2 < a.P) idx = (EPI == Epi::GateUp) ? (size_t)(s2 / a.k) : (size_t)ro;
        asrow[b][rr] = a.act_scale + idx * KBLK;
      }
    }
    f32x4 acc[4][MB];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int b = 0; b < MB; ++b) acc[t][b] = zero4;

    u32x4 wcur[4][2], wnxt[4][2];
    auto load = [&](u32x4 (&buf)[4][2], int kb) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        buf[t][0] = ld16(wrow[t] + kb * 128);
        buf[t][1] = ld16(wrow[t] + kb * 128 + 16);
      }
    };
    load(wcur, 0);
    for (int kb = 0; kb < KBLK; ++kb) {
      if (kb + 1 < KBLK) load(wnxt, kb + 1);
      float bs[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) bs[t] = wsrow[t][kb];
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        if (b >= nmb) continue;
        u32x4 av[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
        if (aok[b]) {
          av[0] = ld16(arow[b] + kb * 128);
          av[1] = ld16(arow[b] + kb * 128 + 16);
        }
        float as[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) as[rr] = asrow[b][rr][kb];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const f32x4 d = mfma_fp8_16x16x128(av, wcur[t], zero4);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) acc[t][b][rr] += d[rr] * (as[rr] * bs[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        wcur[t][0] = wnxt[t][0];
        wcur[t][1] = wnxt[t][1];
      }
    }

#pragma unroll
    for (int b = 0; b < MB; ++b) {
      if (b >= nmb) continue;
      const int rbase = seg0 + (mb0 + b) * kSegRows + 4 * quad;
      if constexpr (EPI == Epi::GateUp) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float* hrow = a.h32 + (size_t)(rbase + r) * a.I + j0 + col;
          hrow[0] = silu_f32_accurate(acc[0][b][r]) * acc[2][b][r];
          hrow[16] = silu_f32_accurate(acc[1][b][r]) * acc[3][b][r];
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
hipError_t launch(const Fp8StreamArgs& a, int E, int mb, hipStream_t stream) {
  const int cols_per_group = (EPI == Epi::GateUp) ? 32 * kWavesPerGroup : 64 * kWavesPerGroup;
  const int extent = (EPI == Epi::GateUp) ? a.I : a.N;
  dim3 grid((extent + cols_per_group - 1) / cols_per_group, E);
  switch (mb) {
    case 1:
      hipLaunchKernelGGL((fp8_stream_kernel<EPI, 1>), grid, dim3(kThreads), 0, stream, a);
      break;
    case 2:
      hipLaunchKernelGGL((fp8_stream_kernel<EPI, 2>), grid, dim3(kThreads), 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL((fp8_stream_kernel<EPI, 4>), grid, dim3(kThreads), 0, stream, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8_gateup_stream(const Fp8Problem& p, const Routing& r, int mb,
                                    hipStream_t stream) {
  Fp8StreamArgs a{p.a_q, p.a_scale, p.w13, p.s13, r.sorted_ids, r.offsets, r.topk_weights,
                  p.h32, nullptr, r.P, r.k, p.H, 2 * p.I, p.I};
  return launch<Epi::GateUp>(a, r.E, mb, stream);
}

hipError_t launch_fp8_down_stream(const Fp8Problem& p, const Routing& r, int mb,
                                  hipStream_t stream) {
  Fp8StreamArgs a{p.hq, p.hs, p.w2, p.s2, r.sorted_ids, r.offsets, r.topk_weights, nullptr,
                  p.out32, r.P, r.k, p.I, p.H, p.I};
  return launch<Epi::Down>(a, r.E, mb, stream);
}

}  // namespace qmoe
