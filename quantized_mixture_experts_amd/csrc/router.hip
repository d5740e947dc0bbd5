// Router on gfx950: per token, the k experts with the largest router logits, and their
// softmax weights, optionally renormalized over the k, with an optional expert-parallel
// map from global to local expert ids.
//
// The indexed MoE kernels take the routed expert ids and weights of every (token, slot)
// pair ("vLLM x Novita AI: Chord W4A16 INT4 MoE Kernel for Kimi K2.x", section "Two
// kernel families": the indexed path consumes the framework's routing), and a layer run
// with expert parallelism holds one GPU's share of the experts (same page, "vLLM
// integration": the EP8 profiles). Ids of experts held elsewhere map to -1, which the
// align step drops.
//
// Selection is by logit value, which orders the experts exactly as their softmax
// probabilities do (exp is increasing) but without exp's rounding: equal logits keep the
// lower expert id first, and -0 equals +0. The weights are exp(l - m) / S with m the
// largest logit and S the sum of exp(l - m) over the k selected experts (renormalized)
// or over all E experts.
//
// One wave per token: lane l holds experts l, l + 64, ...; each of the k rounds finds
// the best unselected expert of every lane and reduces the lanes' candidates with a
// 64-bit key (orderable logit bits, then the inverted id), so one wave-wide maximum
// yields both the value and the lowest id among equals. The keys of the first 512
// experts are formed once and kept in registers; the wave maximum moves data with DPP
// inside 16-lane rows and with permlane swaps across rows (no LDS round trips).
#include <algorithm>

#include "../../include/qmoe.h"
#include "device_common.h"
#include "internal.h"

namespace qmoe {

namespace {

constexpr int kRouterThreads = 256;
constexpr int kRouterWaves = kRouterThreads / kWave;
// Experts per lane held in registers; more experts are read again from memory (the
// token's row stays in the cache).
constexpr int kRegChunks = 8;
constexpr int kMaxChunks = (QMOE_MAX_EXPERTS + kWave - 1) / kWave;  // 64: one bit each

// Order-preserving map of a float to an unsigned integer (-0 folded into +0).
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t key_of(float v, int e) {
  return ((uint64_t)ordered_bits(v) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// x of the lane that DPP control CTRL selects (every lane has a source: quad
// permutations and rotations within a 16-lane row).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, CTRL, 0xF, 0xF, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}

// The larger of x and its counterpart in the paired row (16-lane rows 0<->1, 2<->3) or
// half (rows 0-1 <-> 2-3): a permlane swap of x with itself puts the partner's value in
// one of the two results and the lane's own in the other.
template <bool kHalves>
__device__ __forceinline__ uint64_t max_with_partner(uint64_t x) {
  const uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
  const auto l = kHalves ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                         : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto h = kHalves ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                         : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  return max_u64(((uint64_t)h[0] << 32) | l[0], ((uint64_t)h[1] << 32) | l[1]);
}

// Wave-wide maximum, in every lane.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
  x = max_u64(x, dpp64<0xB1>(x));   // quad_perm [1,0,3,2]
  x = max_u64(x, dpp64<0x4E>(x));   // quad_perm [2,3,0,1]
  x = max_u64(x, dpp64<0x124>(x));  // row_ror:4
  x = max_u64(x, dpp64<0x128>(x));  // row_ror:8: every lane holds its row's maximum
  x = max_with_partner<false>(x);
  return max_with_partner<true>(x);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) x += __shfl_xor(x, d, kWave);
  return x;
}

__global__ void __launch_bounds__(kRouterThreads)
    topk_softmax_kernel(const float* __restrict__ logits, int32_t T, int32_t E, int32_t k,
                        int32_t renormalize, const int32_t* __restrict__ expert_map,
                        int32_t* __restrict__ ids, float* __restrict__ weights) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int nchunks = (E + kWave - 1) / kWave;
  for (int64_t t = (int64_t)blockIdx.x * kRouterWaves + wave; t < T;
       t += (int64_t)gridDim.x * kRouterWaves) {
    const float* row = logits + t * E;
    float reg[kRegChunks];
    uint64_t keys[kRegChunks];  // 0 past the last expert (below every real key)
#pragma unroll
    for (int j = 0; j < kRegChunks; ++j) {
      const int e = lane + kWave * j;
      reg[j] = e < E ? row[e] : 0.f;
      keys[j] = e < E ? key_of(reg[j], e) : 0;
    }
    // Best key of this lane's unselected experts (0: none).
    uint64_t taken = 0;  // bit j: expert lane + 64 j is selected
    auto lane_best = [&]() {
      uint64_t best = 0;
#pragma unroll
      for (int j = 0; j < kRegChunks; ++j)
        if (!((taken >> j) & 1)) best = max_u64(best, keys[j]);
      for (int j = kRegChunks; j < nchunks; ++j) {
        const int e = lane + kWave * j;
        if (e < E && !((taken >> j) & 1)) {
          const uint64_t key = key_of(row[e], e);
          best = key > best ? key : best;
        }
      }
      return best;
    };
    float m = 0.f, sel_sum = 0.f;
    float my_x = 0.f;  // lane s % 64: exp(l - m) of slot s of the current batch of 64
    int my_e = 0;
    for (int i = 0; i < k; ++i) {
      const uint64_t best = wave_max_u64(lane_best());
      const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
      const uint32_t o = (uint32_t)(best >> 32);
      const float v = __builtin_bit_cast(float, (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
      if (e % kWave == lane) taken |= uint64_t(1) << (e / kWave);
      if (i == 0) m = v;  // the first selected logit is the largest
      const float x = expf(v - m);
      sel_sum += x;
      if (lane == (i & (kWave - 1))) {
        my_x = x;
        my_e = e;
      }
      // Every 64 slots the lanes write their slot's id, and the weight as exp(l - m),
      // divided below once the denominator is known (k > 64 only; up to 64 slots stay
      // in registers until the end).
      if ((i & (kWave - 1)) == kWave - 1 && i != k - 1) {
        const int base = i & ~(kWave - 1);
        ids[t * k + base + lane] = expert_map ? expert_map[my_e] : my_e;
        weights[t * k + base + lane] = my_x;
      }
    }
    float denom = sel_sum;
    if (!renormalize) {
      float part = 0.f;
#pragma unroll
      for (int j = 0; j < kRegChunks; ++j)
        if (lane + kWave * j < E) part += expf(reg[j] - m);
      for (int j = kRegChunks; j < nchunks; ++j)
        if (lane + kWave * j < E) part += expf(row[lane + kWave * j] - m);
      denom = wave_sum(part);
    }
    // The last batch of up to 64 slots from registers; each lane divides the earlier
    // slots it wrote (program order: its own stores).
    const int last = (k - 1) & ~(kWave - 1);
    if (lane <= k - 1 - last) {
      ids[t * k + last + lane] = expert_map ? expert_map[my_e] : my_e;
      weights[t * k + last + lane] = my_x / denom;
    }
    for (int s = lane; s < last; s += kWave) weights[t * k + s] = weights[t * k + s] / denom;
  }
}

}  // namespace

hipError_t launch_topk_softmax(const float* logits, int32_t T, int32_t E, int32_t k,
                               int32_t renormalize, const int32_t* expert_map, int32_t* ids,
                               float* weights, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  if (E > kMaxChunks * kWave) return hipErrorInvalidValue;
  const int64_t blocks = std::min<int64_t>((T + kRouterWaves - 1) / kRouterWaves, 8192);
  hipLaunchKernelGGL(topk_softmax_kernel, dim3((unsigned)blocks), dim3(kRouterThreads), 0, stream,
                     logits, T, E, k, renormalize, expert_map, ids, weights);
  return hipGetLastError();
}

}  // namespace qmoe
