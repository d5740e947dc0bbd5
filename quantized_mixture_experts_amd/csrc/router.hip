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
// yields both the value and the lowest id among equals.
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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)x, d, kWave);
    const uint32_t hi = __shfl_xor((uint32_t)(x >> 32), d, kWave);
    const uint64_t y = ((uint64_t)hi << 32) | lo;
    x = y > x ? y : x;
  }
  return x;
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
#pragma unroll
    for (int j = 0; j < kRegChunks; ++j) {
      const int e = lane + kWave * j;
      reg[j] = e < E ? row[e] : 0.f;
    }
    // Best key of this lane's unselected experts (0: none).
    uint64_t taken = 0;  // bit j: expert lane + 64 j is selected
    auto lane_best = [&]() {
      uint64_t best = 0;
#pragma unroll
      for (int j = 0; j < kRegChunks; ++j) {
        const int e = lane + kWave * j;
        if (e < E && !((taken >> j) & 1)) {
          const uint64_t key = key_of(reg[j], e);
          best = key > best ? key : best;
        }
      }
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
      // Every 64 slots (and at the end) the lanes write their slot's id; the weight
      // waits for the denominator, so it goes out as exp(l - m) and is divided below.
      if ((i & (kWave - 1)) == kWave - 1 || i == k - 1) {
        const int base = i & ~(kWave - 1);
        if (lane <= i - base) {
          ids[t * k + base + lane] = expert_map ? expert_map[my_e] : my_e;
          weights[t * k + base + lane] = my_x;
        }
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
    // Each lane divides the slots it wrote (program order: its own stores).
    for (int s = lane; s < k; s += kWave) weights[t * k + s] = weights[t * k + s] / denom;
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
