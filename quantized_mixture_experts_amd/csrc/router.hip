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
// One wave per token. Lane l holds the c = ceil(E / 64) consecutive experts l*c ..
// l*c + c - 1, so lower lanes hold lower ids. Each of the k rounds takes the largest
// remaining value of every lane (its head), reduces the 64 heads to the wave maximum
// (32-bit orderable logit bits: DPP within 16-lane rows, row broadcasts across them),
// and picks the lowest lane whose head equals it (a ballot): that lane's head is the
// lowest id among the equal maxima. Only that lane moves on to its next value.
//  - Up to 512 experts (c <= 8) each lane sorts its values once, in registers, into a
//    descending list (ties: lower id first); a round shifts the winning lane's list.
//  - Above 512 the winning lane scans its experts again (the token's row stays in the
//    cache) for the best one not yet taken.
// The selected values and ids are kept one slot per lane and the exps are
// taken once per batch of 64 slots, all lanes at once.
#include <algorithm>

#include "../../include/qmoe.h"
#include "device_common.h"
#include "internal.h"

namespace qmoe {

namespace {

constexpr int kRouterThreads = 256;
constexpr int kRouterWaves = kRouterThreads / kWave;
// Most experts per lane held in registers as a sorted list (E <= 64 * kRegExperts).
constexpr int kRegExperts = 8;
constexpr int kMaxPerLane = (QMOE_MAX_EXPERTS + kWave - 1) / kWave;  // 64: one bit each

// Order-preserving map of a float to an unsigned integer (-0 folded into +0): the sign
// bit set for positive values, every bit flipped for negative ones. Finite values and
// infinities map above 0, which stands for "no expert".
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ float from_ordered(uint32_t o) {
  return __builtin_bit_cast(float, (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// exp(x) for x <= 0 as 2^(x log2 e) on the hardware exp2: relative error about
// |x| * 2^-24 from the product's rounding plus one ulp (4e-7 at x = -5).
__device__ __forceinline__ float exp_neg(float x) {
  return __builtin_amdgcn_exp2f(x * 1.44269504088896341f);
}

// v with lane `at` (wave-uniform) replaced by the wave-uniform x: the writelane
// intrinsic, declared by its LLVM name (this compiler has no builtin for it).
extern "C" __device__ int qmoe_llvm_writelane(int x, int at, int v) __asm("llvm.amdgcn.writelane.i32");
__device__ __forceinline__ uint32_t write_lane(uint32_t v, uint32_t x, int at) {
  return (uint32_t)qmoe_llvm_writelane((int)x, at, (int)v);
}

// Word 3 of a raw buffer resource (32-bit data format, no swizzle, no index).
constexpr int kRsrcWord3 = 0x00020000;

// x of the lane that DPP control CTRL selects; 0 (no expert) in lanes of rows outside
// ROWS.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xF, true);
}

// Wave-wide maximum (wave-uniform result).
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = umax(x, dpp<0xB1>(x));        // quad_perm [1,0,3,2]
  x = umax(x, dpp<0x4E>(x));        // quad_perm [2,3,0,1]
  x = umax(x, dpp<0x124>(x));       // row_ror:4
  x = umax(x, dpp<0x128>(x));       // row_ror:8: every lane holds its row's maximum
  x = umax(x, dpp<0x142, 0xA>(x));  // row_bcast:15: rows 1, 3 take rows 0, 2
  x = umax(x, dpp<0x143, 0xC>(x));  // row_bcast:31: rows 2, 3 take rows 0-1
  return (uint32_t)__builtin_amdgcn_readlane((int)x, kWave - 1);
}

// Wave-wide sum (wave-uniform result), in the same DPP pattern: 0.0 where a row has no
// source.
__device__ __forceinline__ float wave_sum(float x) {
  auto f = [](uint32_t u) { return __builtin_bit_cast(float, u); };
  auto u = [](float v) { return __builtin_bit_cast(uint32_t, v); };
  x += f(dpp<0xB1>(u(x)));
  x += f(dpp<0x4E>(u(x)));
  x += f(dpp<0x124>(u(x)));
  x += f(dpp<0x128>(u(x)));
  x += f(dpp<0x142, 0xA>(u(x)));
  x += f(dpp<0x143, 0xC>(u(x)));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane((int)u(x), kWave - 1));
}

// Sorts the first C of 8 keys into descending order: the odd-even merge network for 8
// (19 comparators) without the comparators that touch a position >= C. Keys placed
// there below every key of the first C would never move, so the rest sorts the first C
// (12 comparators for 6, 5 for 4: the fewest known for those sizes).
template <int C>
__device__ __forceinline__ void sort_desc(uint64_t (&a)[8]) {
  auto cx = [&](int i, int j) {
    if (j >= C) return;
    const uint64_t hi = a[i] > a[j] ? a[i] : a[j];
    const uint64_t lo = a[i] > a[j] ? a[j] : a[i];
    a[i] = hi;
    a[j] = lo;
  };
  cx(0, 1); cx(2, 3); cx(4, 5); cx(6, 7);
  cx(0, 2); cx(1, 3); cx(4, 6); cx(5, 7);
  cx(1, 2); cx(5, 6);
  cx(0, 4); cx(1, 5); cx(2, 6); cx(3, 7);
  cx(2, 4); cx(3, 5);
  cx(1, 2); cx(3, 4); cx(5, 6);
}

// C: experts per lane, 1..8 held in registers; 0 for more than 512 experts (scanned from
// memory).
template <int C>
__global__ void __launch_bounds__(kRouterThreads)
    topk_softmax_kernel(const float* __restrict__ logits, int32_t T, int32_t E, int32_t k,
                        int32_t renormalize, const int32_t* __restrict__ expert_map,
                        int32_t* __restrict__ ids, float* __restrict__ weights) {
  constexpr bool kWide = C == 0;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int c = kWide ? (E + kWave - 1) / kWave : C;  // experts per lane (E <= 64 c)
  const int e0 = lane * c;                // this lane's first expert
  for (int64_t t = (int64_t)blockIdx.x * kRouterWaves + wave; t < T;
       t += (int64_t)gridDim.x * kRouterWaves) {
    const float* row = logits + t * E;
    float reg[kRegExperts];
    uint32_t s[kRegExperts];  // sorted list: the lane's remaining values, 0 past the end
    uint32_t q = 0;           // nibble n: 7 - (index within the lane) of s[n]
    uint64_t taken = 0;       // wide: bit j set once expert e0 + j is selected
    uint32_t head = 0;        // wide: the lane's best remaining value (0: none) ...
    int head_j = 0;           // ... and its index within the lane
    auto rescan = [&]() {
      head = 0;
      head_j = 0;
      for (int j = 0; j < c; ++j) {
        if (e0 + j < E && !((taken >> j) & 1)) {
          const uint32_t o = ordered_bits(row[e0 + j]);
          if (o > head) {
            head = o;
            head_j = j;
          }
        }
      }
    };
    if constexpr (kWide) {
      rescan();
    } else {
      // value, then 7 - j: equal values keep the lower j first. Past the last expert the
      // value is 0 (below every expert's) and the index is left in place.
      uint64_t key[kRegExperts];
      // The token's row through a buffer resource of E floats: the C loads of a lane share
      // one address register and are all in flight together; loads past the row's end
      // return 0 (the hardware's range check).
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)row, (short)0, E * 4, kRsrcWord3);
#pragma unroll
      for (int j = 0; j < C; ++j)
        reg[j] = __builtin_bit_cast(float,
                                    __builtin_amdgcn_raw_buffer_load_b32(rs, e0 * 4 + j * 4, 0, 0));
#pragma unroll
      for (int j = 0; j < kRegExperts; ++j) {
        const uint32_t o = j < C && e0 + j < E ? ordered_bits(reg[j]) : 0u;
        key[j] = ((uint64_t)o << 32) | (uint32_t)(7 - j);
      }
      sort_desc<C>(key);
#pragma unroll
      for (int j = 0; j < C; ++j) {
        s[j] = (uint32_t)(key[j] >> 32);
        q |= ((uint32_t)key[j] & 15u) << (4 * j);
      }
    }
    float m = 0.f, sel_sum = 0.f;
    uint32_t my_o = 0;  // lane s % 64: the value of slot s of the current batch of 64
    int my_e = 0;       // ... and its expert
    for (int i = 0; i < k; ++i) {
      const uint32_t h = kWide ? head : s[0];
      const uint32_t best = wave_max(h);
      const int win = __builtin_ctzll(__ballot(h == best));  // lowest lane: lowest id
      const int hj = kWide ? head_j : 7 - (int)(q & 15u);
      const int e = win * c + __builtin_amdgcn_readlane(hj, win);
      if constexpr (kWide) {
        if (lane == win) {
          taken |= uint64_t(1) << (e - e0);
          rescan();
        }
      } else {
        // All ones in the winning lane. Kept opaque to the compiler, which would otherwise
        // turn the shift into a dynamically indexed read of the list.
        uint32_t w = lane == win ? ~0u : 0u;
        asm volatile("" : "+v"(w));
#pragma unroll
        for (int j = 0; j + 1 < C; ++j) s[j] = (s[j + 1] & w) | (s[j] & ~w);
        s[C - 1] &= ~w;
        q = ((q >> 4) & w) | (q & ~w);
      }
      if (i == 0) m = from_ordered(best);  // the first selected logit is the largest
      my_o = write_lane(my_o, best, i & (kWave - 1));
      my_e = (int)write_lane((uint32_t)my_e, (uint32_t)e, i & (kWave - 1));
      // Every 64 slots (k > 64 only) the lanes write their slot's id and exp(l - m); the
      // weights are divided below once the denominator is known.
      if ((i & (kWave - 1)) == kWave - 1 && i != k - 1) {
        const int64_t at = t * k + (i & ~(kWave - 1)) + lane;
        const float x = exp_neg(from_ordered(my_o) - m);
        sel_sum += wave_sum(x);
        ids[at] = expert_map ? expert_map[my_e] : my_e;
        weights[at] = x;
      }
    }
    // The last batch of up to 64 slots, from registers.
    const int last = (k - 1) & ~(kWave - 1);
    const bool mine = lane <= k - 1 - last;
    const float x = mine ? exp_neg(from_ordered(my_o) - m) : 0.f;
    sel_sum += wave_sum(x);
    float denom = sel_sum;
    if (!renormalize) {
      float part = 0.f;
      if constexpr (kWide) {
        for (int j = 0; j < c; ++j)
          if (e0 + j < E) part += exp_neg(row[e0 + j] - m);
      } else {
#pragma unroll
        for (int j = 0; j < C; ++j)
          if (e0 + j < E) part += exp_neg(reg[j] - m);
      }
      denom = wave_sum(part);
    }
    if (mine) {
      ids[t * k + last + lane] = expert_map ? expert_map[my_e] : my_e;
      weights[t * k + last + lane] = x / denom;
    }
    // Earlier batches: each lane divides the slots it wrote (program order: its own stores).
    for (int s2 = lane; s2 < last; s2 += kWave) weights[t * k + s2] = weights[t * k + s2] / denom;
  }
}

}  // namespace

hipError_t launch_topk_softmax(const float* logits, int32_t T, int32_t E, int32_t k,
                               int32_t renormalize, const int32_t* expert_map, int32_t* ids,
                               float* weights, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  if (E > kMaxPerLane * kWave) return hipErrorInvalidValue;
  const int64_t blocks = std::min<int64_t>((T + kRouterWaves - 1) / kRouterWaves, 8192);
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kRouterThreads), 0, stream, logits, T,
                       E, k, renormalize, expert_map, ids, weights);
  };
  switch ((E + kWave - 1) / kWave) {
    case 1: launch(topk_softmax_kernel<1>); break;
    case 2: launch(topk_softmax_kernel<2>); break;
    case 3: launch(topk_softmax_kernel<3>); break;
    case 4: launch(topk_softmax_kernel<4>); break;
    case 5: launch(topk_softmax_kernel<5>); break;
    case 6: launch(topk_softmax_kernel<6>); break;
    case 7: launch(topk_softmax_kernel<7>); break;
    case 8: launch(topk_softmax_kernel<8>); break;
    default: launch(topk_softmax_kernel<0>); break;
  }
  return hipGetLastError();
}

}  // namespace qmoe
