// Elementwise kernels of the MoE FFN path: clearing the fp32 combine buffer, the final
// fp32 -> bf16 rounding of the output, the block E4M3 quantizer, and the per-row routing
// of the grouped layouts.
//
// The quantizer follows "SGLang W8A8 Block FP8 quantization kernel config guide",
// background section: E4M3 (max 448), one scale per block from the block's absmax.
// Per block: scale = max(absmax, 1e-10) / 448, q = e4m3(clamp(v / scale, -448, 448))
// with IEEE fp32 division and round-to-nearest-even (gfx950's v_cvt_pk_fp8_f32 emits
// OCP E4M3FN).
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace qmoe {

namespace {

constexpr int kEwThreads = 256;

__global__ void __launch_bounds__(kEwThreads) zero_f32_kernel(float* __restrict__ p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kEwThreads * 4;
  for (int64_t i = ((int64_t)blockIdx.x * kEwThreads + threadIdx.x) * 4; i < n; i += stride) {
    if (i + 4 <= n) {
      *reinterpret_cast<f32x4*>(p + i) = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
      for (int64_t j = i; j < n; ++j) p[j] = 0.f;
    }
  }
}

__global__ void __launch_bounds__(kEwThreads)
    cast_f32_bf16_kernel(const float* __restrict__ src, uint16_t* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kEwThreads * 4;
  for (int64_t i = ((int64_t)blockIdx.x * kEwThreads + threadIdx.x) * 4; i < n; i += stride) {
    if (i + 4 <= n) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(src + i);
      uint32_t lo = f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
      uint32_t hi = f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
      *reinterpret_cast<uint2*>(dst + i) = make_uint2(lo, hi);
    } else {
      for (int64_t j = i; j < n; ++j) dst[j] = f32_to_bf16(src[j]);
    }
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, kWave));
  return v;
}

__device__ __forceinline__ float load_value(const float* p) { return *p; }
// bf16 bit pattern: the top half of the fp32 value (exact).
__device__ __forceinline__ float load_value(const uint16_t* p) {
  return __builtin_bit_cast(float, (uint32_t)*p << 16);
}

// One wave per [br, bc] block; four blocks per work-group. In: fp32 values or bf16 bit
// patterns (widened exactly, so both give the same codes for the same values).
template <typename In>
__global__ void __launch_bounds__(kEwThreads)
    fp8_quantize_blocks_kernel(const In* __restrict__ v, int64_t R, int64_t C, int32_t br,
                               int32_t bc, uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int64_t nbc = (C + bc - 1) / bc, nbr = (R + br - 1) / br;
  const int64_t blk = (int64_t)blockIdx.x * (kEwThreads / kWave) + threadIdx.x / kWave;
  if (blk >= nbr * nbc) return;
  const int lane = lane_id();
  const int64_t bi = blk / nbc, bj = blk % nbc;
  const int64_t r0 = bi * br, c0 = bj * bc;
  const int rows = (int)min<int64_t>(br, R - r0), cols = (int)min<int64_t>(bc, C - c0);
  const int n = rows * cols;
  float amax = 0.f;
  for (int i = lane; i < n; i += kWave) {
    const int64_t r = r0 + i / cols, c = c0 + i % cols;
    amax = fmaxf(amax, fabsf(load_value(v + r * C + c)));
  }
  amax = wave_max(amax);
  const float s = fmaxf(amax, 1e-10f) / 448.0f;
  if (lane == 0) scale[blk] = s;
  for (int i = lane; i < n; i += kWave) {
    const int64_t r = r0 + i / cols, c = c0 + i % cols;
    const float t = fminf(fmaxf(load_value(v + r * C + c) / s, -448.0f), 448.0f);
    const uint32_t packed = __builtin_amdgcn_cvt_pk_fp8_f32(t, t, 0u, false);
    q[r * C + c] = (uint8_t)(packed & 0xFFu);
  }
}

// Per-row routing of the contiguous grouped layout: every row is one pair of routing
// weight 1; a row whose index lies outside [0, E) is padding, and its output row is
// cleared when `out` is given (the kernels after it write only the valid rows).
__global__ void __launch_bounds__(kEwThreads)
    grouped_routing_kernel(const int32_t* __restrict__ ids, int32_t E, int32_t n,
                           float* __restrict__ ones, uint16_t* __restrict__ out, int32_t H) {
  const int32_t stride = (int32_t)gridDim.x * kEwThreads;
  for (int32_t i = (int32_t)blockIdx.x * kEwThreads + threadIdx.x; i < n; i += stride)
    ones[i] = 1.f;
  if (!out) return;
  const int pieces = H >> 3;
  const int64_t total = (int64_t)n * pieces;
  for (int64_t i = (int64_t)blockIdx.x * kEwThreads + threadIdx.x; i < total;
       i += (int64_t)stride) {
    const int32_t row = (int32_t)(i / pieces);
    const int32_t e = ids[row];
    if (e < 0 || e >= E)
      reinterpret_cast<u32x4*>(out + (size_t)row * H)[i - (int64_t)row * pieces] =
          u32x4{0u, 0u, 0u, 0u};
  }
}

int grid_for(int64_t n) {
  int64_t g = (n / 4 + kEwThreads - 1) / kEwThreads;
  if (g < 1) g = 1;
  if (g > 4096) g = 4096;
  return (int)g;
}

}  // namespace

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_f32_kernel, dim3(grid_for(n)), dim3(kEwThreads), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_cast_f32_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(cast_f32_bf16_kernel, dim3(grid_for(n)), dim3(kEwThreads), 0, stream, src,
                     dst, n);
  return hipGetLastError();
}

namespace {
template <typename In>
hipError_t launch_quantize(const In* v, int64_t R, int64_t C, int32_t br, int32_t bc, uint8_t* q,
                           float* scale, hipStream_t stream) {
  const int64_t nblk = ((R + br - 1) / br) * ((C + bc - 1) / bc);
  if (nblk <= 0) return hipSuccess;
  const int64_t per = kEwThreads / kWave;
  hipLaunchKernelGGL(fp8_quantize_blocks_kernel<In>, dim3((unsigned)((nblk + per - 1) / per)),
                     dim3(kEwThreads), 0, stream, v, R, C, br, bc, q, scale);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_fp8_quantize_blocks(const float* v, int64_t R, int64_t C, int32_t br, int32_t bc,
                                      uint8_t* q, float* scale, hipStream_t stream) {
  return launch_quantize(v, R, C, br, bc, q, scale, stream);
}

hipError_t launch_fp8_quantize_blocks_bf16(const uint16_t* v, int64_t R, int64_t C, int32_t br,
                                           int32_t bc, uint8_t* q, float* scale,
                                           hipStream_t stream) {
  return launch_quantize(v, R, C, br, bc, q, scale, stream);
}

hipError_t launch_grouped_routing(const int32_t* ids, int32_t E, int32_t n, float* ones,
                                  uint16_t* out, int32_t H, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (out && (!ids || H % 8)) return hipErrorInvalidValue;
  const int64_t work = out ? (int64_t)n * (H / 8) : n;
  const int32_t blocks = (int32_t)std::min<int64_t>((work + kEwThreads - 1) / kEwThreads, 1024);
  hipLaunchKernelGGL(grouped_routing_kernel, dim3(blocks), dim3(kEwThreads), 0, stream, ids, E, n,
                     ones, out, H);
  return hipGetLastError();
}

namespace {
// out[sid] = bf16(out32[sid]) for the routed rows of a one-pair-per-row layout (k = 1: the
// pair id is the row), found through the sorted rows below num_tokens_padded; the other
// rows of out are left as they are. One work-group per (16 sorted rows, 1024 columns); a
// thread takes 4 columns of every row, all rows' loads issued before any store.
constexpr int kCastRowCols = 4 * kEwThreads;
__global__ void __launch_bounds__(kEwThreads)
    cast_routed_rows_kernel(const float* __restrict__ out32, const int32_t* __restrict__ sorted_ids,
                            const int32_t* __restrict__ ntp, int32_t P, int32_t H,
                            uint16_t* __restrict__ out) {
  const int rb = blockIdx.x;
  if (rb * 16 >= ntp[0]) return;
  const int c = blockIdx.y * kCastRowCols + 4 * (int)threadIdx.x;
  if (c >= H) return;
  int sid[16];
  f32x4 v[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) sid[m] = sorted_ids[rb * 16 + m];
#pragma unroll
  for (int m = 0; m < 16; ++m)
    v[m] = *reinterpret_cast<const f32x4*>(out32 + (size_t)(sid[m] < P ? sid[m] : 0) * H + c);
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    if (sid[m] >= P) continue;
    const uint32_t lo = (uint32_t)f32_to_bf16(v[m].x) | ((uint32_t)f32_to_bf16(v[m].y) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(v[m].z) | ((uint32_t)f32_to_bf16(v[m].w) << 16);
    *reinterpret_cast<uint2*>(out + (size_t)sid[m] * H + c) = uint2{lo, hi};
  }
}
}  // namespace

hipError_t launch_cast_routed_rows(const float* out32, const int32_t* sorted_ids,
                                   const int32_t* ntp, int32_t P, int32_t L, int32_t H,
                                   uint16_t* out, hipStream_t stream) {
  if (L <= 0 || P <= 0) return hipSuccess;
  if (H % 4) return hipErrorInvalidValue;
  const dim3 grid((L + 15) / 16, (H + kCastRowCols - 1) / kCastRowCols);
  hipLaunchKernelGGL(cast_routed_rows_kernel, grid, dim3(kEwThreads), 0, stream, out32, sorted_ids,
                     ntp, P, H, out);
  return hipGetLastError();
}

}  // namespace qmoe
