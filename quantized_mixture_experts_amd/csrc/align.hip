// Token -> expert align on gfx950.
//
// Sorts the flat (token, slot) pair indices i = t*k + s by expert, stable in i, and
// pads each expert's segment to a multiple of block_m (the sorted_ids / expert_ids /
// num_tokens_padded contract of the indexed MoE kernels in "vLLM x Novita AI: Chord
// W4A16 INT4 MoE Kernel for Kimi K2.x", section "Two kernel families"; padding lives
// in the routing indices, Figure 3).
//
// One work-group per expert, no workspace and no atomics on the output order:
//   1. every work-group builds the full per-expert histogram in LDS (LDS atomics only
//      count; the order they land in does not matter);
//   2. an exclusive scan of the padded counts gives every segment offset;
//   3. work-group e compacts the indices of expert e in ascending order: per pass each
//      thread counts the matches in its run of consecutive indices and a work-group
//      scan orders the runs (deterministic);
//   4. it writes its segment's sentinel padding and expert_ids, and a strided share
//      of the tail past off[E].
// The result is bit-identical to a stable counting sort on the host.
#include "device_common.h"
#include "internal.h"

namespace qmoe {

namespace {

constexpr int kAlignThreads = 256;
constexpr int kAlignWaves = kAlignThreads / kWave;
// Pair ids per thread and pass: all of a pass's loads are in flight at once, so a pass
// costs one memory latency instead of kRun.
constexpr int kRun = 16;

// Exclusive scan of v over the work-group; returns this thread's prefix, writes the
// total to *total. Uses kAlignWaves ints of LDS at `tmp`.
__device__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int n = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += n;
  }
  if (lane == kWave - 1) tmp[wave] = incl;
  __syncthreads();
  int wave_base = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < kAlignWaves; ++w) {
    int tw = tmp[w];
    if (w < wave) wave_base += tw;
    sum += tw;
  }
  __syncthreads();
  *total = sum;
  return wave_base + incl - v;
}

__global__ void __launch_bounds__(kAlignThreads)
    align_kernel(const int32_t* __restrict__ ids, int32_t P, int32_t E, int32_t B, int32_t L,
                 int32_t NB, int32_t* __restrict__ sorted_ids, int32_t* __restrict__ expert_ids,
                 int32_t* __restrict__ num_tokens_padded, int32_t* __restrict__ expert_offsets,
                 int32_t tile_m, int32_t* __restrict__ tile_offsets) {
  extern __shared__ int32_t lds[];
  int32_t* cnt = lds;          // [E]
  int32_t* off = lds + E;      // [E + 1]
  int32_t* toff = off + E + 1; // [E + 1] (tiles of tile_m rows per expert)
  int32_t* tmp = toff + E + 1; // [kAlignWaves]

  const int tid = threadIdx.x;
  const int me = blockIdx.x;

  for (int e = tid; e < E; e += kAlignThreads) cnt[e] = 0;
  __syncthreads();
  for (int base = 0; base < P; base += kAlignThreads * kRun) {
    int v[kRun];
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
      const int i = base + j * kAlignThreads + tid;
      v[j] = i < P ? ids[i] : -1;
    }
#pragma unroll
    for (int j = 0; j < kRun; ++j)
      if ((unsigned)v[j] < (unsigned)E) atomicAdd(&cnt[v[j]], 1);
  }
  __syncthreads();

  // Exclusive scans of padded rows and of row tiles over experts, chunked so one
  // thread owns a contiguous run of experts.
  const int per = (E + kAlignThreads - 1) / kAlignThreads;
  const int e0 = tid * per;
  int my_rows = 0, my_tiles = 0;
  for (int e = e0; e < e0 + per && e < E; ++e) {
    my_rows += (cnt[e] + B - 1) / B * B;
    if (tile_m > 0) my_tiles += (cnt[e] + tile_m - 1) / tile_m;
  }
  int total_rows, total_tiles;
  int rbase = block_exclusive_scan(my_rows, tmp, &total_rows);
  int tbase = block_exclusive_scan(my_tiles, tmp, &total_tiles);
  for (int e = e0; e < e0 + per && e < E; ++e) {
    off[e] = rbase;
    toff[e] = tbase;
    rbase += (cnt[e] + B - 1) / B * B;
    if (tile_m > 0) tbase += (cnt[e] + tile_m - 1) / tile_m;
  }
  if (tid == 0) {
    off[E] = total_rows;
    toff[E] = total_tiles;
  }
  __syncthreads();

  const int seg0 = off[me], seg1 = off[me + 1], c = cnt[me], ntp = off[E];
  if (me == 0) {
    if (tid == 0) num_tokens_padded[0] = ntp;
    if (expert_offsets)
      for (int e = tid; e <= E; e += kAlignThreads) expert_offsets[e] = off[e];
    if (tile_offsets)
      for (int e = tid; e <= E; e += kAlignThreads) tile_offsets[e] = toff[e];
  }
  // Sentinel padding of this segment and this work-group's share of the tail.
  for (int r = seg0 + c + tid; r < seg1; r += kAlignThreads) sorted_ids[r] = P;
  for (int r = ntp + me * kAlignThreads + tid; r < L; r += E * kAlignThreads) sorted_ids[r] = P;
  for (int b = seg0 / B + tid; b < seg1 / B; b += kAlignThreads) expert_ids[b] = me;
  for (int b = ntp / B + me * kAlignThreads + tid; b < NB; b += E * kAlignThreads)
    expert_ids[b] = -1;

  // Stable compaction of this expert's pair indices: per pass each thread takes a run
  // of kRun consecutive indices, counts its matches, and an exclusive scan over the
  // work-group places the runs in order. The next pass's ids are loaded before this
  // pass's scan.
  if (c == 0) return;
  auto load_run = [&](int base, int (&v)[kRun]) {
    const int i0 = base + tid * kRun;
#pragma unroll
    for (int j = 0; j < kRun; ++j) v[j] = (i0 + j < P) ? ids[i0 + j] : -1;
  };
  int cur[kRun], nxt[kRun];
  load_run(0, cur);
  int running = 0;
  for (int base = 0; base < P && running < c; base += kAlignThreads * kRun) {
    load_run(base + kAlignThreads * kRun, nxt);
    int n = 0;
#pragma unroll
    for (int j = 0; j < kRun; ++j) n += (cur[j] == me);
    int all;
    int pos = seg0 + running + block_exclusive_scan(n, tmp, &all);
    const int i0 = base + tid * kRun;
#pragma unroll
    for (int j = 0; j < kRun; ++j)
      if (cur[j] == me) sorted_ids[pos++] = i0 + j;
    running += all;  // the same in every thread: the loop condition is uniform
#pragma unroll
    for (int j = 0; j < kRun; ++j) cur[j] = nxt[j];
  }
}

}  // namespace

size_t align_lds_bytes(int32_t E) {
  return sizeof(int32_t) * ((size_t)E + 2 * ((size_t)E + 1) + kAlignWaves);
}

hipError_t launch_align(const int32_t* ids, int32_t P, int32_t E, int32_t B, int32_t L, int32_t NB,
                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntp,
                        int32_t* expert_offsets, int32_t tile_m, int32_t* tile_offsets,
                        hipStream_t stream) {
  hipLaunchKernelGGL(align_kernel, dim3(E), dim3(kAlignThreads), align_lds_bytes(E), stream, ids, P,
                     E, B, L, NB, sorted_ids, expert_ids, ntp, expert_offsets, tile_m,
                     tile_offsets);
  return hipGetLastError();
}

}  // namespace qmoe
