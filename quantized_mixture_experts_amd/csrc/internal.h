// Host-side declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qmoe {

// --- router (router.hip) ---------------------------------------------------
// Top-k experts by router logit with softmax weights (renormalized over the k or not),
// ids mapped through expert_map when it is not null. E <= QMOE_MAX_EXPERTS, 1 <= k <= E.
hipError_t launch_topk_softmax(const float* logits, int32_t T, int32_t E, int32_t k,
                               int32_t renormalize, const int32_t* expert_map, int32_t* ids,
                               float* weights, hipStream_t stream);

// --- align (align.hip) -----------------------------------------------------
size_t align_lds_bytes(int32_t E);
hipError_t launch_align(const int32_t* ids, int32_t P, int32_t E, int32_t B, int32_t L, int32_t NB,
                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntp,
                        int32_t* expert_offsets, int32_t tile_m, int32_t* tile_offsets,
                        hipStream_t stream);

// Masked grouped layout: the align outputs from the per-expert counts (no sort), the
// routing weight 1 of every row, and (out != null) cleared output rows past each count.
hipError_t launch_masked_align(const int32_t* masked_m, int32_t E, int32_t max_m, int32_t B,
                               int32_t L, int32_t NB, int32_t* sorted_ids, int32_t* expert_ids,
                               int32_t* ntp, int32_t* expert_offsets, int32_t tile_m,
                               int32_t* tile_offsets, float* ones, uint16_t* out, int32_t H,
                               hipStream_t stream);

// --- elementwise helpers (elementwise.hip) --------------------------------
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t stream);
hipError_t launch_cast_f32_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t stream);
hipError_t launch_fp8_quantize_blocks(const float* v, int64_t R, int64_t C, int32_t br, int32_t bc,
                                      uint8_t* q, float* scale, hipStream_t stream);
hipError_t launch_fp8_quantize_blocks_bf16(const uint16_t* v, int64_t R, int64_t C, int32_t br,
                                           int32_t bc, uint8_t* q, float* scale,
                                           hipStream_t stream);
// Contiguous grouped layout: ones[0, n) = 1 and, when out is not null, output row r
// (H bf16) cleared where ids[r] lies outside [0, E) (a padding row).
hipError_t launch_grouped_routing(const int32_t* ids, int32_t E, int32_t n, float* ones,
                                  uint16_t* out, int32_t H, hipStream_t stream);
// One pair per row (k = 1): out[sid] = bf16(out32[sid]) for every sorted row below
// num_tokens_padded whose pair id sid is below P; other rows of out are not written.
hipError_t launch_cast_routed_rows(const float* out32, const int32_t* sorted_ids,
                                   const int32_t* ntp, int32_t P, int32_t L, int32_t H,
                                   uint16_t* out, hipStream_t stream);

// --- grouped expert GEMMs ---------------------------------------------------
// Routing view shared by the expert GEMMs: segments of the sorted pair list, each a
// multiple of kSegRows rows, expert e owning [offsets[e], offsets[e+1]).
constexpr int kSegRows = 16;

struct Routing {
  const int32_t* sorted_ids;    // [L]
  const int32_t* offsets;       // [E + 1]
  const int32_t* tile_offsets;  // [E + 1], tiles of the prefill GEMM's row-tile size
  const int32_t* expert_ids;    // [L / block_m], expert of each align block (16 or 32 rows)
  const int32_t* ntp;           // rows in use (offsets[E]), on the device
  const float* topk_weights;    // [P]
  int32_t P, k, E, L;
};

// The 4-bit weight formats: INT4 codes with bf16 scales (mx = false), MXFP4 E2M1 codes
// with E8M0 scales (mx = true, s13 / s2 then point at the scale bytes), or NVFP4 E2M1
// codes with E4M3 scales per 16 k and fp32 scales per expert g13 / g2 (mx = nv = true).
struct W4A16Problem {
  const uint16_t* x;  // [T, H] bf16
  uint16_t* xs;       // [L, H] bf16: x gathered by sorted row, operand k order
  const uint8_t* w13;
  const uint16_t* s13;
  const uint8_t* w2;
  const uint16_t* s2;
  uint16_t* h;    // [L, I] bf16
  float* out32;   // [T, H]
  int32_t T, H, I;
  bool mx;
  bool nv = false;
  const float* g13 = nullptr;  // [E]
  const float* g2 = nullptr;   // [E]
  // One pair per row (k = 1, the grouped layouts): the decode gate_up clears only the
  // routed rows of out32 (the others are never read: the cast takes the routed rows).
  bool routed_rows_only = false;
};

struct Fp8Problem {
  const uint8_t* a_q;    // [T, H]
  const float* a_scale;  // [T, H/128]
  const uint8_t* w13;    // [E, 2I, H]
  const float* s13;      // [E, 2I/128, H/128]
  const uint8_t* w2;     // [E, H, I]
  const float* s2;       // [E, H/128, I/128]
  float* h32;            // [L, I]
  uint8_t* hq;           // [L, I]
  float* hs;             // [L, I/128]
  float* out32;          // [T, H]
  int32_t T, H, I;
};

// xs[r] = x[token of sorted row r] in the GEMM operand k order (natural k order for
// the MXFP4 kernels).
hipError_t launch_gather_rows(const uint16_t* x, const Routing& r, const int32_t* ntp, int32_t H,
                              uint16_t* xs, hipStream_t stream, bool natural = false);

// Decode profile: weights streamed once per pass of 16*mb rows of an expert. mb = 2
// (K a multiple of 512) needs align blocks of 32 rows; the general kernel takes mb = 1.
hipError_t launch_w4a16_gateup_stream(const W4A16Problem& p, const Routing& r, int mb,
                                      hipStream_t stream);
// Whether the decode gate_up launch also clears out32 (then no separate clearing launch
// is needed before down).
bool w4a16_stream_zeroes_output(int32_t H);
// Whether the decode gate_up launch with mb blocks per pass reads the activation rows of x
// itself (then the gathered copy xs is not needed).
bool w4a16_stream_reads_rows(int32_t H, int mb);
hipError_t launch_w4a16_down_stream(const W4A16Problem& p, const Routing& r, int mb,
                                    hipStream_t stream);
// Work-groups of a persistent launch: one per compute unit, a multiple of the XCD count.
int persistent_grid();
// Tile kernels with one work-group per tile instead of the persistent grid (tuning).
void set_tiled_one_per_tile(bool on);
// Prefill profile (W4A16 / MXFP4): row tiles of each expert segment on the matrix
// cores, 256 rows, or 128 when the experts hold few rows (w4a16_tiled_rows). Needs H and
// I multiples of 256; align must have produced tile_offsets for tiles of tile_rows rows.
// down writes y[P, H] (fp32 row per pair, not yet weighted) and launch_combine_rows sums
// each token's top-k rows, times their routing weights, into the bf16 output.
bool w4a16_tiled_supported(int32_t H, int32_t I);
int32_t w4a16_tiled_rows(double rows_per_expert);
hipError_t launch_w4a16_gateup_tiled(const W4A16Problem& p, const Routing& r, int tile_rows,
                                     hipStream_t stream);
// out16 != null (one pair per row, k = 1, routing weights 1): down writes bf16(row)
// straight into the output row of each pair instead of fp32 rows into y, so no combine
// pass is needed.
// kslices > 1 (split-K): each output tile's K is split into that many slices (it must
// divide I / 256), slice q writing its partial rows to y + q * P * H (y is [kslices, P, H]).
hipError_t launch_w4a16_down_tiled(const W4A16Problem& p, const Routing& r, int tile_rows,
                                   float* y, hipStream_t stream, uint16_t* out16 = nullptr,
                                   int kslices = 1);
// out[t] = bf16 of the sum over the K slices (in order) of the sums over token t's valid
// slots (in order) of the rows of y ([slices, T*k, H]).
// wts: the routing weights [T * k] to apply to the rows of y, or null when y's rows are
// already weighted.
hipError_t launch_combine_rows(const float* y, const int32_t* topk_ids, const float* wts,
                               int32_t T, int32_t k, int32_t E, int32_t H, uint16_t* out,
                               hipStream_t stream, int32_t slices = 1);

// Prefill profile (block FP8): 128-row tiles; needs H % 256 == 0 and I % 128 == 0 and
// at most 64 k blocks; align must have produced tile_offsets for fp8_tiled_rows() rows.
// gate_up writes hq and hs (h quantized to E4M3 per row and 128 columns), down writes
// y[P, H].
bool fp8_tiled_supported(int32_t H, int32_t I);
int32_t fp8_tiled_rows();
hipError_t launch_fp8_gateup_tiled(const Fp8Problem& p, const Routing& r, hipStream_t stream);
hipError_t launch_fp8_down_tiled(const Fp8Problem& p, const Routing& r, float* y,
                                 hipStream_t stream);

hipError_t launch_fp8_gateup_stream(const Fp8Problem& p, const Routing& r, int mb,
                                    hipStream_t stream);
hipError_t launch_fp8_down_stream(const Fp8Problem& p, const Routing& r, int mb,
                                  hipStream_t stream);

}  // namespace qmoe
