// W4A16 grouped expert GEMMs, prefill profile (row tiles of 256, MFMA-bound).
//
// Method: BF16 activations times INT4 group-32 weights with BF16 scales, fp32
// accumulation ("vLLM x Novita AI: Chord W4A16 INT4 MoE Kernel for Kimi K2.x": summary;
// "vLLM integration"). With hundreds of routed rows per expert the product is a grouped
// GEMM over the expert segments of the sorted row list (same page, "Two kernel
// families": the indexed path consumes sorted ids, expert ids and the padded count), and
// prefill is bound by the matrix units (same page, "Kernel optimizations"), so the
// kernel is laid out for the matrix cores.
//
// gfx950 mapping. A work-group owns one (row tile of an expert segment, 256 weight rows)
// output tile at a time over eight waves, two per SIMD; the row tile is 256 rows, or 128
// when the experts hold few rows. The launch is persistent (one work-group per compute
// unit, a static XCD-major deal of the tiles): the copy pipeline runs on from one tile
// into the next, so a tile's start and its epilogue do not wait for a pipeline refill. Each wave owns all the tile's rows and 32 weight rows (two
// 16-column MFMA tiles), so every weight element is dequantized exactly once per tile and
// reused for 16 (or 8) row blocks:
//   * activation rows (bf16, tiled layout: the operand of one 16-row block and k group
//     is 1 KB contiguous), weight words and block scales move global -> LDS by buffer
//     loads into LDS: activations through a ring of seven 16 KB stages, six k groups
//     ahead; weight words and scales through per-wave staging one 256-deep block ahead.
//     Completion is tracked with counted vmcnt waits (the compiler does not track these
//     asynchronous LDS writes), and one barrier per k group publishes a stage;
//   * staged weight words are read into registers, and a 4x4 permlane transpose
//     regroups them so that every lane quarter holds its k slice of each group (the B
//     operand layout of v_mfma_f32_16x16x32_bf16);
//   * dequantization folds the scale into the operand: OR-ing a code into fp16 1024.0
//     gives 1024 + code exactly, v_fma_mix_f32 forms (1024 + code) * s - 1032 * s =
//     (code - 8) * s exactly in fp32 (1032 * s is exact for a bf16 s), and
//     v_cvt_pk_bf16_f32 rounds it to the bf16 operand; 16 row blocks share each operand;
//   * 32 accumulator tiles (128 fp32 per lane) per wave.
// gate_up stores h = SiLU(gate) * up (bf16, tiled layout); down stores the routing-
// weighted rows per (token, slot) pair in fp32 and a combine kernel sums the top-k rows
// of every token, so the prefill output does not depend on atomic ordering.
//
// MXFP4 weights (MX = true; E2M1 codes with E8M0 scales per 32 k, the weight-only MXFP4
// format of the "xiaotu-moe" project page, overview): an operand word is one
// v_cvt_scalef32_pk_bf16_fp4 of the code word with the group's power-of-two scale,
// exact, in natural k order (the activation rows and h use the natural-order tiled
// layout); the scales are copied one byte per group. NVFP4 (NV = true): E4M3 scales per
// 16 k (two bytes per group, copied like the INT4 scales) times an fp32 scale per expert;
// an operand word is the pair converted to fp32, multiplied by that scale and rounded
// once to bf16.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace qmoe {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;
constexpr int kColTiles = 2;                      // 16-column MFMA tiles per wave
constexpr int kPieces = kColTiles * 4;            // dequantized operand words per lane and group
constexpr int kStages = 7;                        // LDS ring of activation k groups
constexpr int kGroupsPerBlock = 8;                // k groups per 256-deep weight block

// Tile height TR (rows per work-group tile): 256, or 128 when the experts hold few
// rows (a 256-row tile would be mostly padding).
template <int TR>
struct Tile {
  static constexpr int kRowBlocks = TR / 16;              // 16-row MFMA tiles per wave
  static constexpr int kCopiesPerWave = kRowBlocks / kWaves;  // 1 KB copies per wave and group
  // LDS layout in 16 B units (see the kernel).
  static constexpr int kWBase = kStages * kRowBlocks * kWave;
  static constexpr int kSBase = kWBase + kWaves * 2 * kColTiles * kWave;
  static constexpr int kEBase = kSBase + kWaves * kColTiles * 16;
  // down: the pair id of each of the tile's rows, in two buffers (the current item's, and
  // the next one's, copied while the current item runs), so the epilogue needs one round
  // trip (the routing weights) instead of two per row block.
  static constexpr int kIdUnits = TR / 4;
  static constexpr int kSmemUnits = kEBase + 2 * kIdUnits;
  static_assert(kRowBlocks == kPieces || kRowBlocks == 2 * kPieces,
                "a dequantized piece spans one or two row blocks");
  static_assert(kCopiesPerWave >= 1 && kRowBlocks % kWaves == 0, "copies per wave");
};
// Word 3 of a raw buffer resource (32-bit data format, no swizzle, no index).
constexpr int kRsrcWord3 = 0x00020000;
// Routed rows per expert up to which the tile kernels use 128-row tiles.
constexpr double kSmallTileRows = 136.0;

enum class TEpi { GateUp, Down };

struct TiledArgs {
  const uint16_t* act;          // [L, K] activation rows, tiled layout
  const uint8_t* w;             // [E, N, K/2]
  const uint16_t* s;            // [E, N, K/32] bf16 (INT4) or E8M0 bytes (MXFP4)
  const int32_t* sorted_ids;    // [L]
  const int32_t* offsets;       // [E + 1] segment starts (multiples of 16)
  const int32_t* tile_offsets;  // [E + 1] row tiles per expert (launch's height), exclusive scan
  const float* topk_weights;    // [P]
  uint16_t* h;                  // gate_up output [L, I], tiled layout
  float* y;                     // down output [P, N] per routed pair
  int32_t P, E, K, N, I;
  int32_t col_tiles;            // output column tiles per row tile
  uint32_t act_bytes;           // size of act (L * K * 2 < 2^32, host-checked)
  const float* g = nullptr;     // NVFP4: [E] fp32 scale per expert of this projection
  uint16_t* out16 = nullptr;    // down with one pair per row: bf16 output [P, N] instead of y
  int32_t kslices = 1;          // split-K (down): K slices per output tile; y is [kslices, P, N]
};

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Largest e with toff[e] <= m, for 0 <= m < toff[E] (skips empty experts). Scalar
// loads: toff is written by an earlier launch.
__device__ __forceinline__ int expert_of_tile(const int32_t* toff, int E, int m) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ld_invariant(toff, mid) <= m) lo = mid;
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

// One MFMA accumulating in place. Written as assembly so that the 256 accumulator values
// stay pinned in AGPRs (the register allocator otherwise shuffles them through VGPRs).
// The compiler does not see the operand reads, so the code around it keeps VALU writes
// of MFMA operands at least two instructions away: operands come from LDS reads or
// from VALU work of the previous step, and each step opens with `s_nop 1`.
__device__ __forceinline__ void mfma_acc(f32x4& acc, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Orders every later read of the accumulators after at least 24 wait states following
// the last MFMA (more than an MFMA-write to VALU-read dependency requires). The
// accumulators pass through volatile statements, which keep their program order.
template <int RB>
__device__ __forceinline__ void drain_acc(f32x4 (&acc)[RB][kColTiles]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int m = 0; m < RB; ++m)
#pragma unroll
    for (int t = 0; t < kColTiles; ++t) asm volatile("" : "+a"(acc[m][t]));
}

template <TEpi EPI, bool MX, bool NV, int TR>
__global__ void __launch_bounds__(kThreads) w4a16_tiled_kernel(TiledArgs a) {
  constexpr int kTileRows = TR;
  constexpr int kRowBlocks = Tile<TR>::kRowBlocks;
  constexpr int kCopiesPerWave = Tile<TR>::kCopiesPerWave;
  constexpr int kWBase = Tile<TR>::kWBase;
  constexpr int kSBase = Tile<TR>::kSBase;
  constexpr int kEBase = Tile<TR>::kEBase;
  constexpr int kSmemUnits = Tile<TR>::kSmemUnits;
  // One LDS array (150 KB at TR = 256, 95 KB at 128), in 16 B units:
  //   activation ring [stage][row block][lane], TR / 16 KB per k group;
  //   per wave, the block's weight words [tile][8-row half][row][slot] (whole 128 B
  //   lines, pieces swizzled; see copy_words);
  //   per wave, the block's scales [tile][row] (16 B = eight groups per weight row).
  //   down: two buffers of the tile rows' pair ids (TR * 4 B each).
  // A single object also keeps the compiler from adding conservative waits between the
  // asynchronous copies and the reads of other staging areas.
  __shared__ u32x4 smem[kSmemUnits];
  auto a_at = [&](int st, int rb) { return &smem[(st * kRowBlocks + rb) * kWave]; };
  auto w_at = [&](int wv, int t, int h8) {
    return &smem[kWBase + ((wv * kColTiles + t) * 2 + h8) * kWave];
  };
  auto s_at = [&](int wv, int t) { return &smem[kSBase + (wv * kColTiles + t) * 16]; };

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int col = lane & 15, quad = lane >> 4;

  // Persistent schedule. The grid is at most one work-group per compute unit; the items
  // (row tile, column tile, K slice; with a.kslices > 1, split-K for down, the slices of
  // an output tile are neighbours) are dealt XCD-major: XCD x owns the contiguous range
  // [x per, (x + 1) per), and its wpx work-groups take every wpx-th item of it, so the
  // items that run at once on one XCD are neighbours sharing activation rows in its L2.
  const int total = ld_invariant(a.tile_offsets, a.E) * a.col_tiles * a.kslices;
  const int wpx = gridDim.x / kNumXcd;
  const int xcd = blockIdx.x % kNumXcd;
  const int per = (total + kNumXcd - 1) / kNumXcd;
  const int iend = min(total, (xcd + 1) * per);
  int item_k = xcd * per + blockIdx.x / kNumXcd;
  if (item_k >= iend) return;
  const int K = a.K, KG = K >> 5;
  // An item's 256-deep weight blocks: all of K, or its slice. Offsets below keep the
  // full-K strides and start at the slice's first block; the loop runs over the slice.
  const int nblocks = (K >> 8) / a.kslices;
  const int nsteps = nblocks * kGroupsPerBlock;

  // Weight row of tile t for column c of this wave in column tile ctile.
  auto weight_row = [&](int ctile, int t, int c) {
    if constexpr (EPI == TEpi::GateUp) {
      const int j = ctile * 128 + wave * (kColTiles * 8) + (t % (kColTiles / 2)) * 16 + c;
      return (t < kColTiles / 2) ? j : a.I + j;
    } else {
      return ctile * 256 + wave * (kColTiles * 16) + t * 16 + c;
    }
  };
  // Byte offsets stay 32-bit (host-checked). Weight words: lane (col, quad) takes 16 B of
  // row col at quarter `quad` of a 64 B half line. Scales: lane l takes word l % 4 of the
  // 16 B (eight groups) of row l / 4. MXFP4 scales are one byte per group: the block's
  // eight are words 0 and 1 of the 16 B window (words 2 and 3 hold the next block's, or
  // zeros past the buffer, unused). A copy's vector offset is a fixed per-lane part plus
  // its item's uniform part (the buffer's range check covers both); the scalar offset
  // is the step's position within the item.
  constexpr uint32_t kScaleBytes = (MX && !NV) ? 1u : 2u;
  const int hsh = NV ? 8 * (quad >> 1) : 0;  // NVFP4: byte of this lane's 16-k half
  const uint32_t a_lane = (uint32_t)lane * 16u;
  // Weight words are copied a whole 128 B line (one 256-deep block of a row) per eight
  // lanes: lane l takes row 8 h8 + l / 8 of the tile and puts the line's 16 B piece p
  // into LDS slot p ^ sw(l / 8) ^ 4 h8 of that row. (With the MFMA's lane order, sixteen
  // rows across sixteen lanes, the address path moves a third of the bytes per clock.)
  // Lane (col, quad) then reads piece 4 hf + quad of row col: the four lanes of a row
  // take four neighbouring pieces, so sw moves a row's lowest bit to the top of the
  // mask, which puts neighbouring rows' pieces in opposite halves of the line's banks.
  // (Measured: the MFMA-order reads of this layout have no bank conflicts.)
  auto sw = [](int r) { return ((r & 1) << 2) | (r >> 1); };
  uint32_t w_lane[2];
#pragma unroll
  for (int h8 = 0; h8 < 2; ++h8)
    w_lane[h8] = (uint32_t)(8 * h8 + (lane >> 3)) * (uint32_t)(K >> 1) +
                 16u * (uint32_t)((lane & 7) ^ sw(lane >> 3) ^ (4 * h8));
  int w_rd[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
    w_rd[hf] =
        (col >> 3) * kWave + (col & 7) * 8 + ((4 * hf + quad) ^ sw(col & 7) ^ (4 * (col >> 3)));
  const uint32_t s_lane = (uint32_t)(lane >> 2) * (uint32_t)KG * kScaleBytes + 4u * (lane & 3);
  const __amdgpu_buffer_rsrc_t ars =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.act, (short)0, (int)a.act_bytes, kRsrcWord3);

  // What the copies need of an item: the uniform parts of their offsets (weight tile 1
  // lies a fixed distance past tile 0: I rows for gate_up, 16 for down) and its expert's
  // weight and scale buffers. What the epilogue needs of the current item: Rows.
  const uint32_t tile1_rows = EPI == TEpi::GateUp ? (uint32_t)a.I : 16u;
  const uint32_t w_tile1 = tile1_rows * (uint32_t)(K >> 1);
  const uint32_t s_tile1 = tile1_rows * (uint32_t)KG * kScaleBytes;
  struct Src {
    uint32_t abase[kCopiesPerWave], wbase, sbase;
    const uint8_t* wb;  // the expert's weight words and scales
    const uint8_t* sb;
    float gsc;  // NVFP4: the expert's global scale
  };
  const int w_records = (int)((uint32_t)a.N * (uint32_t)(K >> 1));
  const int s_records = (int)((uint32_t)a.N * (uint32_t)KG * kScaleBytes);
  struct Rows {
    int row0, rb_last, ctile, slice;
  };
  auto item_rows = [&](int ik, int& e) {
    Rows it;
    const int item = ik / a.kslices;
    it.slice = ik - item * a.kslices;
    const int rtile = item / a.col_tiles;
    it.ctile = item - rtile * a.col_tiles;
    e = expert_of_tile(a.tile_offsets, a.E, rtile);
    it.row0 = ld_invariant(a.offsets, e) + (rtile - ld_invariant(a.tile_offsets, e)) * kTileRows;
    it.rb_last = (ld_invariant(a.offsets, e + 1) >> 4) - 1;
    return it;
  };
  auto item_src = [&](const Rows& it, int e) {
    Src c;
    const uint32_t kb_first = (uint32_t)(it.slice * nblocks);
#pragma unroll
    for (int i = 0; i < kCopiesPerWave; ++i) {
      const int rb = min((it.row0 >> 4) + wave * kCopiesPerWave + i, it.rb_last);
      c.abase[i] = (uint32_t)rb * (uint32_t)(KG * 1024) + kb_first * kGroupsPerBlock * 1024u;
    }
    const uint32_t wr = (uint32_t)weight_row(it.ctile, 0, 0);
    c.wbase = wr * (uint32_t)(K >> 1) + kb_first * 128u;
    c.sbase = wr * (uint32_t)KG * kScaleBytes + kb_first * kGroupsPerBlock * kScaleBytes;
    c.wb = a.w + (size_t)e * a.N * (size_t)(K >> 1);
    c.sb = reinterpret_cast<const uint8_t*>(a.s) + (size_t)e * a.N * (size_t)KG * kScaleBytes;
    c.gsc = 1.f;
    if constexpr (NV)
      c.gsc = __builtin_bit_cast(float, ld_invariant(reinterpret_cast<const int32_t*>(a.g), e));
    return c;
  };
  // cur: the item being computed; nrows / nsrc: the next one of this work-group. The
  // copies read from cp: cur's source until step 1 of cur's last block, from there on
  // (the first copy of a group or block past cur's end) the next item's, with goff and
  // boff the group and block that item starts at in cur's numbering. Without a next item
  // cp stays and the copies past the end repeat cur's last group and block.
  int e_cur = 0, e_nxt = 0;
  Rows cur = item_rows(item_k, e_cur);
  Src cp = item_src(cur, e_cur);
  float gsc_cur = cp.gsc;
  int goff = 0, boff = 0;
  bool has_next = item_k + wpx < iend;
  Rows nrows = cur;
  Src nsrc = cp;
  if (has_next) {
    nrows = item_rows(item_k + wpx, e_nxt);
    nsrc = item_src(nrows, e_nxt);
  }

  // All global reads of the loop are asynchronous LDS copies whose completion this code
  // tracks itself with vmcnt (the compiler does not count these). They are issued in a
  // fixed order and never skipped, so the counts below hold at every step: past the end
  // of an item they fetch the next item's first groups and weight block, or, after the
  // work-group's last item, repeat the last group or block. Per 8-group block and wave:
  // kCopiesPerWave activation copies every step, the next block's weight words at j = 1
  // (2 kColTiles: two 8-row halves per tile), its scales at j = 2 (kColTiles).
  // Anything else issued between them (the epilogue's stores and loads, the next item's
  // pair ids) is younger than the copies a later wait counts on; since loads complete in
  // issue order, it can only make such a wait wait longer, never too little. Reads past a
  // buffer's size return zeros.
  // Activation group gg of cur's numbering (gg >= nsteps: the next item's).
  auto copy_act = [&](int gg, int st_, int i) {
    const int gl = min(gg - goff, nsteps - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        ars, (__attribute__((address_space(3))) void*)a_at(st_, wave * kCopiesPerWave + i), 16,
        (int)(a_lane + cp.abase[i]), gl * 1024, 0, 0);
  };
  // Weight words and scales of block kb of cur's numbering (kb >= nblocks: the next
  // item's).
  auto copy_words = [&](int kb, int t, int h8) {
    const int kl = min(kb - boff, nblocks - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        __builtin_amdgcn_make_buffer_rsrc((void*)cp.wb, (short)0, w_records, kRsrcWord3),
        (__attribute__((address_space(3))) void*)w_at(wave, t, h8), 16,
        (int)(w_lane[h8] + cp.wbase + (t ? w_tile1 : 0u)), kl * 128, 0, 0);
  };
  auto copy_scale = [&](int kb, int t) {
    const int kl = min(kb - boff, nblocks - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        __builtin_amdgcn_make_buffer_rsrc((void*)cp.sb, (short)0, s_records, kRsrcWord3),
        (__attribute__((address_space(3))) void*)s_at(wave, t), 4,
        (int)(s_lane + cp.sbase + (t ? s_tile1 : 0u)), kl * 8 * (int)kScaleBytes, 0, 0);
  };
  auto copy_group = [&](int g, int st_) {
#pragma unroll
    for (int i = 0; i < kCopiesPerWave; ++i) copy_act(g, st_, i);
  };
  auto copy_block_words = [&](int kb) {
#pragma unroll
    for (int t = 0; t < kColTiles; ++t)
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) copy_words(kb, t, h8);
  };
  auto copy_scales = [&](int kb) {
#pragma unroll
    for (int t = 0; t < kColTiles; ++t) copy_scale(kb, t);
  };
  // down: the pair ids of an item's rows (row0 + 64 wave + lane, clamped into the segment;
  // rows past it are not stored) into id buffer buf, by the first TR / 64 waves.
  auto copy_ids = [&](const Rows& it, int buf) {
    if (EPI == TEpi::Down && wave < kTileRows / kWave) {
      const int r = min(it.row0 + wave * kWave + lane, it.rb_last * 16 + 15);
      __builtin_amdgcn_global_load_lds(
          (const void*)(a.sorted_ids + r),
          (__attribute__((address_space(3))) void*)&smem[kEBase + buf * Tile<TR>::kIdUnits +
                                                         wave * (kWave / 4)],
          4, 0, 0);
    }
  };

  f32x4 acc[kRowBlocks][kColTiles];
#pragma unroll
  for (int m = 0; m < kRowBlocks; ++m)
#pragma unroll
    for (int t = 0; t < kColTiles; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint32_t mask = opaque_sgpr(0x000F000Fu);
  const uint32_t magic = opaque_vgpr(0x64006400u);

  // tw: the current half block's words, transposed so that word g of lane quarter q is
  // slice q of group g. scur: the current block's scales. Step g runs the MFMAs of group
  // g on operands dequantized during step g-1 (buffer g % 2) and dequantizes group g+1
  // into the other buffer, spread between the MFMAs so the VALU work overlaps them.
  // wnext / snext: staged words or scales read from LDS one step before they are used.
  uint32_t tw[kColTiles][4];
  u32x4 scur[kColTiles];
  u32x4 bq[2][kColTiles];
  u32x4 wnext[kColTiles], snext[kColTiles];
  auto read_staged_half = [&](int hf) {
#pragma unroll
    for (int t = 0; t < kColTiles; ++t) wnext[t] = w_at(wave, t, 0)[w_rd[hf]];
  };
  auto read_staged_scales = [&]() {
#pragma unroll
    for (int t = 0; t < kColTiles; ++t) snext[t] = s_at(wave, t)[col];
  };
  auto take_half = [&]() {
#pragma unroll
    for (int t = 0; t < kColTiles; ++t) {
      tw[t][0] = wnext[t].x;
      tw[t][1] = wnext[t].y;
      tw[t][2] = wnext[t].z;
      tw[t][3] = wnext[t].w;
      transpose4_rows(tw[t]);
    }
  };
  auto wait_lds_reads = [] {
    // lgkmcnt(0), other counters left alone
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
  };
  auto next_stage = [](int s_) { return s_ == kStages - 1 ? 0 : s_ + 1; };

  // Issue schedule (per wave). Step g issues, after its barrier (one copy per MFMA of the
  // last three row blocks), the copies of activation group g + kStages into the stage
  // group g has just released (kCopiesPerWave); at block position j = 1 the next block's
  // weight words (whole lines, 2 kColTiles), at j = 2 its scales (kColTiles). The staged
  // words are read into registers one step or more before use (j = 0: second half of
  // this block, before the copies at j = 1 overwrite it; j = 6: first half and scales of
  // the next block). The prologue issues the same sequence for the steps before group 0
  // of the work-group's first item; a later item's first groups and block come from the
  // previous item's last steps.
  // The first item's pair ids: older than every copy below, so the waits below cover it.
  copy_ids(cur, 0);
  copy_group(0, 0);  // step -7 (j = 1)
  copy_block_words(0);
  copy_group(1, 1);  // step -6 (j = 2)
  copy_scales(0);
  copy_group(2, 2);  // step -5
  copy_group(3, 3);  // step -4
  copy_group(4, 4);  // step -3
  copy_group(5, 5);  // step -2 (j = 6): younger than the scales are copies 2..5
  wait_vmcnt<4 * kCopiesPerWave>();
  read_staged_half(0);
  read_staged_scales();
  // step -1 (j = 7): group 0's copies; younger are the words, the scales and copies 1..5
  wait_vmcnt<3 * kColTiles + 5 * kCopiesPerWave>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  copy_group(6, 6);
  __builtin_amdgcn_sched_barrier(0);
  // Activation operands are read from LDS in groups of four row blocks, a whole group
  // ahead, into two register sets: the compiler waits for all outstanding LDS reads
  // (lgkmcnt(0)) before the first use of each group, and by then they have landed.
  u32x4 ra[2][4];
  // An operand set stays allocated until it is refilled: otherwise the register allocator
  // hands a just-read operand register to the next dequantized weights, and every such
  // write needs a wait state after the MFMA that read it.
  auto keep_live = [](const u32x4 (&v)[4]) {
    asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]));
  };
  {
    const u32x4* as0 = a_at(0, 0) + lane;
#pragma unroll
    for (int r = 0; r < 4; ++r) ra[0][r] = as0[r * kWave];
  }
  take_half();
#pragma unroll
  for (int t = 0; t < kColTiles; ++t) scur[t] = snext[t];
#pragma unroll
  for (int p = 0; p < kPieces; ++p) {
    const int t = p >> 2, i = p & 3;
    if constexpr (NV) {
      bq[0][t][i] = nvfp4_pair(tw[t][0], e4m3_low(scur[t][0] >> hsh) * gsc_cur, i);
      continue;
    } else if constexpr (MX) {
      bq[0][t][i] = fp4_pair(tw[t][0], e8m0_scale(scur[t][0]), i);
      continue;
    }
    const float sc = bf16_lo(scur[t][0]);
    const uint32_t pr = ((tw[t][0] >> (4 * i)) & mask) | magic;
    const f16x2 hv = __builtin_bit_cast(f16x2, pr);
    const f32x2 f = {__builtin_fmaf((float)hv.x, sc, -1032.0f * sc),
                     __builtin_fmaf((float)hv.y, sc, -1032.0f * sc)};
    bq[0][t][i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
  }

  int st = 0;    // stage of group g
  int ibuf = 0;  // id buffer of cur
  for (;;) {
  for (int kb = 0; kb < nblocks; ++kb) {
    auto step = [&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int g = kb * kGroupsPerBlock + j;
      const int jn = (j + 1) & 7;
      // From step 1 of the last block on, the copies fetch the next item's data.
      if (j == 1 && kb == nblocks - 1 && has_next) {
        cp = nsrc;
        goff = nsteps;
        boff = nblocks;
      }
      // NVFP4: the global scale of the item whose group jn this step dequantizes (the
      // last step of an item dequantizes the next item's group 0).
      const float gsc = (j == 7 && kb == nblocks - 1) ? cp.gsc : gsc_cur;
      // Operand registers written by VALU instructions at the end of the last step.
      asm volatile("s_nop 1");
      if (j == 3) {
        take_half();
      } else if (j == 7) {
        take_half();
#pragma unroll
        for (int t = 0; t < kColTiles; ++t) scur[t] = snext[t];
      }
      __builtin_amdgcn_sched_barrier(0);
      const u32x4* as = a_at(st, 0) + lane;
      const int stn = next_stage(st);
      const u32x4* asn = a_at(stn, 0) + lane;
      const u32x4 (&bc)[kColTiles] = bq[j & 1];
      u32x4 (&bn)[kColTiles] = bq[(j + 1) & 1];
      float sc = 0.f, cc = 0.f;
      uint32_t pr = 0;
      float flo = 0.f, fhi = 0.f;
      // Row block m: its four MFMAs, each followed by about a quarter of piece m of the
      // next group's operands (fenced, so the VALU work issues while the matrix pipe is
      // busy); the next four row blocks' operands are requested after each group's
      // first MFMA.
#pragma unroll
      for (int m = 0; m < kRowBlocks; ++m) {
        const int q = m >> 2, r = m & 3;
        // With 16 row blocks, row blocks 2p and 2p + 1 carry piece p of the next group's
        // operands: its scale and codes, the two products, then the conversion (behind the
        // next piece's mask, since a bf16 conversion right behind an MFMA needs a wait
        // state). With 8 row blocks, row block p carries all of piece p.
        constexpr bool kTwoPerPiece = kRowBlocks == 2 * kPieces;
        const int p = kTwoPerPiece ? m >> 1 : m, odd = kTwoPerPiece ? m & 1 : 0;
        const int t = p >> 2, i = p & 3;
        const u32x4& a0 = ra[q & 1][r];
        // This step's copies, issued after the barrier one per MFMA of row blocks
        // kRowBlocks-3 .. kRowBlocks-1 (a run of copies stalls the wave), in a fixed
        // order: activation group g + kStages, then at j = 1 the next block's weight
        // words, at j = 2 its scales.
        auto copy_slot = [&](int k) {
          if (m < kRowBlocks - 3) return;
          const int c = (m - (kRowBlocks - 3)) * kColTiles + k;
          if (c < kCopiesPerWave) {
            copy_act(g + kStages, st, c);
          } else if (c < kCopiesPerWave + 2 * kColTiles) {
            const int w = c - kCopiesPerWave;
            if (j == 1) copy_words(kb + 1, w >> 1, w & 1);
            else if (j == 2 && w < kColTiles) copy_scale(kb + 1, w);
          }
        };
        mfma_acc(acc[m][0], a0, bc[0]);
        __builtin_amdgcn_sched_barrier(0);
        copy_slot(0);
        // After the group's first MFMA, so that the wait before it does not cover them.
        if (r == 0 && q < kRowBlocks / 4 - 1) {
          keep_live(ra[(q + 1) & 1]);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) ra[(q + 1) & 1][rr] = as[(4 * (q + 1) + rr) * kWave];
        }
        uint32_t shv = 0;
        if constexpr (NV) {
          // The lane's scale for group jn (byte 2 jn + its half), at the tile's first piece.
          if (!odd && i == 0) sc = e4m3_low(scur[t][jn >> 1] >> (16 * (jn & 1) + hsh)) * gsc;
        } else if constexpr (MX) {
          // The tile's scale for group jn (byte jn of the block), at its first piece.
          if (!odd && i == 0) sc = e8m0_scale(scur[t][jn >> 2] >> (8 * (jn & 3)));
        } else if (!kTwoPerPiece) {
          if (i == 0) {
            const uint32_t sw = scur[t][jn >> 1];
            sc = (jn & 1) ? bf16_hi(sw) : bf16_lo(sw);
            cc = -1032.0f * sc;
          }
          pr = ((tw[t][jn & 3] >> (4 * i)) & mask) | magic;
        } else if (!odd) {
          if (i == 0) {
            const uint32_t sw = scur[t][jn >> 1];
            sc = (jn & 1) ? bf16_hi(sw) : bf16_lo(sw);
            cc = -1032.0f * sc;
          }
          if (m == 0) pr = (tw[0][jn & 3] & mask) | magic;
        } else if (p + 1 < kPieces) {
          shv = tw[(p + 1) >> 2][jn & 3] >> (4 * ((p + 1) & 3));
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_acc(acc[m][1], a0, bc[1]);
        __builtin_amdgcn_sched_barrier(0);
        copy_slot(1);
        if constexpr (NV) {
          if (odd || !kTwoPerPiece) bn[t][i] = nvfp4_pair(tw[t][jn & 3], sc, i);
        } else if constexpr (MX) {
          if (odd || !kTwoPerPiece) bn[t][i] = fp4_pair(tw[t][jn & 3], sc, i);
        } else if (!kTwoPerPiece) {
          const f16x2 hv = __builtin_bit_cast(f16x2, pr);
          const f32x2 f = {__builtin_fmaf((float)hv.x, sc, cc), __builtin_fmaf((float)hv.y, sc, cc)};
          bn[t][i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
        } else if (!odd) {
          const f16x2 hv = __builtin_bit_cast(f16x2, pr);
          flo = __builtin_fmaf((float)hv.x, sc, cc);
          fhi = __builtin_fmaf((float)hv.y, sc, cc);
        } else {
          if (p + 1 < kPieces) pr = (shv & mask) | magic;
          const f32x2 f = {flo, fhi};
          bn[t][i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
        }
        __builtin_amdgcn_sched_barrier(0);
        if (m == kRowBlocks - 4) {
          // Every read of this stage has been issued. Once they have completed and
          // group g+1's copies have landed (vmcnt: at most the younger copies of groups
          // g+2 .. g+6 and the weight copies of the last six steps, positions j+2 .. j+7
          // of the block, are pending; loads complete in issue order), the barrier lets
          // group g + kStages reuse this stage, and the next step's first reads go out
          // while the last row blocks' MFMAs run (register set 0 is free again).
          wait_lds_reads();
          constexpr int kLater = (kStages - 2) * kCopiesPerWave;
          constexpr int w1 = 2 * kColTiles, w2 = kColTiles;
          constexpr int kPrev = w1 + w2 - ((j == 1 || j == 0) ? w1 : 0) -
                                ((j == 2 || j == 1) ? w2 : 0);
          wait_vmcnt<kLater + kPrev>();
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
          // After the item's first barrier every wave has finished the previous item's
          // epilogue, which read the id buffer that the next item's pair ids go to.
          if (j == 0 && kb == 0 && has_next) copy_ids(nrows, ibuf ^ 1);
          // (This step's copies follow, spread over the next MFMAs.)
          if (j == 0) {
            // Second half of this block's words (copied at j = 1 of the last block;
            // younger are its scales and six steps of activation copies), read before
            // the copies at j = 1, behind the next barrier, overwrite them.
            wait_vmcnt<6 * kCopiesPerWave + kColTiles>();
            read_staged_half(1);
          } else if (j == 6) {
            // Next block's first half and scales (copied at j = 1 and 2): younger are
            // three steps of activation copies.
            wait_vmcnt<3 * kCopiesPerWave>();
            read_staged_half(0);
            read_staged_scales();
          }
          keep_live(ra[0]);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) ra[0][rr] = asn[rr * kWave];
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      st = stn;
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
    step(std::integral_constant<int, 4>{});
    step(std::integral_constant<int, 5>{});
    step(std::integral_constant<int, 6>{});
    step(std::integral_constant<int, 7>{});
  }
  // The matrix-core results must be settled before ordinary instructions read them.
  drain_acc(acc);

  // Epilogue of cur. Lane (col, quad) holds rows 4*quad + r of each 16-row block, column
  // col.
  if constexpr (EPI == TEpi::GateUp) {
#pragma unroll
    for (int m = 0; m < kRowBlocks; ++m) {
      const int rb = (cur.row0 >> 4) + m;
      if (rb > cur.rb_last) break;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tp = 0; tp < kColTiles / 2; ++tp) {
        const int j = cur.ctile * 128 + wave * (kColTiles * 8) + tp * 16 + col;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gv = acc[m][tp][r], uv = acc[m][tp + kColTiles / 2][r];
          a.h[tiled_offset<MX>(rb * 16 + 4 * quad + r, j, a.I)] = f32_to_bf16(silu_f32(gv) * uv);
        }
      }
    }
  } else {
    // Rows of the pairs (ids from LDS, four row blocks per read batch), unweighted: the
    // combine applies the routing weights, so the epilogue makes no global reads.
    const int* ep = reinterpret_cast<const int*>(&smem[kEBase + ibuf * Tile<TR>::kIdUnits]);
#pragma unroll
    for (int m0 = 0; m0 < kRowBlocks; m0 += 4) {
      if ((cur.row0 >> 4) + m0 > cur.rb_last) break;
      u32x4 pv[4];
#pragma unroll
      for (int mm = 0; mm < 4; ++mm)
        pv[mm] = *reinterpret_cast<const u32x4*>(ep + (m0 + mm) * 16 + 4 * quad);
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        const int m = m0 + mm;
        if ((cur.row0 >> 4) + m > cur.rb_last) break;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int pair = (int)pv[mm][r];
          if (pair < a.P) {
            if (a.out16) {
              // one pair per row, of routing weight 1: the pair's output row is final
              uint16_t* orow = a.out16 + (size_t)pair * a.N;
#pragma unroll
              for (int t = 0; t < kColTiles; ++t)
                orow[weight_row(cur.ctile, t, col)] = f32_to_bf16(acc[m][t][r]);
            } else {
              float* yrow = a.y + ((size_t)cur.slice * a.P + pair) * a.N;
#pragma unroll
              for (int t = 0; t < kColTiles; ++t) yrow[weight_row(cur.ctile, t, col)] = acc[m][t][r];
            }
          }
        }
      }
    }
  }
  if (!has_next) break;
  // On to the next item: its first groups, block and pair ids are already on their way.
  item_k += wpx;
  cur = nrows;
  gsc_cur = cp.gsc;
  goff = 0;
  boff = 0;
  ibuf ^= 1;
  has_next = item_k + wpx < iend;
  if (has_next) {
    nrows = item_rows(item_k + wpx, e_nxt);
    nsrc = item_src(nrows, e_nxt);
  }
#pragma unroll
  for (int m = 0; m < kRowBlocks; ++m)
#pragma unroll
    for (int t = 0; t < kColTiles; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // The next item's first operands, read by the last step, are read again here so that
  // they hold no registers during the epilogue (st is the stage of its group 0).
  {
    const u32x4* as0 = a_at(st, 0) + lane;
#pragma unroll
    for (int r = 0; r < 4; ++r) ra[0][r] = as0[r * kWave];
  }
  }
  // No copy may still be landing in LDS when the work-group's LDS is released.
  wait_vmcnt<0>();
}

// out[t, :] = bf16(sum over the K slices q (in order) of the sum over the valid slots s of
// token t (in slot order) of w[t*k + s] * y[q, t*k + s, :]), w the routing weights (or 1
// when wts is null: rows already weighted). A thread owns 8 columns of one token; the
// rows of up to kSlotBatch slots of a slice are requested before any is summed.
constexpr int kCombineThreads = 256;
constexpr int kSlotBatch = 8;

__global__ void __launch_bounds__(kCombineThreads)
    combine_rows_kernel(const float* __restrict__ y, const int32_t* __restrict__ ids,
                        const float* __restrict__ wts, int32_t T, int32_t k, int32_t E,
                        int32_t H, int32_t slices, uint16_t* __restrict__ out) {
  const int64_t slice_stride = (int64_t)T * k * H;
  const int chunks = H >> 3;
  const int64_t items = (int64_t)T * chunks;
  for (int64_t i = (int64_t)blockIdx.x * kCombineThreads + threadIdx.x; i < items;
       i += (int64_t)gridDim.x * kCombineThreads) {
    const int64_t t = i / chunks;
    const int c = (int)(i - t * chunks) * 8;
    f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < slices; ++q) {
      const float* yq = y + q * slice_stride;
      for (int s0 = 0; s0 < k; s0 += kSlotBatch) {
        f32x4 vl[kSlotBatch], vh[kSlotBatch];
        float wv[kSlotBatch];
        bool ok[kSlotBatch];
#pragma unroll
        for (int s = 0; s < kSlotBatch; ++s) {
          const int64_t pair = t * k + s0 + s;
          const int id = (s0 + s < k) ? ids[pair] : -1;
          ok[s] = id >= 0 && id < E;
          wv[s] = (wts && ok[s]) ? wts[pair] : 1.f;
          const float* row = yq + (ok[s] ? pair : 0) * H + c;
          vl[s] = *reinterpret_cast<const f32x4*>(row);
          vh[s] = *reinterpret_cast<const f32x4*>(row + 4);
        }
#pragma unroll
        for (int s = 0; s < kSlotBatch; ++s) {
          if (ok[s]) {
            if (wts) {
              lo += wv[s] * vl[s];
              hi += wv[s] * vh[s];
            } else {
              lo += vl[s];
              hi += vh[s];
            }
          }
        }
      }
    }
    u32x4 o;
    o.x = (uint32_t)f32_to_bf16(lo.x) | ((uint32_t)f32_to_bf16(lo.y) << 16);
    o.y = (uint32_t)f32_to_bf16(lo.z) | ((uint32_t)f32_to_bf16(lo.w) << 16);
    o.z = (uint32_t)f32_to_bf16(hi.x) | ((uint32_t)f32_to_bf16(hi.y) << 16);
    o.w = (uint32_t)f32_to_bf16(hi.z) | ((uint32_t)f32_to_bf16(hi.w) << 16);
    *reinterpret_cast<u32x4*>(out + t * H + c) = o;
  }
}

std::atomic<bool> g_one_per_tile{false};

template <TEpi EPI, int TR>
void launch_tiled_rows(const TiledArgs& a, int64_t items, bool mx, bool nv, hipStream_t stream) {
  // persistent: at most one work-group per compute unit, a multiple of the XCD count
  // (or, for tuning, one per tile: then each work-group runs a single item)
  const int all = xcd_major_grid((int)items);
  const dim3 grid(g_one_per_tile.load() ? all : std::min(all, persistent_grid()));
  if (nv)
    hipLaunchKernelGGL((w4a16_tiled_kernel<EPI, true, true, TR>), grid, dim3(kThreads), 0, stream,
                       a);
  else if (mx)
    hipLaunchKernelGGL((w4a16_tiled_kernel<EPI, true, false, TR>), grid, dim3(kThreads), 0, stream,
                       a);
  else
    hipLaunchKernelGGL((w4a16_tiled_kernel<EPI, false, false, TR>), grid, dim3(kThreads), 0,
                       stream, a);
}

template <TEpi EPI>
hipError_t launch_tiled(const TiledArgs& a, int64_t P, int E, int tile_rows, bool mx, bool nv,
                        hipStream_t stream) {
  if (tile_rows != 128 && tile_rows != 256) return hipErrorInvalidValue;
  // at most this many row tiles, times the column tiles and K slices of each
  const int64_t items = (P / tile_rows + E) * a.col_tiles * a.kslices;
  if (items <= 0) return hipSuccess;
  if (items > (int64_t(1) << 30)) return hipErrorInvalidValue;
  if (tile_rows == 128)
    launch_tiled_rows<EPI, 128>(a, items, mx, nv, stream);
  else
    launch_tiled_rows<EPI, 256>(a, items, mx, nv, stream);
  return hipGetLastError();
}

}  // namespace

void set_tiled_one_per_tile(bool on) { g_one_per_tile.store(on); }

bool w4a16_tiled_supported(int32_t H, int32_t I) { return H % 256 == 0 && I % 256 == 0; }

int32_t w4a16_tiled_rows(double rows_per_expert) {
  // Measured on MI355X (hidden 7168, intermediate 2048, 48 experts): 128-row tiles win
  // while the experts average up to about kSmallTileRows routed rows.
  return rows_per_expert <= kSmallTileRows ? 128 : 256;
}

hipError_t launch_w4a16_gateup_tiled(const W4A16Problem& p, const Routing& r, int tile_rows,
                                     hipStream_t stream) {
  TiledArgs a{p.xs, p.w13, p.s13, r.sorted_ids, r.offsets, r.tile_offsets, r.topk_weights,
              p.h, nullptr, r.P, r.E, p.H, 2 * p.I, p.I, p.I / 128,
              (uint32_t)((uint64_t)r.L * p.H * 2u)};
  a.g = p.g13;
  return launch_tiled<TEpi::GateUp>(a, r.P, r.E, tile_rows, p.mx, p.nv, stream);
}

hipError_t launch_w4a16_down_tiled(const W4A16Problem& p, const Routing& r, int tile_rows,
                                   float* y, hipStream_t stream, uint16_t* out16, int kslices) {
  if (kslices < 1 || (p.I / 256) % kslices || (out16 && kslices != 1)) return hipErrorInvalidValue;
  TiledArgs a{p.h, p.w2, p.s2, r.sorted_ids, r.offsets, r.tile_offsets, r.topk_weights,
              nullptr, y, r.P, r.E, p.I, p.H, p.I, p.H / 256,
              (uint32_t)((uint64_t)r.L * p.I * 2u)};
  a.g = p.g2;
  a.out16 = out16;
  a.kslices = kslices;
  return launch_tiled<TEpi::Down>(a, r.P, r.E, tile_rows, p.mx, p.nv, stream);
}

hipError_t launch_combine_rows(const float* y, const int32_t* topk_ids, const float* wts,
                               int32_t T, int32_t k, int32_t E, int32_t H, uint16_t* out,
                               hipStream_t stream, int32_t slices) {
  const int64_t items = (int64_t)T * (H / 8);
  if (items <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((items + kCombineThreads - 1) / kCombineThreads, 16384);
  hipLaunchKernelGGL(combine_rows_kernel, dim3((unsigned)blocks), dim3(kCombineThreads), 0,
                     stream, y, topk_ids, wts, T, k, E, H, slices, out);
  return hipGetLastError();
}

}  // namespace qmoe
