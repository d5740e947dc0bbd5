// W8A8 block-FP8 grouped expert GEMMs, prefill profile (row tiles of 128, MFMA-bound).
//
// Method ("SGLang W8A8 Block FP8 quantization kernel config guide", background
// section): E4M3 activations with one fp32 scale per token and 128-column group (As),
// E4M3 weights with one fp32 scale per [128, 128] block (Bs); the per-expert product is
// C = sum over 128-deep k blocks of (A_q B_q^T)_block * As * Bs. With hundreds of rows
// per expert it is a grouped GEMM over the expert segments of the sorted row list
// ("vLLM x Novita AI: Chord W4A16 INT4 MoE Kernel for Kimi K2.x", "Two kernel
// families").
//
// gfx950 mapping. A work-group owns one (128-row tile of an expert segment, 256 weight
// rows) output tile; its eight waves, two per SIMD, each own 64 rows and 64 weight rows:
// 4 x 4 MFMA tiles, 64 fp32 accumulators per lane, kept in VGPRs because every 128-deep
// block is promoted with a VALU multiply-add:
//   * one v_mfma_scale_f32_16x16x128_f8f6f4 (block scales pinned to 1.0) is one k block;
//     its fp32 result d is added as acc += d * (As[row] * Bs), the scales being general
//     fp32 values (a power-of-two block scale cannot carry them);
//   * activation rows (gathered by token for gate_up, sorted rows of h for down), their
//     scales and the weights of each k block go global -> LDS by buffer loads to LDS
//     into a ring of three stages, eight lanes per 128 B row line (the MFMA's lane order,
//     sixteen rows per sixteen lanes, moves a third of the bytes per clock), placed with
//     a swizzle that keeps the MFMA-order reads free of bank conflicts; every wave waits
//     on its own copies with vmcnt (the compiler does not count these) before the
//     stage's barrier, which sits in the middle of the step so the last MFMAs cover it;
// gate_up quantizes SiLU(gate) * up to E4M3 per row and 128 columns in its epilogue (the
// tile's 128 h columns are one block; the rows' maxima meet through LDS); down stores
// the routing-weighted rows per (token, slot) pair, summed per token by the combine
// kernel.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace qmoe {

namespace {

constexpr int kTileRows = 128;
constexpr int kRowBlocks = kTileRows / 16;  // 8
// Eight waves: wave (wr, wc) owns row half wr (four 16-row blocks) and column quarter wc
// (four 16-column MFMA tiles) of the 128 x 256 tile, two waves per SIMD so that one
// wave's LDS and barrier waits are covered by the other's MFMAs.
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;
constexpr int kRowHalves = 2;
constexpr int kMyBlocks = kRowBlocks / kRowHalves;  // 4 row blocks per wave
constexpr int kColTiles = 4;                        // MFMA column tiles per wave
constexpr int kTileCols = 16;                       // column tiles per work-group tile
constexpr int kStages = 3;
constexpr int kScaleRowsPerWave = kTileRows / kWaves;  // 16 activation scale rows per wave
// Vector memory instructions per wave and step: one activation row block (two planes),
// the activation scales, two of the sixteen weight column tiles (two planes each).
constexpr int kCopiesPerStep = 2 + 1 + 2 * 2;
constexpr int kMaxKBlocks = 64;  // per-wave weight-scale rows held in LDS (K <= 8192)

// LDS layout in 16 B units: per stage the activation blocks and the weight column tiles,
// each 16 rows as [8-row half][row][slot] (see the copies), and the activation scales
// (per wave 64 floats: its 16 rows, then three copies of them, so that every lane of the
// copy is active and the loop body stays one basic block); then per wave the weight
// block scales for the whole K (two rows: gate and up for gate_up, the same block twice
// for down); then the gate_up epilogue's partial row maxima.
constexpr int kAUnits = kRowBlocks * 2 * kWave;       // 1024
constexpr int kAsUnits = kWaves * 64 / 4;             // 128
constexpr int kBUnits = kTileCols * 2 * kWave;        // 2048
constexpr int kStageUnits = kAUnits + kAsUnits + kBUnits;
constexpr int kBsBase = kStages * kStageUnits;
// gate_up epilogue: per tile row, the four column quarters' partial absolute maxima of h.
constexpr int kAmaxBase = kBsBase + kWaves * 2 * (kMaxKBlocks / 4);
constexpr int kSmemUnits = kAmaxBase + kTileRows * 4 / 4;
static_assert(kSmemUnits * 16 <= 160 * 1024, "LDS budget");

enum class FEpi { GateUp, Down };

struct Fp8TiledArgs {
  const uint8_t* act;           // gate_up: a_q [T, K]; down: hq [L, K]
  const float* act_scale;       // gate_up: a_scale [T, K/128]; down: hs [L, K/128]
  const uint8_t* w;             // [E, N, K]
  const float* ws;              // [E, N/128, K/128]
  const int32_t* sorted_ids;    // [L]
  const int32_t* offsets;       // [E + 1]
  const int32_t* tile_offsets;  // [E + 1], 128-row tiles
  const float* topk_weights;    // [P]
  uint8_t* hq;                  // gate_up output [L, I], E4M3
  float* hs;                    // gate_up output scales [L, I/128]
  float* y;                     // down output [P, N]
  int32_t P, k, E, K, N, I;
  int32_t col_tiles;
  // Sizes in bytes of act, act_scale, ws and one expert's weights (N * K), each < 2^31
  // (host-checked): the copies go through buffer resources of these sizes.
  uint32_t act_bytes, scale_bytes, ws_bytes, w_expert_bytes;
};

// Word 3 of a raw buffer resource (32-bit data format, no swizzle, no index).
constexpr int kRsrcWord3 = 0x00020000;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ int expert_of_tile(const int32_t* toff, int E, int m) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (toff[mid] <= m) lo = mid;
    else hi = mid;
  }
  return lo;
}

// LDS destination operand of a buffer load to LDS.
#define QMOE_LDS(p) ((__attribute__((address_space(3))) void*)(p))

template <FEpi EPI>
__global__ void __launch_bounds__(kThreads) fp8_tiled_kernel(Fp8TiledArgs a) {
  __shared__ u32x4 smem[kSmemUnits];

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wr = wave / (kWaves / kRowHalves), wc = wave % (kWaves / kRowHalves);
  const int col = lane & 15, quad = lane >> 4;

  const int total = a.tile_offsets[a.E] * a.col_tiles;
  const int per = (total + kNumXcd - 1) / kNumXcd;
  const int xi = blockIdx.x / kNumXcd;
  const int item = (blockIdx.x % kNumXcd) * per + xi;
  if (xi >= per || item >= total) return;
  // Items are ordered expert-major, then column tile, then row tile: the row tiles of
  // one (expert, column tile) are neighbours, run together on one XCD and share the
  // weight tile (the larger of the two operand streams here) in its L2.
  const int e = expert_of_tile(a.tile_offsets, a.E, item / a.col_tiles);
  const int ntile_e = a.tile_offsets[e + 1] - a.tile_offsets[e];
  const int local = item - a.tile_offsets[e] * a.col_tiles;
  const int ctile = local / ntile_e, rt = local - ctile * ntile_e;
  const int seg1 = a.offsets[e + 1];
  const int row0 = a.offsets[e] + rt * kTileRows;
  const int rb0 = row0 >> 4;
  const int rb_last = (seg1 >> 4) - 1;
  const int K = a.K, KB = K >> 7;

  // Weight row of column tile tt (0..15) of the work-group tile, column c: for gate_up,
  // quarter tt / 4 covers 32 h columns, its tiles 0-1 the gate rows and 2-3 the up rows
  // (a wave's gate and up rows lie in two [128, 128] weight blocks); for down a quarter's
  // 64 rows lie in one block.
  auto weight_row = [&](int tt, int c) {
    if constexpr (EPI == FEpi::GateUp) {
      const int t = tt & 3;
      const int j = ctile * 128 + (tt >> 2) * 32 + (t & 1) * 16 + c;
      return (t < 2) ? j : a.I + j;
    } else {
      return ctile * 256 + tt * 16 + c;
    }
  };
  // Activation row (of the act matrix) for tile row r; padding rows read row 0.
  auto act_row = [&](int r) {
    if constexpr (EPI == FEpi::GateUp) {
      const int sid = a.sorted_ids[r];
      return sid < a.P ? sid / a.k : 0;
    } else {
      return r;
    }
  };

  // Operand copies. A copy instruction moves 8 rows x 128 B (one k block of each row):
  // lane l takes row l / 8 of the eight and a 16 B piece of it, so every eight
  // consecutive lanes read one whole 128 B line. (With the MFMA's own lane order, where
  // consecutive lanes are consecutive rows, the address path delivers a third of the
  // bytes per clock.) The copy lands lane-linear in LDS; the piece a lane fetches is its
  // slot XOR (row ^ half) within the row, so that the MFMA-order reads below, which take
  // pieces 2 quad and 2 quad + 1 of row col for sixteen rows at once, fall on distinct
  // banks. In LDS a 16-row block is [half (rows 0-7, 8-15)][row][slot], 128 units of 16 B.
  // Copies go through buffer resources (32-bit byte offsets; weights per expert).
  const int crow = lane >> 3, cslot = lane & 7;
  auto piece_of = [&](int h8) { return (uint32_t)(cslot ^ crow ^ h8) * 16u; };
  const __amdgpu_buffer_rsrc_t ars =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.act, (short)0, (int)a.act_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)a.act_scale, (short)0, (int)a.scale_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.w + (size_t)e * a.N * (size_t)K), (short)0, (int)a.w_expert_bytes, kRsrcWord3);
  // Wave w copies activation row block w, the scales of rows 16w .. 16w+15 and weight
  // column tiles 4 wc + 2 wr and 4 wc + 2 wr + 1.
  uint32_t a_off[2];
  {
    const int rb = min(rb0 + wave, rb_last);
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8)
      a_off[h8] = (uint32_t)act_row(rb * 16 + 8 * h8 + crow) * (uint32_t)K + piece_of(h8);
  }
  uint32_t s_off;
  {
    const int r = min(row0 + wave * kScaleRowsPerWave + (lane & (kScaleRowsPerWave - 1)),
                      rb_last * 16 + 15);  // lanes 16..63 repeat lanes 0..15
    s_off = (uint32_t)act_row(r) * (uint32_t)KB * 4u;
  }
  const int my_tile0 = wc * kColTiles + 2 * wr;
  uint32_t w_off[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8)
      w_off[i][h8] = (uint32_t)weight_row(my_tile0 + i, 8 * h8 + crow) * (uint32_t)K + piece_of(h8);
  // Read side: this lane's two pieces (k bytes 32 quad .. 32 quad + 31 of row col) of a
  // 16-row block, in 16 B units from the block's start.
  int rd_off[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
    rd_off[hh] = (col >> 3) * kWave + (col & 7) * 8 + ((2 * quad + hh) ^ (col & 7) ^ (col >> 3));

  auto stage_at = [&](int st) { return &smem[st * kStageUnits]; };
  auto copy_step = [&](int g, int st) {
    const int kb = min(g, KB - 1);
    u32x4* s = stage_at(st);
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, QMOE_LDS(s + (wave * 2 + h8) * kWave), 16,
                                               (int)a_off[h8], kb * 128, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, QMOE_LDS(s + kAUnits + wave * 16), 4, (int)s_off,
                                             kb * 4, 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wrs, QMOE_LDS(s + kAUnits + kAsUnits + ((my_tile0 + i) * 2 + h8) * kWave), 16,
            (int)w_off[i][h8], kb * 128, 0, 0);
  };

  // Weight block scales of this wave for the whole K: row 0 for tiles 0-1, row 1 for
  // tiles 2-3 (gate / up for gate_up; down has one block row, copied to both).
  u32x4* bs_lds = &smem[kBsBase + wave * 2 * (kMaxKBlocks / 4)];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int nb = weight_row(wc * kColTiles + 2 * h, 0) >> 7;
    const uint32_t off = ((uint32_t)(e * (a.N >> 7) + nb) * KB + min(lane, KB - 1)) * 4u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        __builtin_amdgcn_make_buffer_rsrc((void*)a.ws, (short)0, (int)a.ws_bytes, kRsrcWord3),
        QMOE_LDS(bs_lds + h * (kMaxKBlocks / 4)), 4, (int)off, 0, 0, 0);
  }

  f32x4 acc[kMyBlocks][kColTiles];
#pragma unroll
  for (int m = 0; m < kMyBlocks; ++m)
#pragma unroll
    for (int t = 0; t < kColTiles; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  // Prologue: the two block-scale copies, then steps 0 .. kStages-1.
#pragma unroll
  for (int g = 0; g < kStages; ++g) copy_step(g, g);
  wait_vmcnt<(kStages - 1) * kCopiesPerStep>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

  const int rbt0 = wr * kMyBlocks;  // first row block of this wave within the tile
  // Scales of tile row r were copied by wave r / 16, to its 64-float slice.
  auto as_blk = [&](const u32x4* s, int rbt) {
    return *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(s + kAUnits) +
                                           rbt * 64 + 4 * quad);
  };
  // A step's first operands: its weight tiles, the first row block of activations and
  // their scales, the weight block scales. Read for step g + 1 right after step g's
  // barrier (its copies are complete by then), so that these reads overlap step g's last
  // MFMAs instead of stalling the start of step g + 1.
  // Two operand sets, used by alternate steps (the loop runs two steps per pass): a step
  // reads the next step's first operands into the other set, with no register copies
  // between steps that would wait for those reads.
  struct Ops {
    u32x4 bv[kColTiles][2], av[2];
    f32x4 as4;
    float bs0, bs1;
  };
  auto read_first = [&](const u32x4* s, int g, Ops& o) {
#pragma unroll
    for (int t = 0; t < kColTiles; ++t)
#pragma unroll
      for (int p = 0; p < 2; ++p)
        o.bv[t][p] = s[kAUnits + kAsUnits + (wc * kColTiles + t) * 2 * kWave + rd_off[p]];
    o.av[0] = s[rbt0 * 2 * kWave + rd_off[0]];
    o.av[1] = s[rbt0 * 2 * kWave + rd_off[1]];
    o.as4 = as_blk(s, rbt0);
    const int gc = min(g, KB - 1);
    o.bs0 = reinterpret_cast<const float*>(bs_lds)[gc];
    o.bs1 = reinterpret_cast<const float*>(bs_lds + kMaxKBlocks / 4)[gc];
  };
  Ops opa, opb;
  read_first(stage_at(0), 0, opa);
  int st = 0;
  auto step = [&](int g, Ops& cur, Ops& nxt) {
    const u32x4* s = stage_at(st);
    const int stn = (st == kStages - 1) ? 0 : st + 1;
    u32x4 av[2] = {cur.av[0], cur.av[1]};
    f32x4 as4 = cur.as4;
    const float bs0 = cur.bs0, bs1 = cur.bs1;
    // Row block m's operands are read one block ahead; the stage's last reads are issued
    // before the next-to-last block's MFMAs, so the barrier can follow those and the last
    // block's MFMAs cover it. The four MFMA results of block m are promoted into the
    // accumulators while block m+1's MFMAs run (no VALU waits on a fresh MFMA result).
    f32x4 dprev[kColTiles];
    // down: one block scale for all four tiles (one product per row block).
    constexpr bool kOneScale = EPI == FEpi::Down;
    f32x4 scprev0 = zero4, scprev1 = zero4;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m <= kMyBlocks; ++m) {
      f32x4 dcur[kColTiles];
      u32x4 avn[2] = {av[0], av[1]};
      f32x4 as4n = as4;
      if (m < kMyBlocks) {
        if (m + 1 < kMyBlocks) {
          avn[0] = s[(rbt0 + m + 1) * 2 * kWave + rd_off[0]];
          avn[1] = s[(rbt0 + m + 1) * 2 * kWave + rd_off[1]];
          as4n = as_blk(s, rbt0 + m + 1);
        }
#pragma unroll
        for (int t = 0; t < kColTiles; ++t) {
          const u32x4 bb[2] = {cur.bv[t][0], cur.bv[t][1]};
          dcur[t] = mfma_fp8_16x16x128(av, bb, zero4);
        }
      }
      if (m > 0) {
#pragma unroll
        for (int t = 0; t < kColTiles; ++t) {
          const f32x4 sc = (kOneScale || t < 2) ? scprev0 : scprev1;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[m - 1][t][r] = __builtin_fmaf(dprev[t][r], sc[r], acc[m - 1][t][r]);
        }
      }
      if (m < kMyBlocks) {
#pragma unroll
        for (int t = 0; t < kColTiles; ++t) dprev[t] = dcur[t];
        scprev0 = as4 * bs0;
        if (!kOneScale) scprev1 = as4 * bs1;
      }
      if (m == kMyBlocks - 2) {
        // All reads of this stage were issued; once they and the copies of step g+1
        // (younger: the copies of step g+2) have completed, the barrier frees the stage
        // for step g + kStages.
        __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0)
        wait_vmcnt<(kStages - 2) * kCopiesPerStep>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        copy_step(g + kStages, st);
        // Step g + 1's stage is complete (every wave waited for its copies before the
        // barrier); past the last step it holds re-read blocks, never used.
        read_first(stage_at(stn), g + 1, nxt);
        __builtin_amdgcn_sched_barrier(0);
      }
      av[0] = avn[0];
      av[1] = avn[1];
      as4 = as4n;
      // Keep each block's LDS reads in its own iteration: a compiler-level memory fence,
      // no instruction.
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
    st = stn;
  };
  int g = 0;
  for (; g + 1 < KB; g += 2) {
    step(g, opa, opb);
    step(g + 1, opb, opa);
  }
  if (g < KB) step(g, opa, opb);
  wait_vmcnt<0>();

  if constexpr (EPI == FEpi::GateUp) {
    // h = SiLU(gate) * up in fp32, then the E4M3 quantization of every row's block of
    // 128 h columns (the tile's columns are exactly one such block) with the block
    // quantizer's arithmetic: s = max(absmax, 1e-10) / 448, q = e4m3(clamp(h / s)).
    float hv[kMyBlocks][2][4];
#pragma unroll
    for (int m = 0; m < kMyBlocks; ++m)
#pragma unroll
      for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          hv[m][tp][r] = silu_f32_accurate(acc[m][tp][r]) * acc[m][tp + 2][r];
    // Row maxima: over this lane's two columns, the 16 lanes of its row quarter, then the
    // four column quarters (waves) through LDS.
    float* amax_lds = reinterpret_cast<float*>(&smem[kAmaxBase]);
#pragma unroll
    for (int m = 0; m < kMyBlocks; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = fmaxf(fabsf(hv[m][0][r]), fabsf(hv[m][1][r]));
#pragma unroll
        for (int d = 8; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, kWave));
        if (col == 0) amax_lds[((rbt0 + m) * 16 + 4 * quad + r) * 4 + wc] = v;
      }
    __syncthreads();
    const int nblk = a.I >> 7;
#pragma unroll
    for (int m = 0; m < kMyBlocks; ++m) {
      const int rb = rb0 + rbt0 + m;
      if (rb > rb_last) break;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rb * 16 + 4 * quad + r;
        const f32x4 am =
            *reinterpret_cast<const f32x4*>(&amax_lds[((rbt0 + m) * 16 + 4 * quad + r) * 4]);
        const float amax = fmaxf(fmaxf(am[0], am[1]), fmaxf(am[2], am[3]));
        const float sc = fmaxf(amax, 1e-10f) / 448.0f;
        if (wc == 0 && col == 0) a.hs[(size_t)row * nblk + ctile] = sc;
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
          const int j = ctile * 128 + wc * 32 + tp * 16 + col;
          const float t = fminf(fmaxf(hv[m][tp][r] / sc, -448.0f), 448.0f);
          a.hq[(size_t)row * a.I + j] =
              (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(t, t, 0u, false) & 0xFFu);
        }
      }
    }
  } else {
    // Every pair id of this wave's rows, then every routing weight, requested before any
    // is used (two round trips per tile instead of two per row block).
    int pair[kMyBlocks][4];
    float wt[kMyBlocks][4];
#pragma unroll
    for (int m = 0; m < kMyBlocks; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        pair[m][r] = a.sorted_ids[min(rb0 + rbt0 + m, rb_last) * 16 + 4 * quad + r];
#pragma unroll
    for (int m = 0; m < kMyBlocks; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) wt[m][r] = a.topk_weights[min(pair[m][r], a.P - 1)];
#pragma unroll
    for (int m = 0; m < kMyBlocks; ++m) {
      if (rb0 + rbt0 + m > rb_last) break;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (pair[m][r] >= a.P) continue;
        float* yrow = a.y + (size_t)pair[m][r] * a.N;
#pragma unroll
        for (int t = 0; t < kColTiles; ++t)
          yrow[weight_row(wc * kColTiles + t, col)] = wt[m][r] * acc[m][t][r];
      }
    }
  }
}

template <FEpi EPI>
hipError_t launch_fp8_tiled(const Fp8TiledArgs& a, int64_t max_row_tiles, hipStream_t stream) {
  const int64_t items = max_row_tiles * a.col_tiles;
  if (items <= 0) return hipSuccess;
  if (items > (int64_t(1) << 30)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fp8_tiled_kernel<EPI>), dim3(xcd_major_grid((int)items)), dim3(kThreads),
                     0, stream, a);
  return hipGetLastError();
}

}  // namespace

bool fp8_tiled_supported(int32_t H, int32_t I) {
  return H % 256 == 0 && I % 128 == 0 && H / 128 <= kMaxKBlocks && I / 128 <= kMaxKBlocks;
}

int32_t fp8_tiled_rows() { return kTileRows; }

hipError_t launch_fp8_gateup_tiled(const Fp8Problem& p, const Routing& r, hipStream_t stream) {
  Fp8TiledArgs a{p.a_q, p.a_scale, p.w13, p.s13, r.sorted_ids, r.offsets, r.tile_offsets,
                 r.topk_weights, p.hq, p.hs, nullptr, r.P, r.k, r.E, p.H, 2 * p.I, p.I, p.I / 128,
                 (uint32_t)((uint64_t)p.T * p.H), (uint32_t)((uint64_t)p.T * (p.H / 128) * 4u),
                 (uint32_t)((uint64_t)r.E * (2 * p.I / 128) * (p.H / 128) * 4u),
                 (uint32_t)((uint64_t)2 * p.I * p.H)};
  return launch_fp8_tiled<FEpi::GateUp>(a, (int64_t)r.P / kTileRows + r.E, stream);
}

hipError_t launch_fp8_down_tiled(const Fp8Problem& p, const Routing& r, float* y,
                                 hipStream_t stream) {
  Fp8TiledArgs a{p.hq, p.hs, p.w2, p.s2, r.sorted_ids, r.offsets, r.tile_offsets,
                 r.topk_weights, nullptr, nullptr, y, r.P, r.k, r.E, p.I, p.H, p.I, p.H / 256,
                 (uint32_t)((uint64_t)r.L * p.I), (uint32_t)((uint64_t)r.L * (p.I / 128) * 4u),
                 (uint32_t)((uint64_t)r.E * (p.H / 128) * (p.I / 128) * 4u),
                 (uint32_t)((uint64_t)p.H * p.I)};
  return launch_fp8_tiled<FEpi::Down>(a, (int64_t)r.P / kTileRows + r.E, stream);
}

}  // namespace qmoe
