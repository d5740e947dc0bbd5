// C ABI of the MoE expert FFN library: argument checks, schedule choice, workspace
// layout and the launch sequence. Everything here is host code; no call reads a
// device value back, allocates, frees or synchronizes.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/qmoe.h"
#include "internal.h"

namespace qmoe {
namespace {

thread_local char g_last_error[512] = "";

qmoe_status fail(qmoe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

qmoe_status hip_fail(hipError_t err, const char* what) {
  (void)hipGetLastError();  // clear the sticky launch error
  return fail(QMOE_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr size_t kRegionAlign = 256;
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

enum Format { kW4A16 = 0, kFp8 = 1, kMxfp4 = 2, kNvfp4 = 3 };
// Compute units the planner fills (MI355X: 256). A plan is pure host computation, so the
// device is not queried; a GPU with fewer units only gets more tiles per unit.
constexpr double kPlanComputeUnits = 256.0;
// The 4-bit formats share the W4A16 kernels, workspace and limits.
bool four_bit(int fmt) { return fmt == kW4A16 || fmt == kMxfp4 || fmt == kNvfp4; }

// Rows per weight pass of the FP8 decode kernels, in 16-row blocks: four, measured on
// MI355X at hidden 7168, intermediate 2048, 32 experts (one / two / four blocks: 0.30 /
// 0.30 / 0.30 ms at 8 rows per expert, 0.52 / 0.37 / 0.36 ms at 16, 0.79 / 0.57 / 0.43
// ms at 32): a pass serves up to 64 rows for one read of the weights, and an empty
// block costs little next to the FP8 weight stream.
int decode_mb_for(double) { return 4; }
// Routed rows per expert above which the 4-bit persistent decode kernel serves two
// 16-row blocks per weight pass, measured on MI355X for hidden 7168, intermediate 2048,
// 48 experts (one vs two blocks per pass: W4A16 at 14 rows 0.342 vs 0.355 ms, at 16
// rows 0.427 vs 0.370 ms; MXFP4 at 10 rows 0.297 vs 0.287 ms, at 8 rows 0.253 vs
// 0.281 ms). Below these, most experts fit one block and a second one costs MFMA and
// activation work for nothing.
double two_block_rows(int fmt) { return fmt == kMxfp4 || fmt == kNvfp4 ? 11.0 : 15.0; }

constexpr size_t kNoRegion = ~size_t(0);

// Schedule overrides of qmoe_set_tuning (0: the library's own choice).
std::atomic<int32_t> g_tune_tile_rows{0}, g_tune_rows_per_pass{0}, g_tune_kslices{0};

struct Plan {
  int fmt = 0;
  int schedule = QMOE_SCHEDULE_DECODE;
  int mb = 1;
  bool tiled = false;  // 4-bit prefill on the tile kernels
  int32_t tile_rows = 256;  // their row tile
  int32_t kslices = 1;      // split-K of the prefill down GEMM (4-bit tile kernels)
  int32_t block_m = kSegRows;
  int64_t P = 0, L = 0, NB = 0;
  // Workspace regions, indexed by the QMOE_REGION_* values: byte offset (kNoRegion when
  // the plan has no such region) and size.
  size_t off[QMOE_NUM_REGIONS];
  size_t len[QMOE_NUM_REGIONS];
  size_t off_sorted = 0, off_expert_ids = 0, off_ntp = 0, off_offsets = 0, off_tiles = 0;
  size_t off_xs = 0, off_h = 0, off_h32 = 0, off_hq = 0, off_hs = 0, off_out32 = 0, off_y = 0;
  size_t total = 0;
};

qmoe_status check_shape(int fmt, int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                        int32_t schedule) {
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0)
    return fail(QMOE_ERR_INVALID_ARG, "sizes must be positive (T >= 0): T=%d H=%d I=%d E=%d k=%d",
                T, H, I, E, k);
  if (k > E) return fail(QMOE_ERR_INVALID_ARG, "top-k %d exceeds expert count %d", k, E);
  if (E > QMOE_MAX_EXPERTS)
    return fail(QMOE_ERR_UNSUPPORTED, "expert count %d exceeds %d", E, QMOE_MAX_EXPERTS);
  if (schedule < QMOE_SCHEDULE_AUTO || schedule > QMOE_SCHEDULE_PREFILL)
    return fail(QMOE_ERR_INVALID_ARG, "unknown schedule %d", schedule);
  const int q = four_bit(fmt) ? 32 : 128;
  if (H % q || I % q)
    return fail(QMOE_ERR_UNSUPPORTED, "%s needs H and I multiples of %d (H=%d I=%d)",
                fmt == kW4A16   ? "W4A16 group-32"
                : fmt == kMxfp4 ? "MXFP4 block-32"
                : fmt == kNvfp4 ? "NVFP4 (32-column packing)"
                                : "block FP8 [128,128]",
                q, H, I);
  const int64_t P = (int64_t)T * k;
  const int64_t L = P + (int64_t)E * (2 * kSegRows - 1);  // the largest align block
  if (L >= (int64_t(1) << 31) || (int64_t)L * (int64_t)I >= (int64_t(1) << 40))
    return fail(QMOE_ERR_UNSUPPORTED, "too many routed pairs: T*k=%lld", (long long)P);
  return QMOE_OK;
}

// tok_e_hint > 0 replaces the routed-rows-per-expert estimate T * k / E that picks the
// schedule (the grouped layouts pass the caller's expected rows per expert).
// direct_out: the forward writes the output rows without per-pair fp32 rows (one pair of
// weight 1 per row: the grouped layouts), so the plan has no Y region.
Plan make_plan(int fmt, int32_t T, int32_t H, int32_t I, int32_t E, int32_t k, int32_t schedule,
               double tok_e_hint = -1.0, bool direct_out = false) {
  Plan p;
  p.fmt = fmt;
  p.P = (int64_t)T * k;
  const double tok_e = tok_e_hint > 0 ? tok_e_hint : E > 0 ? (double)p.P / E : 0.0;
  p.schedule = schedule;
  // Crossover of the two profiles, measured on MI355X for hidden 7168, intermediate 2048,
  // 48 experts (quantized_mixture_experts_amd.tune_schedule): the decode profile streams
  // the weights once per pass of one or two 16-row blocks and the tile kernels use
  // 128-row tiles at these sizes, so decode wins up to about 44 routed rows per expert
  // for W4A16 (40: 0.69 vs 0.71 ms; 48: 0.72 vs 0.71 ms), about 60 for MXFP4 (56: 0.61
  // vs 0.64 ms; 64: 0.69 vs 0.64 ms) and about 20 for block FP8 with four blocks per
  // pass (16: 0.36 vs 0.38 ms; 24: 0.40 vs 0.39 ms).
  // (NVFP4, with the same sweep: 32: 0.47 vs 0.56 ms; 40: 0.57 vs 0.56 ms.) With few
  // experts the routed pairs are few and the prefill tiles leave most of the GPU idle:
  // the 4-bit decode profile stays ahead up to about ten times the crossover in routed
  // pairs at any rows per expert (W4A16 at 8, 4 and 2 experts, top-2, top-1, top-1:
  // decode ahead up to 48, 96 and 192 rows per expert, prefill from 64, 128 and 256).
  const double crossover = fmt == kMxfp4 ? 60.0 : fmt == kFp8 ? 20.0 : fmt == kNvfp4 ? 36.0 : 44.0;
  if (schedule == QMOE_SCHEDULE_AUTO)
    p.schedule = (tok_e <= crossover || (four_bit(fmt) && (double)p.P <= 10.2 * crossover))
                     ? QMOE_SCHEDULE_DECODE
                     : QMOE_SCHEDULE_PREFILL;
  p.tiled = p.schedule == QMOE_SCHEDULE_PREFILL &&
            (four_bit(fmt) ? w4a16_tiled_supported(H, I) : fp8_tiled_supported(H, I));
  // Rows per weight pass of the stream kernels and the align block size. The 4-bit
  // persistent kernel serves two 16-row blocks per pass above two_block_rows() routed
  // rows per expert (align then pads segments to 32 rows so a pass stays in one expert); the
  // FP8 stream kernels take mb within segments of any multiple of 16.
  auto set_blocks = [&] {
    if (four_bit(fmt)) {
      // Two blocks per pass also need enough routed pairs: with few experts a second pass
      // over an expert's weights costs less than the work-groups that two-block passes
      // leave idle (W4A16 at 8, 4 and 2 experts: one block ahead up to 24, 48 and 96 rows
      // per expert, two from 32, 64 and 128, i.e. above about 15 x two_block_rows pairs).
      p.mb = (!p.tiled && tok_e > two_block_rows(fmt) && (double)p.P > 15.0 * two_block_rows(fmt))
                 ? 2 : 1;
      if (!p.tiled && g_tune_rows_per_pass.load()) p.mb = g_tune_rows_per_pass.load() / kSegRows;
      p.block_m = kSegRows * p.mb;
    } else {
      p.mb = p.schedule == QMOE_SCHEDULE_DECODE ? decode_mb_for(tok_e) : 2;
      p.block_m = kSegRows;
    }
    p.L = p.P + (int64_t)E * (p.block_m - 1);
    p.NB = (p.L + p.block_m - 1) / p.block_m;
  };
  set_blocks();
  if (four_bit(fmt)) p.tile_rows = g_tune_tile_rows.load() ? g_tune_tile_rows.load()
                                                           : w4a16_tiled_rows(tok_e);
  // 256-row tiles that would not fill the GPU while 128-row tiles fit in one wave: the
  // smaller tiles keep more compute units busy for the same one wave (measured on MI355X at
  // hidden 7168, intermediate 2048: 8 experts, top-2, at 160 and 192 rows per expert, and
  // 4 or 2 experts, top-1, at 256 to 512, 128-row tiles 5-11 % faster; where 128-row tiles
  // need a second wave, 256-row ones stay faster, e.g. 4 experts at 512 rows by 13 %).
  // Rows per expert are counted high, as for split-K below.
  if (four_bit(fmt) && p.tiled && !g_tune_tile_rows.load() && p.tile_rows == 256 && p.P > 0) {
    const double e_eff = std::min<double>(E, (double)p.P);
    const double rows_e = (double)p.P / e_eff;
    const double sd = std::sqrt(rows_e * std::max(0.0, 1.0 - (double)k / E));
    auto gate_up_items = [&](double tr) {
      return e_eff * std::ceil((rows_e + 2.0 * sd) / tr) * (I / 128);
    };
    if (gate_up_items(256.0) < kPlanComputeUnits && gate_up_items(128.0) <= kPlanComputeUnits)
      p.tile_rows = 128;
  }
  // Split-K of the 4-bit prefill down GEMM where its output tiles would not fill the chip
  // ([CHORD] "Kernel optimizations": a shape guard decides when down splits K): the tile
  // kernels hold one work-group per compute unit, so when the expected tiles leave most of
  // the kPlanComputeUnits idle, each tile's K (I / 256 blocks) is split into the largest
  // power of two of slices that still fits one wave. The routed rows of an expert are
  // counted high: mean plus two standard deviations of a uniform top-k routing's count,
  // Binomial(T, k / E), whose variance is rows * (1 - k / E). A split that spills into a
  // second wave costs more than it saves (measured on MI355X at 1024 tokens, 2 experts,
  // top-1: an expert one 256-row tile larger than its mean, 2 slices, +8 %).
  if (p.tiled && four_bit(fmt) && !direct_out && p.P > 0) {
    const double e_eff = std::min<double>(E, (double)p.P);
    const double rows_e = (double)p.P / e_eff;
    const double sd = std::sqrt(rows_e * std::max(0.0, 1.0 - (double)k / E));
    const double tiles = e_eff * std::ceil((rows_e + 2.0 * sd) / p.tile_rows);
    const double items = tiles * (H / 256);
    const int nblk = I / 256;
    while (p.kslices * 2 <= nblk && nblk % (p.kslices * 2) == 0 &&
           items * p.kslices * 2 <= kPlanComputeUnits)
      p.kslices *= 2;
    const int32_t ks = g_tune_kslices.load();
    if (ks) p.kslices = nblk % ks == 0 ? ks : 1;
  }
  // The 4-bit tile kernels address activation rows with 32-bit byte offsets, and one
  // expert's weights (I * H bytes of codes in either GEMM) through a buffer resource whose
  // size is a signed 32-bit count; larger shapes run on the stream kernels.
  if (p.tiled && four_bit(fmt) &&
      ((uint64_t)p.L * (uint64_t)std::max(H, I) * 2u >= (uint64_t(1) << 32) ||
       (uint64_t)I * (uint64_t)H >= (uint64_t(1) << 31))) {
    p.tiled = false;
    set_blocks();
  }
  // The block-FP8 tile kernels copy activation rows (T x H codes for gate_up, L x I for
  // down) and one expert's weights (2I x H codes) through buffer resources whose size is
  // a signed 32-bit count.
  if (p.tiled && fmt == kFp8 &&
      ((uint64_t)T * (uint64_t)H >= (uint64_t(1) << 31) ||
       (uint64_t)p.L * (uint64_t)I >= (uint64_t(1) << 31) ||
       (uint64_t)2 * I * (uint64_t)H >= (uint64_t(1) << 31))) {
    p.tiled = false;
    set_blocks();
  }
  for (int i = 0; i < QMOE_NUM_REGIONS; ++i) {
    p.off[i] = kNoRegion;
    p.len[i] = 0;
  }
  size_t cur = 0;
  auto take = [&](int region, size_t bytes) {
    p.off[region] = cur;
    p.len[region] = bytes;
    cur = round_up(cur + bytes, kRegionAlign);
  };
  take(QMOE_REGION_SORTED_IDS, sizeof(int32_t) * p.L);
  take(QMOE_REGION_EXPERT_IDS, sizeof(int32_t) * p.NB);
  take(QMOE_REGION_NUM_TOKENS_PADDED, sizeof(int32_t));
  take(QMOE_REGION_EXPERT_OFFSETS, sizeof(int32_t) * (E + 1));
  take(QMOE_REGION_TILE_OFFSETS, sizeof(int32_t) * (E + 1));
  if (four_bit(fmt)) {
    take(QMOE_REGION_XS, sizeof(uint16_t) * (size_t)p.L * H);
    take(QMOE_REGION_H, sizeof(uint16_t) * (size_t)p.L * I);
  } else {
    if (!p.tiled) take(QMOE_REGION_H32, sizeof(float) * (size_t)p.L * I);  // quantized afterwards
    take(QMOE_REGION_HQ, (size_t)p.L * I);
    take(QMOE_REGION_HS, sizeof(float) * (size_t)p.L * (I / 128));
  }
  if (p.tiled) {
    if (!direct_out) take(QMOE_REGION_Y, sizeof(float) * (size_t)p.kslices * p.P * H);
  } else {
    take(QMOE_REGION_OUT32, sizeof(float) * (size_t)T * H);
  }
  p.total = cur;
  p.off_sorted = p.off[QMOE_REGION_SORTED_IDS];
  p.off_expert_ids = p.off[QMOE_REGION_EXPERT_IDS];
  p.off_ntp = p.off[QMOE_REGION_NUM_TOKENS_PADDED];
  p.off_offsets = p.off[QMOE_REGION_EXPERT_OFFSETS];
  p.off_tiles = p.off[QMOE_REGION_TILE_OFFSETS];
  p.off_xs = p.off[QMOE_REGION_XS];
  p.off_h = p.off[QMOE_REGION_H];
  p.off_h32 = p.off[QMOE_REGION_H32];
  p.off_hq = p.off[QMOE_REGION_HQ];
  p.off_hs = p.off[QMOE_REGION_HS];
  p.off_out32 = p.off[QMOE_REGION_OUT32];
  p.off_y = p.off[QMOE_REGION_Y];
  return p;
}

// Optional event pairs around each stage launch (qmoe_timing_begin / _end).
struct StageTimer {
  std::mutex mu;
  bool on = false;
  int cap = 0;
  int used[QMOE_NUM_STAGES] = {};
  std::vector<hipEvent_t> ev[QMOE_NUM_STAGES];  // 2 per recorded forward

  void clear() {
    for (auto& v : ev) {
      for (hipEvent_t e : v) (void)hipEventDestroy(e);
      v.clear();
    }
    for (int& u : used) u = 0;
    cap = 0;
    on = false;
  }
};
StageTimer g_timer;

// Runs `launch` (returning hipError_t) bracketed by the stage's events if recording.
template <typename F>
hipError_t staged(int stage, hipStream_t s, F&& launch) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_timer.mu);
    if (g_timer.on && g_timer.used[stage] < g_timer.cap) {
      const int i = g_timer.used[stage]++;
      e0 = g_timer.ev[stage][2 * i];
      e1 = g_timer.ev[stage][2 * i + 1];
    }
  }
  if (e0) {
    hipError_t err = hipEventRecord(e0, s);
    if (err != hipSuccess) return err;
  }
  hipError_t err = launch();
  if (err == hipSuccess && e1) err = hipEventRecord(e1, s);
  return err;
}

// Pointer to a workspace region; null for a region the plan does not have.
template <typename T>
T* region(void* ws, size_t off) {
  return off == kNoRegion ? nullptr : reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

Routing routing_view(const Plan& p, void* workspace, const float* topk_weights, int32_t k,
                     int32_t E) {
  Routing r{};
  r.sorted_ids = region<int32_t>(workspace, p.off_sorted);
  r.offsets = region<int32_t>(workspace, p.off_offsets);
  r.tile_offsets = region<int32_t>(workspace, p.off_tiles);
  r.expert_ids = region<int32_t>(workspace, p.off_expert_ids);
  r.ntp = region<int32_t>(workspace, p.off_ntp);
  r.topk_weights = topk_weights;
  r.P = (int32_t)p.P;
  r.k = k;
  r.E = E;
  r.L = (int32_t)p.L;
  return r;
}

// align of the indexed forwards: the routed pairs sorted to expert segments of block_m
// rows (and the prefill tiles' offsets when the plan uses the tile kernels).
hipError_t w4a16_align(const Plan& p, const int32_t* topk_ids, int32_t E, void* workspace,
                       hipStream_t s) {
  return staged(QMOE_STAGE_ALIGN, s, [&] {
    return launch_align(topk_ids, (int32_t)p.P, E, p.block_m, (int32_t)p.L, (int32_t)p.NB,
                        region<int32_t>(workspace, p.off_sorted),
                        region<int32_t>(workspace, p.off_expert_ids),
                        region<int32_t>(workspace, p.off_ntp),
                        region<int32_t>(workspace, p.off_offsets), p.tiled ? p.tile_rows : 0,
                        p.tiled ? region<int32_t>(workspace, p.off_tiles) : nullptr, s);
  });
}

// The 4-bit forward after align: row gather (where the kernels need it), gate_up, down,
// combine or cast. direct_out (one pair of weight 1 per row, the grouped layouts): on the
// prefill tiles, down writes the bf16 output rows itself and there is no combine pass.
qmoe_status w4a16_after_align(const Plan& p, const uint16_t* x, const uint8_t* w13,
                              const uint16_t* s13, const uint8_t* w2, const uint16_t* s2,
                              const int32_t* topk_ids, const float* topk_weights, int32_t T,
                              int32_t H, int32_t I, int32_t E, int32_t k, uint16_t* out,
                              void* workspace, hipStream_t s, const float* g13 = nullptr,
                              const float* g2 = nullptr, bool direct_out = false) {
  const Routing r = routing_view(p, workspace, topk_weights, k, E);
  const bool mx = p.fmt == kMxfp4 || p.fmt == kNvfp4;  // FP4 codes, natural k order
  W4A16Problem prob{x, region<uint16_t>(workspace, p.off_xs), w13, s13, w2, s2,
                    region<uint16_t>(workspace, p.off_h), region<float>(workspace, p.off_out32),
                    T, H, I, mx};
  prob.nv = p.fmt == kNvfp4;
  prob.g13 = g13;
  prob.g2 = g2;
  // One pair per row: the routing pass has cleared the padding rows of out, gate_up
  // clears the routed rows of out32, and only those are cast.
  prob.routed_rows_only = direct_out;
  const int32_t* ntp = region<int32_t>(workspace, p.off_ntp);

  if (p.tiled) {
    const int32_t tm = p.tile_rows;
    hipError_t err = staged(QMOE_STAGE_ALIGN, s, [&] {
      return launch_gather_rows(x, r, ntp, H, prob.xs, s, mx);
    });
    if (err != hipSuccess) return hip_fail(err, "gather launch");
    err = staged(QMOE_STAGE_GATE_UP, s, [&] { return launch_w4a16_gateup_tiled(prob, r, tm, s); });
    if (err != hipSuccess) return hip_fail(err, "gate_up launch");
    float* y = region<float>(workspace, p.off_y);
    err = staged(QMOE_STAGE_DOWN, s, [&] {
      return launch_w4a16_down_tiled(prob, r, tm, y, s, direct_out ? out : nullptr, p.kslices);
    });
    if (err != hipSuccess) return hip_fail(err, "down launch");
    if (!direct_out) {
      err = staged(QMOE_STAGE_CAST, s, [&] {
        return launch_combine_rows(y, topk_ids, topk_weights, T, k, E, H, out, s, p.kslices);
      });
      if (err != hipSuccess) return hip_fail(err, "combine launch");
    }
    return QMOE_OK;
  }

  hipError_t err = hipSuccess;
  if (!w4a16_stream_zeroes_output(H)) {
    err = staged(QMOE_STAGE_ZERO, s, [&] { return launch_zero_f32(prob.out32, (int64_t)T * H, s); });
    if (err != hipSuccess) return hip_fail(err, "zero launch");
  }
  // The gathered activation rows belong to the align stage's timing; the persistent
  // decode gate_up reads the rows of x itself.
  if (!w4a16_stream_reads_rows(H, p.mb)) {
    err = staged(QMOE_STAGE_ALIGN, s, [&] {
      return launch_gather_rows(x, r, ntp, H, prob.xs, s, mx);
    });
    if (err != hipSuccess) return hip_fail(err, "gather launch");
  }
  err = staged(QMOE_STAGE_GATE_UP, s, [&] { return launch_w4a16_gateup_stream(prob, r, p.mb, s); });
  if (err != hipSuccess) return hip_fail(err, "gate_up launch");
  err = staged(QMOE_STAGE_DOWN, s, [&] { return launch_w4a16_down_stream(prob, r, p.mb, s); });
  if (err != hipSuccess) return hip_fail(err, "down launch");
  err = staged(QMOE_STAGE_CAST, s, [&] {
    return direct_out ? launch_cast_routed_rows(prob.out32, r.sorted_ids, ntp, r.P, r.L, H, out, s)
                      : launch_cast_f32_bf16(prob.out32, out, (int64_t)T * H, s);
  });
  if (err != hipSuccess) return hip_fail(err, "cast launch");
  return QMOE_OK;
}

// The indexed 4-bit forward after argument checks: align, then the rest.
qmoe_status w4a16_run(const Plan& p, const uint16_t* x, const uint8_t* w13, const uint16_t* s13,
                      const uint8_t* w2, const uint16_t* s2, const int32_t* topk_ids,
                      const float* topk_weights, int32_t T, int32_t H, int32_t I, int32_t E,
                      int32_t k, uint16_t* out, void* workspace, hipStream_t s,
                      const float* g13 = nullptr, const float* g2 = nullptr) {
  hipError_t err = w4a16_align(p, topk_ids, E, workspace, s);
  if (err != hipSuccess) return hip_fail(err, "align launch");
  return w4a16_after_align(p, x, w13, s13, w2, s2, topk_ids, topk_weights, T, H, I, E, k, out,
                           workspace, s, g13, g2);
}

// Grouped layouts: the rows arrive grouped by expert (the layout an expert-parallel
// dispatch hands over), each row one pair of routing weight 1, so the forward is the
// indexed one with k = 1 and the row's expert as its only id. `route` is m_indices
// (contiguous) or masked_m (masked, then M is max_m and there are E * M rows).
//   masked: the align outputs come from the counts alone (no sort), in the same pass as
//     the unit weights;
//   contiguous: the unit weights (and cleared padding rows) in one pass, then align over
//     m_indices, which need not be sorted;
//   either: on the prefill tiles down writes the bf16 rows itself (no per-pair fp32 rows,
//     no combine); on the decode schedule gate_up reads the rows of `a` directly.
qmoe_status w4a16_grouped(bool masked, const uint16_t* a, const uint8_t* w13, const uint16_t* s13,
                          const uint8_t* w2, const uint16_t* s2, const int32_t* route,
                          int32_t M, int32_t H, int32_t I, int32_t E, int32_t expected_m,
                          int32_t schedule, uint16_t* out, void* workspace,
                          size_t* workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  if (M < 0)
    return fail(QMOE_ERR_INVALID_ARG, "%s must be >= 0 (got %d)", masked ? "max_m" : "row count",
                M);
  if (expected_m < 0)
    return fail(QMOE_ERR_INVALID_ARG, "expected_m must be >= 0 (got %d)", expected_m);
  const int64_t rows = masked ? (int64_t)std::max(E, 0) * M : M;
  if (rows > INT32_MAX)
    return fail(QMOE_ERR_UNSUPPORTED, "too many rows: %lld", (long long)rows);
  const int32_t T = (int32_t)rows;
  qmoe_status st = check_shape(kW4A16, T, H, I, E, 1, schedule);
  if (st != QMOE_OK) return st;
  if (!workspace_bytes) return fail(QMOE_ERR_INVALID_ARG, "workspace_bytes is NULL");
  const Plan p = make_plan(kW4A16, T, H, I, E, 1, schedule, expected_m > 0 ? expected_m : -1.0,
                           /*direct_out=*/true);
  const size_t off_ones = p.total;
  const size_t total = off_ones + round_up(sizeof(float) * (size_t)T, kRegionAlign);
  if (!workspace) {
    *workspace_bytes = total;
    return QMOE_OK;
  }
  if (*workspace_bytes < total)
    return fail(QMOE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", *workspace_bytes, total);
  if (T == 0) return QMOE_OK;
  const void* ptrs[] = {a, w13, s13, w2, s2, out};
  for (const void* q : ptrs)
    if (!q) return fail(QMOE_ERR_INVALID_ARG, "NULL tensor pointer");
  for (const void* q : ptrs)
    if (!aligned(q, 16)) return fail(QMOE_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (!route || !aligned(route, 4))
    return fail(QMOE_ERR_INVALID_ARG, "%s must be a 4-byte aligned device pointer",
                masked ? "masked_m" : "m_indices");
  if (!aligned(workspace, kRegionAlign))
    return fail(QMOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");

  hipStream_t s = static_cast<hipStream_t>(stream);
  float* ones = region<float>(workspace, off_ones);
  // The kernels write only the valid rows: the routing pass clears the others.
  uint16_t* clear = out;
  hipError_t err;
  if (masked) {
    err = staged(QMOE_STAGE_ALIGN, s, [&] {
      return launch_masked_align(route, E, M, p.block_m, (int32_t)p.L, (int32_t)p.NB,
                                 region<int32_t>(workspace, p.off_sorted),
                                 region<int32_t>(workspace, p.off_expert_ids),
                                 region<int32_t>(workspace, p.off_ntp),
                                 region<int32_t>(workspace, p.off_offsets),
                                 p.tiled ? p.tile_rows : 0,
                                 p.tiled ? region<int32_t>(workspace, p.off_tiles) : nullptr,
                                 ones, clear, H, s);
    });
    if (err != hipSuccess) return hip_fail(err, "masked align launch");
  } else {
    err = staged(QMOE_STAGE_ALIGN, s, [&] {
      return launch_grouped_routing(route, E, T, ones, clear, H, s);
    });
    if (err != hipSuccess) return hip_fail(err, "grouped routing launch");
    err = w4a16_align(p, route, E, workspace, s);
    if (err != hipSuccess) return hip_fail(err, "align launch");
  }
  // topk_ids is only read by the combine pass, which the grouped layouts do not run
  return w4a16_after_align(p, a, w13, s13, w2, s2, masked ? nullptr : route, ones, T, H, I, E, 1,
                           out, workspace, s, nullptr, nullptr, /*direct_out=*/true);
}

}  // namespace
}  // namespace qmoe

using namespace qmoe;

extern "C" {

int32_t qmoe_abi_version(void) { return QMOE_ABI_VERSION; }

const char* qmoe_status_string(int32_t status) {
  switch (status) {
    case QMOE_OK: return "ok";
    case QMOE_ERR_INVALID_ARG: return "invalid argument";
    case QMOE_ERR_UNSUPPORTED: return "unsupported shape or format";
    case QMOE_ERR_WORKSPACE: return "workspace too small";
    case QMOE_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* qmoe_last_error(void) { return g_last_error; }

qmoe_status moe_align(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t block_m,
                      int32_t* sorted_ids, int32_t* expert_ids, int32_t* num_tokens_padded,
                      int32_t* expert_offsets, void* stream) {
  g_last_error[0] = 0;
  if (T < 0 || k <= 0 || E <= 0)
    return fail(QMOE_ERR_INVALID_ARG, "bad sizes T=%d k=%d E=%d", T, k, E);
  if (E > QMOE_MAX_EXPERTS)
    return fail(QMOE_ERR_UNSUPPORTED, "expert count %d exceeds %d", E, QMOE_MAX_EXPERTS);
  if (block_m < 1 || block_m > 256 || (block_m & (block_m - 1)))
    return fail(QMOE_ERR_INVALID_ARG, "block_m %d must be a power of two in [1, 256]", block_m);
  const int64_t P = (int64_t)T * k, L = P + (int64_t)E * (block_m - 1);
  if (L >= (int64_t(1) << 31)) return fail(QMOE_ERR_UNSUPPORTED, "too many routed pairs");
  if ((P > 0 && !topk_ids) || !sorted_ids || !expert_ids || !num_tokens_padded)
    return fail(QMOE_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned(topk_ids, 4) || !aligned(sorted_ids, 4) || !aligned(expert_ids, 4) ||
      !aligned(num_tokens_padded, 4) || !aligned(expert_offsets, 4))
    return fail(QMOE_ERR_INVALID_ARG, "pointers must be 4-byte aligned");
  const int64_t NB = (L + block_m - 1) / block_m;
  hipError_t err = launch_align(topk_ids, (int32_t)P, E, block_m, (int32_t)L, (int32_t)NB,
                                sorted_ids, expert_ids, num_tokens_padded, expert_offsets, 0,
                                nullptr, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "align launch");
  return QMOE_OK;
}

qmoe_status moe_topk_softmax(const float* logits, int32_t T, int32_t E, int32_t k,
                             int32_t renormalize, const int32_t* expert_map, int32_t* topk_ids,
                             float* topk_weights, void* stream) {
  g_last_error[0] = 0;
  if (T < 0 || E <= 0 || k <= 0 || k > E)
    return fail(QMOE_ERR_INVALID_ARG, "bad sizes T=%d E=%d k=%d", T, E, k);
  if (E > QMOE_MAX_EXPERTS)
    return fail(QMOE_ERR_UNSUPPORTED, "expert count %d exceeds %d", E, QMOE_MAX_EXPERTS);
  if (T > 0 && (!logits || !topk_ids || !topk_weights))
    return fail(QMOE_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned(logits, 4) || !aligned(expert_map, 4) || !aligned(topk_ids, 4) ||
      !aligned(topk_weights, 4))
    return fail(QMOE_ERR_INVALID_ARG, "pointers must be 4-byte aligned");
  hipError_t err = launch_topk_softmax(logits, T, E, k, renormalize ? 1 : 0, expert_map, topk_ids,
                                       topk_weights, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "router launch");
  return QMOE_OK;
}

qmoe_status qmoe_plan(int32_t format, int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                      int32_t schedule, int32_t* chosen, int32_t* block_m,
                      size_t* workspace_bytes) {
  g_last_error[0] = 0;
  if (format != kW4A16 && format != kFp8 && format != kMxfp4 && format != kNvfp4)
    return fail(QMOE_ERR_INVALID_ARG, "unknown format %d", format);
  qmoe_status st = check_shape(format, T, H, I, E, k, schedule);
  if (st != QMOE_OK) return st;
  Plan p = make_plan(format, T, H, I, E, k, schedule);
  if (chosen) *chosen = p.schedule;
  if (block_m) *block_m = p.block_m;
  if (workspace_bytes) *workspace_bytes = p.total;
  return QMOE_OK;
}

qmoe_status qmoe_set_tuning(int32_t tile_rows, int32_t rows_per_pass, int32_t kslices,
                            int32_t tile_grid) {
  g_last_error[0] = 0;
  if (tile_rows != 0 && tile_rows != 128 && tile_rows != 256)
    return fail(QMOE_ERR_INVALID_ARG, "tile_rows %d: 0, 128 or 256", tile_rows);
  if (rows_per_pass != 0 && rows_per_pass != 16 && rows_per_pass != 32)
    return fail(QMOE_ERR_INVALID_ARG, "rows_per_pass %d: 0, 16 or 32", rows_per_pass);
  if (kslices < 0 || kslices > 64 || (kslices & (kslices - 1)))
    return fail(QMOE_ERR_INVALID_ARG, "kslices %d: 0 or a power of two up to 64", kslices);
  if (tile_grid != 0 && tile_grid != 1)
    return fail(QMOE_ERR_INVALID_ARG, "tile_grid %d: 0 or 1", tile_grid);
  g_tune_tile_rows.store(tile_rows);
  g_tune_rows_per_pass.store(rows_per_pass);
  g_tune_kslices.store(kslices);
  set_tiled_one_per_tile(tile_grid == 1);
  return QMOE_OK;
}

qmoe_status qmoe_workspace_regions(int32_t format, int32_t T, int32_t H, int32_t I, int32_t E,
                                   int32_t k, int32_t schedule, int64_t* offsets, int64_t* sizes) {
  g_last_error[0] = 0;
  if (format != kW4A16 && format != kFp8 && format != kMxfp4 && format != kNvfp4)
    return fail(QMOE_ERR_INVALID_ARG, "unknown format %d", format);
  if (!offsets) return fail(QMOE_ERR_INVALID_ARG, "offsets is NULL");
  qmoe_status st = check_shape(format, T, H, I, E, k, schedule);
  if (st != QMOE_OK) return st;
  const Plan p = make_plan(format, T, H, I, E, k, schedule);
  for (int i = 0; i < QMOE_NUM_REGIONS; ++i) {
    const bool has = p.off[i] != kNoRegion;
    offsets[i] = has ? (int64_t)p.off[i] : -1;
    if (sizes) sizes[i] = has ? (int64_t)p.len[i] : 0;
  }
  return QMOE_OK;
}

namespace {
qmoe_status four_bit_forward(int fmt, const uint16_t* x, const uint8_t* w13, const void* s13,
                             const uint8_t* w2, const void* s2, const int32_t* topk_ids,
                             const float* topk_weights, int32_t T, int32_t H, int32_t I,
                             int32_t E, int32_t k, int32_t schedule, uint16_t* out,
                             void* workspace, size_t* workspace_bytes, void* stream,
                             const float* g13 = nullptr, const float* g2 = nullptr) {
  g_last_error[0] = 0;
  qmoe_status st = check_shape(fmt, T, H, I, E, k, schedule);
  if (st != QMOE_OK) return st;
  if (!workspace_bytes) return fail(QMOE_ERR_INVALID_ARG, "workspace_bytes is NULL");
  const Plan p = make_plan(fmt, T, H, I, E, k, schedule);
  if (!workspace) {
    *workspace_bytes = p.total;
    return QMOE_OK;
  }
  if (*workspace_bytes < p.total)
    return fail(QMOE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", *workspace_bytes, p.total);
  if (T == 0) return QMOE_OK;
  const void* ptrs[] = {x, w13, s13, w2, s2, topk_ids, topk_weights, out};
  for (const void* q : ptrs)
    if (!q) return fail(QMOE_ERR_INVALID_ARG, "NULL tensor pointer");
  for (const void* q : ptrs)
    if (!aligned(q, 16)) return fail(QMOE_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (!aligned(workspace, kRegionAlign))
    return fail(QMOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (fmt == kNvfp4 && (!g13 || !g2 || !aligned(g13, 4) || !aligned(g2, 4)))
    return fail(QMOE_ERR_INVALID_ARG, "g13 and g2 must be 4-byte aligned device pointers");

  return w4a16_run(p, x, w13, static_cast<const uint16_t*>(s13), w2,
                   static_cast<const uint16_t*>(s2), topk_ids, topk_weights, T, H, I, E, k, out,
                   workspace, static_cast<hipStream_t>(stream), g13, g2);
}
}  // namespace

qmoe_status moe_w4a16_forward(const uint16_t* x, const uint8_t* w13, const uint16_t* s13,
                              const uint8_t* w2, const uint16_t* s2, const int32_t* topk_ids,
                              const float* topk_weights, int32_t T, int32_t H, int32_t I,
                              int32_t E, int32_t k, int32_t schedule, uint16_t* out,
                              void* workspace, size_t* workspace_bytes, void* stream) {
  return four_bit_forward(kW4A16, x, w13, s13, w2, s2, topk_ids, topk_weights, T, H, I, E, k,
                          schedule, out, workspace, workspace_bytes, stream);
}

// Scratch of moe_w4a16_forward_noalloc: one array per GPU, in device memory for the life
// of the process. Host code never uses the name itself (on the host it is only a
// stand-in symbol, not a device address): its device address comes from
// hipGetSymbolAddress, once per device, and only that address is passed on.
static __device__ __align__(256) uint8_t scratch[QMOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on its first use).
qmoe_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return hip_fail(err, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(QMOE_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !ptr) return hip_fail(err, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return QMOE_OK;
}
}  // namespace

qmoe_status moe_w4a16_forward_noalloc(const uint16_t* x, const uint8_t* w13, const uint16_t* s13,
                                      const uint8_t* w2, const uint16_t* s2,
                                      const int32_t* topk_ids, const float* topk_weights,
                                      int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                      int32_t schedule, uint16_t* out, void* stream) {
  g_last_error[0] = 0;
  qmoe_status st = check_shape(kW4A16, T, H, I, E, k, schedule);
  if (st != QMOE_OK) return st;
  const Plan p = make_plan(kW4A16, T, H, I, E, k, schedule);
  if (p.total > (size_t)QMOE_NOALLOC_SCRATCH_BYTES)
    return fail(QMOE_ERR_UNSUPPORTED,
                "this forward needs %zu bytes of scratch; the static scratch holds %zu "
                "(use moe_w4a16_forward with a workspace)",
                p.total, (size_t)QMOE_NOALLOC_SCRATCH_BYTES);
  if (T == 0) return QMOE_OK;
  const void* ptrs[] = {x, w13, s13, w2, s2, topk_ids, topk_weights, out};
  for (const void* q : ptrs)
    if (!q) return fail(QMOE_ERR_INVALID_ARG, "NULL tensor pointer");
  for (const void* q : ptrs)
    if (!aligned(q, 16)) return fail(QMOE_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != QMOE_OK) return st;
  return w4a16_run(p, x, w13, s13, w2, s2, topk_ids, topk_weights, T, H, I, E, k, out, ws,
                   static_cast<hipStream_t>(stream));
}

qmoe_status moe_mxfp4_forward(const uint16_t* x, const uint8_t* w13, const uint8_t* s13,
                              const uint8_t* w2, const uint8_t* s2, const int32_t* topk_ids,
                              const float* topk_weights, int32_t T, int32_t H, int32_t I,
                              int32_t E, int32_t k, int32_t schedule, uint16_t* out,
                              void* workspace, size_t* workspace_bytes, void* stream) {
  return four_bit_forward(kMxfp4, x, w13, s13, w2, s2, topk_ids, topk_weights, T, H, I, E, k,
                          schedule, out, workspace, workspace_bytes, stream);
}

qmoe_status moe_nvfp4_forward(const uint16_t* x, const uint8_t* w13, const uint8_t* s13,
                              const float* g13, const uint8_t* w2, const uint8_t* s2,
                              const float* g2, const int32_t* topk_ids,
                              const float* topk_weights, int32_t T, int32_t H, int32_t I,
                              int32_t E, int32_t k, int32_t schedule, uint16_t* out,
                              void* workspace, size_t* workspace_bytes, void* stream) {
  return four_bit_forward(kNvfp4, x, w13, s13, w2, s2, topk_ids, topk_weights, T, H, I, E, k,
                          schedule, out, workspace, workspace_bytes, stream, g13, g2);
}

qmoe_status moe_w4a16_grouped_contiguous(const uint16_t* a, const uint8_t* w13,
                                         const uint16_t* s13, const uint8_t* w2,
                                         const uint16_t* s2, const int32_t* m_indices, int32_t M,
                                         int32_t H, int32_t I, int32_t E, int32_t expected_m,
                                         int32_t schedule, uint16_t* out, void* workspace,
                                         size_t* workspace_bytes, void* stream) {
  return w4a16_grouped(false, a, w13, s13, w2, s2, m_indices, M, H, I, E, expected_m, schedule,
                       out, workspace, workspace_bytes, stream);
}

qmoe_status moe_w4a16_grouped_masked(const uint16_t* a, const uint8_t* w13, const uint16_t* s13,
                                     const uint8_t* w2, const uint16_t* s2,
                                     const int32_t* masked_m, int32_t max_m, int32_t H, int32_t I,
                                     int32_t E, int32_t expected_m, int32_t schedule,
                                     uint16_t* out, void* workspace, size_t* workspace_bytes,
                                     void* stream) {
  return w4a16_grouped(true, a, w13, s13, w2, s2, masked_m, max_m, H, I, E, expected_m, schedule,
                       out, workspace, workspace_bytes, stream);
}

qmoe_status moe_fp8_block_forward(const uint8_t* a_q, const float* a_scale, const uint8_t* w13,
                                  const float* s13, const uint8_t* w2, const float* s2,
                                  const int32_t* topk_ids, const float* topk_weights, int32_t T,
                                  int32_t H, int32_t I, int32_t E, int32_t k, int32_t schedule,
                                  uint16_t* out, void* workspace, size_t* workspace_bytes,
                                  void* stream) {
  g_last_error[0] = 0;
  qmoe_status st = check_shape(kFp8, T, H, I, E, k, schedule);
  if (st != QMOE_OK) return st;
  if (!workspace_bytes) return fail(QMOE_ERR_INVALID_ARG, "workspace_bytes is NULL");
  const Plan p = make_plan(kFp8, T, H, I, E, k, schedule);
  if (!workspace) {
    *workspace_bytes = p.total;
    return QMOE_OK;
  }
  if (*workspace_bytes < p.total)
    return fail(QMOE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", *workspace_bytes, p.total);
  if (T == 0) return QMOE_OK;
  const void* ptrs[] = {a_q, a_scale, w13, s13, w2, s2, topk_ids, topk_weights, out};
  for (const void* q : ptrs)
    if (!q) return fail(QMOE_ERR_INVALID_ARG, "NULL tensor pointer");
  for (const void* q : ptrs)
    if (!aligned(q, 16)) return fail(QMOE_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (!aligned(workspace, kRegionAlign))
    return fail(QMOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");

  hipStream_t s = static_cast<hipStream_t>(stream);
  Routing r{};
  r.sorted_ids = region<int32_t>(workspace, p.off_sorted);
  r.offsets = region<int32_t>(workspace, p.off_offsets);
  r.tile_offsets = region<int32_t>(workspace, p.off_tiles);
  r.expert_ids = region<int32_t>(workspace, p.off_expert_ids);
  r.ntp = region<int32_t>(workspace, p.off_ntp);
  r.topk_weights = topk_weights;
  r.P = (int32_t)p.P;
  r.k = k;
  r.E = E;
  r.L = (int32_t)p.L;
  Fp8Problem prob{a_q, a_scale, w13, s13, w2, s2,
                  region<float>(workspace, p.off_h32), region<uint8_t>(workspace, p.off_hq),
                  region<float>(workspace, p.off_hs), region<float>(workspace, p.off_out32),
                  T, H, I};

  if (p.tiled) {
    hipError_t err = staged(QMOE_STAGE_ALIGN, s, [&] {
      return launch_align(topk_ids, r.P, E, p.block_m, r.L, (int32_t)p.NB,
                          region<int32_t>(workspace, p.off_sorted),
                          region<int32_t>(workspace, p.off_expert_ids),
                          region<int32_t>(workspace, p.off_ntp),
                          region<int32_t>(workspace, p.off_offsets), fp8_tiled_rows(),
                          region<int32_t>(workspace, p.off_tiles), s);
    });
    if (err != hipSuccess) return hip_fail(err, "align launch");
    // gate_up writes h already quantized (E4M3 per row and 128 columns).
    err = staged(QMOE_STAGE_GATE_UP, s, [&] { return launch_fp8_gateup_tiled(prob, r, s); });
    if (err != hipSuccess) return hip_fail(err, "gate_up launch");
    float* y = region<float>(workspace, p.off_y);
    err = staged(QMOE_STAGE_DOWN, s, [&] { return launch_fp8_down_tiled(prob, r, y, s); });
    if (err != hipSuccess) return hip_fail(err, "down launch");
    err = staged(QMOE_STAGE_CAST, s, [&] {
      return launch_combine_rows(y, topk_ids, nullptr, T, k, E, H, out, s);
    });
    if (err != hipSuccess) return hip_fail(err, "combine launch");
    return QMOE_OK;
  }

  hipError_t err = staged(QMOE_STAGE_ZERO, s, [&] {
    return launch_zero_f32(prob.out32, (int64_t)T * H, s);
  });
  if (err != hipSuccess) return hip_fail(err, "zero launch");
  err = staged(QMOE_STAGE_ALIGN, s, [&] {
    return launch_align(topk_ids, r.P, E, p.block_m, r.L, (int32_t)p.NB,
                        region<int32_t>(workspace, p.off_sorted),
                        region<int32_t>(workspace, p.off_expert_ids),
                        region<int32_t>(workspace, p.off_ntp),
                        region<int32_t>(workspace, p.off_offsets), 0, nullptr, s);
  });
  if (err != hipSuccess) return hip_fail(err, "align launch");
  err = staged(QMOE_STAGE_GATE_UP, s, [&] { return launch_fp8_gateup_stream(prob, r, p.mb, s); });
  if (err != hipSuccess) return hip_fail(err, "gate_up launch");
  err = staged(QMOE_STAGE_REQUANT, s, [&] {
    return launch_fp8_quantize_blocks(prob.h32, p.L, I, 1, 128, prob.hq, prob.hs, s);
  });
  if (err != hipSuccess) return hip_fail(err, "h requant launch");
  err = staged(QMOE_STAGE_DOWN, s, [&] { return launch_fp8_down_stream(prob, r, p.mb, s); });
  if (err != hipSuccess) return hip_fail(err, "down launch");
  err = staged(QMOE_STAGE_CAST, s, [&] {
    return launch_cast_f32_bf16(prob.out32, out, (int64_t)T * H, s);
  });
  if (err != hipSuccess) return hip_fail(err, "cast launch");
  return QMOE_OK;
}

namespace {
qmoe_status check_quantize_args(const void* v, int64_t R, int64_t C, int32_t br, int32_t bc,
                                const uint8_t* q, const float* scale, size_t v_align) {
  if (R < 0 || C < 0) return fail(QMOE_ERR_INVALID_ARG, "negative size");
  if (br < 1 || br > 128 || bc < 1 || bc > 1024 || (int64_t)br * bc > 16384)
    return fail(QMOE_ERR_UNSUPPORTED, "block [%d, %d] outside [1..128] x [1..1024]", br, bc);
  if (R == 0 || C == 0) return QMOE_OK;
  if (!v || !q || !scale) return fail(QMOE_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned(v, v_align) || !aligned(scale, 4))
    return fail(QMOE_ERR_INVALID_ARG, "pointers must be aligned (values %zu bytes, scales 4)",
                v_align);
  return QMOE_OK;
}
}  // namespace

qmoe_status qmoe_fp8_quantize_blocks(const float* v, int64_t R, int64_t C, int32_t br, int32_t bc,
                                     uint8_t* q, float* scale, void* stream) {
  g_last_error[0] = 0;
  const qmoe_status st = check_quantize_args(v, R, C, br, bc, q, scale, 4);
  if (st != QMOE_OK || R == 0 || C == 0) return st;
  hipError_t err = launch_fp8_quantize_blocks(v, R, C, br, bc, q, scale,
                                              static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "quantize launch");
  return QMOE_OK;
}

qmoe_status qmoe_fp8_quantize_blocks_bf16(const uint16_t* v, int64_t R, int64_t C, int32_t br,
                                          int32_t bc, uint8_t* q, float* scale, void* stream) {
  g_last_error[0] = 0;
  const qmoe_status st = check_quantize_args(v, R, C, br, bc, q, scale, 2);
  if (st != QMOE_OK || R == 0 || C == 0) return st;
  hipError_t err = launch_fp8_quantize_blocks_bf16(v, R, C, br, bc, q, scale,
                                                   static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "quantize launch");
  return QMOE_OK;
}

qmoe_status qmoe_timing_begin(int32_t max_calls) {
  g_last_error[0] = 0;
  if (max_calls < 1 || max_calls > 100000)
    return fail(QMOE_ERR_INVALID_ARG, "max_calls %d outside [1, 100000]", max_calls);
  std::lock_guard<std::mutex> lk(g_timer.mu);
  g_timer.clear();
  for (auto& v : g_timer.ev) {
    v.resize(2 * (size_t)max_calls, nullptr);
    for (hipEvent_t& e : v) {
      hipError_t err = hipEventCreate(&e);
      if (err != hipSuccess) {
        g_timer.clear();
        return hip_fail(err, "hipEventCreate");
      }
    }
  }
  g_timer.cap = max_calls;
  g_timer.on = true;
  return QMOE_OK;
}

qmoe_status qmoe_timing_pause(int32_t paused) {
  g_last_error[0] = 0;
  std::lock_guard<std::mutex> lk(g_timer.mu);
  if (g_timer.cap == 0) return fail(QMOE_ERR_INVALID_ARG, "timing not begun");
  g_timer.on = paused == 0;
  return QMOE_OK;
}

qmoe_status qmoe_timing_end(float* ms_sum, int32_t* count) {
  g_last_error[0] = 0;
  if (!ms_sum || !count) return fail(QMOE_ERR_INVALID_ARG, "NULL output");
  std::lock_guard<std::mutex> lk(g_timer.mu);
  g_timer.on = false;
  qmoe_status st = QMOE_OK;
  for (int stg = 0; stg < QMOE_NUM_STAGES; ++stg) {
    float sum = 0.f;
    for (int i = 0; i < g_timer.used[stg]; ++i) {
      hipEvent_t e0 = g_timer.ev[stg][2 * i], e1 = g_timer.ev[stg][2 * i + 1];
      float ms = 0.f;
      hipError_t err = hipEventSynchronize(e1);
      if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
      if (err != hipSuccess) {
        st = hip_fail(err, "stage event");
        break;
      }
      sum += ms;
    }
    ms_sum[stg] = sum;
    count[stg] = g_timer.used[stg];
  }
  g_timer.clear();
  return st;
}

}  // extern "C"
