/*
 * qmoe.h - C ABI of the MI355X (gfx950) routed, weight-quantized MoE expert FFN.
 *
 * One routed MoE layer's expert FFN, on one GPU:
 *   align (sort token slots to experts) -> gate_up grouped GEMM with INT4 group-32
 *   dequantization (or block FP8) -> SiLU(gate) * up -> down grouped GEMM ->
 *   top-k weighted combine (scatter-add) -> bf16 output.
 *
 * Sources (web pages, cited by title and section):
 *   [CHORD] "vLLM x Novita AI: Chord W4A16 INT4 MoE Kernel for Kimi K2.x" (Novita AI
 *           blog): summary; "Two kernel families"; "vLLM integration"; "Kernel
 *           optimizations" (indexed kernels; H200 and Blackwell indexed decode;
 *           SM90 grouped kernels); Figure 3 (where the padding lives); "Measurements"
 *           (the grouped prefill and decode rows).
 *   [XT]    "xiaotu-moe" (PyPI project page): overview (the MoE engine's weight
 *           formats: BF16, FP8 (WNA16), MXFP4 (E2M1), NVFP4).
 *   [LSG]   "guqiong96/Lsglang" README (SkillsMP page): quick start (an NVFP4-W4A16
 *           checkpoint), supported quant formats.
 *   [SGL]   "SGLang W8A8 Block FP8 quantization kernel config guide" (xdnf.cn):
 *           background section (E4M3, [BLOCK_N, BLOCK_K] weight blocks, per-token-group
 *           activation scales As, weight block scales Bs); kernel dispatch section
 *           (cdiv(N, block_n) == Bs.shape[0], cdiv(K, block_k) == Bs.shape[1]).
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller. The library never
 *     allocates or frees caller memory and never synchronizes the stream; all work is
 *     enqueued on `stream` (a hipStream_t passed as void*, NULL = the null stream).
 *   - Tensors are dense, row-major, contiguous. bf16 values travel as uint16_t bit
 *     patterns; E4M3 values as uint8_t bit patterns of OCP E4M3FN (max 448).
 *   - Pointers must be 16-byte aligned unless stated otherwise.
 *   - Arguments are checked before anything touches the GPU; a failed check returns
 *     QMOE_ERR_INVALID_ARG or QMOE_ERR_UNSUPPORTED and enqueues nothing. A failed
 *     launch returns QMOE_ERR_HIP (the HIP error state is read and cleared).
 *     qmoe_last_error() then returns a message for the calling thread.
 *   - Entry points are thread-safe; calls that share output or workspace memory on
 *     the same GPU must be ordered by the caller (same stream or events).
 *   - Nothing reads a device value back to the host: every launch is sized for the
 *     worst case and surplus work-groups exit on the device, so a forward can be
 *     captured into a hipGraph ([CHORD] "vLLM integration": over-allocated align
 *     buffers consumed without reading the routed count back).
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QMOE_ABI_VERSION 1

typedef enum qmoe_status {
  QMOE_OK = 0,
  QMOE_ERR_INVALID_ARG = 1, /* NULL or misaligned pointer, negative or inconsistent size */
  QMOE_ERR_UNSUPPORTED = 2, /* well-formed but outside the supported shapes            */
  QMOE_ERR_WORKSPACE = 3,   /* workspace smaller than the size the query returned       */
  QMOE_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed               */
} qmoe_status;

/* Schedules of the forward passes. AUTO picks from routed tokens per expert,
 * tok_e = T*k/E (a host-side quantity; no device readback): the bandwidth-bound
 * decode profile up to the crossover (measured: 44 for W4A16, 60 for MXFP4, 36 for
 * NVFP4, 20 for block FP8), the MFMA-bound prefill profile above it
 * ([CHORD] "Kernel optimizations": the per-expert routed token count, not the total,
 * decides which schedule wins; profiles tune on token counts). DECODE and PREFILL
 * force one profile; both give results within the same tolerance. */
typedef enum qmoe_schedule {
  QMOE_SCHEDULE_AUTO = 0,
  QMOE_SCHEDULE_DECODE = 1,
  QMOE_SCHEDULE_PREFILL = 2
} qmoe_schedule;

/* Limits: 1 <= E <= QMOE_MAX_EXPERTS, 1 <= k <= E, T*k + E*(block_m-1) < 2^31. */
#define QMOE_MAX_EXPERTS 4096

/* ABI version of the loaded library (QMOE_ABI_VERSION it was built with). */
int32_t qmoe_abi_version(void);

/* Static English name of a status code. */
const char* qmoe_status_string(int32_t status);

/* Message describing the last non-OK status returned on the calling thread
 * (empty string if none). Valid until the next call on that thread. */
const char* qmoe_last_error(void);

/*
 * moe_topk_softmax - the router step before align: for each token, the k experts with
 * the largest router logits and their softmax weights ([CHORD] "Two kernel families":
 * the indexed kernels consume the framework's routing, these ids and weights; "vLLM
 * integration": under expert parallelism, the EP8 profiles, a GPU holds a share of the
 * experts).
 *
 *   logits        [T, E] fp32, finite.
 *   k             1 <= k <= E <= QMOE_MAX_EXPERTS.
 *   renormalize   nonzero: the k weights sum to 1; zero: they are the selected experts'
 *                 full softmax probabilities.
 *   expert_map    [E] int32 or NULL. Local id of each (global) expert, or -1 for an
 *                 expert held by another GPU; moe_align and the forwards drop slots whose
 *                 id is outside [0, E_local), so the outputs pass to them unchanged.
 *                 NULL: ids stay global.
 *   topk_ids      [T, k] int32 out: slot s holds the expert with the (s+1)-th largest
 *                 logit (equal logits: the lower expert id first; -0 equals +0), mapped.
 *   topk_weights  [T, k] fp32 out: exp(l - m) / S, m the token's largest logit and S the
 *                 sum of exp(l - m) over the k selected experts (renormalize) or over all
 *                 E experts. Weights of unmapped (-1) slots are kept: they belong to the
 *                 GPU holding that expert.
 * Selection compares logits, which orders the experts as their softmax probabilities do
 * (exp is increasing) without exp's rounding. T = 0 is allowed. 4-byte alignment.
 */
qmoe_status moe_topk_softmax(const float* logits, int32_t T, int32_t E, int32_t k,
                             int32_t renormalize, const int32_t* expert_map, int32_t* topk_ids,
                             float* topk_weights, void* stream);

/*
 * moe_align - sort routed (token, slot) pairs to experts and pad each expert's
 * segment to a multiple of block_m ([CHORD] "Two kernel families": the indexed
 * family consumes sorted_ids / expert_ids / num_tokens_padded; Figure 3: padding
 * lives in the routing indices, -1 marks padding).
 *
 *   topk_ids          [T, k] int32: expert of slot s of token t. Flat pair index
 *                     i = t*k + s. Ids outside [0, E) are dropped (never written).
 *   block_m           power of two, 1 <= block_m <= 256.
 *   sorted_ids        [L] int32, L = T*k + E*(block_m - 1). Expert e owns the segment
 *                     [off[e], off[e+1]) with off[e+1] - off[e] = ceil(c_e / block_m) *
 *                     block_m, c_e = number of pairs routed to e. The segment starts
 *                     with e's pair indices in ascending order; its remaining slots,
 *                     and every slot from off[E] to L, hold the sentinel T*k.
 *   expert_ids        [ceil(L / block_m)] int32: expert of each block_m-row block;
 *                     -1 for blocks at or past off[E].
 *   num_tokens_padded [1] int32: off[E].
 *   expert_offsets    [E + 1] int32: off, or NULL.
 * All outputs are fully written on every call (no pre-clearing needed). The result is
 * deterministic: bit-identical to a stable counting sort on the host. T = 0 is allowed.
 * Pointers here need only 4-byte alignment.
 */
qmoe_status moe_align(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t block_m,
                      int32_t* sorted_ids, int32_t* expert_ids, int32_t* num_tokens_padded,
                      int32_t* expert_offsets, void* stream);

/*
 * moe_w4a16_forward - routed MoE expert FFN with BF16 activations and INT4 group-32
 * weights with BF16 scales ([CHORD] summary: BF16 activations, INT4 weights, group-32
 * scales; "vLLM integration": uint4 codes, group 32, BF16 scales; "H200 and Blackwell
 * indexed decode": the weight is the code minus the zero point, then scaled).
 *
 *   x            [T, H] bf16.
 *   w13, s13     [E, 2I, H/2] uint8 and [E, 2I, H/32] bf16: fused gate (rows [0, I))
 *                and up (rows [I, 2I)) projections. Byte c/2 of a row holds code c in
 *                its low nibble for even c, high nibble for odd c; weight(n, c) =
 *                (code - 8) * s13[n, c/32].
 *   w2, s2       [E, H, I/2] uint8 and [E, H, I/32] bf16: down projection, same format.
 *   topk_ids     [T, k] int32 (see moe_align); topk_weights [T, k] fp32.
 *   out          [T, H] bf16, overwritten:
 *                out[t] = bf16(sum_s topk_weights[t,s] * FFN_{topk_ids[t,s]}(x[t])),
 *                FFN_e(v) = W2_e (silu(W13_e[0:I] v) * W13_e[I:2I] v), fp32 accumulation.
 *   schedule     a qmoe_schedule value.
 *   workspace    device scratch, 256-byte aligned. If NULL, nothing is launched and the
 *                required size is written to *workspace_bytes (same shapes and schedule).
 *                Otherwise *workspace_bytes is the size provided; less than required ->
 *                QMOE_ERR_WORKSPACE. Contents need no initialization and are clobbered.
 * Requires H % 32 == 0 and I % 32 == 0 (QMOE_ERR_UNSUPPORTED otherwise; [CHORD] "vLLM
 * integration": unsupported schemes fail instead of silently picking a wrong kernel).
 * T = 0 writes nothing and returns QMOE_OK.
 */
qmoe_status moe_w4a16_forward(const uint16_t* x, const uint8_t* w13, const uint16_t* s13,
                              const uint8_t* w2, const uint16_t* s2, const int32_t* topk_ids,
                              const float* topk_weights, int32_t T, int32_t H, int32_t I,
                              int32_t E, int32_t k, int32_t schedule, uint16_t* out,
                              void* workspace, size_t* workspace_bytes, void* stream);

/*
 * moe_w4a16_forward_noalloc - moe_w4a16_forward without a workspace argument, for callers
 * that cannot allocate device memory around the call (code under stream capture into a
 * hipGraph, tight serving loops, harnesses that forbid hipMalloc). Its scratch is a
 * static device array of QMOE_NOALLOC_SCRATCH_BYTES per GPU, held from the library's
 * load until the process ends; nothing is allocated or freed, here or later.
 *   Arguments and result as moe_w4a16_forward (same kernels, same output).
 *   A forward whose plan needs more scratch than that (moe_w4a16_forward's workspace size
 *   for the same shapes and schedule) returns QMOE_ERR_UNSUPPORTED before touching the
 *   GPU: 64 MiB covers decode batches (the 32-token, 48-expert layer of hidden 7168 needs
 *   18 MB), not large prefill batches.
 *   Every call on one GPU shares that GPU's array, so calls that overlap in time on one GPU
 *   (different streams, or different host threads without ordering) race and must be
 *   serialized by the caller; consecutive calls on one stream are safe (every region is
 *   written before it is read in each call).
 */
#define QMOE_NOALLOC_SCRATCH_BYTES (64u << 20)
qmoe_status moe_w4a16_forward_noalloc(const uint16_t* x, const uint8_t* w13, const uint16_t* s13,
                                      const uint8_t* w2, const uint16_t* s2,
                                      const int32_t* topk_ids, const float* topk_weights,
                                      int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                      int32_t schedule, uint16_t* out, void* stream);

/*
 * moe_w4a16_grouped_contiguous - the W4A16 expert FFN on the contiguous grouped layout
 * ([CHORD] "Kernel optimizations", SM90 grouped kernels, and Figure 3: the rows are
 * concatenated expert by expert, each expert's run padded, with an int32 expert index
 * per row and -1 on padding rows). Each row is one (row, expert) pair of weight 1:
 *
 *   a            [M, H] bf16 rows.
 *   m_indices    [M] int32 (4-byte alignment suffices): the row's expert; -1 (any value
 *                outside [0, E)) marks a padding row. Rows need not be sorted.
 *   out          [M, H] bf16, overwritten: out[r] = bf16(FFN_{m_indices[r]}(a[r])) with
 *                FFN_e as in moe_w4a16_forward, and 0 on padding rows.
 *   expected_m   rows per expert the caller expects (a host-side hint that picks the
 *                AUTO schedule); 0 = M / E.
 *   w13, s13, w2, s2, H, I, E, schedule, workspace: as moe_w4a16_forward (the weights
 *   are the same canonical tensors: no separate packing per layout). The workspace
 *   size differs from moe_w4a16_forward's; query it with workspace = NULL.
 * Equal to moe_w4a16_forward with topk_ids = m_indices as [M, 1] and weights 1.
 */
qmoe_status moe_w4a16_grouped_contiguous(const uint16_t* a, const uint8_t* w13,
                                         const uint16_t* s13, const uint8_t* w2,
                                         const uint16_t* s2, const int32_t* m_indices, int32_t M,
                                         int32_t H, int32_t I, int32_t E, int32_t expected_m,
                                         int32_t schedule, uint16_t* out, void* workspace,
                                         size_t* workspace_bytes, void* stream);

/*
 * moe_w4a16_grouped_masked - the W4A16 expert FFN on the masked grouped layout ([CHORD]
 * "Kernel optimizations", SM90 grouped kernels: a fixed budget of max_m rows per expert,
 * a device-side count of the valid rows, a host-side expected count that picks the
 * launch, and a flat output whose rows past the count are not part of the result).
 *
 *   a            [E, max_m, H] bf16 (or [E * max_m, H]): row r of expert g at g*max_m + r.
 *   masked_m     [E] int32 on the device (4-byte alignment suffices): valid rows of each
 *                expert; a count above max_m means max_m, a negative count 0. Read only
 *                on the device, so a forward can be captured into a hipGraph.
 *   out          [E * max_m, H] bf16, overwritten: out[g*max_m + r] = bf16(FFN_g(a[g, r]))
 *                for r < masked_m[g], and 0 on the rows past the count.
 *   expected_m   host-side hint of the valid rows per expert (0 = max_m).
 *   w13, s13, w2, s2, H, I, E, schedule, workspace: as moe_w4a16_grouped_contiguous.
 */
qmoe_status moe_w4a16_grouped_masked(const uint16_t* a, const uint8_t* w13, const uint16_t* s13,
                                     const uint8_t* w2, const uint16_t* s2,
                                     const int32_t* masked_m, int32_t max_m, int32_t H, int32_t I,
                                     int32_t E, int32_t expected_m, int32_t schedule,
                                     uint16_t* out, void* workspace, size_t* workspace_bytes,
                                     void* stream);

/*
 * moe_mxfp4_forward - routed MoE expert FFN with BF16 activations and MXFP4 weights
 * ([XT] overview: MXFP4 (E2M1) is one of the weight-only formats of the MoE engine, beside
 * BF16, FP8 (WNA16) and NVFP4). Reading: the OCP microscaling layout, one E8M0 scale per
 * weight row and 32 consecutive k, with E2M1 codes packed two per byte like the INT4 codes.
 *
 *   w13, s13     [E, 2I, H/2] uint8 and [E, 2I, H/32] uint8: byte c/2 of a row holds
 *                E2M1 code c in its low nibble for even c, high nibble for odd c (bit 3
 *                sign, bits 2..1 exponent with bias 1, bit 0 mantissa; exponent 0 is
 *                0.5 * mantissa); s13 holds E8M0 codes, weight(n, c) = e2m1(code) *
 *                2^(s13[n, c/32] - 127).
 *   w2, s2       [E, H, I/2] and [E, H, I/32] uint8: down projection, same format.
 *   x, topk_ids, topk_weights, T, H, I, E, k, schedule, out, workspace: as
 *   moe_w4a16_forward (out = bf16 of the same FFN sum with these weights).
 * Scale codes must lie in 1..254 and keep every scaled weight a normal bf16 (code 255 is
 * NaN in the format; the matrix-core converts take only the scale's exponent, so code 0
 * and results below the bf16 normal range are not defined here). Requires H % 32 == 0
 * and I % 32 == 0 (QMOE_ERR_UNSUPPORTED otherwise).
 */
qmoe_status moe_mxfp4_forward(const uint16_t* x, const uint8_t* w13, const uint8_t* s13,
                              const uint8_t* w2, const uint8_t* s2, const int32_t* topk_ids,
                              const float* topk_weights, int32_t T, int32_t H, int32_t I,
                              int32_t E, int32_t k, int32_t schedule, uint16_t* out,
                              void* workspace, size_t* workspace_bytes, void* stream);

/*
 * moe_nvfp4_forward - routed MoE expert FFN with BF16 activations and NVFP4 weights
 * ([XT] overview: NVFP4 among the MoE engine's weight formats; [LSG] launch example: an
 * "NVFP4-W4A16" checkpoint, i.e. weight-only). Reading: E2M1 codes packed two per byte
 * like the INT4 codes, one E4M3 scale per weight row and 16 consecutive k, and one fp32
 * scale per expert and projection.
 *
 *   w13, s13, g13  [E, 2I, H/2] uint8, [E, 2I, H/16] uint8 (E4M3FN), [E] fp32 (4-byte
 *                  alignment suffices): weight(n, c) = e2m1(code) * e4m3(s13[n, c/16]) *
 *                  g13[e].
 *   w2, s2, g2     [E, H, I/2], [E, H, I/16], [E]: down projection, same format.
 *   x, topk_ids, topk_weights, T, H, I, E, k, schedule, out, workspace: as
 *   moe_w4a16_forward.
 * The GPU forms each weight as bf16(e2m1 * (e4m3 * g)) (one rounding, as the INT4 prefill
 * path rounds (q - 8) * s), accumulating in fp32. Requires H % 32 == 0 and I % 32 == 0.
 */
qmoe_status moe_nvfp4_forward(const uint16_t* x, const uint8_t* w13, const uint8_t* s13,
                              const float* g13, const uint8_t* w2, const uint8_t* s2,
                              const float* g2, const int32_t* topk_ids,
                              const float* topk_weights, int32_t T, int32_t H, int32_t I,
                              int32_t E, int32_t k, int32_t schedule, uint16_t* out,
                              void* workspace, size_t* workspace_bytes, void* stream);

/*
 * moe_fp8_block_forward - routed MoE expert FFN, W8A8 block FP8 ([SGL] background:
 * E4M3 weights with one fp32 scale per [128, 128] block, activations E4M3 with one fp32
 * scale per token and 128-column group; block scale = absmax / 448).
 *
 *   a_q, a_scale  [T, H] E4M3 and [T, H/128] fp32: x[t, c] = a_q[t, c] * a_scale[t, c/128].
 *   w13, s13      [E, 2I, H] E4M3 and [E, 2I/128, H/128] fp32 (gate rows [0, I), up rows
 *                 [I, 2I)); w2, s2  [E, H, I] E4M3 and [E, H/128, I/128] fp32.
 *   The SiLU(gate) * up output h (fp32) is requantized to E4M3 per token and per 128
 *   consecutive columns (scale = max(absmax, 1e-10) / 448, round to nearest even after
 *   clamping to +-448) before the down projection; accumulation is fp32 throughout.
 *   topk_ids, topk_weights, T, k, schedule, out, workspace: as moe_w4a16_forward.
 * Requires H % 128 == 0 and I % 128 == 0 ([SGL] kernel dispatch: the scale grids must
 * match cdiv(N, 128) x cdiv(K, 128) exactly).
 */
qmoe_status moe_fp8_block_forward(const uint8_t* a_q, const float* a_scale, const uint8_t* w13,
                                  const float* s13, const uint8_t* w2, const float* s2,
                                  const int32_t* topk_ids, const float* topk_weights, int32_t T,
                                  int32_t H, int32_t I, int32_t E, int32_t k, int32_t schedule,
                                  uint16_t* out, void* workspace, size_t* workspace_bytes,
                                  void* stream);

/*
 * qmoe_fp8_quantize_blocks - block E4M3 quantizer ([SGL] background: each
 * [BLOCK_N, BLOCK_K] block gets its own absmax-derived scale).
 *   v      [R, C] fp32 (4-byte alignment suffices).
 *   q      [R, C] E4M3 out; scale [ceil(R/br), ceil(C/bc)] fp32 out.
 *   Per block: scale = max(absmax, 1e-10) / 448 and q = e4m3_rne(clamp(v / scale,
 *   -448, 448)), computed in fp32 with IEEE division. br in [1, 128], bc in [1, 1024],
 *   br * bc <= 16384. Per-token-group activations use br = 1, bc = 128; weights 128, 128.
 */
qmoe_status qmoe_fp8_quantize_blocks(const float* v, int64_t R, int64_t C, int32_t br, int32_t bc,
                                     uint8_t* q, float* scale, void* stream);

/*
 * qmoe_fp8_quantize_blocks_bf16 - the same quantizer on bf16 values (bit patterns, 2-byte
 * alignment), widened exactly to fp32 first, so the codes and scales equal those of
 * qmoe_fp8_quantize_blocks on the widened values. With br = 1, bc = 128 it turns a
 * model's bf16 activations [T, H] into the W8A8 path's a_q and a_s ([SGL] background:
 * per-token-group activation scales As).
 */
qmoe_status qmoe_fp8_quantize_blocks_bf16(const uint16_t* v, int64_t R, int64_t C, int32_t br,
                                          int32_t bc, uint8_t* q, float* scale, void* stream);

/*
 * qmoe_plan - the schedule and align block size a forward would use.
 *   format      0 = W4A16, 1 = W8A8 block FP8, 2 = MXFP4, 3 = NVFP4 (weight-only).
 *   schedule    requested qmoe_schedule (AUTO resolves here).
 *   chosen      out: QMOE_SCHEDULE_DECODE or QMOE_SCHEDULE_PREFILL.
 *   block_m     out: align block size of that schedule: 16, or 32 when the 4-bit
 *               decode kernel serves two 16-row blocks per weight pass (more than 15
 *               routed rows per expert for W4A16, 11 for MXFP4 and NVFP4, and more than
 *               15 times as many routed pairs in all).
 * AUTO picks the decode profile up to a crossover in routed rows per expert (W4A16 44,
 * MXFP4 60, NVFP4 36, block FP8 20) and, for the 4-bit formats, at any rows per expert
 * up to about ten times that many routed pairs in all (few experts).
 *   workspace_bytes out (may be NULL): workspace the forward needs.
 * Pure host computation; touches no GPU.
 */
qmoe_status qmoe_plan(int32_t format, int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                      int32_t schedule, int32_t* chosen, int32_t* block_m,
                      size_t* workspace_bytes);

/*
 * qmoe_workspace_regions - where a forward keeps its intermediate results inside its
 * workspace (diagnostics: once a forward has completed on its stream, the caller may read
 * them, for instance to compare the block-FP8 path's quantized h with a reference).
 *   format, T, H, I, E, k, schedule: as qmoe_plan (the indexed forwards' workspace; the
 *               grouped entry points' workspace starts with the same regions for their
 *               row count and k = 1, except Y, which they do not use).
 *   offsets     [QMOE_NUM_REGIONS] int64 out: byte offset of each region from the start
 *               of the workspace, or -1 when the plan has no such region.
 *   sizes       [QMOE_NUM_REGIONS] int64 out, or NULL: the region's size in bytes (0 when
 *               absent).
 * The regions, by sorted row r (the align order, L = T*k + E*(block_m - 1) rows):
 *   SORTED_IDS int32 [L], EXPERT_IDS int32 [ceil(L / block_m)], NUM_TOKENS_PADDED int32
 *   [1], EXPERT_OFFSETS int32 [E + 1], TILE_OFFSETS int32 [E + 1] (prefill tiles);
 *   XS (4-bit formats) bf16 [L, H], the gathered activation rows in the GEMM operand
 *   layout; H (4-bit formats) bf16 [L, I], SiLU(gate) * up in that layout;
 *   H32 (block FP8, decode schedule) fp32 [L, I], SiLU(gate) * up before quantization;
 *   HQ (block FP8) E4M3 codes [L, I] of h, HS (block FP8) fp32 [L, I / 128] scales;
 *   OUT32 fp32 [T, H] (decode schedule); Y fp32 [S, T*k, H] (prefill tiles: one row per
 *   routed pair and K slice, before its routing weight; S > 1 when the down GEMM splits K because its output
 *   tiles would not fill the GPU, S = Y's size / (4 T k H)). Rows at or past
 *   num_tokens_padded, padding rows, and the regions a schedule does not use hold
 *   unspecified values.
 * Pure host computation; touches no GPU.
 */
enum {
  QMOE_REGION_SORTED_IDS = 0,
  QMOE_REGION_EXPERT_IDS = 1,
  QMOE_REGION_NUM_TOKENS_PADDED = 2,
  QMOE_REGION_EXPERT_OFFSETS = 3,
  QMOE_REGION_TILE_OFFSETS = 4,
  QMOE_REGION_XS = 5,
  QMOE_REGION_H = 6,
  QMOE_REGION_H32 = 7,
  QMOE_REGION_HQ = 8,
  QMOE_REGION_HS = 9,
  QMOE_REGION_OUT32 = 10,
  QMOE_REGION_Y = 11,
  QMOE_NUM_REGIONS = 12
};
qmoe_status qmoe_workspace_regions(int32_t format, int32_t T, int32_t H, int32_t I, int32_t E,
                                   int32_t k, int32_t schedule, int64_t* offsets, int64_t* sizes);

/*
 * qmoe_set_tuning - schedule overrides for tuning and measurement: the per-shape kernel
 * configuration that a tuning run picks by timing the candidates ("SGLang W8A8 Block FP8
 * quantization kernel config guide", tuning section; the shape guards of "vLLM x Novita
 * AI: Chord W4A16 INT4 MoE Kernel for Kimi K2.x", "Kernel optimizations"). Process-wide;
 * 0 keeps the library's own choice. They apply to every later qmoe_plan,
 * qmoe_workspace_regions and forward call of the 4-bit formats (W4A16, MXFP4, NVFP4):
 *   tile_rows      128 or 256: row tile of the prefill tile kernels.
 *   rows_per_pass  16 or 32: rows per weight pass of the decode kernels (the align block).
 *   kslices        1, 2, 4, ..., 64: K slices of the prefill down GEMM, used where it
 *                  divides I / 256 (else 1); the grouped entry points never split K.
 *   tile_grid      1: one work-group per prefill tile instead of the persistent grid of
 *                  one work-group per compute unit.
 * A change between qmoe_plan and the forward it sized changes the workspace that forward
 * needs: set them before planning, and not while another thread plans or runs a forward.
 * Invalid values return QMOE_ERR_INVALID_ARG and change nothing. Touches no GPU.
 */
qmoe_status qmoe_set_tuning(int32_t tile_rows, int32_t rows_per_pass, int32_t kslices,
                            int32_t tile_grid);

/*
 * Stage timing (diagnostics and benchmarking). The stages of a forward, in launch
 * order, are QMOE_STAGE_ZERO (clear the fp32 combine buffer), QMOE_STAGE_ALIGN,
 * QMOE_STAGE_GATE_UP (gate_up GEMM + SiLU*up), QMOE_STAGE_REQUANT (block-FP8 only:
 * E4M3 requantization of h), QMOE_STAGE_DOWN (down GEMM; on the decode schedule with the
 * weighted scatter-add) and QMOE_STAGE_CAST (fp32 -> bf16 output; on the prefill tiles
 * the routing-weighted sum of each token's top-k rows).
 *
 * qmoe_timing_begin(max_calls): the next max_calls forward calls in this process
 *   record a HIP event pair around each stage's launch, on the forward's stream.
 *   Event handles are created here (host-side objects; no device memory is touched).
 * qmoe_timing_pause(paused): between begin and end, paused != 0 stops recording and
 *   paused == 0 resumes it, keeping what was recorded (a caller can time a sample of its
 *   forwards; a stream in which every launch is bracketed by events runs its kernels
 *   more slowly, since the pauses the events add between kernels move the GPU's power
 *   state). QMOE_ERR_INVALID_ARG outside begin / end.
 * qmoe_timing_end(ms_sum, count): stops recording, waits for the recorded events and
 *   writes, per stage, the summed event-to-event milliseconds and the number of
 *   forwards recorded. Both arrays hold QMOE_NUM_STAGES entries.
 * Not meant to be used from several threads at once.
 */
enum {
  QMOE_STAGE_ZERO = 0,
  QMOE_STAGE_ALIGN = 1,
  QMOE_STAGE_GATE_UP = 2,
  QMOE_STAGE_REQUANT = 3,
  QMOE_STAGE_DOWN = 4,
  QMOE_STAGE_CAST = 5,
  QMOE_NUM_STAGES = 6
};
qmoe_status qmoe_timing_begin(int32_t max_calls);
qmoe_status qmoe_timing_pause(int32_t paused);
qmoe_status qmoe_timing_end(float* ms_sum, int32_t* count);

#ifdef __cplusplus
}
#endif

#endif /* QMOE_H */
