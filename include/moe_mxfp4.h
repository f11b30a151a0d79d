/*
 * moe_mxfp4.h -- C ABI of the routed-expert MXFP4 MoE layer for AMD MI355X (gfx950).
 *
 * The layer: for every token t and top-k slot s with a resident expert id
 * e = topk_ids[t,s] in [0, E):
 *     [g | u] = W13_e x_t          (W13_e = [w1_e; w3_e], gate rows then up rows)
 *     h       = silu(g) * u        (silu(z) = z / (1 + exp(-z)))
 *     y       = W2_e h
 *     acc_t  += topk_weights[t,s] * y      (fp32, slots in ascending order)
 *     out_t   = round_to_nearest_even_bf16(acc_t)
 * Expert weights are MXFP4: E2M1 codes, two per byte along K (element 2j in
 * bits 3:0), with one E8M0 scale byte (value 2^(b-127)) per 32 consecutive K.
 * Sources: pegainfer PR #867 ("K3 model line ... MegaMoE(situ) transport"),
 * commits b49a9f04 (FP4 B operand, gran_k 32), 88ec37ec (packed [gate; up]
 * regions), 53edfa98 (route metadata with deterministic token*topk+slot
 * order; topk-slot-order f32 combine, no atomics, single bf16 round);
 * batchgen PR #307 ("mxfp4 marlin grouped gemm ...": repack as a pure nibble
 * rearrangement, E8M0 edge bytes 0x00/0xFF raise, w1||w3 fused repack,
 * hard-fail contract); b12x PR #339 (commits "FC2-only route validation":
 * ids outside the resident count contribute an exact zero without mutating
 * caller tensors; "large-token FC2 fused-sum epilogue": caller-owned fp32
 * token accumulator, cast once).
 *
 * Conventions for every entry point:
 *  - Device pointers are HIP device addresses owned by the caller; the library
 *    never allocates device memory and never frees caller memory.
 *  - Every device pointer must be 16-byte aligned (MOE_ERR_ALIGN otherwise).
 *  - bf16 tensors are passed as uint16_t bit patterns; shapes are row-major.
 *  - Work is enqueued on the given stream (0 = the null stream).  Only
 *    moe_mxfp4_plan synchronises (once, to read back its validation word).
 *  - On failure the call returns a non-zero moe_status before launching any
 *    work (host-checkable errors) and moe_mxfp4_last_error() names what was
 *    expected and what was passed.  Nothing falls back to another path.
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = 1,          /* null pointer, bad enum, negative count */
  MOE_ERR_SHAPE = 2,        /* dimension not supported (see moe_mxfp4_config) */
  MOE_ERR_ALIGN = 3,        /* a device pointer is not 16-byte aligned */
  MOE_ERR_CAPACITY = 4,     /* num_tokens > max_tokens */
  MOE_ERR_SCALE_BYTE = 5,   /* a weight scale byte is not accepted (plan) */
  MOE_ERR_WORKSPACE = 6,    /* workspace or repacked buffer too small */
  MOE_ERR_UNSUPPORTED = 7,  /* device is not gfx950 */
  MOE_ERR_HIP = 8,          /* a HIP runtime call failed (text from hipGetErrorString) */
  MOE_ERR_TIMEOUT = 9       /* a wait of a fused forward passed its time bound (moe_mxfp4_fused_status) */
} moe_status;

typedef enum {
  MOE_ACT_BF16 = 0,   /* bf16 activations x bf16-dequantised MXFP4 weights on bf16 MFMA */
  MOE_ACT_MXFP8 = 1   /* activations quantised to MXFP8 (E4M3 + E8M0 per 32) before FC1
                         and FC2, on the gfx950 scaled F8F6F4 MFMA with FP4 weights */
} moe_act;

typedef struct {
  int32_t hidden;        /* H: multiple of 128, 128..16384 */
  int32_t intermediate;  /* I: multiple of 128, 128..16384 */
  int32_t num_experts;   /* E resident experts, 1..1024; ids outside [0,E) contribute exact zero */
  int32_t top_k;         /* k: 1..32 */
  int32_t max_tokens;    /* capacity T_max (1..65536) used to size the workspace */
  int32_t act;           /* moe_act */
} moe_mxfp4_config;

typedef struct moe_mxfp4_plan_s* moe_mxfp4_plan_t;

/* Sizes in bytes of the repacked-weight buffer and of the forward workspace
 * for a configuration.  Host only; no device access. */
moe_status moe_mxfp4_query_sizes(const moe_mxfp4_config* cfg, size_t* repacked_bytes,
                                 size_t* workspace_bytes);

/* Repack checkpoint-layout MXFP4 weights into the kernels' operand order and
 * validate their scale bytes (batchgen PR #307: repack is a pure nibble
 * rearrangement carrying the E8M0 bytes unchanged; edge bytes raise).
 *   w13_codes  [E, 2I, H/2]  u8, rows 0..I-1 = w1 (gate), rows I..2I-1 = w3 (up)
 *   w13_scales [E, 2I, H/32] u8 E8M0
 *   w2_codes   [E, H, I/2]   u8
 *   w2_scales  [E, H, I/32]  u8 E8M0
 *   repacked   caller buffer of repacked_bytes (query_sizes); must outlive the plan
 * Scale bytes 0x00 and 0xFF are rejected; with MOE_ACT_BF16 also 0x01, 0xFD and
 * 0xFE (their bf16 weights would be subnormal or overflow).  The error text
 * names the first offending (matrix, expert, row, group, byte).  The source
 * buffers are only read and may be freed after this call returns.
 * Synchronises the stream once.  *out receives a host-side plan object. */
moe_status moe_mxfp4_plan(const moe_mxfp4_config* cfg, const uint8_t* w13_codes,
                          const uint8_t* w13_scales, const uint8_t* w2_codes,
                          const uint8_t* w2_scales, void* repacked, size_t repacked_bytes,
                          hipStream_t stream, moe_mxfp4_plan_t* out);

/* One forward pass of the layer for num_tokens tokens (0 <= T <= max_tokens).
 *   hidden        [T, H] bf16
 *   topk_ids      [T, k] int32; ids outside [0, E) contribute an exact zero
 *   topk_weights  [T, k] fp32; ignored for invalid ids
 *   acc_fp32      [T, H] fp32 or NULL: if given, every element is overwritten
 *                 with the fp32 token accumulator (tokens without a valid
 *                 route get +0.0)
 *   out_bf16      [T, H] bf16: overwritten with RNE_bf16(acc)
 *   workspace     caller buffer of workspace_bytes (query_sizes); its contents
 *                 on entry do not matter (the call sets every word it reads,
 *                 including the work counters of the large-batch kernels,
 *                 which its first kernel zeroes on the stream)
 * Intermediate precision: g and u are fp32 sums; h is rounded to bf16 (bf16
 * activations) or requantised to MXFP8 before FC2; batches that take the
 * 128-row-tile kernels (T*k >= 16*E) also round each route's y to bf16 before
 * the fp32 slot-order sum (b12x PR #339: the fused-sum epilogue reduces bf16
 * routed outputs).
 * Enqueue-only: no host synchronisation and no allocation, so the call can be
 * captured in a HIP graph.  Inputs and the repacked weights are never written.
 * Concurrent calls sharing one workspace race. */
moe_status moe_mxfp4_forward(moe_mxfp4_plan_t plan, const uint16_t* hidden,
                             const int32_t* topk_ids, const float* topk_weights,
                             int32_t num_tokens, float* acc_fp32, uint16_t* out_bf16,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The same forward as moe_mxfp4_forward for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): it takes no workspace.  Its scratch (route metadata, h, the
 * per-route outputs) lives in a fixed 48 MiB device array of the library, one
 * copy per GPU, held until the process ends; num_tokens is limited to what
 * fits it (at hidden 7168, intermediate 2048, top-8 about 190 tokens), and a
 * larger batch returns MOE_ERR_CAPACITY naming the bytes it needs.  Arguments
 * and outputs are those of moe_mxfp4_forward; the results are bitwise equal
 * to it.  Nothing is allocated and nothing synchronises.  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (on concurrent
 * streams or threads) race. */
moe_status moe_mxfp4_forward_noalloc(moe_mxfp4_plan_t plan, const uint16_t* hidden, const int32_t* topk_ids,
                                     const float* topk_weights, int32_t num_tokens, float* acc_fp32,
                                     uint16_t* out_bf16, hipStream_t stream);

/* The same forward as moe_mxfp4_forward, the whole layer in one kernel
 * launch, for decode-sized batches: a MOE_ACT_BF16 plan and at most 256 routes
 * (num_tokens * top_k), else MOE_ERR_SHAPE.  The pages' fused MoE launch
 * (pegainfer PR #867: dispatch, FC1, activation, FC2 and combine in one kernel)
 * is the model; here every workgroup routes the batch itself and the FC2 and
 * combine work waits on counters of the work it reads.  Arguments, ownership
 * and outputs are those of moe_mxfp4_forward.  It always runs the 16-row
 * streaming kernels' arithmetic: where moe_mxfp4_forward takes those too
 * (fewer than 16 routes per resident expert, or hidden not a multiple of 256)
 * the outputs are bitwise equal; otherwise both meet the same tolerance of the
 * exact result.  Differences:
 *  - the launch is cooperative (every workgroup resident at once), which HIP
 *    graph capture may not accept: use moe_mxfp4_forward under capture;
 *  - the workspace holds the counters: it must be zero before the first fused
 *    forward that uses it (a zero-filled workspace is ready; the calls keep it
 *    consistent afterwards), and concurrent calls sharing one workspace race;
 *  - each wait is bounded in time (100 ms, or MOE_FUSED_SPIN_TICKS ticks of the
 *    100 MHz device clock from the environment); past the bound the kernel
 *    still ends, its outputs are not valid and moe_mxfp4_fused_status reports
 *    MOE_ERR_TIMEOUT.
 * Enqueue-only: no host synchronisation and no allocation. */
moe_status moe_mxfp4_forward_fused(moe_mxfp4_plan_t plan, const uint16_t* hidden,
                                   const int32_t* topk_ids, const float* topk_weights,
                                   int32_t num_tokens, float* acc_fp32, uint16_t* out_bf16,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Whether the plan's last moe_mxfp4_forward_fused on this workspace completed
 * every wait: MOE_OK, or MOE_ERR_TIMEOUT.  Synchronises the stream. */
moe_status moe_mxfp4_fused_status(moe_mxfp4_plan_t plan, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* Route metadata only (the first stage of forward), for checking:
 *   counts  [E] int32, offsets [E+1] int32 (exclusive prefix sum of counts),
 *   perm    [T*k] int32: the first offsets[E] entries are the flat route
 *           indices f = t*k+s of valid routes ordered by (expert, f); the rest
 *           is left untouched,
 *   rowpos  [T*k] int32: row of route f in that order, or -1 if invalid.
 * (pegainfer PR #867, commit 53edfa98: race-free per-expert compaction with
 * deterministic token*topk+slot entry order.)  Uses the workspace. */
moe_status moe_mxfp4_route(moe_mxfp4_plan_t plan, const int32_t* topk_ids, int32_t num_tokens,
                           int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* rowpos,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Regions of the forward workspace that hold an intermediate of the last
 * forward on it, for checking (moe_mxfp4_workspace_region). */
typedef enum {
  MOE_WS_H_CODES = 0,   /* MOE_ACT_MXFP8: the requantised gated activation h as
                           E4M3FN codes, u8 [T_max * k, I]; row r belongs to the
                           r-th valid route in (expert, t*k+s) order (the perm
                           of moe_mxfp4_route), rows past the valid routes are
                           unspecified */
  MOE_WS_H_SCALES = 1   /* MOE_ACT_MXFP8: its E8M0 bytes, u8 [T_max * k, I/32] */
} moe_ws_region;

/* Byte offset and size of a workspace region of the plan's layout, so a
 * checker can read an intermediate back (pegainfer PR #867, commit 53edfa98:
 * the chain's requantised activation scales are compared bit for bit).  The
 * MXFP8 path quantises h from fp32; where the exact h sits within fp32
 * rounding of a rounding or scale decision, either side is correct, so the
 * layer output alone cannot show which one the kernels took.  Host only.
 * MOE_ERR_ARG for an unknown region or a MOE_ACT_BF16 plan (which keeps h in
 * bf16 and has neither region). */
moe_status moe_mxfp4_workspace_region(moe_mxfp4_plan_t plan, int32_t region, size_t* offset, size_t* bytes);

/* MXFP8 quantisation of a bf16 matrix [rows, cols] (cols a multiple of 32),
 * as applied to the activations in MOE_ACT_MXFP8 mode (pegainfer PR #867,
 * commit 33d22f80: gran-32 e4m3 activation quant with UE8M0 scales):
 * per block of 32 along a row, e = floor(log2(amax / 448)) clamped to
 * [-127, 127] (amax = 0 gives -127), codes = E4M3FN round-to-nearest-even of
 * the block scaled by 2^-e and saturated to +-448, scale byte = e + 127.
 *   codes [rows, cols] u8, scales [rows, cols/32] u8. */
moe_status moe_mxfp8_quantize(const uint16_t* x_bf16, int32_t rows, int32_t cols,
                              uint8_t* codes, uint8_t* scales, hipStream_t stream);

/* Router top-k upstream of the layer: the topk_ids / topk_weights that
 * moe_mxfp4_forward consumes, from fp32 router logits [num_tokens, num_experts]
 * (row-major).  The contract follows the pages (pegainfer PR #867, commit
 * b49a9f04: batched router top-k over E in {224, 896}; b12x PR #339: top-16
 * kept in registers, a fixed tie order, a sequential fp32 normalisation of
 * the route weights); the scoring function is not on the pages and the
 * reading taken is the top-k softmax:
 *   topk_ids     [num_tokens, top_k] int32: the top_k largest logits of the
 *                row in descending order; equal logits rank the lower expert
 *                id first; a NaN logit counts as -inf (ranked last, weight 0);
 *   topk_weights [num_tokens, top_k] fp32: exp(l_s - l_0) / sum_j exp(l_j - l_0)
 *                over the selected logits l_0 >= l_1 >= ..., exp in fp32, the
 *                sum over slots in ascending order.
 * Ids are exact; weights are within a few fp32 rounding steps of the exact
 * softmax.  Requires 1 <= num_experts <= 1024 and 1 <= top_k <= min(32,
 * num_experts); num_tokens = 0 is a no-op.  Pointers are device memory,
 * 16-byte aligned; nothing is allocated; the call only enqueues on stream. */
moe_status moe_router_topk(const float* logits, int32_t num_tokens, int32_t num_experts,
                           int32_t top_k, int32_t* topk_ids, float* topk_weights,
                           hipStream_t stream);

/* Peak micro-benchmarks: the measured ceilings a benchmark reports its
 * kernels against beside the published peaks (the pages record each run's
 * GPU operating state because the clock policy moved their numbers: b12x PR
 * #339, maintenance-window and extent-benchmark commits).  Not part of the
 * layer.  `sink` is device memory of at least `grid` floats (one per
 * workgroup; the values mean nothing); 1 <= grid <= 16384.  Enqueue-only. */
typedef enum {
  MOE_PROBE_READ = 0,      /* grid-stride 128-bit loads over src[bytes] */
  MOE_PROBE_READ_NT = 1,   /* the same with non-temporal loads */
  MOE_PROBE_COPY = 2       /* dst[bytes] = src[bytes] in 128-bit words */
} moe_probe_memory_kind;
/* bytes a multiple of 16; src (and dst for a copy) 16-byte aligned. */
moe_status moe_probe_memory(int32_t kind, const void* src, void* dst, size_t bytes, float* sink, int32_t grid,
                            hipStream_t stream);

typedef enum {
  MOE_PROBE_MFMA_BF16 = 0,   /* independent chains of v_mfma_f32_32x32x16_bf16 */
  MOE_PROBE_MFMA_F8F4 = 1    /* v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 A x E2M1 B */
} moe_probe_mfma_kind;
/* `iters` >= 1 rounds of eight independent MFMAs per wave, 256-thread
 * workgroups; *flops receives the launch's multiply-add work (2 per MAC). */
moe_status moe_probe_mfma(int32_t kind, int32_t iters, float* sink, int32_t grid, double* flops,
                          hipStream_t stream);

/* One v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 A, E2M1 B, one E8M0 scale per
 * 32 K of each) per problem, on operands given in the instruction's lane
 * order: a measurement of how the matrix core sums a block of 128 products,
 * which bounds how far the MXFP8 path's fp32 h may sit from the exact h.
 *   a_lanes  [n][64][32] u8  lane l: A row l%16, K 16q..16q+15 then 64+16q.., q = l/16
 *   b_lanes  [n][64][16] u8  lane l: B row l%16, E2M1 K 32q..32q+31, element 2j in bits 3:0
 *   a_scales, b_scales [n][64] u8  lane l: the scale of its row's K group q
 *   c, d     [n][64][4] fp32 lane l: accumulator rows 4q..4q+3 of column l%16
 * 1 <= n <= 65536; device pointers, 16-byte aligned; enqueue-only. */
moe_status moe_probe_mfma_f8f4_blocks(const uint8_t* a_lanes, const uint8_t* b_lanes, const uint8_t* a_scales,
                                      const uint8_t* b_scales, const float* c, float* d, int32_t n,
                                      hipStream_t stream);

/* Record one event at each stage boundary of subsequent forward calls of this
 * plan: events[0] before the first kernel, then after route, FC1, FC2 and the
 * combine (n = 5).  Pass n = 0 to stop.  The events are owned by the caller
 * and must stay valid while set.  Used to time each kernel on its stream. */
moe_status moe_mxfp4_set_stage_events(moe_mxfp4_plan_t plan, hipEvent_t* events, int32_t n);

/* Release a plan (host memory only; the repacked buffer stays the caller's). */
void moe_mxfp4_destroy(moe_mxfp4_plan_t plan);

/* Text of the last error on the calling thread ("" if none). */
const char* moe_mxfp4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
