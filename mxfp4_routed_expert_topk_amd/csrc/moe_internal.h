// Internal declarations of the MXFP4 routed-expert MoE library (gfx950).
//
// Repacked weight layout (one layout serves the bf16 MFMA and the scaled
// F8F6F4 MFMA paths).  A matrix with N rows and K columns (K-major codes
// [N][K/2] in the checkpoint) is cut into tiles of 16 rows x 128 K:
//   NB = N/16 row blocks, KB = K/128 column blocks.
//   codes:  tile (nb, kb) holds 1024 bytes at ((e*NB + nb)*KB + kb)*1024;
//           lane l (0..63) of a wave owns bytes [16l, 16l+16): row 16*nb + l%16,
//           checkpoint bytes [64*kb + 16*(l/16), +16), i.e. the 32 consecutive K
//           values 128*kb + 32*(l/16) + [0, 32), nibbles copied unchanged.
//   scales: KB4 = ceil(KB/4) groups of four column blocks; group (nb, c) holds
//           256 bytes at ((e*NB + nb)*KB4 + c)*256; byte 4l + j is the E8M0 scale
//           of row 16*nb + l%16 for K group 4*(4c + j) + l/16 (its 32 K values are
//           exactly lane l's in column block 4c + j); padding bytes are 127.
// FC1 (W13, N = 2I) interleaves gate and up row blocks: row block 2j holds
// gate rows [16j, 16j+16) and row block 2j+1 holds up rows [I+16j, I+16j+16),
// so one workgroup owning a block pair has the gate and up columns of the
// same 16 intermediate outputs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kTileN = 16;          // rows per repacked tile
constexpr int kTileK = 128;         // K per repacked tile
constexpr int kTileBytes = 1024;    // codes per tile
constexpr int kScaleGroupBytes = 256;
constexpr int kRsrcWord3 = 0x00020000;   // buffer resource word 3: raw buffer, 32-bit data format
constexpr int kRouteChunk = 1024;   // routes per route workgroup
constexpr int kBM = 16;             // rows per FC tile (one MFMA M block)
// K column blocks from which the decode kernels split K four ways (else two):
// a function of K alone, so a row's fp32 summation order depends neither on
// the batch nor on the kernel (the fused decode kernel uses the same split).
constexpr int kKsplit4Blocks = 32;
constexpr int kMaxDimension = 16384;  // largest hidden / intermediate size a plan accepts
constexpr int kMaxTopK = 32;          // largest top-k a plan accepts
// Work counters of the prefill FC kernels: one per XCD chunk of the work list,
// eight for FC1 then eight for FC2.
constexpr int kXcds = 8;
constexpr int kSchedCounters = 2 * kXcds;

struct MatLayout {
  int32_t n, k;        // logical rows / columns
  int32_t nb, kb, kb4; // row blocks, column blocks, scale groups per row block
  size_t codes_per_expert;   // bytes
  size_t scales_per_expert;  // bytes
};

inline MatLayout make_mat_layout(int n, int k) {
  MatLayout m;
  m.n = n; m.k = k;
  m.nb = n / kTileN; m.kb = k / kTileK; m.kb4 = (m.kb + 3) / 4;
  m.codes_per_expert = (size_t)m.nb * m.kb * kTileBytes;
  m.scales_per_expert = (size_t)m.nb * m.kb4 * kScaleGroupBytes;
  return m;
}

// Offsets of every region inside the repacked buffer and the workspace.
struct Layout {
  int32_t H, I, E, k, Tmax, act;
  int32_t Rmax;          // Tmax * k
  int32_t tiles_max;     // upper bound of FC tiles (16 rows each)
  int32_t route_blocks;  // ceil(Rmax / kRouteChunk)
  MatLayout w13, w2;
  // repacked buffer
  size_t rp_w13_codes, rp_w13_scales, rp_w2_codes, rp_w2_scales, rp_status, rp_bytes;
  // workspace
  size_t ws_counts, ws_offsets, ws_perm, ws_rowpos, ws_tiles, ws_tile_count, ws_blockcounts;
  size_t ws_xq, ws_xs, ws_h, ws_hq, ws_hs, ws_y, ws_sync, ws_sched, ws_bytes;
};

Layout make_layout(int H, int I, int E, int k, int Tmax, int act);

// ---------------------------------------------------------------- launchers
// All launchers enqueue on `stream` and return the launch status.
hipError_t launch_repack(const Layout& L, const uint8_t* w13c, const uint8_t* w13s,
                         const uint8_t* w2c, const uint8_t* w2s, uint8_t* repacked,
                         hipStream_t stream);

struct RouteOut {
  int32_t* counts;      // [E]
  int32_t* offsets;     // [E+1]
  int32_t* perm;        // [Rmax]
  int32_t* rowpos;      // [Rmax]
  int2* tiles;          // [tiles_max] (expert, first row) of each bm-row FC tile
  int32_t* tile_count;  // [1]
  int32_t* blockcounts; // [route_blocks * E] scratch
  int32_t* sched;       // [kSchedCounters] work counters of the prefill FC kernels (or null); the
                        // route kernels zero them, so each forward's FC launches start from zero
};
hipError_t launch_route(const Layout& L, const int32_t* ids, int32_t T, const RouteOut& o, int bm,
                        hipStream_t stream);

hipError_t launch_quant_bf16(const uint16_t* x, int32_t rows, int32_t cols, uint8_t* codes,
                             uint8_t* scales, hipStream_t stream);
hipError_t launch_quant_f32(const float* x, const int32_t* rows_dev, int32_t rows_max,
                            int32_t cols, uint8_t* codes, uint8_t* scales, hipStream_t stream);

struct FcArgs {
  const uint8_t* codes;     // repacked codes of the matrix (all experts)
  const uint8_t* scales;    // repacked scales of the matrix
  MatLayout mat;
  const int2* tiles;
  const int32_t* tile_count;
  const int32_t* offsets;   // [E+1]
  const int32_t* perm;      // FC1: gather rows of x through perm/k
  int32_t top_k;
  const void* a;            // FC1: x bf16 [T,H] (or E4M3 codes); FC2: h [R,I] bf16 (or E4M3 codes)
  const uint8_t* a_scales;  // MXFP8: E8M0 per 32 of the A rows
  int32_t lda;              // elements per A row
  int32_t a_rows;           // rows of A (FC1: tokens; FC2: routes)
  void* out;                // FC1: h ([R,I] bf16, or fp32 for MXFP8); FC2: y [R,H] fp32
  int32_t ldo;              // elements per output row
  uint8_t* out_codes;       // MXFP8 prefill FC1: h as E4M3 codes [R,I] (instead of fp32 `out`)
  uint8_t* out_scales;      // ... and its E8M0 bytes [R,I/32]
  int32_t* sched;           // bf16 prefill: kXcds work counters of this launch, zero on entry
  const int32_t* route_ids; // per-route decode kernels: topk_ids [T*k] (the tile of route f is ids[f])
  int32_t num_experts;      // ... ids outside [0, num_experts) get no tile
};
// `tokens` (the batch size) only picks a schedule; results do not depend on it.
hipError_t launch_fc1_bf16(const FcArgs& a, int tiles_max, int tokens, hipStream_t stream);
hipError_t launch_fc2_bf16(const FcArgs& a, int tiles_max, int tokens, hipStream_t stream);
hipError_t launch_fc1_mx(const FcArgs& a, int tiles_max, int tokens, hipStream_t stream);
hipError_t launch_fc2_mx(const FcArgs& a, int tiles_max, int tokens, hipStream_t stream);
// Smallest bf16 batches (routes <= kPerRouteMaxRoutes): no route stage.  FC1
// runs one tile per route (h row f for route f); FC2 runs one workgroup per
// (token, block of output columns) over the token's valid routes and sums them
// in slot order in its epilogue, writing acc and out itself.  (At 64 routes the
// chain measured faster: per-route FC1 tiles read an expert's weights once per
// route, grouped tiles once per 16 rows.)
constexpr int kPerRouteMaxRoutes = 32;
hipError_t launch_fc1_bf16_per_route(const FcArgs& a, int routes, hipStream_t stream);
hipError_t launch_fc2_sum_per_route(const FcArgs& a, const float* weights, int32_t T, int32_t H, float* acc,
                                    uint16_t* out, hipStream_t stream);

// Prefill (MFMA-bound) FC kernels over 128-row tiles, bf16 path (needs
// N % 256 == 0).  Persistent: `sched` holds the launch's work counters.
constexpr int kPrefillRows = 128;
hipError_t launch_fc1_prefill(const FcArgs& a, int tiles_max, hipStream_t stream);
hipError_t launch_fc2_prefill(const FcArgs& a, int tiles_max, hipStream_t stream);
// Prefill FC kernels of the MXFP8 path over 128-row tiles (needs N % 256 == 0
// and A plus its scales addressable with 32-bit offsets).  FC1 writes h already
// requantised to MXFP8 (out_codes / out_scales) by the rule launch_quant_f32
// applies to an fp32 h.
constexpr int kPrefillMxRows = 128;
hipError_t launch_fc1_prefill_mx(const FcArgs& a, int tiles_max, hipStream_t stream);
hipError_t launch_fc2_prefill_mx(const FcArgs& a, int tiles_max, hipStream_t stream);

// The whole bf16 decode layer in one cooperative launch (fused.hip), for at
// most kFusedMaxRoutes routes.  `sync` is kFusedSyncBytes of workspace, zero
// before its first use (the kernel keeps it consistent afterwards).
constexpr int kFusedMaxRoutes = 256;
constexpr int kFusedMaxTiles = kFusedMaxRoutes / kBM + kFusedMaxRoutes;   // tile list bound, any E
constexpr size_t kFusedSyncBytes = 4 * (2 * (size_t)kFusedMaxTiles + 2);   // two counts per tile, two words
hipError_t launch_fused_decode(const FcArgs& f1, const FcArgs& f2, const int32_t* ids, const float* weights,
                               int32_t T, int32_t k, int32_t E, int32_t H, float* acc, uint16_t* out,
                               const RouteOut& route, uint8_t* sync, uint32_t gen, long long spin_ticks,
                               hipStream_t stream);

// Router top-k (E <= kRouterMaxExperts, k <= 32).
constexpr int kRouterMaxExperts = 1024;
hipError_t launch_router_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* ids, float* weights,
                              hipStream_t stream);

// Peak micro-benchmarks (probe.hip).  `sink` holds one float per workgroup
// (grid <= kProbeSinkFloats).
constexpr int kProbeSinkFloats = 16384;
hipError_t launch_probe_memory(int kind, const void* src, void* dst, size_t bytes, float* sink, int grid,
                               hipStream_t stream);
hipError_t launch_probe_mfma(int kind, int iters, float* sink, int grid, double* flops, hipStream_t stream);
hipError_t launch_probe_mfma_blocks(const uint8_t* a, const uint8_t* b, const uint8_t* sa, const uint8_t* sb,
                                    const float* c, float* d, int n, hipStream_t stream);

// y: per-route output rows, fp32 or (y_bf16) bf16.
hipError_t launch_combine(const void* y, bool y_bf16, const int32_t* rowpos, const float* w, int32_t T, int32_t k,
                          int32_t H, float* acc, uint16_t* out, hipStream_t stream);

// ---------------------------------------------------------------- device helpers
#if defined(__HIPCC__)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// E8M0 byte -> fp32 power of two (exact for bytes 1..254).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) { return __uint_as_float(b << 23); }

// Eight E2M1 codes (one dword, element 2j in the low nibble of byte j) -> eight
// bf16 values times the power-of-two scale, on the gfx950 scaled converter
// (it takes the exponent of `scale` only).
__device__ __forceinline__ bf16x8_t dequant8(uint32_t w, float scale) {
  bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  bf16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// silu(z) = z / (1 + e^-z) in fp32, the quotient on the hardware reciprocal
// (at most 1 ulp; h is rounded to bf16 or requantised to E4M3 right after).
// z -> -inf gives -0 (1/inf = 0), NaN stays NaN.  Measured 1 % faster in the
// prefill FC1 epilogues than the IEEE division sequence.
__device__ __forceinline__ float silu_f32(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// MXFP8 scale rule of the MXFP8 x MXFP4 workload: e = floor(log2(amax / 448)),
// clamped to [-127, 127], amax = 0 -> -127; the block is scaled by 2^-e,
// saturated to +-448 and rounded to nearest even E4M3FN (subnormals included);
// the scale byte is e + 127.
// floor(log2(amax / 448)) for finite amax >= 0, clamped to [-127, 127].
__device__ __forceinline__ int mx_scale_exp(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int ex = (int)((u >> 23) & 0xFFu);
  if (ex == 0) return -127;                      // zero or subnormal: far below 448 * 2^-127
  const uint32_t man = u & 0x7FFFFFu;
  int e = (ex - 127) - 8 - (man < 0x600000u ? 1 : 0);   // 448 = 1.75 * 2^8
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Scaled values -> E4M3FN codes, saturated to +-448 and rounded to nearest
// even (subnormals included): clamp with v_med3_f32, then v_cvt_pk_fp8_f32
// converts two values to the low (word_sel false) or high 16 bits of a dword,
// first value in the lower byte.  Infinities clamp to +-448 like any value
// beyond it; NaN inputs are outside the contract.  An exhaustive run over
// every finite fp32 bit pattern gave the same code as the integer rounding
// (round the fp32 mantissa to three bits with the carry into the exponent,
// rebias 127 -> 7; below 2^-6 the code is the value times 512 rounded to
// nearest even), and the quantiser's parity test checks every tie of the
// E4M3 grid against the oracle.
__device__ __forceinline__ float e4m3_clamp(float v) { return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f); }

// codes of a, b in bytes 0, 1 (bits 16..31 zero)
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false) & 0xFFFFu;
}

// codes of a, b, c, d in bytes 0..3
__device__ __forceinline__ uint32_t e4m3_quad(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), lo, true);
}
#endif

}  // namespace moe
