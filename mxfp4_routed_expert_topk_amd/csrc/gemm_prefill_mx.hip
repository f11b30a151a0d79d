// Grouped FC1 / FC2 for large batches on the MXFP8 path: E4M3 activations
// with one E8M0 per 32 along K times E2M1 weights with one E8M0 per 32, on
// the gfx950 scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4, which applies both
// block scales inside the instruction (the OCP MX product; the MXFP8 x MXFP4
// variant of the grouped GEMM).
//
// Work item = (128-row tile of one expert's rows, slice of 16 * WV * kNBW
// weight rows: 512 or 256).  The weights are what the batch streams from HBM (an expert
// holds 23.4 MB of codes and scales at hidden 7168 / intermediate 2048, while
// its ~85 routed rows of E4M3 activations hold 0.6 MB), so one tile covers
// every row an expert has in a balanced batch and each weight byte is read
// once.  A workgroup of WV waves (eight for FC1 where the matrix's rows come
// in 512s, one workgroup per CU; else four, two per CU) runs one stage per
// 128-K column block, loading stage st + kDepth while stage st multiplies:
//  * weights: the repacked 1 KB tile is already the MFMA's B operand (lane l
//    holds the 32 codes of row l%16, K group l/16), so each wave loads its
//    kNBW row blocks straight into registers, with their E8M0 bytes, into a ring
//    of kDepth + 1 register sets (buffer loads: one VGPR offset, SGPR bases);
//  * activations: the tile's rows (gathered through the route permutation
//    for FC1) are shared by the waves, so they are copied global->LDS by
//    buffer_load ... lds into 128-byte rows under the same conflict-free
//    chunk swizzle as the bf16 prefill kernel; each lane reads its A operand
//    (bytes 16(l/16).. and 64+16(l/16).. of row l%16) with two ds_read_b128.
//    Each row's four E8M0 bytes of the stage follow the rows as one dword
//    per row (half-wave dword copies, one per wave), read with ds_read_u8.
// Every stage issues the same group of loads (past the end: zero loads with
// an out-of-range offset), so the wait before each stage counts them exactly
// and the compiler never waits for weights still in flight at the MFMAs.
// Each wave owns all rows x 16 kNBW columns (kNBW/2 gate/up pairs for FC1):
// 2*LIVE 16-row blocks by kNBW row blocks.  Four row blocks per wave rather
// than two halve how often a tile's activations are copied (once per 256
// columns, not 128) at two workgroups per CU instead of three: measured 11%
// faster at 4096 tokens and 384 experts.  32-row blocks wholly past the tile's rows
// are neither copied nor multiplied.
//
// K order: a row's sum runs over the 128-K column blocks in ascending order,
// each block one MFMA step, whatever the tile height.
//
// FC1: row blocks come in (gate j, up j) pairs (interleaved repack); the
// epilogue requantises h = silu(g) * u to MXFP8 (E4M3 codes, one E8M0 per 32
// columns), which FC2 reads.  FC2: y rows in route-row order, rounded to bf16
// (the combine sums them in fp32).
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kRows = kPrefillMxRows;       // rows per tile
constexpr int kNBW = 4;                     // row blocks (16 output columns each) per wave
// Stages loaded ahead of the one multiplied: three for tiles of at most 96
// rows, whose accumulators leave room for a fourth ring slot, else two.
template <int LIVE>
constexpr int depth_for() { return LIVE <= 3 ? 3 : 2; }
constexpr int kMaxDepth = 3;
// Cache policy of FC2's weight loads: non-temporal (measured 3 % faster in FC2;
// the same policy made FC1 6 % slower).
constexpr int kNonTemporal = 2;
constexpr int kBufs = kMaxDepth + 1;        // LDS stage buffers
constexpr int kStageA = kRows * kTileK;       // 128 rows x 128 E4M3
constexpr int kStageBytes = kStageA + kRows * 4;   // + each row's four E8M0 bytes of the stage

// vmcnt <= n with lgkmcnt 0 (every LDS read of the previous stage returned)
#define MOE_WAIT_VM_LGKM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | ((((n) >> 4) & 3) << 14))

__device__ __forceinline__ int swz(int c, int r) { return c ^ (r & 7) ^ ((r >> 3) & 1); }

static_assert((kMaxDepth - 1) * (16 / 4 + 1 + 2 * kNBW) <= 63, "vmcnt holds at most 63");

// Stages s0 + P .. s0 + N - 1 that lie below s0 + n, ring slots P .. N - 1.
template <int P, int N, class F>
__device__ __forceinline__ void ring_pass(F& f, int s0, int n) {
  if constexpr (P < N) {
    if (P < n) {
      f(std::integral_constant<int, P>{}, s0 + P);
      ring_pass<P + 1, N>(f, s0, n);
    }
  }
}

// WV waves per workgroup: 8 (one workgroup per CU, 512 columns) or 4 (two per
// CU, 256 columns).
template <bool FC1, int LIVE, int WV, int kDepth = depth_for<LIVE>()>
__device__ __forceinline__ void tile_body(const FcArgs& a, uint8_t* sa, int e, int row0, int rows, int slice) {
  static_assert(WV == 4 || WV == 8, "four or eight waves per workgroup");
  constexpr int kWaves = WV;
  constexpr int kBlocks = kWaves * kNBW;      // output columns per workgroup / 16
  constexpr int kCopySlots = 16 / kWaves;     // 8-row activation copies per wave and stage, at most
  constexpr int kScaleLanes = kRows / kWaves; // rows whose scale dword one wave copies
  constexpr int MB = 2 * LIVE;            // 16-row MFMA blocks
  constexpr int GROUPS = 4 * LIVE;        // 8-row copy groups of the live rows
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const MatLayout M = a.mat;
  const int S = M.kb;                     // one stage per 128-K column block
  const int sgroups = a.lda / 32;         // E8M0 bytes per activation row

  // Buffer resources over the whole activation matrix and its scales: every
  // address is a 32-bit offset from an SGPR base.
  const __amdgpu_buffer_rsrc_t racts =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.a), (short)0, a.a_rows * a.lda, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rascl = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.a_scales), (short)0, a.a_rows * sgroups, kRsrcWord3);
  // activation copies: group g (rows 8g .. 8g+7) is copied by wave g % kWaves;
  // lane L fills row 8g + L/8 at chunk position L%8.  Every wave issues NA
  // copies per stage: a wave with fewer live groups than that fills rows past
  // the live ones (read by no MFMA) with an out-of-range zero copy, so that
  // every wave issues the same count and the waits below are constants.
  constexpr int NA = (GROUPS + kWaves - 1) / kWaves;
  static_assert(NA <= kCopySlots, "copy slots");
  uint32_t aoff[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    const int r = 8 * (wave + kWaves * j) + (lane >> 3);
    const int rr = min(r, rows - 1);
    const int ar = FC1 ? a.perm[row0 + rr] / a.top_k : row0 + rr;
    aoff[j] = (uint32_t)ar * (uint32_t)a.lda + swz(lane & 7, r) * 16;
  }
  // scale copy of each stage: lane L < kScaleLanes of wave w copies the
  // stage's four E8M0 bytes (one dword: sgroups is a multiple of 4) of row
  // kScaleLanes w + L to dword (kScaleLanes w + L) after the stage's rows
  uint32_t soff;
  {
    const int rr = min(kScaleLanes * wave + (lane & (kScaleLanes - 1)), rows - 1);
    const int ar = FC1 ? a.perm[row0 + rr] / a.top_k : row0 + rr;
    soff = (uint32_t)ar * (uint32_t)sgroups;
  }
  // this wave's two weight row blocks, as buffer resources sized to them
  const int nb0 = slice * kBlocks + wave * kNBW;
  const uint32_t bstride = (uint32_t)M.kb * kTileBytes, sstride = (uint32_t)M.kb4 * kScaleGroupBytes;
  const __amdgpu_buffer_rsrc_t rcode = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.codes) + ((size_t)e * M.nb + nb0) * bstride, (short)0, (int)(kNBW * bstride), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rscale = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.scales) + ((size_t)e * M.nb + nb0) * sstride, (short)0, (int)(kNBW * sstride),
      kRsrcWord3);

  f32x4_t acc[MB][kNBW];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < kNBW; ++j) acc[mb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // weight ring: stage st in slot st % kRing; stage st + kDepth is loaded at
  // the top of stage st into the slot stage st-1 has just finished with
  constexpr int kRing = kDepth + 1;
  u32x4_t bq[kRing][kNBW];
  uint32_t bs[kRing][kNBW];
  // A lane's scale dword covers the four stages of a group.  With a ring of
  // four slots (slot = stage % 4) only slot 0 holds a group's first stage: it
  // alone loads scales, and they are kept in `gsc` for the group's four stages
  // (loaded with every stage they moved four times the bytes through the load
  // path).  Other ring sizes load them with every stage.
  constexpr bool kGroupScales = kRing % 4 == 0;
  uint32_t gsc[kNBW];

  // Stage s >= S (the loads issued "past the end", see run_stage): the
  // per-lane offset is set to kPastEnd and the scalar one to 0, which puts the
  // address beyond its buffer resource's range (the range check takes the
  // per-lane offset; every resource here is under 2^31 bytes): the load
  // returns zeros without a memory request and still counts in vmcnt, which
  // is all it is there for.
  constexpr uint32_t kPastEnd = 0x80000000u;
  // activation copies of stage s into stage buffer `bi`
  auto issue_lds = [&](int bi, int s) {
    uint8_t* buf = sa + bi * kStageBytes;
    const bool real = s < S;
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const bool live = real && wave + kWaves * j < GROUPS;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(racts, (lds_void_t*)(buf + (wave + kWaves * j) * 1024), 16,
                                               live ? aoff[j] : kPastEnd, live ? s * kTileK : 0, 0, 0);
    }
    if (lane < kScaleLanes)   // part of the wave: one operation all the same
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rascl, (lds_void_t*)(buf + kStageA + kScaleLanes * 4 * wave), 4,
                                               real ? soff : kPastEnd, real ? 4 * s : 0, 0, 0);
  };
  auto load_regs = [&](u32x4_t (&q)[kNBW], uint32_t (&sb)[kNBW], int s, bool with_scales) {
    const bool real = s < S;
#pragma unroll
    for (int j = 0; j < kNBW; ++j)
      q[j] = __builtin_amdgcn_raw_buffer_load_b128(rcode, real ? lane * 16 : kPastEnd,
                                                   real ? j * bstride + s * kTileBytes : 0, FC1 ? 0 : kNonTemporal);
    // the dword of the lane's four E8M0 bytes in the stage's scale group (its
    // byte s % 4 is taken at the MFMA): loaded as a byte, the value would be
    // zero-extended by a copy that waits for the load right after it is issued.
    // Past the end: the last stage's dword again (an out-of-range offset here
    // makes the compiler branch around the loads, and its waits then count
    // the loads of later stages too).
    if (with_scales) {
      const int sg = (min(s, S - 1) >> 2) * kScaleGroupBytes;
#pragma unroll
      for (int j = 0; j < kNBW; ++j)
        sb[j] = __builtin_amdgcn_raw_buffer_load_b32(rscale, lane * 4, j * sstride + sg, 0);
    }
  };

  // A operand position of this lane inside a staged 16-row block
  const int rl = lane & 15, q = lane >> 4;
  const int lo_off = rl * kTileK + swz(q, rl) * 16;
  const int hi_off = rl * kTileK + swz(4 + q, rl) * 16;

  // Every stage issues the same loads -- one group: this wave's activation
  // copies and weight loads of stage st + kDepth (past the end: zero loads
  // into the buffer and ring slot of stage st-1, which no later stage
  // reads) -- so the wait at each stage counts them exactly,
  // and the compiler, seeing the same operations on every path around the
  // loop, places its own waits for the weight registers no earlier than that.
  auto run_stage = [&](auto pc, int st) {
    constexpr int p = decltype(pc)::value;   // ring slot of stage st
    // this wave's loads of stage st have landed (the kDepth - 1 groups after
    // it may still be in flight) and its LDS reads of stage st-1 have
    // returned; the barrier extends both to every wave
    constexpr int kLater = [] {   // loads of the kDepth - 1 groups issued after stage st's
      int n = 0;
      for (int d = 1; d < kDepth; ++d) n += NA + 1 + kNBW + (!kGroupScales || (p + d) % 4 == 0 ? kNBW : 0);
      return n;
    }();
    MOE_WAIT_VM_LGKM(kLater);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue_lds((st + kDepth) % kRing, st + kDepth);   // into the buffer of stage st-1
    load_regs(bq[(p + kDepth) % kRing], bs[(p + kDepth) % kRing], st + kDepth,
              !kGroupScales || (p + kDepth) % 4 == 0);
    if constexpr (kGroupScales && p % 4 == 0) {
#pragma unroll
      for (int j = 0; j < kNBW; ++j) gsc[j] = bs[p][j];
    }
    const uint8_t* cur = sa + (st % kRing) * kStageBytes;
    const int sh = 8 * (st & 3);
    const uint8_t* curs = cur + kStageA;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(cur + mb * 16 * kTileK + lo_off);
      const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(cur + mb * 16 * kTileK + hi_off);
      const int sc = curs[(mb * 16 + rl) * 4 + q];
      const i32x8_t Af = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                          (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
      for (int j = 0; j < kNBW; ++j) {
        const i32x8_t Bf = {(int)bq[p][j][0], (int)bq[p][j][1], (int)bq[p][j][2], (int)bq[p][j][3], 0, 0, 0, 0};
        acc[mb][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Af, Bf, acc[mb][j], 0, 4, 0, sc, 0,
                                                                      (int)(((kGroupScales ? gsc[j] : bs[p][j]) >> sh) & 0xFFu));
      }
    }
    // The stage's MFMAs stay above the next barrier (this empty statement
    // reads their results), so their ring slot is free when the next stage's
    // loads overwrite it: no second register set and no copies (a copy of a
    // register still being loaded would make the compiler wait for the load).
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < kNBW; ++j) asm volatile("" ::"v"(acc[mb][j]));
  };

  // one group after another: the waits count whole groups in issue order
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    issue_lds(d, d);
    load_regs(bq[d], bs[d], d, !kGroupScales || d % 4 == 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  int s0 = 0;
  for (; s0 + kRing <= S; s0 += kRing) ring_pass<0, kRing>(run_stage, s0, kRing);
  ring_pass<0, kRing - 1>(run_stage, s0, S - s0);   // the last S % kRing stages
  // the last stages' zero copies still write LDS: drain them before the
  // workgroup can end and its LDS be handed to the next one
  MOE_WAIT_VM_LGKM(0);

  // ---- epilogue.  16x16 D layout: lane holds column l%16, rows 4(l/16) + i.
  if constexpr (FC1) {
    // h = silu(g) * u, requantised to MXFP8 here: the wave's two gate/up pairs
    // are h columns 16 (nb0/2) + [0, 32), one whole 32-element scale block
    // (nb0 is a multiple of 4), held by the 16 lanes of a row (column rl and
    // 16 + rl).  Its amax is reduced over those lanes; every lane shuffles, so
    // the stores alone are guarded by the row count.
    static_assert(kNBW == 4, "one 32-column scale block of h per wave");
    // The codes go through the wave's 4 KB of the (now idle) stage ring and
    // leave as 16-byte row chunks: stored from the MFMA layout they would be
    // byte stores, 16 bytes of a row per store, which measured 12 % of FC1.
    // The barrier finds every wave done reading the ring.
    static_assert(kWaves * 4096 <= kBufs * kStageBytes && MB * 16 * 32 <= 4096, "code staging fits the ring");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    uint8_t* const stg = sa + wave * 4096;                   // [MB * 16][32] E4M3
    const int hc = (nb0 / 2) * kTileN;   // first h column of the block
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mb + 4 * q + i;
        const float h0 = silu_f32(acc[mb][0][i]) * acc[mb][1][i];
        const float h1 = silu_f32(acc[mb][2][i]) * acc[mb][3][i];
        float m = fmaxf(fabsf(h0), fabsf(h1));
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, kWave));
        const int ex = mx_scale_exp(m);
        const float inv = __uint_as_float((uint32_t)(127 - ex) << 23);   // 2^-e
        const uint32_t c2 = e4m3_pair(h0 * inv, h1 * inv);
        stg[r * 32 + rl] = (uint8_t)c2;
        stg[r * 32 + 16 + rl] = (uint8_t)(c2 >> 8);
        if (r < rows && rl == 0) a.out_scales[(size_t)(row0 + r) * (a.ldo / 32) + hc / 32] = (uint8_t)(ex + 127);
      }
    }
    asm volatile("" ::: "memory");
    for (int k = 0; k < MB / 2; ++k) {                         // 32 rows of 32 B per pass
      const int rr = k * 32 + (lane >> 1), half = lane & 1;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stg + rr * 32 + half * 16);
      if (rr < rows)
        *(__attribute__((address_space(1))) u32x4_t*)(a.out_codes + (size_t)(row0 + rr) * a.ldo + hc + half * 16) = v;
    }
    return;
  }
  // FC2: y rounded to bf16.  The rows go through the wave's share of the
  // (now idle) stage ring and leave as 16-byte row chunks (stored from the
  // MFMA layout they would be 2-byte stores, 32 bytes of a row per store);
  // the barrier finds every wave done reading the ring.
  constexpr int kShare = kBufs * kStageBytes / kWaves / 4096 * 4096;
  constexpr int RP = kShare / 128;                     // staged rows of 64 bf16 per pass
  static_assert(RP % 16 == 0 && RP >= 16, "whole 16-row blocks per pass");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  uint8_t* const stg = sa + wave * kShare;
  const int c0 = nb0 * kTileN;                         // the wave's first output column
#pragma unroll
  for (int p0 = 0; p0 < MB * 16; p0 += RP) {
#pragma unroll
    for (int mb = p0 / 16; mb < MB && mb < (p0 + RP) / 16; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < kNBW; ++j)
          *reinterpret_cast<uint16_t*>(stg + (16 * mb + 4 * q + i - p0) * 128 + (j * kTileN + rl) * 2) =
              f32_to_bf16_rne(acc[mb][j][i]);
    asm volatile("" ::: "memory");
    const int nrows = min(RP, MB * 16 - p0);
    for (int k = 0; k < nrows / 8; ++k) {              // 8 rows of 128 B per pass
      const int rr = k * 8 + (lane >> 3), ch = lane & 7;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stg + rr * 128 + ch * 16);
      const int gr = p0 + rr;
      if (gr < rows)
        *(__attribute__((address_space(1))) u32x4_t*)(static_cast<uint16_t*>(a.out) + (size_t)(row0 + gr) * a.ldo +
                                                       c0 + ch * 8) = v;
    }
    asm volatile("" ::: "memory");
  }
}

template <bool FC1, int WV>
__global__ __launch_bounds__(WV * kWave, 8 / WV) void fc_pre_mx(FcArgs a, int slices) {
  __shared__ __align__(1024) uint8_t sa[kBufs * kStageBytes];
  const int ntiles = *a.tile_count;
  // tiles dealt to the XCDs round-robin: XCD x takes tiles x, x + 8, ...,
  // each with all its column slices in a row, so the slices of a tile share
  // its activation rows in one L2
  const int xcd = blockIdx.x % kXcds, qq = blockIdx.x / kXcds;
  const int q = qq / slices, slice = qq - q * slices;
  const int tile = xcd + kXcds * q;
  if (tile >= ntiles) return;
  const int2 td = a.tiles[tile];
  const int e = td.x, row0 = td.y;
  const int rows = min(kRows, a.offsets[e + 1] - row0);
  switch ((rows + 31) >> 5) {
    case 1: tile_body<FC1, 1, WV>(a, sa, e, row0, rows, slice); break;
    case 2: tile_body<FC1, 2, WV>(a, sa, e, row0, rows, slice); break;
    case 3: tile_body<FC1, 3, WV>(a, sa, e, row0, rows, slice); break;
    default: tile_body<FC1, 4, WV>(a, sa, e, row0, rows, slice); break;
  }
}

template <bool FC1, int WV>
hipError_t launch_waves(const FcArgs& a, int tiles_max, hipStream_t stream) {
  const int slices = a.mat.nb / (WV * kNBW);
  const long long grid = (long long)(tiles_max + kXcds - 1) / kXcds * slices * kXcds;
  hipLaunchKernelGGL((fc_pre_mx<FC1, WV>), dim3((unsigned)grid), dim3(WV * kWave), 0, stream, a, slices);
  return hipGetLastError();
}

// FC1: eight waves (512 columns) where the matrix's rows allow it: the staged
// activation rows then serve twice the columns (measured 4 % faster at 4096
// tokens than two four-wave workgroups per CU); else four.  FC2 (K = I: 16
// stages at intermediate 2048, so the ring's fill and the epilogue weigh
// more): four, two workgroups per CU, one filling the gaps of the other
// (measured 676 -> 642 us at 4096 tokens and 384 experts).
template <bool FC1>
hipError_t launch(const FcArgs& a, int tiles_max, hipStream_t stream) {
  if (FC1 && a.mat.nb % (8 * kNBW) == 0) return launch_waves<FC1, 8>(a, tiles_max, stream);
  return launch_waves<FC1, 4>(a, tiles_max, stream);
}

}  // namespace

hipError_t launch_fc1_prefill_mx(const FcArgs& a, int tiles_max, hipStream_t s) { return launch<true>(a, tiles_max, s); }
hipError_t launch_fc2_prefill_mx(const FcArgs& a, int tiles_max, hipStream_t s) {
  return launch<false>(a, tiles_max, s);
}

}  // namespace moe
