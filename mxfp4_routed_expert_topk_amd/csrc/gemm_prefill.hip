// Grouped FC1 / FC2 for large batches (prefill): MFMA-bound tiles.
//
// Work item = (BM-row tile of one expert's rows, 256-column slice of the
// weight rows).  A workgroup of four waves runs over 64-K stages.  Each wave
// owns all BM rows x one 64-column quarter on v_mfma_f32_32x32x16_bf16: its
// weight chunks (the 16 code bytes a lane multiplies in each of its two
// 32-column blocks, and the dwords holding their E8M0 bytes) come straight
// from global memory into a per-wave register ring, several stages ahead, and
// are dequantised in registers with the gfx950 scaled converter (value *
// 2^(scale-127), exact in bf16), every converted fragment feeding BM/32
// MFMAs.  The activation rows, which the four waves share, pass through a
// ring of LDS stages written by global_load_lds_dwordx4 (no staging
// registers).  32-row blocks that lie wholly past the tile's rows (Zipf-routed
// experts leave many) issue no MFMA and their activation rows are not copied;
// tiles with fewer live rows keep more stages in flight.
//
// Step order inside a stage: the first MFMA of a step (its operands were read
// a step earlier), then the step's share of the next stage's loads, then the
// next step's LDS reads, then the other MFMAs; scheduling groups pin the
// first MFMA ahead of the reads.  The compiler stops counting LDS reads
// precisely once an LDS-DMA copy is issued behind them and waits for
// lgkmcnt(0) at their first use; in this order that wait only ever covers
// reads that are a full step old.  The last step's MFMAs but its first wait
// for the next stage: issued right after its barrier and first LDS reads,
// they cover the latency of those reads (measured 2 % faster on the
// 4096-token Zipf and 1536-token layers than a stage that ends with them).
//
// MFMA K order: in the stage covering K [64q, 64q+64) of a 128-K column block
// (q = 0, 1), step s (16 K) of lane l (column n = l%32, half h = l/32)
// multiplies K = 64q + 32h + 8s + [0, 8): for the weights that is dword s of
// the repacked 16-byte chunk lane' = n%16 + 16h + 32q of row block n/16; the
// activation lane reads the same eight K values of its row.  A row's sum over
// K is therefore taken in one fixed order whatever the tile height.
//
// Activations sit in LDS as 128-byte rows (one coalesced 1 KB global_load_lds
// per eight rows) whose eight 16-byte K chunks are permuted per row by
// swz(c, r) = c ^ (r & 7) ^ ((r >> 3) & 1).  gfx950 LDS serves a ds_read_b128
// quarter-wave (16 lanes) from 64 four-byte banks: the sixteen rows a
// quarter-wave reads then hit sixteen distinct 16-byte bank groups (measured:
// the plain (r & 7) swizzle leaves rows r and r + 8 colliding, about 1.6x
// slower; unswizzled rows about 6x slower).
//
// Work order: the flat list of (tile, column slice) items is cut into eight
// contiguous chunks, one per XCD (workgroups are dispatched round-robin over
// the XCDs).  The grid is persistent (as many workgroups as the device holds):
// a workgroup takes the next item of its XCD's chunk from that chunk's counter
// and, once the chunk is done, items left in the other chunks.  Under skewed
// (Zipf) routing the chunks' work differs by tens of percent -- an XCD whose
// chunk holds the most popular experts' full tiles would otherwise finish
// last while the others idle.  Within a chunk items run tile by tile, the
// slices of one tile consecutively: they fall within one XCD's concurrent
// workgroups and share the tile's activation rows in its L2.
#include <algorithm>
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glob_void_t;

constexpr int kStageK = 64;              // K per pipeline stage (half a repacked tile)
constexpr int kHalfTile = kTileBytes / 2;
// Stages loaded ahead: the LDS ring holds kRingBytes of activation rows, so
// tiles with fewer live rows keep more stages in flight (their K loop is bound
// by the weight stream, not by the MFMAs).  A ring of D + 1 slots divides the
// stage counts of the layer's two GEMMs (K / 64 = 112 and 32), which leaves no
// stages to the loop's tail.
constexpr int kRingBytes = 64 * 1024;
template <int LIVE>
constexpr int depth_for() { return LIVE <= 2 ? 7 : 3; }


// Workgroup shape: W waves side by side over the columns (64 each, four
// 16-column row blocks), every wave over all BM rows.
template <int BM, int W_>
struct Cfg {
  static constexpr int W = W_;
  static constexpr int kBlocks = 4 * W;                  // repacked row blocks per workgroup
  static constexpr int nA = BM / 8 / W;                  // 1 KB copies of eight activation rows per stage
  static constexpr int MI = BM / 32;                     // 32-row MFMA blocks per wave
  // activation copies per wave when only the first `live` 32-row blocks hold rows
  static constexpr int nA_live(int live) { return (4 * live + W - 1) / W < nA ? (4 * live + W - 1) / W : nA; }
  // workgroups per CU that the activation ring allows (at most two), and the
  // waves per SIMD that gives
  static constexpr int kPerCU = 2 * kRingBytes <= 160 * 1024 ? 2 : 1;
  static constexpr int kWavesPerSimd = kPerCU * W / 4;
  static_assert(nA * 8 * W == BM, "copies split evenly over the waves");
  // a wave's share of the ring when it stages its outputs
  static constexpr int kStageOut = kRingBytes / W;
  static_assert(BM * 64 <= kStageOut && kStageOut % (32 * 128) == 0, "output staging fits the ring");
};

// A value every lane holds alike, moved to a scalar register.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <class T>
__device__ __forceinline__ T* uni(T* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u), hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// A 16-byte store through a global (not generic) pointer: a flat store would
// also count in lgkmcnt, and the LDS-only barrier between items would then
// wait for the item's output stores.
__device__ __forceinline__ void store16(void* p, u32x4_t v) {
  *(__attribute__((address_space(1))) u32x4_t*)p = v;
}

// LDS position of K chunk c (0..7) in staged activation row r.
__device__ __forceinline__ int swz(int c, int r) { return c ^ (r & 7) ^ ((r >> 3) & 1); }

// s_waitcnt with vmcnt <= n and lgkmcnt 0 (gfx9 encoding): before a stage's
// barrier every LDS read of the previous stage has returned, whatever MFMA
// the compiler placed after the barrier still reads its result.
#define MOE_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | ((((n) >> 4) & 3) << 14))

// Byte offset of stage st's scale dwords in a row block's scale groups: one
// group per four 128-K blocks, a dword per chunk lane of the half tile.
__device__ __forceinline__ size_t scale_off(int st) {
  return (size_t)(st >> 3) * kScaleGroupBytes + (size_t)(st & 1) * 128;   // group of 4 blocks, half of the lanes
}

// Stages ring_pass runs: s0 + P .. s0 + N - 1 that lie below s0 + n, ring slots P .. N - 1.
template <int P, int N, class F>
__device__ __forceinline__ void ring_pass(F& f, int s0, int n) {
  if constexpr (P < N) {
    if (P < n) {
      f(std::integral_constant<int, P>{}, s0 + P);
      ring_pass<P + 1, N>(f, s0, n);
    }
  }
}

// NT: the weight loads carry the non-temporal hint.
// The K loop with the weights in registers: only the activation rows, which
// the four waves share, go through LDS (a ring of D + 1 stages); each wave
// loads its own weight chunks -- the 16 code bytes a lane multiplies in each
// of its two 32-column blocks and the dwords holding their E8M0 bytes --
// straight into a ring of D + 1 register sets, D stages ahead.  Every stage
// issues the same group of loads (past the last stage: activation copies of
// the last stage again, into the slot no later stage reads, and weight loads
// outside their buffer resource, which return zeros without a memory request),
// so the wait before each stage counts them exactly and the compiler never
// waits at the MFMAs for weights still in flight.
template <class C, int LIVE, int D, bool NT>
__device__ __forceinline__ void k_loop_r(uint8_t* smem, const uint8_t* const (&srcA)[C::nA],
                                         __amdgpu_buffer_rsrc_t rcode, __amdgpu_buffer_rsrc_t rscale,
                                         const uint32_t (&coff)[2], const uint32_t (&soff)[2], int S, int wave,
                                         int lane, f32x16_t (&acc)[C::MI][2]) {
  constexpr int NJ = 2;
  constexpr int W = C::W;
  constexpr int NA = C::nA_live(LIVE);   // activation copies per wave and stage
  constexpr int R = D + 1;               // ring slots
  // A scale dword covers four 128-K blocks, i.e. eight stages; even stages
  // take the dwords of the tile's lanes 0..31, odd stages those of lanes
  // 32..63 (the two K halves).  Only ring slot 0 loads them, both halves
  // (R = 4 or 8 stages per ring pass, a pass lies in one group), and the pass
  // keeps them in `gsc` (loaded with every stage they moved four to eight
  // times the bytes through the load path).
  static_assert(8 % R == 0, "a ring pass lies inside one scale group");
  // loads per wave of the stage in ring slot `slot`
  constexpr auto group_size = [](int slot) { return NA + NJ + (slot == 0 ? 2 * NJ : 0); };
  constexpr int G0 = group_size(0);
  constexpr uint32_t kPastEnd = 0x80000000u;
  constexpr int kSlot = NA * W * 1024;   // the stage's live activation rows
  static_assert(R * kSlot <= kRingBytes && (D - 1) * G0 <= 63, "activation ring, vmcnt range");
  const int n32 = lane & 31, h = lane >> 5;
  const int aoff = n32 * (kStageK * 2);
  u32x4_t bc[R][NJ];
  uint32_t sraw[2][NJ];   // slot 0's scale dwords, [K half][row block pair]
  uint32_t gsc[2][NJ];    // the current pass's

  // loads [first, last) of stage st's group into ring slot `slot`
  auto issue = [&](auto slot_c, int st, int first, int last) {
    constexpr int slot = decltype(slot_c)::value;
    constexpr int G = group_size(slot);
    const bool real = st < S;
    const int sa = min(st, S - 1);
    uint8_t* buf = smem + slot * kSlot;
#pragma unroll
    for (int c = 0; c < G; ++c) {
      if (c < first || c >= last) continue;
      if (c < NA) {
        __builtin_amdgcn_global_load_lds((glob_void_t*)(srcA[c] + (size_t)sa * (kStageK * 2)),
                                         (lds_void_t*)(buf + (wave + W * c) * 1024), 16, 0, 0);
      } else if (c < NA + NJ) {
        const int nj = c - NA;
        bc[slot][nj] = __builtin_amdgcn_raw_buffer_load_b128(rcode, real ? coff[nj] : kPastEnd,
                                                             real ? st * kHalfTile : 0, NT ? 2 : 0);
      } else {
        const int hf = (c - NA - NJ) / NJ, nj = (c - NA - NJ) % NJ;
        sraw[hf][nj] = __builtin_amdgcn_raw_buffer_load_b32(rscale, real ? soff[nj] : kPastEnd,
                                                            real ? (int)scale_off(st + hf) : 0, 0);
      }
    }
  };

  // The last step's MFMAs (all but its first) are held back and issued after
  // the next stage's barrier, behind that stage's first activation reads, so
  // the LDS latency after the barrier runs under MFMAs.  Every accumulator
  // still takes its K steps in order.  Before the first stage the held-back
  // operands are zeros (adding 0 * finite leaves the +0 accumulators as they
  // are).
  bf16x8_t Dc[LIVE], DB[NJ];
#pragma unroll
  for (int mi = 0; mi < LIVE; ++mi) Dc[mi] = bf16x8_t{};
#pragma unroll
  for (int nj = 0; nj < NJ; ++nj) DB[nj] = bf16x8_t{};

  auto run_stage = [&](auto pc, int st) {
    constexpr int p = decltype(pc)::value;   // ring slot of stage st
    constexpr int q = (p + D) % R;           // slot of stage st - 1, refilled with stage st + D
    // this wave's group of stage st has landed (the D - 1 groups after it may
    // still be in flight) and its LDS reads of stage st - 1 have returned; the
    // barrier extends both to every wave
    constexpr int kLater = [] {   // loads of the D - 1 groups issued after stage st's
      int n = 0;
      for (int d = 1; d < D; ++d) n += NA + NJ + ((p + d) % R == 0 ? 2 * NJ : 0);   // group_size((p + d) % R)
      return n;
    }();
    MOE_WAIT_VMCNT(kLater);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // raised issue priority while the wave multiplies (measured 1-2 % faster
    // on the 4096-token Zipf and 1536-token layers)
    __builtin_amdgcn_s_setprio(1);
    const uint8_t* arow = smem + p * kSlot + aoff;
    const int sh = ((st >> 1) & 3) * 8;
    bf16x8_t Ac[LIVE], An[LIVE];
#pragma unroll
    for (int mi = 0; mi < LIVE; ++mi)
      Ac[mi] = *reinterpret_cast<const bf16x8_t*>(arow + mi * 32 * (kStageK * 2) + swz(4 * h, n32) * 16);
#pragma unroll
    for (int mi = 0; mi < LIVE; ++mi)
#pragma unroll
      for (int nj = 0; nj < NJ; ++nj)
        if (mi + nj > 0) acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Dc[mi], DB[nj], acc[mi][nj], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, LIVE, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NJ * LIVE - 1, 0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (p == 0) {
#pragma unroll
      for (int nj = 0; nj < NJ; ++nj) {
        gsc[0][nj] = sraw[0][nj];
        gsc[1][nj] = sraw[1][nj];
      }
    }
    float bs[NJ];
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) bs[nj] = e8m0_to_f32((gsc[p & 1][nj] >> sh) & 0xFFu);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8_t B[NJ];
#pragma unroll
      for (int nj = 0; nj < NJ; ++nj) B[nj] = dequant8(bc[p][nj][s], bs[nj]);
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ac[0], B[0], acc[0][0], 0, 0, 0);
      constexpr int Gq = group_size(q);
      issue(std::integral_constant<int, q>{}, st + D, s * Gq / 4, (s + 1) * Gq / 4);
      if (s < 3) {
#pragma unroll
        for (int mi = 0; mi < LIVE; ++mi)
          An[mi] =
              *reinterpret_cast<const bf16x8_t*>(arow + mi * 32 * (kStageK * 2) + swz(4 * h + s + 1, n32) * 16);
#pragma unroll
        for (int mi = 0; mi < LIVE; ++mi)
#pragma unroll
          for (int nj = 0; nj < NJ; ++nj)
            if (mi + nj > 0)
              acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ac[mi], B[nj], acc[mi][nj], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, LIVE, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, NJ * LIVE - 1, 0);
      } else {
#pragma unroll
        for (int mi = 0; mi < LIVE; ++mi) Dc[mi] = Ac[mi];
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj) DB[nj] = B[nj];
      }
      __builtin_amdgcn_sched_barrier(0);
      if (s < 3) {
#pragma unroll
        for (int mi = 0; mi < LIVE; ++mi) Ac[mi] = An[mi];
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // one group after another: the waits count whole groups in issue order
  auto prologue = [&](auto pc, int st) {
    issue(pc, st, 0, group_size(decltype(pc)::value));
    __builtin_amdgcn_sched_barrier(0);
  };
  ring_pass<0, D>(prologue, 0, D);
  int s0 = 0;
  for (; s0 + R <= S; s0 += R) ring_pass<0, R>(run_stage, s0, R);
  ring_pass<0, R - 1>(run_stage, s0, S - s0);   // the last S % R stages
#pragma unroll
  for (int mi = 0; mi < LIVE; ++mi)
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj)
      if (mi + nj > 0) acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Dc[mi], DB[nj], acc[mi][nj], 0, 0, 0);
  // the copies past the end still write LDS: drained before the ring is reused
  MOE_WAIT_VMCNT(0);
}

template <bool FC1, int BM, int W>
__device__ __noinline__ void fc_pre_item(const FcArgs& a, uint8_t* smem, int slices, int ntiles, int w,
                                            int* s_item, int* counter);

// Workgroup barrier for LDS only: this wave's LDS accesses have completed (no
// wait for its global stores), then s_barrier; the empty asm statements keep
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0) alone
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// W = 4 waves side by side: each owns all BM rows x one 64-column group, so
// every weight fragment is dequantised once per workgroup; two workgroups per
// CU.  (Eight waves over 512 columns, one workgroup per CU, give each staged
// activation row twice the columns but meet at every stage barrier with no
// second workgroup to fill the gaps: measured slower.)
template <bool FC1, int BM, int W>
__global__ __launch_bounds__(W * kWave)
__attribute__((amdgpu_waves_per_eu(Cfg<BM, W>::kWavesPerSimd, Cfg<BM, W>::kWavesPerSimd)))
void fc_pre(FcArgs a, int slices) {
  using C = Cfg<BM, W>;
  __shared__ __align__(1024) uint8_t smem[kRingBytes];
  __shared__ int s_item;

  const int ntiles = *a.tile_count;
  const int total = ntiles * slices;
  const int chunk = (total + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds;
  const bool leader = threadIdx.x == 0;
  // Persistent: take items of this XCD's chunk from its counter, then those
  // left in the other chunks.  The leader's atomic for the next item goes out
  // once the current item's K loop is done, so its latency hides under the
  // epilogue without holding an item back; the result is passed on through
  // LDS, and the bare barrier at the top of the loop finds every wave done
  // reading the stage buffers without waiting for the item's output stores.
  int v = 0, c = xcd;
  if (leader) s_item = atomicAdd(&a.sched[c], 1);
  lds_barrier();
  int i = s_item;
  for (;;) {
    const int base = c * chunk, len = min(chunk, total - base);
    if (i >= len) {                          // chunk c is done: the next one
      if (++v == kXcds) break;
      c = (xcd + v) % kXcds;
      lds_barrier();                         // every wave has read s_item
      if (leader) s_item = atomicAdd(&a.sched[c], 1);
      lds_barrier();
      i = s_item;
      continue;
    }
    fc_pre_item<FC1, BM, W>(a, smem, slices, ntiles, base + i, &s_item, &a.sched[c]);
    lds_barrier();
    i = s_item;
  }
}

// Item w of the work list: (tile w / slices, column slice w % slices).
// Kept out of line: inlined into the persistent loop, the item needs more than
// 256 VGPRs and the spill reloads in its epilogue wait (vmcnt(0)) for every
// output store already issued.  After the K loop the leader takes the next
// item from `counter` and, after the epilogue, stores it to *s_item (the K loop's barriers come after every
// wave's read of *s_item; an empty item takes a barrier of its own).
template <bool FC1, int BM, int W>
__device__ __noinline__ void fc_pre_item(const FcArgs& a, uint8_t* smem, int slices, int ntiles, int w,
                                            int* s_item, int* counter) {
  using C = Cfg<BM, W>;
  constexpr int MI = C::MI;
  constexpr int NJ = 2;                      // 32-column MFMA blocks per wave (its 64 columns)
  // Everything that describes the item is the same in every lane: taken
  // through readfirstlane, it lives in scalar registers and the stage loop's
  // control is a scalar branch (arguments of a function call arrive in vector
  // registers, and so does what is loaded through them).
  slices = uni(slices);
  const int tile = uni(w) / slices, slice = uni(w) - tile * slices;
  if (tile >= uni(ntiles)) {
    lds_barrier();   // every wave has read s_item before it is rewritten
    if (threadIdx.x == 0) *s_item = atomicAdd(counter, 1);
    return;
  }
  const int2 td = a.tiles[tile];
  const int e = uni(td.x), row0 = uni(td.y);
  const int rows = uni(min(BM, a.offsets[e + 1] - row0));
  MatLayout M = a.mat;
  M.nb = uni(M.nb);
  M.kb = uni(M.kb);
  M.kb4 = uni(M.kb4);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = uni(t >> 6);
  const int nb0 = slice * C::kBlocks;
  const int live = (rows + 31) >> 5;         // 32-row blocks holding a row, 1..MI
  const uint8_t* const codes = uni(a.codes);
  const uint8_t* const scales = uni(a.scales);
  const uint8_t* const act = uni(static_cast<const uint8_t*>(a.a));
  const int lda = uni(a.lda), top_k = uni(a.top_k), ldo = uni(a.ldo);
  void* const out = uni(a.out);

  // activation chunks this lane copies: copy i = wave + W j writes rows
  // 8i..8i+7 (128 bytes each); lane L fills row 8i + L/8 at position L%8 with
  // the K chunk c that the swizzle places there.
  const uint8_t* srcA[C::nA];
#pragma unroll
  for (int j = 0; j < C::nA; ++j) {
    const int r = 8 * (wave + W * j) + (lane >> 3);
    const int rr = min(r, rows - 1);
    const int ar = FC1 ? a.perm[row0 + rr] / top_k : row0 + rr;
    srcA[j] = act + (size_t)ar * lda * 2 + swz(lane & 7, r) * 16;
  }
  // the wave's four weight row blocks as buffer resources sized to them; lane
  // (n32, h) multiplies 16-byte chunk (n32 % 16) + 16 h of each stage's half
  // tile of row block 2 nj + n32 / 16, and the dword of the same index in the
  // stage's half of the scale group
  const uint32_t bstride = (uint32_t)M.kb * kTileBytes, sstride = (uint32_t)M.kb4 * kScaleGroupBytes;
  const size_t blk0 = (size_t)e * M.nb + nb0 + wave * (2 * NJ);
  const __amdgpu_buffer_rsrc_t rcode = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(codes) + blk0 * bstride, (short)0, (int)(2 * NJ * bstride), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rscale = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(scales) + blk0 * sstride, (short)0, (int)(2 * NJ * sstride), kRsrcWord3);
  uint32_t coff[NJ], soff[NJ];
  {
    const int lp = (lane & 15) + 16 * (lane >> 5), rb = (lane >> 4) & 1;
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) {
      coff[nj] = (uint32_t)(2 * nj + rb) * bstride + lp * 16;
      soff[nj] = (uint32_t)(2 * nj + rb) * sstride + lp * 4;
    }
  }

  f32x16_t acc[MI][NJ];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mi][nj][i] = 0.f;

  const int S = 2 * M.kb;    // stages
  static_assert(MI == 4, "128-row tiles");
  // Cache policy of the weight loads: an expert with one tile has its weights
  // read by this item alone, so they stream non-temporally; an expert with
  // more tiles (Zipf-popular ones) is read again by its other tiles' items,
  // so they stay cacheable (measured: non-temporal everywhere 2.5 % faster on
  // the 1536-token uniform layer and 2.6 % slower on the 4096-token Zipf one;
  // chosen per tile, 2.2 % and 1.2 % faster than plain loads everywhere).
  const bool single = uni(a.offsets[e + 1] - a.offsets[e]) <= BM;
  if (single) {
    switch (live) {
      case 1: k_loop_r<C, 1, depth_for<1>(), true>(smem, srcA, rcode, rscale, coff, soff, S, wave, lane, acc); break;
      case 2: k_loop_r<C, 2, depth_for<2>(), true>(smem, srcA, rcode, rscale, coff, soff, S, wave, lane, acc); break;
      case 3: k_loop_r<C, 3, depth_for<3>(), true>(smem, srcA, rcode, rscale, coff, soff, S, wave, lane, acc); break;
      default: k_loop_r<C, 4, depth_for<4>(), true>(smem, srcA, rcode, rscale, coff, soff, S, wave, lane, acc); break;
    }
  } else {
    switch (live) {
      case 1: k_loop_r<C, 1, depth_for<1>(), false>(smem, srcA, rcode, rscale, coff, soff, S, wave, lane, acc); break;
      case 2: k_loop_r<C, 2, depth_for<2>(), false>(smem, srcA, rcode, rscale, coff, soff, S, wave, lane, acc); break;
      case 3: k_loop_r<C, 3, depth_for<3>(), false>(smem, srcA, rcode, rscale, coff, soff, S, wave, lane, acc); break;
      default: k_loop_r<C, 4, depth_for<4>(), false>(smem, srcA, rcode, rscale, coff, soff, S, wave, lane, acc); break;
    }
  }
  const int next = threadIdx.x == 0 ? atomicAdd(counter, 1) : 0;
  const int n32 = lane & 31, h = lane >> 5;

  // ---- epilogue.  32x32 D layout: lane holds column n32, rows 8(i/4) + 4h + (i%4).
  // The wave's outputs go through its own share of the (now idle) activation
  // ring and leave in 16-byte row chunks: written straight from the MFMA
  // layout they would take one store instruction per accumulator register (a
  // column's values are four rows apart), which measured 9 % of FC1 and 20 %
  // of FC2.  The barrier finds every wave done reading the ring.
  lds_barrier();
  uint8_t* const stg = smem + wave * C::kStageOut;
  if constexpr (FC1) {
    // h = silu(g) * u, row-major [BM][32] bf16: columns 0..15 of a block pair
    // are gate j, 16..31 up j (interleaved row blocks)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      if (mi >= live) break;
#pragma unroll
      for (int nj = 0; nj < NJ; ++nj) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = mi * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
          const float v = acc[mi][nj][i];
          const float u = __shfl_xor(v, 16, kWave);
          if (n32 < 16)
            *reinterpret_cast<uint16_t*>(stg + r * 64 + (nj * 16 + n32) * 2) = f32_to_bf16_rne(silu_f32(v) * u);
        }
      }
    }
    asm volatile("" ::: "memory");
    const int hc0 = ((nb0 + wave * (2 * NJ)) >> 1) * kTileN;   // the wave's first h column
    for (int k = 0; k < 2 * live; ++k) {                        // 16 rows of 64 B per pass
      const int rr = k * 16 + (lane >> 2), c4 = lane & 3;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stg + rr * 64 + c4 * 16);
      if (rr < rows) store16(static_cast<uint16_t*>(out) + (size_t)(row0 + rr) * ldo + hc0 + c4 * 8, v);
    }
  } else {
    // y rounded to bf16 (the routes' outputs are summed in fp32 by the
    // combine), RB rows at a time: row-major [RB][64] bf16
    constexpr int RB0 = C::kStageOut / 128, RB = RB0 < BM ? RB0 : BM, MG = RB / 32;
    const int c0 = (nb0 + wave * (2 * NJ)) * kTileN;           // the wave's first output column
#pragma unroll
    for (int g = 0; g < MI / MG; ++g) {
      if (MG * g >= live) break;
#pragma unroll
      for (int m2 = 0; m2 < MG; ++m2) {
        const int mi = MG * g + m2;
        if (mi >= live) break;
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = m2 * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
            *reinterpret_cast<uint16_t*>(stg + r * 128 + (nj * 32 + n32) * 2) = f32_to_bf16_rne(acc[mi][nj][i]);
          }
      }
      asm volatile("" ::: "memory");
      const int nrows = min(RB, live * 32 - g * RB);
      for (int k = 0; k < nrows / 8; ++k) {                     // 8 rows of 128 B per pass
        const int rr = k * 8 + (lane >> 3), ch = lane & 7;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stg + rr * 128 + ch * 16);
        const int gr = g * RB + rr;
        if (gr < rows) store16(static_cast<uint16_t*>(out) + (size_t)(row0 + gr) * ldo + c0 + ch * 8, v);
      }
      asm volatile("" ::: "memory");
    }
  }
  if (threadIdx.x == 0) *s_item = next;
}

template <bool FC1>
hipError_t launch_cfg(const FcArgs& a, int tiles_max, hipStream_t stream) {
  using C = Cfg<kPrefillRows, 4>;
  const int slices = a.mat.nb / C::kBlocks;
  const long long items = (long long)tiles_max * slices;
  // as many workgroups as the device holds at once (kPerCU per CU), a multiple
  // of the XCD count, and no more than there can be items
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const long long resident = (long long)cus * C::kPerCU / kXcds * kXcds;
  const long long grid = std::max<long long>(kXcds, std::min(resident, (items + kXcds - 1) / kXcds * kXcds));
  hipLaunchKernelGGL((fc_pre<FC1, kPrefillRows, 4>), dim3((unsigned)grid), dim3(4 * kWave), 0, stream, a, slices);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fc1_prefill(const FcArgs& a, int tiles_max, hipStream_t s) { return launch_cfg<true>(a, tiles_max, s); }
hipError_t launch_fc2_prefill(const FcArgs& a, int tiles_max, hipStream_t s) { return launch_cfg<false>(a, tiles_max, s); }

}  // namespace moe
