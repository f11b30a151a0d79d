// Route metadata of a decode-sized batch (R <= 256 routes) computed by one
// wave; see route.hip for the method and the (expert, f) row order.  Used by
// the one-wave route kernel and, into LDS, by the fused decode kernel.
#pragma once

#include "moe_internal.h"

namespace moe {

// Mask of the lanes of this wave that hold the same valid expert id.
__device__ __forceinline__ uint64_t match_expert(int e, bool valid) {
  uint64_t todo = __ballot(valid);
  uint64_t mine = 0;
  while (todo) {
    const int leader = __ffsll((unsigned long long)todo) - 1;
    const int el = __builtin_amdgcn_readlane(e, leader);
    const uint64_t m = __ballot(valid && e == el);
    if (valid && e == el) mine = m;
    todo &= ~m;
  }
  return mine;
}

// One wave: everything for R <= 256 routes (decode batches).  No workgroup
// barriers: lane l holds routes l, l+64, ... in f order; a 64-route chunk at
// a time gets its ranks from ballots (match_expert), plus a running per-expert
// count in LDS that one lane per expert advances after the chunk -- the same
// (expert, f) order as the chunked kernels.

// Orders the calling wave's LDS accesses for the compiler and the hardware
// (the LDS serves one wave's instructions in issue order; the wait makes the
// results of earlier ones land first).  Not a workgroup barrier: the other
// waves of a larger workgroup do not take part.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0) alone
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// `s_cnt` is E ints of LDS, private to the calling wave.  The outputs may be
// global or LDS; a caller with other waves orders their reads after this with
// its own barrier.
__device__ inline void route_wave(const int32_t* ids, int R, int E, int bm, const RouteOut& o, int* s_cnt) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int e = lane; e < E; e += kWave) s_cnt[e] = 0;
  wave_lds_sync();
  for (int f = lane; f < R; f += kWave) {
    const int e = ids[f];
    if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
  }
  wave_lds_sync();
  // exclusive scans of the counts and of the tile counts, 16 experts per lane
  // step (ascending expert order; one wave, so lane order is the scan order)
  int run = 0, trun = 0;
  for (int base = 0; base < E; base += kWave) {
    const int e = base + lane;
    const int c = e < E ? s_cnt[e] : 0;
    const int nt = (c + bm - 1) / bm;
    int incl = c, tincl = nt;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int t1 = __shfl_up(incl, d, kWave), t2 = __shfl_up(tincl, d, kWave);
      if (lane >= d) {
        incl += t1;
        tincl += t2;
      }
    }
    const int off = run + incl - c, toff = trun + tincl - nt;
    if (e < E) {
      o.counts[e] = c;
      o.offsets[e] = off;
      for (int i = 0; i < nt; ++i) o.tiles[toff + i] = make_int2(e, off + i * bm);
      s_cnt[e] = off;   // running row position from here on
    }
    run += __shfl(incl, kWave - 1, kWave);
    trun += __shfl(tincl, kWave - 1, kWave);
  }
  if (lane == 0) {
    o.offsets[E] = run;
    *o.tile_count = trun;
  }
  wave_lds_sync();
  // rows: chunk by chunk in f order
  const uint64_t below = lane ? (~0ull >> (kWave - lane)) : 0ull;
  for (int base = 0; base < R; base += kWave) {
    const int f = base + lane;
    const int e = f < R ? ids[f] : -1;
    const bool valid = f < R && e >= 0 && e < E;
    const uint64_t mine = match_expert(e, valid);
    if (f < R) {
      if (valid) {
        const int pos = s_cnt[e] + __popcll(mine & below);
        o.perm[pos] = f;
        o.rowpos[f] = pos;
      } else {
        o.rowpos[f] = -1;
      }
    }
    wave_lds_sync();   // every lane has read s_cnt before the leaders advance it
    if (valid && __popcll(mine & below) == 0) s_cnt[e] += __popcll(mine);
    wave_lds_sync();
  }
}

}  // namespace moe
