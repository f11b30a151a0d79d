// Route metadata: per-expert counts, offsets, stable permutation, row of each
// route, and the list of bm-row FC tiles (16 for the streaming kernels, 64 or
// 128 for the prefill kernels).
//
// A route is a (token, slot) pair with flat index f = t*k + s.  Ids outside
// [0, E) get no row (exact-zero contribution; b12x PR #339, commit "FC2-only
// route validation").  Rows are ordered by (expert, f) -- the deterministic
// token*topk+slot entry order of pegainfer PR #867, commit 53edfa98 -- and
// the result does not depend on thread timing: counts use integer LDS
// atomics (order-free), ranks come from wave ballots and fixed-order prefix
// sums, never from atomic return values.
//
// Decode-sized problems (T*k <= 256) run in one wave, mid-sized ones
// (<= 1024) as one workgroup; larger ones as count -> scan -> scatter over
// 1024-route chunks.
#include "route_wave.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Inclusive scan across the 1024 threads of a workgroup; `tmp` holds 16 ints.
__device__ int block_inclusive_scan(int v, int* tmp) {
  const int lane = lane_id(), w = threadIdx.x / kWave;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int t = __shfl_up(v, d, kWave);
    if (lane >= d) v += t;
  }
  if (lane == kWave - 1) tmp[w] = v;
  __syncthreads();
  if (w == 0) {
    int s = lane < kWaves ? tmp[lane] : 0;
#pragma unroll
    for (int d = 1; d < kWaves; d <<= 1) {
      int t = __shfl_up(s, d, kWave);
      if (lane >= d) s += t;
    }
    if (lane < kWaves) tmp[lane] = s;
  }
  __syncthreads();
  int r = v + (w > 0 ? tmp[w - 1] : 0);
  __syncthreads();
  return r;
}

// Counts per expert, offsets, tile list.  `cnt` is the per-expert total
// (thread e holds expert e).  Writes counts/offsets/tiles/tile_count.
__device__ void finish_counts(int e, int cnt, int E, int bm, int* tmp, const RouteOut& o, int* s_offsets) {
  const int c = e < E ? cnt : 0;
  const int incl = block_inclusive_scan(c, tmp);
  const int off = incl - c;
  const int nt = (c + bm - 1) / bm;
  const int tincl = block_inclusive_scan(nt, tmp);
  const int toff = tincl - nt;
  if (e < E) {
    o.counts[e] = c;
    o.offsets[e] = off;
    if (s_offsets) s_offsets[e] = off;
    for (int i = 0; i < nt; ++i) o.tiles[toff + i] = make_int2(e, off + i * bm);
  }
  if (e == E - 1) {
    o.offsets[E] = incl;
    *o.tile_count = tincl;
  }
}

// Ranks of this workgroup's chunk of routes [base, base+1024) and scatter.
// `wbase[e]` is the first row of expert e for this chunk.
__device__ void scatter_chunk(const int32_t* ids, int R, int E, int base, const int* wbase,
                              uint8_t* wcnt, const RouteOut& o) {
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int f = base + threadIdx.x;
  const int e = f < R ? ids[f] : -1;
  const bool valid = f < R && e >= 0 && e < E;
  for (int i = threadIdx.x; i < kWaves * E; i += kThreads) wcnt[i] = 0;
  __syncthreads();
  const uint64_t mine = match_expert(e, valid);
  const uint64_t below = lane ? (~0ull >> (kWave - lane)) : 0ull;
  const int rank_in_wave = __popcll(mine & below);
  if (valid && rank_in_wave == 0) wcnt[w * E + e] = (uint8_t)__popcll(mine);
  __syncthreads();
  if (f < R) {
    if (valid) {
      int pos = wbase[e] + rank_in_wave;
      for (int v = 0; v < w; ++v) pos += wcnt[v * E + e];
      o.perm[pos] = f;
      o.rowpos[f] = pos;
    } else {
      o.rowpos[f] = -1;
    }
  }
}

// One workgroup: everything for R <= 1024.
__global__ __launch_bounds__(kThreads) void route_fused(const int32_t* ids, int R, int E, int bm, RouteOut o) {
  __shared__ int s_cnt[1024];
  __shared__ int s_off[1024];
  __shared__ int tmp[kWaves];
  __shared__ uint8_t wcnt[kWaves * 1024];
  if (o.sched != nullptr && threadIdx.x < kSchedCounters) o.sched[threadIdx.x] = 0;
  const int t = threadIdx.x;
  s_cnt[t] = 0;
  __syncthreads();
  if (t < R) {
    const int e = ids[t];
    if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  finish_counts(t, s_cnt[t], E, bm, tmp, o, s_off);
  __syncthreads();
  scatter_chunk(ids, R, E, 0, s_off, wcnt, o);
}

constexpr int kSmallRoutes = 64;   // routes the one-wave kernel takes (route_wave.h)

// One wave: everything for R <= kSmallRoutes (decode batches).
__global__ __launch_bounds__(kWave) void route_small(const int32_t* ids, int R, int E, int bm, RouteOut o) {
  __shared__ int s_cnt[1024];    // per-expert count, then running row position
  if (o.sched != nullptr && threadIdx.x < kSchedCounters) o.sched[threadIdx.x] = 0;
  route_wave(ids, R, E, bm, o, s_cnt);
}

// Chunked: per-chunk counts.
__global__ __launch_bounds__(kThreads) void route_count(const int32_t* ids, int R, int E, int32_t* blockcounts) {
  __shared__ int s_cnt[1024];
  const int t = threadIdx.x;
  s_cnt[t] = 0;
  __syncthreads();
  const int f = blockIdx.x * kThreads + t;
  if (f < R) {
    const int e = ids[f];
    if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  if (t < E) blockcounts[(size_t)blockIdx.x * E + t] = s_cnt[t];
}

// Chunked: totals, offsets, tiles; blockcounts become each chunk's first row
// per expert.  Thread e walks expert e's counts down the chunks eight at a
// time, the eight loads issued together (one load and, in the second pass, one
// store after the other waited for each load in turn: 15 us at 32 chunks).
constexpr int kScanBatch = 8;

__global__ __launch_bounds__(kThreads) void route_scan(int E, int nblk, int bm, RouteOut o) {
  __shared__ int tmp[kWaves];
  if (o.sched != nullptr && threadIdx.x < kSchedCounters) o.sched[threadIdx.x] = 0;
  const int e = threadIdx.x;
  int total = 0;
  if (e < E)
    for (int b0 = 0; b0 < nblk; b0 += kScanBatch) {
      int c[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) c[j] = b0 + j < nblk ? o.blockcounts[(size_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) total += c[j];
    }
  finish_counts(e, total, E, bm, tmp, o, nullptr);
  __syncthreads();
  if (e < E) {
    int run = o.offsets[e];
    for (int b0 = 0; b0 < nblk; b0 += kScanBatch) {
      int c[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) c[j] = b0 + j < nblk ? o.blockcounts[(size_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) {
        if (b0 + j < nblk) o.blockcounts[(size_t)(b0 + j) * E + e] = run;
        run += c[j];
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void route_scatter(const int32_t* ids, int R, int E, RouteOut o) {
  __shared__ int s_base[1024];
  __shared__ uint8_t wcnt[kWaves * 1024];
  const int t = threadIdx.x;
  if (t < E) s_base[t] = o.blockcounts[(size_t)blockIdx.x * E + t];
  __syncthreads();
  scatter_chunk(ids, R, E, blockIdx.x * kThreads, s_base, wcnt, o);
}

}  // namespace

hipError_t launch_route(const Layout& L, const int32_t* ids, int32_t T, const RouteOut& o, int bm,
                        hipStream_t stream) {
  const int R = T * L.k;
  const int E = L.E;
  if (R <= kSmallRoutes) {
    hipLaunchKernelGGL(route_small, dim3(1), dim3(kWave), 0, stream, ids, R, E, bm, o);
    return hipGetLastError();
  }
  if (R <= kThreads) {
    hipLaunchKernelGGL(route_fused, dim3(1), dim3(kThreads), 0, stream, ids, R, E, bm, o);
    return hipGetLastError();
  }
  const int nblk = (R + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(route_count, dim3(nblk), dim3(kThreads), 0, stream, ids, R, E, o.blockcounts);
  hipLaunchKernelGGL(route_scan, dim3(1), dim3(kThreads), 0, stream, E, nblk, bm, o);
  hipLaunchKernelGGL(route_scatter, dim3(nblk), dim3(kThreads), 0, stream, ids, R, E, o);
  return hipGetLastError();
}

}  // namespace moe
