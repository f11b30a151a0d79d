// The whole decode layer in one launch: route -> FC1 + SiLU gate -> FC2 ->
// slot-order combine, for batches of at most kFusedMaxRoutes routes on the
// bf16 path.  The pages' fused kernel (pegainfer PR #867, commit 33d22f80 and
// the "mega MoE" path: dispatch, FC1, activation, FC2 and combine in one
// launch) was 5-8 % faster per layer than the multi-launch chain; at decode
// sizes the chain here spends a good part of its time between launches.
//
// Every workgroup routes the batch itself into LDS (one wave, the same code
// and row order as the stand-alone route kernel), so no barrier follows the
// routing.  Work is a list of items in dependency order -- FC1 items (tile,
// group of weight row blocks), then FC2 items, then combine items (token,
// 1024 columns) -- and workgroup b takes items b, b + G, b + 2G, ...  An item
// waits only for items of smaller index: an FC2 item for the FC1 items of
// its tile, a combine item for the FC2 items of the tiles its routes sit in.
// A workgroup finishes its own earlier items before it waits, and the launch
// is cooperative (every workgroup resident at once), so every wait ends.
// Each wait is also bounded in time: past the bound the item is skipped and
// the error word takes the forward's generation, which makes every later wait
// of that forward give up at once; the kernel always runs to its end.
//
// FC1 and FC2 items run the stand-alone decode kernels' K loop (dec_core.h)
// with the same K split per matrix, so every output element is
// summed over the same K ranges in the same order: the result is bitwise the
// multi-launch forward's wherever that runs the decode kernels (it takes the
// 128-row prefill kernels from 16 routes per expert on).  The combine item is
// the combine kernel's arithmetic.
//
// Cross-workgroup order: a workgroup that finished an item's stores waits
// for them (the barrier), one thread fences at agent scope (the L2s of the
// XCDs are not coherent with each other inside a kernel; the fence writes
// them back) and adds one to the item's counter.  Waiters poll with acquire
// loads and fence again before reading.  The counters start at zero: the
// last workgroup to finish (a count of finished workgroups says which) sets
// them back to zero, so the next call, ordered after this kernel on the
// stream, finds them so (a zero-filled workspace starts them).  A plain
// atomic add per item: 128 workgroups finishing items of one tile at once
// made a compare-and-swap loop retry its way to milliseconds.
#include <atomic>

#include "dec_core.h"
#include "route_wave.h"

namespace moe {
namespace {

// One work item of the 16-row decode FC kernels (FC1 with the SiLU gate, or
// FC2): tile td = (expert, first row), group of SUBS x NBW weight row blocks,
// on SUBS x KSPLIT waves: wave w takes K range w % KSPLIT of row blocks
// NBW (SUBS group + w / KSPLIT) ..; the KSPLIT partial sums of a row block are
// added in range order.  Every output element sees the K loop (dec_core.h)
// and the range order of the 16-row kernels, whatever SUBS is.  The item ends
// with all of its stores issued (a caller running items back to back puts a
// barrier between them: the next item writes the same partial-sum LDS).
template <bool FC1, bool MX, int NBW, int KSPLIT, int SUBS, int P>
__device__ __forceinline__ void dec_item(const FcArgs& a, int2 td, int group) {
  static_assert(!FC1 || NBW % 2 == 0, "FC1 groups hold gate/up pairs");
  const int e = td.x, row0 = td.y;
  const int rows = min(kBM, a.offsets[e + 1] - row0);
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int sub = wv / KSPLIT, wave = wv % KSPLIT;   // column sub-group, K range
  const int m = lane & 15, kq = lane >> 4;
  const int mr = min(m, rows - 1);
  const long long arow = FC1 ? (long long)(a.perm[row0 + mr] / a.top_k) : (long long)(row0 + mr);
  const int nb0 = (group * SUBS + sub) * NBW;
  int lo, hi;
  dec_krange<KSPLIT>(a.mat.kb, wave, &lo, &hi);
  f32x4_t acc[NBW];
  dec_kloop<FC1, MX, NBW, P>(a, e, nb0, arow, lo, hi, acc);

  __shared__ float red[SUBS * KSPLIT][NBW][4][kWave];
#pragma unroll
  for (int j = 0; j < NBW; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wv][j][i][lane] = acc[j][i];
  __syncthreads();
  float (*rs)[NBW][4][kWave] = red + sub * KSPLIT;   // this sub-group's KSPLIT partial sets

  constexpr int NEPI = FC1 ? NBW / 2 : NBW;   // output column blocks of the group
  for (int c = wave; c < NEPI; c += KSPLIT) {
    float v0[4], v1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j0 = FC1 ? 2 * c : c;
      float s0 = rs[0][j0][i][lane], s1 = FC1 ? rs[0][j0 + 1][i][lane] : 0.f;
#pragma unroll
      for (int w = 1; w < KSPLIT; ++w) {
        s0 += rs[w][j0][i][lane];
        if (FC1) s1 += rs[w][j0 + 1][i][lane];
      }
      v0[i] = s0;
      v1[i] = s1;
    }
    // D layout: lane holds rows 4*kq + i, column m
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * kq + i;
      if (r >= rows) continue;
      const size_t orow = (size_t)(row0 + r) * a.ldo;
      if constexpr (FC1) {
        const float hv = silu_f32(v0[i]) * v1[i];
        const size_t col = (size_t)(nb0 / 2 + c) * kTileN + m;
        if constexpr (MX) static_cast<float*>(a.out)[orow + col] = hv;
        else static_cast<uint16_t*>(a.out)[orow + col] = f32_to_bf16_rne(hv);
      } else {
        static_cast<float*>(a.out)[orow + (size_t)(nb0 + c) * kTileN + m] = v0[i];
      }
    }
  }
}

constexpr int kThreads = 4 * kWave;
constexpr int kNBW = 2;                                // weight row blocks per wave and item
constexpr int kP = 3;                                  // K blocks loaded ahead
constexpr int kCombineCols = 4 * kThreads;             // output columns per combine item
constexpr int kMaxTiles = kFusedMaxTiles;

struct FusedArgs {
  FcArgs f1, f2;                 // weights, activations and outputs; route fields are set in the kernel
  const int32_t* ids;
  const float* weights;
  int T, k, E, H;
  float* acc;                    // or null
  uint16_t* out;
  RouteOut route;                // the route outputs, published by workgroup 0
  uint32_t* fc1_done;            // [kMaxTiles] finished FC1 items per tile
  uint32_t* fc2_done;            // [kMaxTiles] the same for FC2
  uint32_t* wg_done;             // finished workgroups
  uint32_t* error;               // the generation of a forward whose wait timed out
  uint32_t gen;
  long long spin_ticks;          // bound of one wait in s_memrealtime ticks (100 MHz)
};

// A run of this workgroup's items -- item indices first, first + G, ...
// below end, the run's kind starting at item `base` with g items per tile --
// made visible to every workgroup, then counted per tile (all threads call
// it; the barrier completes every wave's stores, thread 0's fence writes
// them back for the other XCDs).
__device__ void publish_run(uint32_t* counts, int first, int end, int G, int g, int base) {
  if (first >= end) return;   // uniform: nothing to publish, no fence (each one writes back the L2)
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    for (int i = first; i < end; i += G)
      __hip_atomic_fetch_add(&counts[(i - base) / g], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Thread 0: poll until *c == target, the error word holds this forward's
// generation, or the time bound passes (then set the error word).  True when
// the target was seen.  The poll count is capped as well, so the wait ends
// whatever the clock does.
constexpr int kMaxPolls = 1 << 22;
__device__ bool poll(const uint32_t* c, uint32_t target, const FusedArgs& p) {
  const long long t0 = (long long)__builtin_amdgcn_s_memrealtime();
  for (int n = 0; n < kMaxPolls; ++n) {
    // relaxed: an acquire load invalidates the L2 on every poll, under the
    // feet of the workgroups still streaming weights through it; the caller
    // fences once when the count is there
    if (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == target) return true;
    if (__hip_atomic_load(p.error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == p.gen) return false;
    if ((long long)__builtin_amdgcn_s_memrealtime() - t0 > p.spin_ticks) break;
    __builtin_amdgcn_s_sleep(8);
  }
  __hip_atomic_store(p.error, p.gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return false;
}

template <int KS1, int KS2>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void fused_decode(FusedArgs p) {
  __shared__ int s_cnt[1024];                       // route scratch
  __shared__ int l_counts[1024], l_offsets[1025], l_perm[kFusedMaxRoutes], l_rowpos[kFusedMaxRoutes];
  __shared__ int2 l_tiles[kMaxTiles];
  __shared__ int l_tile_count;
  __shared__ uint16_t l_tile_of_row[kFusedMaxRoutes];  // tile index of each route row
  __shared__ int l_ok;

  const int R = p.T * p.k;
  const int t = threadIdx.x;
  if (t < kWave) {
    RouteOut lo{};
    lo.counts = l_counts;
    lo.offsets = l_offsets;
    lo.perm = l_perm;
    lo.rowpos = l_rowpos;
    lo.tiles = l_tiles;
    lo.tile_count = &l_tile_count;
    route_wave(p.ids, R, p.E, kBM, lo, s_cnt);
  }
  __syncthreads();
  const int ntiles = l_tile_count;
  for (int i = t; i < ntiles; i += kThreads) {
    const int2 td = l_tiles[i];
    const int rows = min(kBM, l_offsets[td.x + 1] - td.y);
    for (int r = 0; r < rows; ++r) l_tile_of_row[td.y + r] = (uint16_t)i;
  }
  if (blockIdx.x == 0) {   // the same route outputs as the multi-launch forward leaves in the workspace
    for (int i = t; i < p.E; i += kThreads) {
      p.route.counts[i] = l_counts[i];
      p.route.offsets[i] = l_offsets[i];
    }
    if (t == 0) {
      p.route.offsets[p.E] = l_offsets[p.E];
      *p.route.tile_count = ntiles;
    }
    for (int i = t; i < R; i += kThreads) {
      p.route.rowpos[i] = l_rowpos[i];
      if (i < l_offsets[p.E]) p.route.perm[i] = l_perm[i];
    }
    for (int i = t; i < ntiles; i += kThreads) p.route.tiles[i] = l_tiles[i];
  }
  __syncthreads();

  FcArgs a1 = p.f1, a2 = p.f2;
  a1.tiles = a2.tiles = l_tiles;
  a1.tile_count = a2.tile_count = &l_tile_count;
  a1.offsets = a2.offsets = l_offsets;
  a1.perm = a2.perm = l_perm;
  constexpr int S1 = 4 / KS1, S2 = 4 / KS2;        // column sub-groups per item
  const int g1 = a1.mat.nb / (kNBW * S1), g2 = a2.mat.nb / (kNBW * S2);
  const int n1 = ntiles * g1, n2 = ntiles * g2;
  const int chunks = (p.H + kCombineCols - 1) / kCombineCols;
  const int total = n1 + n2 + p.T * chunks;

  // This workgroup's items come in three runs (FC1, FC2, combine).  The FC1
  // and FC2 runs are each published once, at their end: one fence per run
  // instead of one per item (a fence writes back the L2).
  const int G = gridDim.x;
  int it = blockIdx.x;
  for (; it < n1; it += G) {
    const int tile = it / g1;
    dec_item<true, false, kNBW, KS1, S1, kP>(a1, l_tiles[tile], it - tile * g1);
    __syncthreads();   // the epilogue's reads of the partial sums are done before the next item writes them
  }
  publish_run(p.fc1_done, blockIdx.x, min(it, n1), G, g1, 0);
  const int f2_first = it;
  for (; it < n1 + n2; it += G) {
    const int j = it - n1, tile = j / g2;
    if (t == 0) {
      l_ok = poll(&p.fc1_done[tile], g1, p);
      __threadfence();
    }
    __syncthreads();
    const bool ok = l_ok;
    __syncthreads();   // every thread has read l_ok before thread 0 may write it again
    if (!ok) continue;
    dec_item<false, false, kNBW, KS2, S2, kP>(a2, l_tiles[tile], j - tile * g2);
    __syncthreads();
  }
  publish_run(p.fc2_done, f2_first, min(it, n1 + n2), G, g2, n1);
  for (; it < total; it += G) {
    {
      const int j = it - n1 - n2, tok = j / chunks, c = (j - tok * chunks) * kCombineCols + 4 * t;
      if (t == 0) {
        bool ok = true;
        for (int s = 0; s < p.k && ok; ++s) {
          const int r = l_rowpos[tok * p.k + s];
          if (r >= 0) ok = poll(&p.fc2_done[l_tile_of_row[r]], g2, p);
        }
        l_ok = ok;
        __threadfence();
      }
      __syncthreads();
      if (l_ok && c < p.H) {
        // slot-order fp32 sum, one RNE cast (the combine kernel's arithmetic)
        const float* y = static_cast<const float*>(a2.out);
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s = 0; s < p.k; ++s) {
          const int r = l_rowpos[tok * p.k + s];
          if (r < 0) continue;
          const float ws = p.weights[(size_t)tok * p.k + s];
          const float4 v = *reinterpret_cast<const float4*>(y + (size_t)r * p.H + c);
          acc.x = fmaf(ws, v.x, acc.x);
          acc.y = fmaf(ws, v.y, acc.y);
          acc.z = fmaf(ws, v.z, acc.z);
          acc.w = fmaf(ws, v.w, acc.w);
        }
        if (p.acc) *reinterpret_cast<float4*>(p.acc + (size_t)tok * p.H + c) = acc;
        const uint32_t lo = f32_to_bf16_rne(acc.x) | ((uint32_t)f32_to_bf16_rne(acc.y) << 16);
        const uint32_t hi = f32_to_bf16_rne(acc.z) | ((uint32_t)f32_to_bf16_rne(acc.w) << 16);
        *reinterpret_cast<uint2*>(p.out + (size_t)tok * p.H + c) = make_uint2(lo, hi);
      }
      __syncthreads();   // l_ok is rewritten by the next item
    }
  }
  // the last workgroup to get here sets the counters back to zero for the next call
  __syncthreads();
  if (t == 0) {
    // relaxed: every counter this workgroup added to was already published; only
    // the last workgroup, which resets them, needs to see the others' adds
    const uint32_t done = __hip_atomic_fetch_add(p.wg_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    l_ok = done == gridDim.x - 1;
    if (l_ok) __threadfence();
  }
  __syncthreads();
  if (l_ok) {
    for (int i = t; i < ntiles; i += kThreads) {
      __hip_atomic_store(&p.fc1_done[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.fc2_done[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (t == 0) __hip_atomic_store(p.wg_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Workgroups that fit the device at once (0 if it cannot launch cooperatively),
// asked once per device and kernel.
template <int KS1, int KS2>
hipError_t resident_workgroups(int* out) {
  constexpr int kDevices = 64;
  static std::atomic<int> cache[kDevices];   // 0: not asked yet; -1: no cooperative launch
  int dev = 0;
  hipError_t e;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if (dev < kDevices && cache[dev].load() != 0) {
    *out = max(0, cache[dev].load());
    return hipSuccess;
  }
  int cus = 0, per_cu = 0, coop = 0;
  if ((e = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fused_decode<KS1, KS2>, kThreads, 0)) !=
      hipSuccess)
    return e;
  const int n = coop ? per_cu * cus : 0;
  if (dev < kDevices) cache[dev].store(n > 0 ? n : -1);
  *out = n;
  return hipSuccess;
}

template <int KS1, int KS2>
hipError_t launch(FusedArgs& p, int items_max, hipStream_t stream) {
  int resident = 0;
  hipError_t e;
  if ((e = resident_workgroups<KS1, KS2>(&resident)) != hipSuccess) return e;
  if (resident <= 0) return hipErrorNotSupported;
  const int grid = max(1, min(resident, items_max));
  void* args[] = {&p};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(fused_decode<KS1, KS2>), dim3(grid),
                                    dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_fused_decode(const FcArgs& f1, const FcArgs& f2, const int32_t* ids, const float* weights,
                               int32_t T, int32_t k, int32_t E, int32_t H, float* acc, uint16_t* out,
                               const RouteOut& route, uint8_t* sync, uint32_t gen, long long spin_ticks,
                               hipStream_t stream) {
  FusedArgs p{};
  p.f1 = f1;
  p.f2 = f2;
  p.ids = ids;
  p.weights = weights;
  p.T = T;
  p.k = k;
  p.E = E;
  p.H = H;
  p.acc = acc;
  p.out = out;
  p.route = route;
  p.fc1_done = reinterpret_cast<uint32_t*>(sync);
  p.fc2_done = p.fc1_done + kMaxTiles;
  p.wg_done = p.fc2_done + kMaxTiles;
  p.error = p.wg_done + 1;
  p.gen = gen;
  p.spin_ticks = spin_ticks;
  // the K split of each matrix is the stand-alone kernels' (a function of K alone)
  const bool ks1 = dec_ksplit(f1.mat.kb) == 4, ks2 = dec_ksplit(f2.mat.kb) == 4;
  const int R = T * k;
  const int tiles = R / kBM + min(E, R);
  const int items = tiles * (f1.mat.nb / (kNBW * (ks1 ? 1 : 2)) + f2.mat.nb / (kNBW * (ks2 ? 1 : 2))) +
                    T * ((H + kCombineCols - 1) / kCombineCols);
  if (ks1 && ks2) return launch<4, 4>(p, items, stream);
  if (ks1) return launch<4, 2>(p, items, stream);
  if (ks2) return launch<2, 4>(p, items, stream);
  return launch<2, 2>(p, items, stream);
}

}  // namespace moe
