// Grouped FC1 / FC2 over MXFP4 expert weights, 16-row tiles (decode sizes).
//
// Work item = (16-row tile, group of NBW 16-row weight blocks).  K is split
// into KSPLIT contiguous ranges (a function of K only, so the fp32 summation
// order of a row does not depend on the batch), and the KSPLIT partial sums
// are added in range order 0, 1, ..., KSPLIT-1.  A workgroup has WAVES waves:
// with WAVES = KSPLIT each wave runs the shared K loop (dec_core.h) over one
// range and the sums meet in LDS; with WAVES = KSPLIT / 2 a wave runs two
// adjacent ranges as one loop with one parked partial sum (the same bits);
// with one wave the sums are added in registers.
//
// Tiles come from the route stage (the rows of one expert, 16 at a time;
// tiles past the device-side tile count exit at once) or, for the smallest
// batches, one per route: the tile of route f = t*k + s is the single row of
// token t on expert ids[f] (no route stage at all; an invalid id exits), and
// its output row is f.  An MFMA row does not mix with the others, so a row
// computed alone or within a 16-row tile gets the same bits.  Lanes of rows
// past a tile's end load a copy of its last row: their MFMA output rows are
// never stored.
//
// FC1 (pegainfer PR #867, commit 53edfa98: gather fused into the FC1 input,
// "gate|up split-half"; batchgen PR #307: w1||w3 fused): row blocks come in
// (gate j, up j) pairs; the epilogue computes h = silu(g) * u in fp32 and
// stores it (bf16 for the bf16 path, fp32 for the MXFP8 path, which
// requantises it in a separate pass).  FC2: fp32 y rows.
#include "dec_core.h"

namespace moe {
namespace {

template <bool FC1, bool MX, int NBW, int KSPLIT, int P, bool PER_ROUTE, bool GRP, int WAVES = KSPLIT>
__global__ __launch_bounds__(kWave * WAVES) void fc_dec(FcArgs a) {
  static_assert(!FC1 || NBW % 2 == 0, "FC1 groups hold gate/up pairs");
  constexpr int R = KSPLIT / WAVES;   // K ranges per wave
  static_assert(R * WAVES == KSPLIT && R <= 2 && (R == 1 || (GRP && !PER_ROUTE)),
                "two ranges per wave run on the group schedule");
  const int tile = blockIdx.y;
  int e, row0, rows;
  if constexpr (PER_ROUTE) {                 // tile = route f, one row
    e = a.route_ids[tile];
    if (e < 0 || e >= a.num_experts) return;
    row0 = tile;
    rows = 1;
  } else {
    const int ntiles = *a.tile_count;
    const int2 td = a.tiles[tile];   // grid.y never exceeds the tile list capacity
    if (tile >= ntiles) return;
    e = td.x;
    row0 = td.y;
    rows = min(kBM, a.offsets[e + 1] - row0);
  }
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int m = lane & 15, kq = lane >> 4;

  const int mr = min(m, rows - 1);
  long long arow;
  if constexpr (PER_ROUTE) arow = FC1 ? (long long)(row0 / a.top_k) : (long long)row0;
  else arow = FC1 ? (long long)(a.perm[row0 + mr] / a.top_k) : (long long)(row0 + mr);

  const int nb0 = blockIdx.x * NBW;
  int lo, hi;
  dec_krange<KSPLIT>(a.mat.kb, wave * R, &lo, &hi);
  f32x4_t acc[NBW];
  f32x4_t first[NBW];   // R = 2: the sum of the wave's first range
  if constexpr (R == 2) {
    int lo1, hi1;
    dec_krange<KSPLIT>(a.mat.kb, wave * R + 1, &lo1, &hi1);
    const int split = hi;
    hi = max(hi, hi1);
    dec_kloop<FC1, MX, NBW, P, !FC1, false, GRP>(a, e, nb0, arow, lo, hi, acc, nullptr, split, first);
  } else if constexpr (PER_ROUTE && !MX) {
    // one token row per tile: each wave stages its K range of it in its own
    // share of the dynamic LDS (launch_dec sizes it: KSPLIT ranges); measured
    // FC1 21.4 -> 19.0 us at one token, 58.5 -> 51.3 us at four
    extern __shared__ __align__(16) uint8_t row_lds[];
    const int per = dec_krange_max(a.mat.kb, KSPLIT);
    dec_kloop<FC1, MX, NBW, P, !FC1, true, GRP>(a, e, nb0, arow, lo, hi, acc, row_lds + wave * per * (kTileK * 2));
  } else {
    dec_kloop<FC1, MX, NBW, P, !FC1, false, GRP>(a, e, nb0, arow, lo, hi, acc);
  }

  // the partial sums of the K ranges, added in range order: in registers
  // with one wave, else parked in LDS by range
  constexpr int NEPI = FC1 ? NBW / 2 : NBW;   // output column blocks of the group
  __shared__ float red[WAVES == 1 ? 1 : KSPLIT][NBW][4][kWave];
  if constexpr (WAVES > 1) {
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (R == 2) red[wave * R][j][i][lane] = first[j][i];
        red[wave * R + R - 1][j][i][lane] = acc[j][i];
      }
    __syncthreads();
  }
#pragma unroll
  for (int c = WAVES == 1 ? 0 : wave; c < NEPI; c += WAVES) {
    float v0[4], v1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j0 = FC1 ? 2 * c : c;
      float s0, s1 = 0.f;
      if constexpr (WAVES == 1 && R == 2) {
        s0 = first[j0][i] + acc[j0][i];
        if (FC1) s1 = first[j0 + 1][i] + acc[j0 + 1][i];
      } else if constexpr (WAVES == 1) {
        s0 = acc[j0][i];
        if (FC1) s1 = acc[j0 + 1][i];
      } else {
        s0 = red[0][j0][i][lane];
        if (FC1) s1 = red[0][j0 + 1][i][lane];
#pragma unroll
        for (int w = 1; w < KSPLIT; ++w) {
          s0 += red[w][j0][i][lane];
          if (FC1) s1 += red[w][j0 + 1][i][lane];
        }
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

// CAP: single-wave workgroups reserve a sixth of the CU's 160 KB of LDS
// (unused: an occupancy cap) so that at most six share a CU.  Measured for
// FC2 at intermediate 2048, same box, against eight per CU (the register
// limit): 270 -> 261 us at 128 tokens, 210 -> 206 us at 64, equal at 16 and
// slightly slower at 8; seven per CU gained half as much, five the same as
// six, four nothing.
constexpr int kOneWaveWgPerCu = 6;
constexpr size_t kOneWaveWgLds = (160 * 1024 / kOneWaveWgPerCu) & ~(size_t)511;

// R = K ranges per wave (the group schedule only; 1 without it).
template <bool FC1, bool MX, int NBW, int KSPLIT, int P, bool PER_ROUTE, int R, bool CAP = false>
hipError_t launch_dec(const FcArgs& a, int tiles_max, hipStream_t stream) {
  const dim3 grid(a.mat.nb / NBW, tiles_max);
  const size_t lds = PER_ROUTE && !MX ? (size_t)KSPLIT * dec_krange_max(a.mat.kb, KSPLIT) * kTileK * 2
                     : CAP && KSPLIT / R == 1 && a.mat.kb % 4 == 0 ? kOneWaveWgLds : 0;
  // whole scale groups per K range: the group schedule (one scale load per
  // four column blocks; measured 6 % faster FC1 and 3 % faster FC2 at 128
  // tokens, 2-7 % faster layers from 1 to 128 tokens)
  if (a.mat.kb % 4 == 0)
    hipLaunchKernelGGL((fc_dec<FC1, MX, NBW, KSPLIT, P, PER_ROUTE, true, KSPLIT / R>), grid,
                       dim3(kWave * (KSPLIT / R)), lds, stream, a);
  else
    hipLaunchKernelGGL((fc_dec<FC1, MX, NBW, KSPLIT, P, PER_ROUTE, false>), grid, dim3(kWave * KSPLIT), lds, stream,
                       a);
  return hipGetLastError();
}

// The K split is fixed per matrix (it sets the fp32 summation order); the
// row-block group width, the load depth and the ranges per wave only change
// the schedule.
constexpr int kSmallTokens = 4;

template <bool FC1, bool MX, int NBW, int P, bool PER_ROUTE = false, int R = 1, bool CAP = false>
hipError_t launch_sched(const FcArgs& a, int tiles_max, hipStream_t stream) {
  if (dec_ksplit(a.mat.kb) == 4) return launch_dec<FC1, MX, NBW, 4, P, PER_ROUTE, R, CAP>(a, tiles_max, stream);
  return launch_dec<FC1, MX, NBW, 2, P, PER_ROUTE, R, CAP>(a, tiles_max, stream);
}

// Schedules (every row-block count here is a multiple of 8: H, I multiples of
// 128).  Up to 4 tokens: two row blocks per workgroup, two column blocks
// loaded ahead, one K range per wave (the most waves for the fewest tiles);
// larger batches: four row blocks (measured 9-10 % faster than two from 8 to
// 16 tokens; eight FC1 row blocks, or three column blocks ahead, were slower
// there; with the group schedule four FC2 row blocks also beat eight by 3-4 %
// at 64 and 128 tokens).  Two K ranges per wave: FC2 (intermediate 2048: one
// wave per workgroup) 286 -> 271 us at 128 tokens, 51 -> 50 us at 8; FC1
// (hidden 7168: two waves) about 1 % faster from 64 tokens, 3 % slower at 8,
// where fewer waves leave the chip short of loads in flight.  The same
// threshold turns on the single-wave workgroup cap (CAP above).
constexpr int kWideTokens = 32;

template <bool FC1, bool MX>
hipError_t launch_fc(const FcArgs& a, int tiles_max, int tokens, hipStream_t stream) {
  if (tokens <= kSmallTokens) return launch_sched<FC1, MX, 2, 2>(a, tiles_max, stream);
  if (tokens < kWideTokens) {
    if (FC1) return launch_sched<FC1, MX, 4, 2>(a, tiles_max, stream);
    return launch_sched<FC1, MX, 4, 2, false, 2>(a, tiles_max, stream);
  }
  return launch_sched<FC1, MX, 4, 2, false, 2, true>(a, tiles_max, stream);
}

}  // namespace

hipError_t launch_fc1_bf16(const FcArgs& a, int tiles_max, int tokens, hipStream_t s) {
  return launch_fc<true, false>(a, tiles_max, tokens, s);
}
hipError_t launch_fc2_bf16(const FcArgs& a, int tiles_max, int tokens, hipStream_t s) {
  return launch_fc<false, false>(a, tiles_max, tokens, s);
}
hipError_t launch_fc1_mx(const FcArgs& a, int tiles_max, int tokens, hipStream_t s) {
  return launch_fc<true, true>(a, tiles_max, tokens, s);
}
hipError_t launch_fc2_mx(const FcArgs& a, int tiles_max, int tokens, hipStream_t s) {
  return launch_fc<false, true>(a, tiles_max, tokens, s);
}
hipError_t launch_fc1_bf16_per_route(const FcArgs& a, int routes, hipStream_t s) {
  return launch_sched<true, false, 2, 2, true>(a, routes, s);
}

}  // namespace moe
