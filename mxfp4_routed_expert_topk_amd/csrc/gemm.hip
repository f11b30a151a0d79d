// Grouped FC1 / FC2 over MXFP4 expert weights, 16-row tiles.
//
// Work item = (16-row tile of one expert's rows, group of NBW 16-row weight
// blocks).  A workgroup of KSPLIT waves splits K into KSPLIT contiguous ranges
// (a function of K only, so the fp32 summation order of a row does not depend
// on the batch); each wave streams its range of the group's repacked tiles
// with 128-bit loads kept P column blocks ahead of the MFMAs, and the KSPLIT
// partial sums are added through LDS in wave order 0, 1, ..., KSPLIT-1.  Row
// tiles come from the route stage; tiles past the device-side tile count exit
// at once.  Lanes of rows past a tile's end load a copy of its last row: their
// MFMA output rows are never stored, and MFMA rows do not mix.
//
// bf16 path: A = bf16 activations, B = E2M1 codes dequantised in registers to
// bf16 by the gfx950 scaled converter (value * 2^(scale-127), exact), on
// v_mfma_f32_16x16x32_bf16.  MXFP8 path: A = E4M3 codes + E8M0 per 32, B = the
// same E2M1 tiles + E8M0, on v_mfma_scale_f32_16x16x128_f8f6f4, which applies
// both block scales inside the instruction.
//
// FC1 (pegainfer PR #867, commit 53edfa98: gather fused into the FC1 input,
// "gate|up split-half"; batchgen PR #307: w1||w3 fused): row blocks come in
// (gate j, up j) pairs; the epilogue computes h = silu(g) * u in fp32 and
// stores it (bf16 for the bf16 path, fp32 for the MXFP8 path, which
// requantises it in a separate pass).  FC2: fp32 y rows in route-row order.
#include "moe_internal.h"

// Weight loads with the non-temporal hint: bit 0 for FC1, bit 1 for FC2.
#ifndef MOE_NT_LOADS
#define MOE_NT_LOADS 1
#endif

namespace moe {
namespace {

template <bool MX>
struct AFrag;
template <>
struct AFrag<false> { uint4 v[4]; };                 // 32 bf16 = K 32*kq .. +32 of one 128-K block
template <>
struct AFrag<true> { uint4 lo, hi; uint32_t scale; };  // 32 E4M3 + E8M0 of group kq

template <bool FC1, bool MX, int NBW, int KSPLIT, int P>
__global__ __launch_bounds__(kWave * KSPLIT) void fc_dec(FcArgs a) {
  static_assert(!FC1 || NBW % 2 == 0, "FC1 groups hold gate/up pairs");
  const int tile = blockIdx.y;
  const int ntiles = *a.tile_count;
  const int2 td = a.tiles[tile];   // grid.y never exceeds the tile list capacity
  if (tile >= ntiles) return;
  const int e = td.x, row0 = td.y;
  const int rows = min(kBM, a.offsets[e + 1] - row0);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int m = lane & 15, kq = lane >> 4;
  const MatLayout M = a.mat;

  const int mr = min(m, rows - 1);
  const long long arow = FC1 ? (long long)(a.perm[row0 + mr] / a.top_k) : (long long)(row0 + mr);

  const int nb0 = blockIdx.x * NBW;
  const uint8_t* cbase = a.codes + ((size_t)e * M.nb + nb0) * M.kb * kTileBytes + lane * 16;
  const size_t cstride = (size_t)M.kb * kTileBytes;
  const uint8_t* sbase = a.scales + ((size_t)e * M.nb + nb0) * M.kb4 * kScaleGroupBytes + lane * 4;
  const size_t sstride = (size_t)M.kb4 * kScaleGroupBytes;

  const int per = (M.kb + KSPLIT - 1) / KSPLIT;
  const int lo = min(M.kb, wave * per), hi = min(M.kb, lo + per);
  const int n = hi - lo;

  f32x4_t acc[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 Wr[P][NBW];
  uint32_t Sr[P][NBW];
  AFrag<MX> Ar[P];

  auto load = [&](uint4 (&w)[NBW], uint32_t (&s)[NBW], AFrag<MX>& af, int kb) {
    kb = min(kb, hi - 1);
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const uint4* wp = reinterpret_cast<const uint4*>(cbase + j * cstride + (size_t)kb * kTileBytes);
      if constexpr ((FC1 && (MOE_NT_LOADS & 1)) || (!FC1 && (MOE_NT_LOADS & 2))) {
        typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wp));  // streamed once
        w[j] = make_uint4(v[0], v[1], v[2], v[3]);
      } else {
        w[j] = *wp;
      }
      s[j] = *reinterpret_cast<const uint32_t*>(sbase + j * sstride + (size_t)(kb >> 2) * kScaleGroupBytes);
    }
    if constexpr (!MX) {
      const uint4* ap = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.a) + arow * a.lda +
                                                       (size_t)kb * kTileK + kq * 32);
#pragma unroll
      for (int q = 0; q < 4; ++q) af.v[q] = ap[q];
    } else {
      const uint8_t* ap = static_cast<const uint8_t*>(a.a) + arow * a.lda + (size_t)kb * kTileK + kq * 16;
      af.lo = *reinterpret_cast<const uint4*>(ap);
      af.hi = *reinterpret_cast<const uint4*>(ap + 64);
      af.scale = a.a_scales[arow * (a.lda / 32) + kb * 4 + kq];
    }
  };

  auto compute = [&](const uint4 (&w)[NBW], const uint32_t (&s)[NBW], const AFrag<MX>& af, int kb) {
    const int sh = (kb & 3) * 8;
    if constexpr (!MX) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x8_t A = __builtin_bit_cast(bf16x8_t, af.v[q]);
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          const uint32_t wd = q == 0 ? w[j].x : q == 1 ? w[j].y : q == 2 ? w[j].z : w[j].w;
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, dequant8(wd, e8m0_to_f32((s[j] >> sh) & 0xFFu)),
                                                           acc[j], 0, 0, 0);
        }
      }
    } else {
      const i32x8_t A = {(int)af.lo.x, (int)af.lo.y, (int)af.lo.z, (int)af.lo.w,
                         (int)af.hi.x, (int)af.hi.y, (int)af.hi.z, (int)af.hi.w};
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const i32x8_t B = {(int)w[j].x, (int)w[j].y, (int)w[j].z, (int)w[j].w, 0, 0, 0, 0};
        acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc[j], 0, 4, 0, (int)af.scale, 0,
                                                                  (int)((s[j] >> sh) & 0xFFu));
      }
    }
  };

  if (n > 0) {
#pragma unroll
    for (int p = 0; p < P; ++p) load(Wr[p], Sr[p], Ar[p], lo + p);
    for (int it = 0; it < n; it += P) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        if (it + p < n) {
          compute(Wr[p], Sr[p], Ar[p], lo + it + p);
          load(Wr[p], Sr[p], Ar[p], lo + it + p + P);
        }
      }
    }
  }

  // every wave parks its partial sums; the epilogue adds them in wave order
  __shared__ float red[KSPLIT][NBW][4][kWave];
#pragma unroll
  for (int j = 0; j < NBW; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][j][i][lane] = acc[j][i];
  __syncthreads();

  constexpr int NEPI = FC1 ? NBW / 2 : NBW;   // output column blocks of the group
  for (int c = wave; c < NEPI; c += KSPLIT) {
    float v0[4], v1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j0 = FC1 ? 2 * c : c;
      float s0 = red[0][j0][i][lane], s1 = FC1 ? red[0][j0 + 1][i][lane] : 0.f;
#pragma unroll
      for (int w = 1; w < KSPLIT; ++w) {
        s0 += red[w][j0][i][lane];
        if (FC1) s1 += red[w][j0 + 1][i][lane];
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

template <bool FC1, bool MX, int NBW, int KSPLIT, int P>
hipError_t launch_dec(const FcArgs& a, int tiles_max, hipStream_t stream) {
  const dim3 grid(a.mat.nb / NBW, tiles_max);
  hipLaunchKernelGGL((fc_dec<FC1, MX, NBW, KSPLIT, P>), grid, dim3(kWave * KSPLIT), 0, stream, a);
  return hipGetLastError();
}

// The K split is fixed per matrix (it sets the fp32 summation order); the
// row-block group width and the load depth only change the schedule.  The
// schedule knobs below are compile-time so variants can be built and timed.
#ifndef MOE_SMALL_T
#define MOE_SMALL_T 16
#endif
#ifndef MOE_FC1_SMALL
#define MOE_FC1_SMALL 2, 2
#endif
#ifndef MOE_FC1_LARGE
#define MOE_FC1_LARGE 4, 2
#endif
#ifndef MOE_FC2_SMALL
#define MOE_FC2_SMALL 2, 2
#endif
#ifndef MOE_FC2_LARGE
#define MOE_FC2_LARGE 8, 2
#endif

template <int NBW, int P>
struct Sched {};

template <bool FC1, bool MX, int NBW, int P>
hipError_t launch_sched(Sched<NBW, P>, const FcArgs& a, int tiles_max, hipStream_t stream) {
  // K split: four ranges for long K (>= kKsplit4Blocks column blocks), two
  // otherwise.  It depends on K alone, so every batch size sums a row in the
  // same order.
  if (a.mat.kb >= kKsplit4Blocks) return launch_dec<FC1, MX, NBW, 4, P>(a, tiles_max, stream);
  return launch_dec<FC1, MX, NBW, 2, P>(a, tiles_max, stream);
}

template <bool FC1, bool MX>
hipError_t launch_fc(const FcArgs& a, int tiles_max, int tokens, hipStream_t stream) {
  // every row-block count here is a multiple of 8 (H, I multiples of 128)
  if (tokens <= MOE_SMALL_T) {
    if (FC1) return launch_sched<FC1, MX>(Sched<MOE_FC1_SMALL>{}, a, tiles_max, stream);
    return launch_sched<FC1, MX>(Sched<MOE_FC2_SMALL>{}, a, tiles_max, stream);
  }
  if (FC1) return launch_sched<FC1, MX>(Sched<MOE_FC1_LARGE>{}, a, tiles_max, stream);
  return launch_sched<FC1, MX>(Sched<MOE_FC2_LARGE>{}, a, tiles_max, stream);
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

}  // namespace moe
