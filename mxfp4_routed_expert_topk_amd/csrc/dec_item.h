// One work item of the 16-row-tile decode FC kernels (FC1 with the SiLU gate,
// or FC2) for the fused decode kernel: the body of gemm.hip's fc_dec, with the
// waves of a workgroup split into column sub-groups.  See gemm.hip for the
// method.  It computes exactly what fc_dec computes (the same K ranges summed
// in the same order; the fused tests compare the two bit for bit).  fc_dec
// keeps its own copy: run through this function, the compiler placed one
// coarse wait for all loads in flight at the head of fc_dec's K loop instead
// of a wait before each use, and the decode FC2 kernel lost 3 %.
#pragma once

#include "moe_internal.h"

#ifndef MOE_NT_LOADS
#define MOE_NT_LOADS 1
#endif

namespace moe {

template <bool MX>
struct AFrag;
template <>
struct AFrag<false> { uint4 v[4]; };                 // 32 bf16 = K 32*kq .. +32 of one 128-K block
template <>
struct AFrag<true> { uint4 lo, hi; uint32_t scale; };  // 32 E4M3 + E8M0 of group kq

// One work item (tile td = (expert, first row), group of SUBS x NBW weight row blocks) on SUBS x KSPLIT
// waves: wave w takes K range w % KSPLIT of row blocks NBW (SUBS group + w /
// KSPLIT) ..; the KSPLIT partial sums of a row block are added in range
// order.  Every output element sees the same K ranges, summed in the same
// order, whatever SUBS is.  The item ends with all of its stores issued (no
// barrier after them: a caller running items back to back puts one between
// them, the next item writes the same partial-sum LDS).
template <bool FC1, bool MX, int NBW, int KSPLIT, int SUBS, int P>
__device__ __forceinline__ void dec_item(const FcArgs& a, int2 td, int group) {
  static_assert(!FC1 || NBW % 2 == 0, "FC1 groups hold gate/up pairs");
  const int e = td.x, row0 = td.y;
  const int rows = min(kBM, a.offsets[e + 1] - row0);
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int sub = wv / KSPLIT, wave = wv % KSPLIT;   // column sub-group, K range
  const int m = lane & 15, kq = lane >> 4;
  const MatLayout M = a.mat;

  const int mr = min(m, rows - 1);
  const long long arow = FC1 ? (long long)(a.perm[row0 + mr] / a.top_k) : (long long)(row0 + mr);

  const int nb0 = (group * SUBS + sub) * NBW;
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

  // every wave parks its partial sums; the epilogue adds them in range order
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

}  // namespace moe
