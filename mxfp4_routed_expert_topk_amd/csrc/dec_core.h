// The K loop of one wave of the 16-row decode FC kernels, shared by every
// kernel that runs it (the grouped decode kernels, the small-batch kernels
// and the single-launch fused forward), so a row's fp32 sum is formed by one
// piece of code wherever it runs.
//
// A wave multiplies one 16-row A tile (row `arow` per lane: lane l holds row
// l%16 of the tile, K group l/16) by NBW consecutive 16-row weight blocks
// starting at block nb0 of expert e, over the 128-K column blocks [lo, hi) in
// ascending order, streaming the repacked 1 KB tiles with 128-bit loads kept
// P column blocks ahead of the MFMAs.
//
// bf16 path: A = bf16 activations, B = E2M1 codes dequantised in registers to
// bf16 by the gfx950 scaled converter (value * 2^(scale-127), exact), four
// v_mfma_f32_16x16x32_bf16 per column block.  MXFP8 path: A = E4M3 codes +
// E8M0 per 32, B = the same E2M1 tiles + E8M0, one
// v_mfma_scale_f32_16x16x128_f8f6f4 per column block, which applies both
// block scales inside the instruction.
#pragma once

#include "moe_internal.h"

namespace moe {

// Largest K range of one wave, in 128-K column blocks (checked against the K
// split at the end of this file).
constexpr int kMaxStagedBlocks = 32;

template <bool MX>
struct AFrag;
template <>
struct AFrag<false> { uint4 v[4]; };                 // 32 bf16 = K 32*kq .. +32 of one 128-K block
template <>
struct AFrag<true> { uint4 lo, hi; uint32_t scale; };  // 32 E4M3 + E8M0 of group kq

// Weight-code loads carry the non-temporal hint: each weight byte is read
// once per forward.
//
// Two load schedules, the same arithmetic.  PIPE = false: each loop turn
// computes and reloads its P column blocks under one condition per block,
// across which the compiler cannot count loads, so each turn starts by
// waiting for every load in flight (the P blocks then arrive as one burst of
// adjacent tiles).  PIPE = true: whole groups of P blocks run with no
// condition (loads past hi fetch block hi - 1 again and go unused) and the
// last n % P blocks follow with no loads, so each compute waits only for its
// own block, P blocks deep.  Measured at hidden 7168 / intermediate 2048 /
// top-8: PIPE 2-5 % faster for the grouped FC2 at every batch size and for
// the FC2 + sum kernel at four tokens; the burst 1 % faster for FC1 at 128
// tokens and 7-10 % faster for the per-route FC1 and the FC2 + sum kernel at
// one token.
//
// GRP (P = 2; lo and hi multiples of four): one group of four column blocks
// per turn, the group's scale dwords loaded once, with its first block (a
// lane's scale dword covers the four blocks of a group: loading it with every
// block moved four times the scale bytes through the load path); measured
// FC1 548 -> 515 us and FC2 287 -> 278 us at 128 tokens.
//
// Two K ranges in one wave (GRP only): with `first` given, the wave runs
// [lo, hi) as one loop but parks the sum of [lo, split) in `first` when the
// loop reaches split and restarts acc from zero, so each range keeps the sum
// it has when a wave of its own computes it (split is a group boundary, met
// at the start of a turn).
//
// ALDS (bf16 only): every lane's A row is the same row (one route per tile).
// Loaded per lane, each column block took four 1 KB load instructions for
// 256 distinct bytes; instead the wave copies its K range of the row to its
// own LDS region `alds` (n * 256 bytes) once, in 1 KB loads issued ahead of
// the weight prologue, and reads the fragments from there (16-lane broadcast
// reads).  Only this wave touches its region, so no barrier is needed.
template <bool FC1, bool MX, int NBW, int P, bool PIPE = false, bool ALDS = false, bool GRP = false>
__device__ __forceinline__ void dec_kloop(const FcArgs& a, int e, int nb0, long long arow, int lo, int hi,
                                          f32x4_t (&acc)[NBW], uint8_t* alds = nullptr, int split = 0,
                                          f32x4_t* first = nullptr) {
  static_assert(!(ALDS && MX), "the staged row is bf16");
  static_assert(!GRP || P == 2, "the group schedule keeps two column blocks in flight");
  const int lane = threadIdx.x & (kWave - 1);
  const int kq = lane >> 4;
  const MatLayout M = a.mat;
  const uint8_t* cbase = a.codes + ((size_t)e * M.nb + nb0) * M.kb * kTileBytes + lane * 16;
  const size_t cstride = (size_t)M.kb * kTileBytes;
  const uint8_t* sbase = a.scales + ((size_t)e * M.nb + nb0) * M.kb4 * kScaleGroupBytes + lane * 4;
  const size_t sstride = (size_t)M.kb4 * kScaleGroupBytes;
  const int n = hi - lo;

#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (first) first[j] = acc[j];
  }

  uint4 Wr[P][NBW];
  uint32_t Sr[P][NBW];
  AFrag<MX> Ar[P];

  // Both layers: at 4-128 tokens non-temporal FC2 codes save 1-2.5% of the
  // layer against plain loads (FC2 itself runs 1-3% slower; FC1 and the
  // combine run faster by more).
  auto load_codes = [&](uint4 (&w)[NBW], int kb) {
    kb = min(kb, hi - 1);
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
      const u32x4_t v = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(cbase + j * cstride + (size_t)kb * kTileBytes));
      w[j] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  };
  auto load_scale = [&](uint32_t (&s)[NBW], int kb) {
    kb = min(kb, hi - 1);
#pragma unroll
    for (int j = 0; j < NBW; ++j)
      s[j] = *reinterpret_cast<const uint32_t*>(sbase + j * sstride + (size_t)(kb >> 2) * kScaleGroupBytes);
  };
  auto load_w = [&](uint4 (&w)[NBW], uint32_t (&s)[NBW], int kb) {
    kb = min(kb, hi - 1);
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
      const u32x4_t v = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(cbase + j * cstride + (size_t)kb * kTileBytes));
      w[j] = make_uint4(v[0], v[1], v[2], v[3]);
      s[j] = *reinterpret_cast<const uint32_t*>(sbase + j * sstride + (size_t)(kb >> 2) * kScaleGroupBytes);
    }
  };
  auto load_a = [&](AFrag<MX>& af, int kb) {
    kb = min(kb, hi - 1);
    if constexpr (ALDS) {
      const uint4* ap = reinterpret_cast<const uint4*>(alds + (kb - lo) * (kTileK * 2) + kq * 64);
#pragma unroll
      for (int q = 0; q < 4; ++q) af.v[q] = ap[q];
    } else if constexpr (!MX) {
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
  auto load = [&](uint4 (&w)[NBW], uint32_t (&s)[NBW], AFrag<MX>& af, int kb) {
    load_w(w, s, kb);
    load_a(af, kb);
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
    if constexpr (ALDS) {
      // the row's bytes [lo, hi) * 256 in 1 KB loads (a fixed count: chunks past
      // the range are clamped to its last 16 bytes, read and written again
      // with the same value, so no load or write sits behind a condition),
      // then the weight loads of the prologue, then the LDS writes, which wait
      // only for the row's loads
      constexpr int kRowLoads = kMaxStagedBlocks * kTileK * 2 / 1024;
      const int nbytes = n * kTileK * 2;
      const uint8_t* row = static_cast<const uint8_t*>(a.a) + (arow * a.lda + (long long)lo * kTileK) * 2;
      uint4 st[kRowLoads];
      int off[kRowLoads];
#pragma unroll
      for (int i = 0; i < kRowLoads; ++i) {
        off[i] = min(i * 1024 + lane * 16, nbytes - 16);
        st[i] = *reinterpret_cast<const uint4*>(row + off[i]);
      }
      if constexpr (GRP) {
        load_codes(Wr[0], lo);
        load_scale(Sr[0], lo);
        load_codes(Wr[1], lo + 1);
      } else {
#pragma unroll
        for (int p = 0; p < P; ++p) load_w(Wr[p], Sr[p], lo + p);
      }
#pragma unroll
      for (int i = 0; i < kRowLoads; ++i) *reinterpret_cast<uint4*>(alds + off[i]) = st[i];
#pragma unroll
      for (int p = 0; p < P; ++p) load_a(Ar[p], lo + p);
    } else if constexpr (GRP) {
      load_codes(Wr[0], lo);
      load_scale(Sr[0], lo);
      load_a(Ar[0], lo);
      load_codes(Wr[1], lo + 1);
      load_a(Ar[1], lo + 1);
    } else {
#pragma unroll
      for (int p = 0; p < P; ++p) load(Wr[p], Sr[p], Ar[p], lo + p);
    }
    if constexpr (GRP) {
      // one group of four column blocks per turn (lo and n are multiples of
      // four): the group's scale dwords arrived with its first block, in
      // Sr[0], and the next group's are loaded with that block's load, two
      // blocks ahead; slots alternate 0, 1, 0, 1
      // (scheduling barriers keep each block's loads where they are written:
      // left free, the scheduler moved the next group's scale loads to the
      // end of the turn, right before their first use)
      for (int it = 0; it < n; it += 4) {
        if (first && lo + it == split) {
#pragma unroll
          for (int j = 0; j < NBW; ++j) {
            first[j] = acc[j];
            acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
        }
        uint32_t cur[NBW];
#pragma unroll
        for (int j = 0; j < NBW; ++j) cur[j] = Sr[0][j];
        compute(Wr[0], cur, Ar[0], lo + it);
        load_codes(Wr[0], lo + it + 2);
        load_a(Ar[0], lo + it + 2);
        __builtin_amdgcn_sched_barrier(0);
        compute(Wr[1], cur, Ar[1], lo + it + 1);
        load_codes(Wr[1], lo + it + 3);
        load_a(Ar[1], lo + it + 3);
        __builtin_amdgcn_sched_barrier(0);
        compute(Wr[0], cur, Ar[0], lo + it + 2);
        load_codes(Wr[0], lo + it + 4);
        load_scale(Sr[0], lo + it + 4);
        load_a(Ar[0], lo + it + 4);
        __builtin_amdgcn_sched_barrier(0);
        compute(Wr[1], cur, Ar[1], lo + it + 3);
        load_codes(Wr[1], lo + it + 5);
        load_a(Ar[1], lo + it + 5);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (PIPE) {
      int it = 0;
      for (; it + P <= n; it += P) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
          compute(Wr[p], Sr[p], Ar[p], lo + it + p);
          load(Wr[p], Sr[p], Ar[p], lo + it + p + P);
        }
      }
#pragma unroll
      for (int p = 0; p < P - 1; ++p)
        if (it + p < n) compute(Wr[p], Sr[p], Ar[p], lo + it + p);
    } else {
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
  }
}

// K range of wave w of KSPLIT: whole groups of four column blocks (the unit of
// the scale layout: one scale dword per lane covers a group), the first
// G % KSPLIT waves of G groups one group more; ranges in order, the last
// clipped to kb.
template <int KSPLIT>
__device__ __forceinline__ void dec_krange(int kb, int w, int* lo, int* hi) {
  const int g = (kb + 3) / 4, q = g / KSPLIT, r = g % KSPLIT;
  const int g0 = w * q + min(w, r);
  *lo = min(kb, 4 * g0);
  *hi = min(kb, 4 * (g0 + q + (w < r ? 1 : 0)));
}

// The longest range dec_krange gives, in column blocks.
__host__ __device__ constexpr int dec_krange_max(int kb, int ksplit) {
  return 4 * (((kb + 3) / 4 + ksplit - 1) / ksplit);
}

// The K split of a matrix: four ranges for long K (>= kKsplit4Blocks column
// blocks), two otherwise -- a function of K alone, so every batch size and
// kernel sums a row in the same order.
__host__ __device__ constexpr int dec_ksplit(int kb) { return kb >= kKsplit4Blocks ? 4 : 2; }

static_assert(dec_krange_max(kMaxDimension / kTileK, 4) <= kMaxStagedBlocks &&
                  dec_krange_max(kKsplit4Blocks - 1, 2) <= kMaxStagedBlocks,
              "every K range fits the staged-row buffer");

}  // namespace moe
