// Grouped FC1 / FC2 over MXFP4 expert weights.
//
// Work item = (16-row tile of one expert's rows, pair of 16-row weight
// blocks).  A workgroup of four waves splits K into four contiguous ranges;
// each wave streams its range of the pair's repacked tiles with 128-bit loads
// and accumulates in MFMA registers; the four partial sums are added through
// LDS in a fixed order (wave 0 + 1 + 2 + 3), so results do not depend on
// timing.  Row tiles come from the route stage (moe_internal.h); tiles past
// the device-side tile count exit at once.
//
// bf16 path: A = bf16 activations, B = E2M1 codes dequantised in registers to
// bf16 by the gfx950 scaled converter (value * 2^(scale-127), exact), on
// v_mfma_f32_16x16x32_bf16.  MXFP8 path: A = E4M3 codes + E8M0 per 32, B = the
// same E2M1 tiles + E8M0, on v_mfma_scale_f32_16x16x128_f8f6f4, which applies
// both block scales inside the instruction.
//
// FC1 (pegainfer PR #867, commit 53edfa98: gather fused into the FC1 input,
// "gate|up split-half"; batchgen PR #307: w1||w3 fused): the pair is (gate
// block j, up block j); the epilogue computes h = silu(g) * u in fp32 and
// stores it (bf16 for the bf16 path, fp32 for the MXFP8 path, which
// requantises it in a separate pass).  FC2: the pair is two consecutive
// blocks of H; fp32 y rows are stored in route-row order.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <bool FC1, bool MX>
__global__ __launch_bounds__(kThreads) void fc_m16(FcArgs a) {
  const int tile = blockIdx.y;
  if (tile >= *a.tile_count) return;
  const int2 td = a.tiles[tile];
  const int e = td.x, row0 = td.y;
  const int rows = min(kBM, a.offsets[e + 1] - row0);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int m = lane & 15, kq = lane >> 4;
  const MatLayout M = a.mat;

  // A row of this lane (rows past the tile's end read nothing and stay 0)
  long long arow = -1;
  if (m < rows) arow = FC1 ? (long long)(a.perm[row0 + m] / a.top_k) : (long long)(row0 + m);

  const int nb0 = 2 * blockIdx.x;
  const uint4* c0 = reinterpret_cast<const uint4*>(a.codes + ((size_t)e * M.nb + nb0) * M.kb * kTileBytes) + lane;
  const uint4* c1 = c0 + (size_t)M.kb * kWave;
  const uint32_t* s0 = reinterpret_cast<const uint32_t*>(a.scales + ((size_t)e * M.nb + nb0) * M.kb4 * kScaleGroupBytes) + lane;
  const uint32_t* s1 = s0 + (size_t)M.kb4 * kWave;

  const int per = (M.kb + kWaves - 1) / kWaves;
  const int kb_lo = min(M.kb, wave * per), kb_hi = min(M.kb, kb_lo + per);

  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};

  for (int kb = kb_lo; kb < kb_hi; ++kb) {
    const uint4 w0 = c0[(size_t)kb * kWave];
    const uint4 w1 = c1[(size_t)kb * kWave];
    const int sh = (kb & 3) * 8;
    const uint32_t sb0 = (s0[(size_t)(kb >> 2) * kWave] >> sh) & 0xFFu;
    const uint32_t sb1 = (s1[(size_t)(kb >> 2) * kWave] >> sh) & 0xFFu;
    if constexpr (!MX) {
      uint4 av[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
      if (arow >= 0) {
        const uint4* ap = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.a) + arow * a.lda +
                                                         (size_t)kb * kTileK + kq * 32);
#pragma unroll
        for (int s = 0; s < 4; ++s) av[s] = ap[s];
      }
      const float f0 = e8m0_to_f32(sb0), f1 = e8m0_to_f32(sb1);
      const uint32_t* w0d = reinterpret_cast<const uint32_t*>(&w0);
      const uint32_t* w1d = reinterpret_cast<const uint32_t*>(&w1);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8_t A = __builtin_bit_cast(bf16x8_t, av[s]);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, dequant8(w0d[s], f0), acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, dequant8(w1d[s], f1), acc1, 0, 0, 0);
      }
    } else {
      // A: E4M3 codes, bytes [0,16) = K 16*kq.., bytes [16,32) = K 64+16*kq..;
      // A scale of this lane = (row m, K group 4*kb + kq).
      uint4 alo = make_uint4(0, 0, 0, 0), ahi = make_uint4(0, 0, 0, 0);
      uint32_t sa = 127u;
      if (arow >= 0) {
        const uint8_t* ap = static_cast<const uint8_t*>(a.a) + arow * a.lda + (size_t)kb * kTileK + kq * 16;
        alo = *reinterpret_cast<const uint4*>(ap);
        ahi = *reinterpret_cast<const uint4*>(ap + 64);
        sa = a.a_scales[arow * (a.lda / 32) + kb * 4 + kq];
      }
      const i32x8_t A = {(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w, (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
      const i32x8_t B0 = {(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, 0, 0, 0, 0};
      const i32x8_t B1 = {(int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w, 0, 0, 0, 0};
      acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B0, acc0, 0, 4, 0, (int)sa, 0, (int)sb0);
      acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B1, acc1, 0, 4, 0, (int)sa, 0, (int)sb1);
    }
  }

  // fixed-order reduction of the four K ranges
  __shared__ float red[kWaves - 1][8][kWave];
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      red[wave - 1][i][lane] = acc0[i];
      red[wave - 1][4 + i][lane] = acc1[i];
    }
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc0[i] += red[w][i][lane];
      acc1[i] += red[w][4 + i][lane];
    }
  }

  // D layout: lane holds rows 4*kq + i, column m
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * kq + i;
    if (r >= rows) continue;
    const size_t orow = (size_t)(row0 + r) * a.ldo;
    if constexpr (FC1) {
      const float hv = silu_f32(acc0[i]) * acc1[i];
      const size_t col = (size_t)blockIdx.x * kTileN + m;
      if constexpr (MX) static_cast<float*>(a.out)[orow + col] = hv;
      else static_cast<uint16_t*>(a.out)[orow + col] = f32_to_bf16_rne(hv);
    } else {
      float* y = static_cast<float*>(a.out);
      y[orow + (size_t)nb0 * kTileN + m] = acc0[i];
      y[orow + (size_t)(nb0 + 1) * kTileN + m] = acc1[i];
    }
  }
}

template <bool FC1, bool MX>
hipError_t launch_fc(const FcArgs& a, int tiles_max, hipStream_t stream) {
  const dim3 grid(a.mat.nb / 2, tiles_max);
  hipLaunchKernelGGL((fc_m16<FC1, MX>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fc1_bf16(const FcArgs& a, int tiles_max, hipStream_t s) { return launch_fc<true, false>(a, tiles_max, s); }
hipError_t launch_fc2_bf16(const FcArgs& a, int tiles_max, hipStream_t s) { return launch_fc<false, false>(a, tiles_max, s); }
hipError_t launch_fc1_mx(const FcArgs& a, int tiles_max, hipStream_t s) { return launch_fc<true, true>(a, tiles_max, s); }
hipError_t launch_fc2_mx(const FcArgs& a, int tiles_max, hipStream_t s) { return launch_fc<false, true>(a, tiles_max, s); }

}  // namespace moe
