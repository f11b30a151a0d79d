// Grouped FC1 / FC2 for large batches (prefill): MFMA-bound tiles.
//
// Work item = (BM-row tile of one expert's rows, 256-column slice of the
// weight rows).  A workgroup of four waves stages, per 128-K column block,
// the BM gathered activation rows (bf16) and the sixteen raw repacked weight
// tiles (E2M1 codes, 16 KB) in LDS, prefetching the next block into
// registers while the current one is multiplied.  Each wave owns a 64-row x
// (256/WN)-column sub-tile on v_mfma_f32_32x32x16_bf16; weights are
// dequantised in registers from the staged codes by the gfx950 scaled
// converter (value * 2^(scale-127), exact in bf16), so a code byte crosses
// LDS once per wave instead of as two bf16 bytes per weight.
//
// MFMA K order: for step s (16 K) of a 128-K block, lane l (column n = l%32,
// half h = l/32) multiplies K = 64h + 32(s/4) + 8(s%4) + [0, 8).  For the
// weights these eight codes are dword s%4 of the repacked 16-byte chunk
// lane' = n%16 + 32h + 16(s/4) of row block n/16 (one ds_read_b128 serves
// four steps); the activation lane reads the same eight K values of its row.
// The row's sum over K is therefore taken in a fixed order independent of
// the tile shape and the batch.
//
// Work order: the flat list (tile, column slice) is cut into eight contiguous
// chunks, one per XCD (workgroups are dispatched round-robin over the XCDs),
// so the tiles of one expert run together on one XCD and share its L2.
#include "moe_internal.h"

namespace moe {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBN = 256;             // weight rows (output columns) per workgroup
constexpr int kBlocks = kBN / kTileN;  // 16 repacked row blocks
constexpr int kArow = 128 * 2 + 16;  // LDS bytes per staged activation row (padded against bank conflicts)

// Global loads of one 128-K column block into the staging registers.
template <int AI>
__device__ __forceinline__ void stage_load(u32x4_t (&ra)[AI], u32x4_t (&rb)[4], uint32_t (&rs)[4],
                                           const uint8_t* abase, const uint32_t (&aoff)[AI], const uint8_t* bptr,
                                           size_t bstride, const uint8_t* sptr, size_t sstride, int wave, int kb) {
#pragma unroll
  for (int i = 0; i < AI; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(abase + aoff[i] + (size_t)kb * 256);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rb[i] = *reinterpret_cast<const u32x4_t*>(bptr + (wave + 4 * i) * bstride + (size_t)kb * kTileBytes);
    rs[i] = *reinterpret_cast<const uint32_t*>(sptr + (wave + 4 * i) * sstride + (size_t)(kb >> 2) * kScaleGroupBytes);
  }
}

template <bool FC1, int WM>
__global__ __launch_bounds__(256) void fc_pre(FcArgs a, int slices) {
  constexpr int BM = 64 * WM;
  constexpr int WN = 4 / WM;                 // waves along N
  constexpr int NJ = kBN / WN / 32;          // 32-column MFMA blocks per wave (4 or 2)
  __shared__ __align__(16) uint8_t sA[BM * kArow];
  __shared__ __align__(16) uint8_t sB[kBlocks * kTileBytes];
  __shared__ __align__(16) uint32_t sS[kBlocks * kWave];

  const int ntiles = *a.tile_count;
  const int total = ntiles * slices;
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int chunk = (total + 7) >> 3;
  const int w = xcd * chunk + q;
  if (q >= chunk || w >= total) return;
  const int tile = w / slices, slice = w - tile * slices;
  const int2 td = a.tiles[tile];
  const int e = td.x, row0 = td.y;
  const int rows = min(BM, a.offsets[e + 1] - row0);
  const MatLayout M = a.mat;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int nb0 = slice * kBlocks;

  // ---- staging assignments
  // A: thread t copies 16-byte column c16 = t%16 of rows t/16 + 16i
  constexpr int AI = BM / 16;
  const int c16 = t & 15;
  const uint8_t* abase = static_cast<const uint8_t*>(a.a) + c16 * 16;
  uint32_t aoff[AI];   // byte offset of each staged row's 128-K block 0 (rows < 2^31 / lda bytes)
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int r = min((t >> 4) + 16 * i, rows - 1);
    const int ar = FC1 ? a.perm[row0 + r] / a.top_k : row0 + r;
    aoff[i] = (uint32_t)ar * (uint32_t)a.lda * 2u;
  }
  // B: thread t copies chunk lane' = t%64 of row blocks t/64 + 4i; scales likewise
  const uint8_t* bptr = a.codes + ((size_t)e * M.nb + nb0) * M.kb * kTileBytes + (size_t)lane * 16;
  const size_t bstride = (size_t)M.kb * kTileBytes;
  const uint8_t* sptr = a.scales + ((size_t)e * M.nb + nb0) * M.kb4 * kScaleGroupBytes + (size_t)lane * 4;
  const size_t sstride = (size_t)M.kb4 * kScaleGroupBytes;

  u32x4_t ra[AI], rb[4];
  uint32_t rs[4];
  f32x16_t acc[2][NJ];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mi][nj][i] = 0.f;

  const int n32 = lane & 31, h = lane >> 5;
  const int KB = M.kb;
  stage_load<AI>(ra, rb, rs, abase, aoff, bptr, bstride, sptr, sstride, wave, 0);
  for (int kb = 0; kb < KB; ++kb) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < AI; ++i) *reinterpret_cast<u32x4_t*>(sA + ((t >> 4) + 16 * i) * kArow + c16 * 16) = ra[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4_t*>(sB + (wave + 4 * i) * kTileBytes + lane * 16) = rb[i];
      sS[(wave + 4 * i) * kWave + lane] = rs[i];
    }
    __syncthreads();
    if (kb + 1 < KB) stage_load<AI>(ra, rb, rs, abase, aoff, bptr, bstride, sptr, sstride, wave, kb + 1);
    const int sh = (kb & 3) * 8;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4_t bc[NJ];
      float bs[NJ];
#pragma unroll
      for (int nj = 0; nj < NJ; ++nj) {
        const int blk = wn * (2 * NJ) + 2 * nj + (n32 >> 4);
        const int lp = (n32 & 15) + 32 * h + 16 * c;
        bc[nj] = *reinterpret_cast<const u32x4_t*>(sB + blk * kTileBytes + lp * 16);
        bs[nj] = e8m0_to_f32((sS[blk * kWave + lp] >> sh) & 0xFFu);
      }
      const uint8_t* ap = sA + (wm * 64 + n32) * kArow + (64 * h + 32 * c) * 2;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const bf16x8_t A0 = *reinterpret_cast<const bf16x8_t*>(ap + s4 * 16);
        const bf16x8_t A1 = *reinterpret_cast<const bf16x8_t*>(ap + 32 * kArow + s4 * 16);
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj) {
          const bf16x8_t B = dequant8(bc[nj][s4], bs[nj]);
          acc[0][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, B, acc[0][nj], 0, 0, 0);
          acc[1][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, B, acc[1][nj], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue.  32x32 D layout: lane holds column n32, rows 8(i/4) + 4h + (i%4).
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = wm * 64 + mi * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        const float v = acc[mi][nj][i];
        if constexpr (FC1) {
          // columns 0..15 of the block pair are gate j, 16..31 up j (interleaved row blocks)
          const float u = __shfl_xor(v, 16, kWave);
          if (n32 < 16 && r < rows) {
            const int j = (nb0 + wn * (2 * NJ) + 2 * nj) >> 1;
            static_cast<uint16_t*>(a.out)[(size_t)(row0 + r) * a.ldo + j * kTileN + n32] =
                f32_to_bf16_rne(silu_f32(v) * u);
          }
        } else {
          if (r < rows)
            static_cast<float*>(a.out)[(size_t)(row0 + r) * a.ldo + (size_t)(nb0 + wn * (2 * NJ) + 2 * nj) * kTileN +
                                       n32] = v;
        }
      }
    }
  }
}

template <bool FC1, int WM>
hipError_t launch_pre(const FcArgs& a, int tiles_max, hipStream_t stream) {
  const int slices = a.mat.nb / kBlocks;
  const long long items = (long long)tiles_max * slices;
  const long long grid = (items + 7) / 8 * 8;
  hipLaunchKernelGGL((fc_pre<FC1, WM>), dim3((unsigned)grid), dim3(256), 0, stream, a, slices);
  return hipGetLastError();
}

}  // namespace

int prefill_rows(int tokens, int top_k, int experts) {
  // rows per expert on average decide the tile height (results do not depend on it)
  return (long long)tokens * top_k >= 96LL * experts ? 128 : 64;
}

hipError_t launch_fc1_prefill(const FcArgs& a, int bm, int tiles_max, hipStream_t s) {
  return bm == 128 ? launch_pre<true, 2>(a, tiles_max, s) : launch_pre<true, 1>(a, tiles_max, s);
}
hipError_t launch_fc2_prefill(const FcArgs& a, int bm, int tiles_max, hipStream_t s) {
  return bm == 128 ? launch_pre<false, 2>(a, tiles_max, s) : launch_pre<false, 1>(a, tiles_max, s);
}

}  // namespace moe
