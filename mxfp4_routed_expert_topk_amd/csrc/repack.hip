// Plan-time repack of checkpoint-layout MXFP4 weights into the tile order of
// moe_internal.h, with validation of every E8M0 scale byte.
//
// The repack is a pure rearrangement of 16-byte runs of codes (nibble order
// inside a byte unchanged) and of scale bytes (batchgen PR #307, repack
// commit: "pure nibble rearrangement carrying E8M0 uint8 scales through",
// w1||w3 repacked together).  Scale bytes 0x00 and 0xFF raise (same commit:
// "edge bytes 0x00/0xFF raise"); the bf16 path also refuses 0x01, 0xFD and
// 0xFE, whose dequantised bf16 weights would be subnormal or overflow.
// The first offending byte is reported through a 64-bit word in the repacked
// buffer: (matrix << 56) | flat scale index, minimised with atomicMin.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ bool bad_scale(uint32_t b, bool bf16_path) {
  if (b == 0x00u || b == 0xFFu) return true;
  return bf16_path && (b == 0x01u || b >= 0xFDu);
}

// codes: one thread per 16-byte run of the destination.
__global__ __launch_bounds__(kThreads) void repack_codes(const uint8_t* __restrict__ src,
                                                         uint8_t* __restrict__ dst, int E, MatLayout m,
                                                         int interleave_half) {
  const size_t runs_per_expert = (size_t)m.nb * m.kb * kWave;
  const size_t total = runs_per_expert * (size_t)E;
  const size_t row_bytes = (size_t)m.k / 2;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (size_t)gridDim.x * kThreads) {
    const int lane = (int)(i % kWave);
    const size_t t = i / kWave;
    const int kb = (int)(t % m.kb);
    const size_t t2 = t / m.kb;
    const int nb = (int)(t2 % m.nb);
    const int e = (int)(t2 / m.nb);
    int row;
    if (interleave_half > 0) {
      const int j = nb >> 1;
      row = (nb & 1 ? interleave_half : 0) + j * kTileN + (lane & 15);
    } else {
      row = nb * kTileN + (lane & 15);
    }
    const uint4* s = reinterpret_cast<const uint4*>(src + ((size_t)e * m.n + row) * row_bytes +
                                                    (size_t)kb * 64 + (lane >> 4) * 16);
    reinterpret_cast<uint4*>(dst)[i] = *s;
  }
}

// scales: one thread per destination dword (4 column blocks of one lane).
__global__ __launch_bounds__(kThreads) void repack_scales(const uint8_t* __restrict__ src,
                                                          uint8_t* __restrict__ dst, int E, MatLayout m,
                                                          int interleave_half, int bf16_path,
                                                          unsigned long long matrix_tag,
                                                          unsigned long long* status) {
  const size_t words_per_expert = (size_t)m.nb * m.kb4 * kWave;
  const size_t total = words_per_expert * (size_t)E;
  const int groups = m.k / 32;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (size_t)gridDim.x * kThreads) {
    const int lane = (int)(i % kWave);
    const size_t t = i / kWave;
    const int c = (int)(t % m.kb4);
    const size_t t2 = t / m.kb4;
    const int nb = (int)(t2 % m.nb);
    const int e = (int)(t2 / m.nb);
    int row;
    if (interleave_half > 0) {
      const int j = nb >> 1;
      row = (nb & 1 ? interleave_half : 0) + j * kTileN + (lane & 15);
    } else {
      row = nb * kTileN + (lane & 15);
    }
    uint32_t word = 0;
    unsigned long long first_bad = ~0ull;
    for (int j = 0; j < 4; ++j) {
      const int kb = 4 * c + j;
      uint32_t b = 127u;
      if (kb < m.kb) {
        const int g = 4 * kb + (lane >> 4);
        const size_t flat = ((size_t)e * m.n + row) * groups + g;
        b = src[flat];
        if (bad_scale(b, bf16_path != 0) && flat < first_bad) first_bad = flat;
      }
      word |= b << (8 * j);
    }
    reinterpret_cast<uint32_t*>(dst)[i] = word;
    if (first_bad != ~0ull) atomicMin(status, (matrix_tag << 56) | first_bad);
  }
}

__global__ void init_status(unsigned long long* status) { *status = ~0ull; }

int grid_for(size_t n) {
  const size_t blocks = (n + kThreads - 1) / kThreads;
  return (int)(blocks < 65536 ? (blocks ? blocks : 1) : 65536);
}

}  // namespace

hipError_t launch_repack(const Layout& L, const uint8_t* w13c, const uint8_t* w13s,
                         const uint8_t* w2c, const uint8_t* w2s, uint8_t* rp, hipStream_t stream) {
  unsigned long long* status = reinterpret_cast<unsigned long long*>(rp + L.rp_status);
  const int bf16_path = L.act == 0;
  hipLaunchKernelGGL(init_status, dim3(1), dim3(1), 0, stream, status);
  const size_t r13 = (size_t)L.E * L.w13.nb * L.w13.kb * kWave;
  const size_t r2 = (size_t)L.E * L.w2.nb * L.w2.kb * kWave;
  hipLaunchKernelGGL(repack_codes, dim3(grid_for(r13)), dim3(kThreads), 0, stream, w13c,
                     rp + L.rp_w13_codes, L.E, L.w13, L.I);
  hipLaunchKernelGGL(repack_codes, dim3(grid_for(r2)), dim3(kThreads), 0, stream, w2c,
                     rp + L.rp_w2_codes, L.E, L.w2, 0);
  const size_t s13 = (size_t)L.E * L.w13.nb * L.w13.kb4 * kWave;
  const size_t s2 = (size_t)L.E * L.w2.nb * L.w2.kb4 * kWave;
  hipLaunchKernelGGL(repack_scales, dim3(grid_for(s13)), dim3(kThreads), 0, stream, w13s,
                     rp + L.rp_w13_scales, L.E, L.w13, L.I, bf16_path, 0ull, status);
  hipLaunchKernelGGL(repack_scales, dim3(grid_for(s2)), dim3(kThreads), 0, stream, w2s,
                     rp + L.rp_w2_scales, L.E, L.w2, 0, bf16_path, 1ull, status);
  return hipGetLastError();
}

}  // namespace moe
