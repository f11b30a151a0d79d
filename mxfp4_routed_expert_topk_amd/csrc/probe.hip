// Peak micro-benchmarks of the device the layer runs on: the measured
// ceilings its kernels are compared with besides the published ones.
//
//  * memory: a grid-stride stream of 128-bit loads over a buffer (plain or
//    non-temporal), or a 128-bit copy -- the HBM ceiling of a weight-streaming
//    kernel;
//  * MFMA: back-to-back independent chains of v_mfma_f32_32x32x16_bf16 (the
//    bf16 prefill kernel's instruction) or v_mfma_scale_f32_16x16x128_f8f6f4
//    with E4M3 A and E2M1 B operands (the MXFP8 x MXFP4 kernel's instruction)
//    on every SIMD -- the matrix-core ceiling of each path.
// The pages time their kernels against the GPU's measured operating point
// (b12x PR #339: replay samples recorded with the GPU's operating state;
// clock policy changed the measured numbers), so the same box measures both.
// Every result feeds a per-workgroup sum into `sink` so nothing is dropped by
// the compiler; the values themselves mean nothing.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float wg_sum_to(float v, float* sink) {
  __shared__ float part[kThreads / kWave];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int w = 0; w < kThreads / kWave; ++w) s += part[w];
    sink[blockIdx.x] = s;
  }
  return v;
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void probe_read(const u32x4_t* __restrict__ src, size_t n, float* sink) {
  uint32_t x = 0;
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
    const u32x4_t v = NT ? __builtin_nontemporal_load(src + i) : src[i];
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  wg_sum_to((float)(x & 0xFFFF), sink);
}

__global__ __launch_bounds__(kThreads) void probe_copy(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                       size_t n) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

constexpr int kChains = 8;   // independent accumulators per wave

__global__ __launch_bounds__(kThreads) void probe_mfma_bf16(int iters, float* sink) {
  f32x16_t acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  bf16x8_t A, B;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    A[i] = (__bf16)(1e-3f * (float)(threadIdx.x + i));
    B[i] = (__bf16)(1e-3f * (float)(blockIdx.x % 7 + i));
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  wg_sum_to(s, sink);
}

__global__ __launch_bounds__(kThreads) void probe_mfma_f8f4(int iters, float* sink) {
  f32x4_t acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  i32x8_t A, B;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    A[i] = (int)(0x38383838u + ((threadIdx.x + i) & 15));    // E4M3 codes in [1, 3)
    B[i] = i < 4 ? (int)(0x22222222u + blockIdx.x % 5) : 0;    // E2M1 codes (16 bytes)
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc[c], 0, 4, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  wg_sum_to(s, sink);
}

// One scaled MFMA per problem on operands given in the instruction's lane
// order (one wave per problem): how the matrix core sums a 128-product block.
__global__ __launch_bounds__(kWave) void probe_mfma_f8f4_blocks(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b,
                                                               const uint8_t* __restrict__ sa,
                                                               const uint8_t* __restrict__ sb,
                                                               const float* __restrict__ c, float* __restrict__ d) {
  const size_t p = blockIdx.x;
  const int l = threadIdx.x;
  const uint32_t* ap = reinterpret_cast<const uint32_t*>(a + (p * kWave + l) * 32);
  const uint32_t* bp = reinterpret_cast<const uint32_t*>(b + (p * kWave + l) * 16);
  i32x8_t A, B;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    A[i] = (int)ap[i];
    B[i] = i < 4 ? (int)bp[i] : 0;
  }
  const float* cp = c + (p * kWave + l) * 4;
  f32x4_t acc = {cp[0], cp[1], cp[2], cp[3]};
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 0, 4, 0, (int)sa[p * kWave + l], 0,
                                                         (int)sb[p * kWave + l]);
  float* dp = d + (p * kWave + l) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) dp[i] = acc[i];
}

}  // namespace

hipError_t launch_probe_mfma_blocks(const uint8_t* a, const uint8_t* b, const uint8_t* sa, const uint8_t* sb,
                                    const float* c, float* d, int n, hipStream_t stream) {
  hipLaunchKernelGGL(probe_mfma_f8f4_blocks, dim3(n), dim3(kWave), 0, stream, a, b, sa, sb, c, d);
  return hipGetLastError();
}

hipError_t launch_probe_memory(int kind, const void* src, void* dst, size_t bytes, float* sink, int grid,
                               hipStream_t stream) {
  const size_t n = bytes / 16;
  const auto* s = static_cast<const u32x4_t*>(src);
  if (kind == 0) hipLaunchKernelGGL(probe_read<false>, dim3(grid), dim3(kThreads), 0, stream, s, n, sink);
  else if (kind == 1) hipLaunchKernelGGL(probe_read<true>, dim3(grid), dim3(kThreads), 0, stream, s, n, sink);
  else hipLaunchKernelGGL(probe_copy, dim3(grid), dim3(kThreads), 0, stream, s, static_cast<u32x4_t*>(dst), n);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(int kind, int iters, float* sink, int grid, double* flops, hipStream_t stream) {
  const double waves = (double)grid * (kThreads / kWave);
  if (kind == 0) {
    hipLaunchKernelGGL(probe_mfma_bf16, dim3(grid), dim3(kThreads), 0, stream, iters, sink);
    *flops = waves * iters * kChains * (2.0 * 32 * 32 * 16);
  } else {
    hipLaunchKernelGGL(probe_mfma_f8f4, dim3(grid), dim3(kThreads), 0, stream, iters, sink);
    *flops = waves * iters * kChains * (2.0 * 16 * 16 * 128);
  }
  return hipGetLastError();
}

}  // namespace moe
