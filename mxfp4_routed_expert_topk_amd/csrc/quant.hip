// MXFP8 activation quantisation: E4M3FN codes with one E8M0 scale per 32
// consecutive elements of a row (pegainfer PR #867, commit 33d22f80: "gran-32
// e4m3 activation quant"; commit 53edfa98: per-token-group FP8 quant of the
// gathered rows and requant of h before W2, with UE8M0 scales).
//
// Scale rule: mx_scale_exp / e4m3_quad (moe_internal.h).  With it the block
// maximum lands in [448, 896) and saturates.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// One thread per 32-element block.
__global__ __launch_bounds__(kThreads) void quant_bf16(const uint16_t* __restrict__ x, int rows, int cols,
                                                       uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int gpr = cols / 32;
  const long long b = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (b >= (long long)rows * gpr) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + b * 32);
  uint4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = src[i];
  const uint32_t* w = reinterpret_cast<const uint32_t*>(v);
  float f[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    f[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
    f[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    amax = fmaxf(amax, fmaxf(fabsf(f[2 * i]), fabsf(f[2 * i + 1])));
  }
  const int e = mx_scale_exp(amax);
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);   // 2^-e, e in [-127, 126]
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    out[i] = e4m3_quad(f[4 * i] * inv, f[4 * i + 1] * inv, f[4 * i + 2] * inv, f[4 * i + 3] * inv);
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + b * 32);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  scales[b] = (uint8_t)(e + 127);
}

// fp32 rows; the live row count is read on the device (rows_dev).
__global__ __launch_bounds__(kThreads) void quant_f32(const float* __restrict__ x, const int32_t* rows_dev,
                                                      int cols, uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales) {
  const int gpr = cols / 32;
  const long long b = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (b >= (long long)(*rows_dev) * gpr) return;
  const float4* src = reinterpret_cast<const float4*>(x + b * 32);
  float f[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 q = src[i];
    f[4 * i] = q.x; f[4 * i + 1] = q.y; f[4 * i + 2] = q.z; f[4 * i + 3] = q.w;
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(q.x), fabsf(q.y)), fmaxf(fabsf(q.z), fabsf(q.w))));
  }
  const int e = mx_scale_exp(amax);
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    out[i] = e4m3_quad(f[4 * i] * inv, f[4 * i + 1] * inv, f[4 * i + 2] * inv, f[4 * i + 3] * inv);
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + b * 32);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  scales[b] = (uint8_t)(e + 127);
}

}  // namespace

hipError_t launch_quant_bf16(const uint16_t* x, int32_t rows, int32_t cols, uint8_t* codes,
                             uint8_t* scales, hipStream_t stream) {
  const long long blocks = ((long long)rows * (cols / 32) + kThreads - 1) / kThreads;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_bf16, dim3((unsigned)blocks), dim3(kThreads), 0, stream, x, rows, cols, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_f32(const float* x, const int32_t* rows_dev, int32_t rows_max, int32_t cols,
                            uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const long long blocks = ((long long)rows_max * (cols / 32) + kThreads - 1) / kThreads;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_f32, dim3((unsigned)blocks), dim3(kThreads), 0, stream, x, rows_dev, cols, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
