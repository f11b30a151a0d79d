// Gather-weight-reduce epilogue: for every token t,
//   acc_t = sum over slots s = 0..k-1 (ascending) with a valid route of
//           w[t,s] * y[row(t,s)]      (fp32, fused multiply-add per term)
//   out_t = RNE_bf16(acc_t)
// Each output element is owned by one thread, so there are no atomics and the
// order is fixed (pegainfer PR #867, commit 53edfa98: "topk-slot-order f32
// accumulation, no atomics, single bf16 round").  The fp32 accumulator, when
// the caller passes one, is overwritten in full and rounded once (b12x PR
// #339: caller-owned fp32 token accumulator cast once; commit "top-k sum
// output store element": the bf16 store rounds the same fp32 value once, to
// nearest even).  Invalid routes are skipped, their weights never read.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kSlotsAhead = 8;   // slots whose y loads are in flight together

// y: fp32 rows (the decode kernels) or bf16 rows (the prefill kernels, which
// land y in bf16 as the pages' fused-sum epilogue reduces bf16 routed outputs:
// half the bytes of the largest intermediate).  A thread owns 4 columns
// (fp32 y) or 8 (bf16 y): one 16-byte load per slot.  The slots are taken
// eight at a time, their loads issued before the first multiply-add, which
// still runs in slot order (an invalid slot loads row 0 and leaves it
// unused).  Measured against one 8-byte load per slot and a wait per slot:
// 121 -> 103 us on the 4096-token Zipf batch, 109 -> 86 us on the 4096-token
// MXFP8 one, 41 -> 34 us at 1536 tokens.
template <bool BF16Y>
__global__ __launch_bounds__(kThreads) void combine(const void* __restrict__ y, const int32_t* __restrict__ rowpos,
                                                    const float* __restrict__ w, int k, int H,
                                                    float* __restrict__ acc_out, uint16_t* __restrict__ out) {
  constexpr int NC = BF16Y ? 8 : 4;   // columns per thread
  const int t = blockIdx.x;
  const int c = (blockIdx.y * kThreads + threadIdx.x) * NC;
  if (c >= H) return;
  float acc[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) acc[i] = 0.f;
  for (int s0 = 0; s0 < k; s0 += kSlotsAhead) {
    int r[kSlotsAhead];
    f32x4_t v[kSlotsAhead];
#pragma unroll
    for (int j = 0; j < kSlotsAhead; ++j) {
      r[j] = s0 + j < k ? rowpos[(size_t)t * k + s0 + j] : -1;
      // every y element is read exactly once: a non-temporal load streams it
      // past the caches (measured 15% faster on 4096-token batches)
      const int rr = r[j] < 0 ? 0 : r[j];
      if (BF16Y)
        v[j] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4_t*>(static_cast<const uint16_t*>(y) + (size_t)rr * H + c));
      else
        v[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(static_cast<const float*>(y) + (size_t)rr * H + c));
    }
#pragma unroll
    for (int j = 0; j < kSlotsAhead; ++j) {
      if (r[j] < 0) continue;
      const float ws = w[(size_t)t * k + s0 + j];
      if constexpr (BF16Y) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t b = __float_as_uint(v[j][q]);
          acc[2 * q] = fmaf(ws, __uint_as_float(b << 16), acc[2 * q]);
          acc[2 * q + 1] = fmaf(ws, __uint_as_float(b & 0xFFFF0000u), acc[2 * q + 1]);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = fmaf(ws, v[j][q], acc[q]);
      }
    }
  }
  if (acc_out) {
#pragma unroll
    for (int i = 0; i < NC; i += 4)
      *reinterpret_cast<float4*>(acc_out + (size_t)t * H + c + i) = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
  }
  uint32_t o[NC / 2];
#pragma unroll
  for (int i = 0; i < NC / 2; ++i) o[i] = f32_to_bf16_rne(acc[2 * i]) | ((uint32_t)f32_to_bf16_rne(acc[2 * i + 1]) << 16);
  if constexpr (BF16Y) *reinterpret_cast<uint4*>(out + (size_t)t * H + c) = make_uint4(o[0], o[1], o[2], o[3]);
  else *reinterpret_cast<uint2*>(out + (size_t)t * H + c) = make_uint2(o[0], o[1]);
}

}  // namespace

hipError_t launch_combine(const void* y, bool y_bf16, const int32_t* rowpos, const float* w, int32_t T, int32_t k,
                          int32_t H, float* acc, uint16_t* out, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int nc = y_bf16 ? 8 : 4;
  const dim3 grid(T, (H / nc + kThreads - 1) / kThreads);
  if (y_bf16) hipLaunchKernelGGL(combine<true>, grid, dim3(kThreads), 0, stream, y, rowpos, w, k, H, acc, out);
  else hipLaunchKernelGGL(combine<false>, grid, dim3(kThreads), 0, stream, y, rowpos, w, k, H, acc, out);
  return hipGetLastError();
}

}  // namespace moe
