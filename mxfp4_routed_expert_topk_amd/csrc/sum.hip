// FC2 with the gather-weight-reduce epilogue, for the smallest bf16 batches
// (at most kPerRouteMaxRoutes routes): every token's routes are summed into
// the fp32 token accumulator inside the FC2 launch, with no per-route output
// in memory and no combine launch (b12x PR #339, commit "large-token FC2
// fused-sum epilogue": the routed outputs reduce straight into the caller's
// fp32 token accumulator; pegainfer PR #867, commit 53edfa98: topk-slot-order
// f32 accumulation, no atomics, one bf16 rounding).
//
// A workgroup owns a block of 16 output columns of every token, so a token's
// slot-order sum needs nothing from another workgroup (on MI355X the L2s of
// the eight XCDs are not coherent inside a kernel: a hand-off between
// workgroups would cost an L2 writeback).  Its waves take the (route, K range)
// units of the batch's valid routes -- route f = t*k + s multiplies h row f
// (FC1's per-route output) by expert ids[f]'s W2 rows of the block over the
// same K ranges as the 16-row FC2 kernel (dec_core.h) -- and park the partial
// sums in LDS.  Then each thread adds the K ranges of a route in range order
// and the routes of its (token, column) in slot order with one fused
// multiply-add per route, exactly as the 16-row FC2 kernel and the combine
// kernel would: the bits are theirs.
#include "dec_core.h"

namespace moe {
namespace {

constexpr int kSumWaves = 16;

template <int KS, int P>
__global__ __launch_bounds__(kWave * kSumWaves) void fc2_sum(FcArgs a, const float* __restrict__ w, int T, int H,
                                                            float* __restrict__ acc_out, uint16_t* __restrict__ out) {
  __shared__ float red[KS][kPerRouteMaxRoutes][kTileN];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int k = a.top_k, R = T * k;             // R <= kPerRouteMaxRoutes = one wave's lanes
  const int nb0 = blockIdx.x;                   // the workgroup's 16-row block of W2 = output columns
  const int my_id = lane < R ? a.route_ids[lane] : -1;
  const uint64_t valid = __ballot(lane < R && my_id >= 0 && my_id < a.num_experts);
  const int units = __popcll(valid) * KS;
  for (int u = wave; u < units; u += kSumWaves) {
    const int vi = u / KS, p = u - vi * KS;
    uint64_t rest = valid;
    for (int i = 0; i < vi; ++i) rest &= rest - 1;
    const int f = __ffsll((unsigned long long)rest) - 1;   // the vi-th valid route
    const int e = a.route_ids[f];
    int lo, hi;
    dec_krange<KS>(a.mat.kb, p, &lo, &hi);
    f32x4_t acc[1];
    dec_kloop<false, false, 1, P>(a, e, nb0, (long long)f, lo, hi, acc);
    if (lane < kTileN) red[p][f][lane] = acc[0][0];    // D row 0 (lanes 0..15 hold its 16 columns)
  }
  __syncthreads();
  for (int i = threadIdx.x; i < T * kTileN; i += kWave * kSumWaves) {
    const int t = i / kTileN, c = i - t * kTileN;
    float s = 0.f;
    for (int sl = 0; sl < k; ++sl) {
      const int f = t * k + sl;
      if (!((valid >> f) & 1ull)) continue;   // invalid route: its weight is never read
      float y = red[0][f][c];
#pragma unroll
      for (int q = 1; q < KS; ++q) y += red[q][f][c];
      s = fmaf(w[f], y, s);
    }
    const size_t o = (size_t)t * H + (size_t)nb0 * kTileN + c;
    if (acc_out) acc_out[o] = s;
    out[o] = f32_to_bf16_rne(s);
  }
}

}  // namespace

hipError_t launch_fc2_sum_per_route(const FcArgs& a, const float* weights, int32_t T, int32_t H, float* acc,
                                    uint16_t* out, hipStream_t stream) {
  const dim3 grid(a.mat.nb), block(kWave * kSumWaves);
  if (dec_ksplit(a.mat.kb) == 4)
    hipLaunchKernelGGL((fc2_sum<4, 2>), grid, block, 0, stream, a, weights, T, H, acc, out);
  else
    hipLaunchKernelGGL((fc2_sum<2, 2>), grid, block, 0, stream, a, weights, T, H, acc, out);
  return hipGetLastError();
}

}  // namespace moe
