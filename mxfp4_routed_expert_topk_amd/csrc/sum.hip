// FC2 with the gather-weight-reduce epilogue, for the smallest bf16 batches
// (at most kPerRouteMaxRoutes routes): every token's routes are summed into
// the fp32 token accumulator inside the FC2 launch, with no per-route output
// in memory and no combine launch (b12x PR #339, commit "large-token FC2
// fused-sum epilogue": the routed outputs reduce straight into the caller's
// fp32 token accumulator; pegainfer PR #867, commit 53edfa98: topk-slot-order
// f32 accumulation, no atomics, one bf16 rounding).
//
// A workgroup owns one token and a block of 16 output columns, so the token's
// slot-order sum needs nothing from another workgroup (on MI355X the L2s of
// the eight XCDs are not coherent inside a kernel: a hand-off between
// workgroups would cost an L2 writeback).  Its waves take the (route, K range)
// units of the token's valid routes -- route f = t*k + s multiplies h row f
// (FC1's per-route output) by expert ids[f]'s W2 rows of the block over the
// same K ranges as the 16-row FC2 kernel (dec_core.h), one unit per wave at
// top-8 -- and park the partial sums in LDS.  Then each of 16 threads adds the
// K ranges of a route in range order and the routes of its column in slot
// order with one fused multiply-add per route, exactly as the 16-row FC2
// kernel and the combine kernel would: the bits are theirs.
#include "dec_core.h"

namespace moe {
namespace {

// Eight waves per workgroup, two column blocks loaded ahead; the widest of
// 64, 32 or 16 output columns per workgroup that still gives at least
// kSumMinGroups workgroups (about two per CU): at hidden 7168 that is 16
// columns at one token, 32 at two and three, 64 from four.  Measured at
// hidden 7168, intermediate 2048, top-8: 30.2 / 90.8 us per layer at 1 / 4
// tokens, against 34.9 / 99.7 us for the route + FC1 + FC2 + combine chain;
// wider workgroups lost at one token, narrower ones at four, sixteen waves
// and deeper loads lost everywhere; by this rule, against 64 columns from two
// tokens and 32 at one: 42.0 -> 40.5 us at two tokens, 61.3 -> 59.1 us at
// three, 25.8 -> 25.7 us at one, and 20.9 -> 19.3 us at one token of the
// K3 shapes (hidden 3584: 16 columns, 224 workgroups).
constexpr int kSumMinGroups = 448;
constexpr int kSumWaves = 8;
constexpr int kSumP = 2;

template <int KS, int NBW, bool GRP>
__global__ __launch_bounds__(kWave * kSumWaves) void fc2_sum(FcArgs a, const float* __restrict__ w, int H,
                                                            float* __restrict__ acc_out, uint16_t* __restrict__ out) {
  __shared__ float red[KS][kMaxTopK][NBW * kTileN];  // k <= kMaxTopK
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int k = a.top_k;
  const int nb0 = blockIdx.x * NBW;             // the workgroup's 16-row blocks of W2 = output columns
  const int t = blockIdx.y;                     // the workgroup's token
  const int f0 = t * k;
  const int my_id = lane < k ? a.route_ids[f0 + lane] : -1;
  const uint64_t valid = __ballot(lane < k && my_id >= 0 && my_id < a.num_experts);   // slots with a route
  const int units = __popcll(valid) * KS;
  // a unit's h row segment, staged by its wave (launch_sum sizes this: one K
  // range per wave)
  extern __shared__ __align__(16) uint8_t row_lds[];
  const int per = dec_krange_max(a.mat.kb, KS);
  for (int u = wave; u < units; u += kSumWaves) {
    const int vi = u / KS, p = u - vi * KS;
    uint64_t rest = valid;
    for (int i = 0; i < vi; ++i) rest &= rest - 1;
    const int s = __ffsll((unsigned long long)rest) - 1;   // the vi-th valid slot
    const int e = a.route_ids[f0 + s];
    int lo, hi;
    dec_krange<KS>(a.mat.kb, p, &lo, &hi);
    f32x4_t acc[NBW];
    // one token: the unit's h row segment staged in LDS (1-token layer 13.6 ->
    // 13.2 us in this kernel); at four tokens the per-lane loads measured
    // 0.7 us faster
    dec_kloop<false, false, NBW, kSumP, (NBW > 2), (NBW <= 2), GRP>(a, e, nb0, (long long)(f0 + s), lo, hi, acc,
                                                                    row_lds + wave * per * (kTileK * 2));
    if (lane < kTileN)                                  // D row 0: lanes 0..15 hold a block's 16 columns
#pragma unroll
      for (int j = 0; j < NBW; ++j) red[p][s][j * kTileN + lane] = acc[j][0];
  }
  __syncthreads();
  if (threadIdx.x < NBW * kTileN) {
    const int c = threadIdx.x;
    float sum = 0.f;
    for (int s = 0; s < k; ++s) {
      if (!((valid >> s) & 1ull)) continue;   // invalid route: its weight is never read
      float y = red[0][s][c];
#pragma unroll
      for (int q = 1; q < KS; ++q) y += red[q][s][c];
      sum = fmaf(w[f0 + s], y, sum);
    }
    const size_t o = (size_t)t * H + (size_t)nb0 * kTileN + c;
    if (acc_out) acc_out[o] = sum;
    out[o] = f32_to_bf16_rne(sum);
  }
}

template <int NBW>
hipError_t launch_sum(const FcArgs& a, const float* weights, int32_t T, int32_t H, float* acc, uint16_t* out,
                      hipStream_t stream) {
  const dim3 grid(a.mat.nb / NBW, T), block(kWave * kSumWaves);
  const int ks = dec_ksplit(a.mat.kb);
  const size_t lds = NBW <= 2 ? (size_t)kSumWaves * dec_krange_max(a.mat.kb, ks) * kTileK * 2 : 0;
  const bool grp = a.mat.kb % 4 == 0;   // whole scale groups per K range
  if (ks == 4) {
    if (grp) hipLaunchKernelGGL((fc2_sum<4, NBW, true>), grid, block, lds, stream, a, weights, H, acc, out);
    else hipLaunchKernelGGL((fc2_sum<4, NBW, false>), grid, block, lds, stream, a, weights, H, acc, out);
  } else {
    if (grp) hipLaunchKernelGGL((fc2_sum<2, NBW, true>), grid, block, lds, stream, a, weights, H, acc, out);
    else hipLaunchKernelGGL((fc2_sum<2, NBW, false>), grid, block, lds, stream, a, weights, H, acc, out);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fc2_sum_per_route(const FcArgs& a, const float* weights, int32_t T, int32_t H, float* acc,
                                    uint16_t* out, hipStream_t stream) {
  // every row-block count is a multiple of 8 (H a multiple of 128)
  if (a.mat.nb / 4 * T >= kSumMinGroups) return launch_sum<4>(a, weights, T, H, acc, out, stream);
  if (a.mat.nb / 2 * T >= kSumMinGroups) return launch_sum<2>(a, weights, T, H, acc, out, stream);
  return launch_sum<1>(a, weights, T, H, acc, out, stream);
}

}  // namespace moe
