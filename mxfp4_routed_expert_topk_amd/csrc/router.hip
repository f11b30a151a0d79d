// Router top-k upstream of the layer: the topk_ids / topk_weights the forward
// consumes, from fp32 router logits [T, E].
//
// The pages fix the contract, not the scoring function: a batched router top-k
// over E in {224, 896} for batch buckets 1..128 (pegainfer PR #867, commit
// b49a9f04), with the top-16 selection kept in registers, a fixed tie order and
// a sequential fp32 normalisation of the route weights (b12x PR #339, the
// paired gather/router path).  Reading taken: ids are the k largest logits in
// descending order, equal logits rank the lower expert id first and NaN counts
// as -inf (ranked last, weight 0); weights are the max-subtracted softmax of
// the selected logits with the sum taken over slots in ascending order.
//
// One wave per token.  Lane l holds the logits of experts l, l+64, ... in
// registers (E <= 1024: at most 16 per lane).  Each of the k rounds takes the
// wave-wide best (largest value, then lowest id) of the entries not yet taken
// with a butterfly over (value, id) pairs -- a strict total order, so every
// lane ends on the same winner -- and the owning lane marks its entry taken.
// Lane s keeps round s's logit; its term exp(l_s - l_0) is computed in fp32,
// every lane adds the k terms in slot order, and lane s divides its own term.
#include <climits>
#include <cmath>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kPerLane = kRouterMaxExperts / kWave;
constexpr int kTokensPerBlock = 4;

__device__ __forceinline__ bool ranks_before(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__global__ __launch_bounds__(kTokensPerBlock* kWave) void router_topk_kernel(const float* logits, int T, int E,
                                                                            int k, int32_t* ids, float* weights) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kTokensPerBlock + (int)(threadIdx.x / kWave);
  if (t >= T) return;   // whole waves
  const float* row = logits + (size_t)t * E;
  float v[kPerLane];
  uint32_t taken = 0;   // bit j: entry lane + 64 j is selected or does not exist
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) {
    const int e = lane + kWave * j;
    const float x = e < E ? row[e] : -INFINITY;
    v[j] = x != x ? -INFINITY : x;
    if (e >= E) taken |= 1u << j;
  }
  float mine = 0.f;
  int my_id = 0;
  for (int s = 0; s < k; ++s) {
    float bv = -INFINITY;
    int bi = INT_MAX;   // "nothing yet": any real entry, -inf included, ranks before it
#pragma unroll
    for (int j = 0; j < kPerLane; ++j)
      if (!((taken >> j) & 1u) && ranks_before(v[j], lane + kWave * j, bv, bi)) {
        bv = v[j];
        bi = lane + kWave * j;
      }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, kWave);
      const int oi = __shfl_xor(bi, off, kWave);
      if (ranks_before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
    if (lane == s) {
      mine = bv;
      my_id = bi;
    }
  }
  const float top = __shfl(mine, 0, kWave);
  const float term = lane < k ? expf(mine - top) : 0.f;
  float total = 0.f;
  for (int s = 0; s < k; ++s) total += __shfl(term, s, kWave);   // slot order, the same sum on every lane
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    weights[(size_t)t * k + lane] = term / total;
  }
}

}  // namespace

hipError_t launch_router_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* ids, float* weights,
                              hipStream_t stream) {
  const unsigned blocks = (unsigned)((T + kTokensPerBlock - 1) / kTokensPerBlock);
  hipLaunchKernelGGL(router_topk_kernel, dim3(blocks), dim3(kTokensPerBlock * kWave), 0, stream, logits, T, E, k, ids,
                     weights);
  return hipGetLastError();
}

}  // namespace moe
