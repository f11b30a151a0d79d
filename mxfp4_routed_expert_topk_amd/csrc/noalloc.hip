// moe_mxfp4_forward_noalloc: the forward with its scratch in a fixed device
// array of this library instead of a caller workspace, for callers that
// cannot allocate (code under graph capture, tight serving loops).
//
// The array is a file-scope device variable: every GPU the library runs on
// holds its own copy (kNoallocScratchBytes) until the process ends.  Host code
// never passes the variable's name to a kernel (on the host it only stands in
// for the symbol): the first call on a device asks HIP for the device address
// of that device's copy (hipGetSymbolAddress, with the device current) and
// keeps it per device; every launch takes that address.
//
// The forward sets every scratch word it reads before reading it (its first
// kernel zeroes the prefill kernels' work counters), so the last call's
// contents never matter; calls that overlap on one GPU share the array and
// race.
#include <mutex>

#include "plan.h"

namespace moe {
namespace {

constexpr size_t kNoallocScratchBytes = 48ull << 20;
constexpr int kMaxDevices = 64;

}  // namespace
}  // namespace moe

static __device__ __align__(256) uint8_t scratch[moe::kNoallocScratchBytes];

namespace moe {
namespace {

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device (null: not asked yet)

// The current device's copy of the scratch array.
moe_status scratch_address(uint8_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
    g_scratch[dev] = ptr;
  }
  *out = static_cast<uint8_t*>(g_scratch[dev]);
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_mxfp4_forward_noalloc(moe_mxfp4_plan_t p, const uint16_t* hidden, const int32_t* topk_ids,
                                                const float* topk_weights, int32_t num_tokens, float* acc_fp32,
                                                uint16_t* out_bf16, hipStream_t stream) {
  if (moe_status s = moe::check_forward_io(p, hidden, topk_ids, topk_weights, num_tokens, acc_fp32, out_bf16))
    return s;
  // the workspace layout of this batch alone, which must fit the array
  const moe::Layout L = moe::make_layout(p->cfg.hidden, p->cfg.intermediate, p->cfg.num_experts, p->cfg.top_k,
                                         num_tokens > 0 ? num_tokens : 1, p->cfg.act);
  if (L.ws_bytes > moe::kNoallocScratchBytes)
    return moe::fail(MOE_ERR_CAPACITY,
                     "num_tokens %d needs %zu bytes of scratch; the fixed scratch of the allocation-free forward "
                     "holds %zu (use moe_mxfp4_forward with a workspace)",
                     num_tokens, L.ws_bytes, moe::kNoallocScratchBytes);
  if (num_tokens == 0) return moe::ok();
  uint8_t* ws = nullptr;
  if (moe_status s = moe::scratch_address(&ws)) return s;
  return moe::forward_with_layout(p, L, hidden, topk_ids, topk_weights, num_tokens, acc_fp32, out_bf16, ws, stream);
}
