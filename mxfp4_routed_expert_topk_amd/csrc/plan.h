// The plan object behind moe_mxfp4_plan_t and the host-side pieces the C-ABI
// sources share (error reporting, the forward's launch sequence).
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/moe_mxfp4.h"
#include "moe_internal.h"

struct moe_mxfp4_plan_s {
  moe_mxfp4_config cfg;
  moe::Layout L;          // buffer layout for cfg.max_tokens
  const uint8_t* repacked;
  hipEvent_t events[5];
  int n_events;
  uint32_t fused_gen;     // generation of this plan's last fused forward (0: none)
};

namespace moe {

// Set the calling thread's error text (printf format) and return s.
moe_status fail(moe_status s, const char* fmt, ...);
moe_status ok();
moe_status hip_fail(hipError_t e, const char* what);

// Enqueue the forward for T tokens over workspace `ws` laid out by L (checked
// arguments; L may be sized for fewer tokens than the plan's capacity).
moe_status forward_with_layout(moe_mxfp4_plan_s* p, const Layout& L, const uint16_t* hidden, const int32_t* topk_ids,
                               const float* topk_weights, int32_t T, float* acc_fp32, uint16_t* out_bf16,
                               uint8_t* ws, hipStream_t stream);

// The argument checks of every forward entry point except the workspace.
moe_status check_forward_io(const moe_mxfp4_plan_s* p, const uint16_t* hidden, const int32_t* topk_ids,
                            const float* topk_weights, int32_t T, const float* acc_fp32, const uint16_t* out_bf16);

}  // namespace moe
