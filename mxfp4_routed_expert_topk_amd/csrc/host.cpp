// C ABI of the MXFP4 routed-expert MoE library: argument validation, buffer
// layout, plan (repack + scale validation) and the forward launch sequence.
//
// Contract conventions follow the pages' hard-fail seams: every violation
// returns an error that names what was expected and what was passed, with no
// fallback path (batchgen PR #307: "every contract violation raises";
// "error names the extension file actually loaded"); forward allocates
// nothing and never writes its inputs (b12x PR #339, commit "FC2-only route
// validation": no caller-tensor mutation, no allocation during graph replay).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <string>

#include "../../include/moe_mxfp4.h"
#include "moe_internal.h"
#include "plan.h"

namespace {

thread_local std::string g_err;

}  // namespace

namespace moe {

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

moe_status ok() {
  g_err.clear();
  return MOE_OK;
}

moe_status hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s failed: %s", what, hipGetErrorString(e));
}

}  // namespace moe

namespace {

using moe::fail;
using moe::hip_fail;
using moe::ok;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

constexpr int32_t kMaxDim = moe::kMaxDimension;
constexpr int32_t kMaxExperts = 1024;
constexpr int32_t kMaxTopK = moe::kMaxTopK;
constexpr int64_t kMaxRoutes = 262144;

moe_status check_config(const moe_mxfp4_config* c) {
  if (!c) return fail(MOE_ERR_ARG, "config pointer is null");
  if (c->hidden < 128 || c->hidden > kMaxDim || c->hidden % 128)
    return fail(MOE_ERR_SHAPE, "hidden must be a multiple of 128 in [128, %d], got %d", kMaxDim, c->hidden);
  if (c->intermediate < 128 || c->intermediate > kMaxDim || c->intermediate % 128)
    return fail(MOE_ERR_SHAPE, "intermediate must be a multiple of 128 in [128, %d], got %d", kMaxDim,
                c->intermediate);
  if (c->num_experts < 1 || c->num_experts > kMaxExperts)
    return fail(MOE_ERR_SHAPE, "num_experts must be in [1, %d], got %d", kMaxExperts, c->num_experts);
  if (c->top_k < 1 || c->top_k > kMaxTopK)
    return fail(MOE_ERR_SHAPE, "top_k must be in [1, %d], got %d", kMaxTopK, c->top_k);
  if (c->max_tokens < 1 || (int64_t)c->max_tokens * c->top_k > kMaxRoutes)
    return fail(MOE_ERR_SHAPE, "max_tokens must be >= 1 with max_tokens*top_k <= %lld, got max_tokens=%d top_k=%d",
                (long long)kMaxRoutes, c->max_tokens, c->top_k);
  if (c->act != MOE_ACT_BF16 && c->act != MOE_ACT_MXFP8)
    return fail(MOE_ERR_ARG, "act must be MOE_ACT_BF16 (0) or MOE_ACT_MXFP8 (1), got %d", c->act);
  return MOE_OK;
}

}  // namespace

namespace moe {

Layout make_layout(int H, int I, int E, int k, int Tmax, int act) {
  Layout L{};
  L.H = H; L.I = I; L.E = E; L.k = k; L.Tmax = Tmax; L.act = act;
  L.Rmax = Tmax * k;
  L.tiles_max = L.Rmax / kBM + (E < L.Rmax ? E : L.Rmax);
  L.route_blocks = (L.Rmax + kRouteChunk - 1) / kRouteChunk;
  L.w13 = make_mat_layout(2 * I, H);
  L.w2 = make_mat_layout(H, I);
  constexpr size_t A = 256;
  size_t o = 0;
  L.rp_w13_codes = o;  o = align_up(o + L.w13.codes_per_expert * E, A);
  L.rp_w13_scales = o; o = align_up(o + L.w13.scales_per_expert * E, A);
  L.rp_w2_codes = o;   o = align_up(o + L.w2.codes_per_expert * E, A);
  L.rp_w2_scales = o;  o = align_up(o + L.w2.scales_per_expert * E, A);
  L.rp_status = o;     o = align_up(o + 8, A);
  L.rp_bytes = o;
  const size_t R = (size_t)L.Rmax;
  o = 0;
  L.ws_counts = o;      o = align_up(o + 4 * (size_t)E, A);
  L.ws_offsets = o;     o = align_up(o + 4 * (size_t)(E + 1), A);
  L.ws_perm = o;        o = align_up(o + 4 * R, A);
  L.ws_rowpos = o;      o = align_up(o + 4 * R, A);
  L.ws_tiles = o;       o = align_up(o + 8 * (size_t)L.tiles_max, A);
  L.ws_tile_count = o;  o = align_up(o + 4, A);
  L.ws_blockcounts = o; o = align_up(o + 4 * (size_t)L.route_blocks * E, A);
  if (act == MOE_ACT_MXFP8) {
    L.ws_xq = o; o = align_up(o + (size_t)Tmax * H, A);
    L.ws_xs = o; o = align_up(o + (size_t)Tmax * (H / 32), A);
    L.ws_h = o;  o = align_up(o + 4 * R * I, A);
    L.ws_hq = o; o = align_up(o + R * I, A);
    L.ws_hs = o; o = align_up(o + R * (I / 32), A);
  } else {
    L.ws_xq = L.ws_xs = L.ws_hq = L.ws_hs = 0;
    L.ws_h = o; o = align_up(o + 2 * R * I, A);
  }
  L.ws_y = o; o = align_up(o + 4 * R * H, A);
  L.ws_sync = o; o = align_up(o + kFusedSyncBytes, A);
  L.ws_sched = o; o = align_up(o + 4 * (size_t)kSchedCounters, A);
  L.ws_bytes = o;
  return L;
}

}  // namespace moe


namespace {

moe::RouteOut route_out(const moe::Layout& L, uint8_t* ws) {
  moe::RouteOut o;
  o.counts = reinterpret_cast<int32_t*>(ws + L.ws_counts);
  o.offsets = reinterpret_cast<int32_t*>(ws + L.ws_offsets);
  o.perm = reinterpret_cast<int32_t*>(ws + L.ws_perm);
  o.rowpos = reinterpret_cast<int32_t*>(ws + L.ws_rowpos);
  o.tiles = reinterpret_cast<int2*>(ws + L.ws_tiles);
  o.tile_count = reinterpret_cast<int32_t*>(ws + L.ws_tile_count);
  o.blockcounts = reinterpret_cast<int32_t*>(ws + L.ws_blockcounts);
  o.sched = reinterpret_cast<int32_t*>(ws + L.ws_sched);
  return o;
}

moe_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(MOE_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950 only", dev, prop.gcnArchName);
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_mxfp4_query_sizes(const moe_mxfp4_config* cfg, size_t* repacked_bytes, size_t* workspace_bytes) {
  if (moe_status s = check_config(cfg)) return s;
  if (!repacked_bytes || !workspace_bytes) return fail(MOE_ERR_ARG, "size output pointers must not be null");
  const moe::Layout L = moe::make_layout(cfg->hidden, cfg->intermediate, cfg->num_experts, cfg->top_k,
                                         cfg->max_tokens, cfg->act);
  *repacked_bytes = L.rp_bytes;
  *workspace_bytes = L.ws_bytes;
  return ok();
}

moe_status moe_mxfp4_plan(const moe_mxfp4_config* cfg, const uint8_t* w13_codes, const uint8_t* w13_scales,
                          const uint8_t* w2_codes, const uint8_t* w2_scales, void* repacked,
                          size_t repacked_bytes, hipStream_t stream, moe_mxfp4_plan_t* out) {
  if (moe_status s = check_config(cfg)) return s;
  if (!out) return fail(MOE_ERR_ARG, "plan output pointer is null");
  *out = nullptr;
  const void* ptrs[] = {w13_codes, w13_scales, w2_codes, w2_scales, repacked};
  const char* names[] = {"w13_codes", "w13_scales", "w2_codes", "w2_scales", "repacked"};
  for (int i = 0; i < 5; ++i) {
    if (!ptrs[i]) return fail(MOE_ERR_ARG, "%s is null", names[i]);
    if (misaligned(ptrs[i])) return fail(MOE_ERR_ALIGN, "%s must be 16-byte aligned, got %p", names[i], ptrs[i]);
  }
  const moe::Layout L = moe::make_layout(cfg->hidden, cfg->intermediate, cfg->num_experts, cfg->top_k,
                                         cfg->max_tokens, cfg->act);
  if (repacked_bytes < L.rp_bytes)
    return fail(MOE_ERR_WORKSPACE, "repacked buffer must hold %zu bytes, got %zu", L.rp_bytes, repacked_bytes);
  if (moe_status s = check_device()) return s;
  uint8_t* rp = static_cast<uint8_t*>(repacked);
  hipError_t e = moe::launch_repack(L, w13_codes, w13_scales, w2_codes, w2_scales, rp, stream);
  if (e != hipSuccess) return hip_fail(e, "repack launch");
  unsigned long long status = 0;
  e = hipMemcpyAsync(&status, rp + L.rp_status, 8, hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(status)");
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  if (status != ~0ull) {
    const int matrix = (int)(status >> 56);
    const unsigned long long flat = status & ((1ull << 56) - 1);
    const moe::MatLayout& m = matrix == 0 ? L.w13 : L.w2;
    const unsigned long long groups = (unsigned long long)m.k / 32;
    const unsigned long long g = flat % groups;
    const unsigned long long row = (flat / groups) % (unsigned long long)m.n;
    const unsigned long long ex = flat / groups / (unsigned long long)m.n;
    const uint8_t* src = matrix == 0 ? w13_scales : w2_scales;
    uint8_t byte = 0;
    if (hipMemcpy(&byte, src + flat, 1, hipMemcpyDeviceToHost) != hipSuccess) byte = 0;
    return fail(MOE_ERR_SCALE_BYTE,
                "%s scale byte 0x%02X at expert %llu, row %llu, group %llu is not accepted "
                "(0x00 and 0xFF never%s)",
                matrix == 0 ? "w13" : "w2", (unsigned)byte, ex, row, g,
                cfg->act == MOE_ACT_BF16 ? "; 0x01, 0xFD, 0xFE not on the bf16 path" : "");
  }
  moe_mxfp4_plan_s* p = new moe_mxfp4_plan_s();
  p->cfg = *cfg;
  p->L = L;
  p->repacked = rp;
  p->n_events = 0;
  p->fused_gen = 0;
  *out = p;
  return ok();
}

static moe_status check_ws(const moe_mxfp4_plan_s* p, void* workspace, size_t workspace_bytes) {
  if (!workspace) return fail(MOE_ERR_ARG, "workspace is null");
  if (misaligned(workspace)) return fail(MOE_ERR_ALIGN, "workspace must be 16-byte aligned, got %p", workspace);
  if (workspace_bytes < p->L.ws_bytes)
    return fail(MOE_ERR_WORKSPACE, "workspace must hold %zu bytes, got %zu", p->L.ws_bytes, workspace_bytes);
  return MOE_OK;
}

// The FC1 and FC2 arguments of one forward: weights, route outputs, the
// activations each reads and the workspace rows each writes.
static void fc_args(const moe_mxfp4_plan_s* p, const moe::Layout& L, uint8_t* ws, const moe::RouteOut& ro,
                    const uint16_t* hidden, int32_t T, moe::FcArgs* f1, moe::FcArgs* f2) {
  const bool mx = p->cfg.act == MOE_ACT_MXFP8;
  *f1 = moe::FcArgs{};
  f1->codes = p->repacked + L.rp_w13_codes;
  f1->scales = p->repacked + L.rp_w13_scales;
  f1->mat = L.w13;
  f1->tiles = ro.tiles;
  f1->tile_count = ro.tile_count;
  f1->offsets = ro.offsets;
  f1->perm = ro.perm;
  f1->top_k = L.k;
  f1->a = mx ? static_cast<const void*>(ws + L.ws_xq) : static_cast<const void*>(hidden);
  f1->a_scales = mx ? ws + L.ws_xs : nullptr;
  f1->lda = L.H;
  f1->a_rows = T;
  f1->out = ws + L.ws_h;
  f1->ldo = L.I;
  f1->out_codes = mx ? ws + L.ws_hq : nullptr;
  f1->out_scales = mx ? ws + L.ws_hs : nullptr;
  f1->sched = ro.sched;
  *f2 = *f1;
  f2->codes = p->repacked + L.rp_w2_codes;
  f2->scales = p->repacked + L.rp_w2_scales;
  f2->mat = L.w2;
  f2->a = mx ? static_cast<const void*>(ws + L.ws_hq) : static_cast<const void*>(ws + L.ws_h);
  f2->a_scales = mx ? ws + L.ws_hs : nullptr;
  f2->lda = L.I;
  f2->a_rows = T * L.k;
  f2->out = ws + L.ws_y;
  f2->ldo = L.H;
  f2->sched = ro.sched + moe::kXcds;
}

// The argument checks every forward entry makes.
static moe_status check_forward(moe_mxfp4_plan_t p, const uint16_t* hidden, const int32_t* topk_ids,
                                const float* topk_weights, int32_t T, float* acc_fp32, uint16_t* out_bf16,
                                void* workspace, size_t workspace_bytes) {
  if (moe_status s = moe::check_forward_io(p, hidden, topk_ids, topk_weights, T, acc_fp32, out_bf16)) return s;
  return check_ws(p, workspace, workspace_bytes);
}

moe_status moe_mxfp4_forward(moe_mxfp4_plan_t p, const uint16_t* hidden, const int32_t* topk_ids,
                             const float* topk_weights, int32_t T, float* acc_fp32, uint16_t* out_bf16,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (moe_status s = check_forward(p, hidden, topk_ids, topk_weights, T, acc_fp32, out_bf16, workspace,
                                   workspace_bytes))
    return s;
  return moe::forward_with_layout(p, p->L, hidden, topk_ids, topk_weights, T, acc_fp32, out_bf16,
                                  static_cast<uint8_t*>(workspace), stream);
}

}  // extern "C"

namespace moe {

moe_status check_forward_io(const moe_mxfp4_plan_s* p, const uint16_t* hidden, const int32_t* topk_ids,
                            const float* topk_weights, int32_t T, const float* acc_fp32, const uint16_t* out_bf16) {
  if (!p) return fail(MOE_ERR_ARG, "plan is null");
  if (T < 0) return fail(MOE_ERR_ARG, "num_tokens must be >= 0, got %d", T);
  if (T > p->cfg.max_tokens)
    return fail(MOE_ERR_CAPACITY, "num_tokens %d exceeds the plan's max_tokens %d", T, p->cfg.max_tokens);
  const void* ptrs[] = {hidden, topk_ids, topk_weights, out_bf16};
  const char* names[] = {"hidden", "topk_ids", "topk_weights", "out_bf16"};
  for (int i = 0; i < 4; ++i) {
    if (!ptrs[i]) return fail(MOE_ERR_ARG, "%s is null", names[i]);
    if (misaligned(ptrs[i])) return fail(MOE_ERR_ALIGN, "%s must be 16-byte aligned, got %p", names[i], ptrs[i]);
  }
  if (acc_fp32 && misaligned(acc_fp32))
    return fail(MOE_ERR_ALIGN, "acc_fp32 must be 16-byte aligned, got %p", (const void*)acc_fp32);
  return MOE_OK;
}

// The forward's launch sequence over a workspace laid out by L (the plan's
// layout, or one sized for the batch at hand: every offset and bound comes from
// L, so a layout for fewer tokens addresses a smaller workspace).  Arguments
// are checked by the caller.
moe_status forward_with_layout(moe_mxfp4_plan_s* p, const Layout& L, const uint16_t* hidden, const int32_t* topk_ids,
                               const float* topk_weights, int32_t T, float* acc_fp32, uint16_t* out_bf16,
                               uint8_t* ws, hipStream_t stream) {
  if (T == 0) return ok();

  const moe::RouteOut ro = route_out(L, ws);
  const bool mx = p->cfg.act == MOE_ACT_MXFP8;
  const int nev = p->n_events;
  hipError_t e;
#define REC(i)                                                                                        \
  do {                                                                                                \
    if (nev > (i) && (e = hipEventRecord(p->events[i], stream)) != hipSuccess)                        \
      return hip_fail(e, "hipEventRecord");                                                           \
  } while (0)
#define CHK(call, what)                                                                               \
  do {                                                                                                \
    if ((e = (call)) != hipSuccess) return hip_fail(e, what);                                         \
  } while (0)

  // Batches with at least 16 rows per expert on average take the 128-row-tile
  // prefill kernels, smaller ones the 16-row weight-streaming kernels.  The
  // prefill kernels cut N into 256-column slices (FC2's N is H; FC1's 2I always
  // divides), and the MXFP8 one addresses its activations with 32-bit offsets.
  const int R = T * L.k;
  const bool large = (int64_t)R >= 16LL * L.E && L.H % 256 == 0;
  const bool prefill = large && !mx;
  const bool prefill_mx = large && mx && (int64_t)T * L.H < (1LL << 31) && (int64_t)R * L.I < (1LL << 31);
  const int bm = prefill ? moe::kPrefillRows : prefill_mx ? moe::kPrefillMxRows : moe::kBM;
  const int tiles_max = R / bm + (L.E < R ? L.E : R);

  moe::FcArgs f1, f2;
  fc_args(p, L, ws, ro, hidden, T, &f1, &f2);
  if (!mx && R <= moe::kPerRouteMaxRoutes) {
    // The smallest batches: two launches, no route stage.  FC1 runs one tile
    // per route (h row f), FC2 sums each token's routes in its epilogue.
    f1.route_ids = f2.route_ids = topk_ids;
    f1.num_experts = f2.num_experts = L.E;
    REC(0);
    REC(1);
    CHK(moe::launch_fc1_bf16_per_route(f1, R, stream), "FC1 launch");
    REC(2);
    CHK(moe::launch_fc2_sum_per_route(f2, topk_weights, T, L.H, acc_fp32, out_bf16, stream), "FC2 launch");
    REC(3);
    REC(4);
    return ok();
  }

  REC(0);
  CHK(moe::launch_route(L, topk_ids, T, ro, bm, stream), "route launch");
  if (mx) CHK(moe::launch_quant_bf16(hidden, T, L.H, ws + L.ws_xq, ws + L.ws_xs, stream), "x quant launch");
  REC(1);

  if (prefill) CHK(moe::launch_fc1_prefill(f1, tiles_max, stream), "FC1 launch");
  else if (prefill_mx) CHK(moe::launch_fc1_prefill_mx(f1, tiles_max, stream), "FC1 launch");
  else CHK(mx ? moe::launch_fc1_mx(f1, tiles_max, T, stream) : moe::launch_fc1_bf16(f1, tiles_max, T, stream),
           "FC1 launch");
  REC(2);

  if (mx && !prefill_mx)   // the MXFP8 prefill FC1 requantises h itself
    CHK(moe::launch_quant_f32(reinterpret_cast<const float*>(ws + L.ws_h), ro.offsets + L.E, T * L.k, L.I,
                              ws + L.ws_hq, ws + L.ws_hs, stream), "h quant launch");
  if (prefill) CHK(moe::launch_fc2_prefill(f2, tiles_max, stream), "FC2 launch");
  else if (prefill_mx) CHK(moe::launch_fc2_prefill_mx(f2, tiles_max, stream), "FC2 launch");
  else CHK(mx ? moe::launch_fc2_mx(f2, tiles_max, T, stream) : moe::launch_fc2_bf16(f2, tiles_max, T, stream),
           "FC2 launch");
  REC(3);

  // the prefill kernels land y in bf16, the decode kernels in fp32
  CHK(moe::launch_combine(ws + L.ws_y, prefill || prefill_mx, ro.rowpos, topk_weights, T, L.k, L.H, acc_fp32,
                          out_bf16, stream), "combine launch");
  REC(4);
#undef REC
#undef CHK
  return ok();
}

}  // namespace moe

extern "C" {

moe_status moe_mxfp4_forward_fused(moe_mxfp4_plan_t p, const uint16_t* hidden, const int32_t* topk_ids,
                                   const float* topk_weights, int32_t T, float* acc_fp32, uint16_t* out_bf16,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (moe_status s = check_forward(p, hidden, topk_ids, topk_weights, T, acc_fp32, out_bf16, workspace,
                                   workspace_bytes))
    return s;
  const moe::Layout& L = p->L;
  if (p->cfg.act != MOE_ACT_BF16)
    return fail(MOE_ERR_SHAPE, "the fused forward takes MOE_ACT_BF16 plans, got act=%d", p->cfg.act);
  if ((int64_t)T * L.k > moe::kFusedMaxRoutes)
    return fail(MOE_ERR_SHAPE, "the fused forward takes at most %d routes (num_tokens*top_k), got %lld",
                moe::kFusedMaxRoutes, (long long)T * L.k);
  if (T == 0) return ok();
  // a process-wide generation: the error word of an earlier forward, of any
  // plan, never matches this one
  static std::atomic<uint32_t> generation{0};
  uint32_t gen;
  do gen = generation.fetch_add(1) + 1;
  while (gen == 0);
  long long spin = 10000000;   // 100 ms of the 100 MHz s_memrealtime clock per wait
  if (const char* env = std::getenv("MOE_FUSED_SPIN_TICKS")) spin = std::atoll(env);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const moe::RouteOut ro = route_out(L, ws);
  moe::FcArgs f1, f2;
  fc_args(p, L, ws, ro, hidden, T, &f1, &f2);
  hipError_t e;
  if (p->n_events > 0 && (e = hipEventRecord(p->events[0], stream)) != hipSuccess)
    return hip_fail(e, "hipEventRecord");
  if ((e = moe::launch_fused_decode(f1, f2, topk_ids, topk_weights, T, L.k, L.E, L.H, acc_fp32, out_bf16, ro,
                                    ws + L.ws_sync, gen, spin, stream)) != hipSuccess)
    return hip_fail(e, "fused decode launch");
  for (int i = 1; i < p->n_events; ++i)   // one kernel: every later stage boundary is its end
    if ((e = hipEventRecord(p->events[i], stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  p->fused_gen = gen;
  return ok();
}

moe_status moe_mxfp4_fused_status(moe_mxfp4_plan_t p, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  if (!p) return fail(MOE_ERR_ARG, "plan is null");
  if (moe_status s = check_ws(p, workspace, workspace_bytes)) return s;
  if (p->fused_gen == 0) return ok();
  hipError_t e;
  if ((e = hipStreamSynchronize(stream)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  uint32_t word = 0;
  const uint8_t* err = static_cast<const uint8_t*>(workspace) + p->L.ws_sync + 4 * (2 * (size_t)moe::kFusedMaxTiles + 1);
  if ((e = hipMemcpy(&word, err, 4, hipMemcpyDeviceToHost)) != hipSuccess) return hip_fail(e, "hipMemcpy");
  if (word == p->fused_gen)
    return fail(MOE_ERR_TIMEOUT, "a wait of the last fused forward (generation %u) passed its time bound; "
                "its outputs are not valid", word);
  return ok();
}

moe_status moe_mxfp4_route(moe_mxfp4_plan_t p, const int32_t* topk_ids, int32_t T, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* rowpos, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (!p) return fail(MOE_ERR_ARG, "plan is null");
  if (T < 0) return fail(MOE_ERR_ARG, "num_tokens must be >= 0, got %d", T);
  if (T > p->cfg.max_tokens)
    return fail(MOE_ERR_CAPACITY, "num_tokens %d exceeds the plan's max_tokens %d", T, p->cfg.max_tokens);
  if (moe_status s = check_ws(p, workspace, workspace_bytes)) return s;
  const void* ptrs[] = {topk_ids, counts, offsets, perm, rowpos};
  const char* names[] = {"topk_ids", "counts", "offsets", "perm", "rowpos"};
  for (int i = 0; i < 5; ++i) {
    if (!ptrs[i]) return fail(MOE_ERR_ARG, "%s is null", names[i]);
    if (misaligned(ptrs[i])) return fail(MOE_ERR_ALIGN, "%s must be 16-byte aligned, got %p", names[i], ptrs[i]);
  }
  moe::RouteOut o = route_out(p->L, static_cast<uint8_t*>(workspace));
  o.counts = counts;
  o.offsets = offsets;
  o.perm = perm;
  o.rowpos = rowpos;
  hipError_t e = moe::launch_route(p->L, topk_ids, T, o, moe::kBM, stream);
  if (e != hipSuccess) return hip_fail(e, "route launch");
  return ok();
}

moe_status moe_mxfp4_workspace_region(moe_mxfp4_plan_t p, int32_t region, size_t* offset, size_t* bytes) {
  if (!p) return fail(MOE_ERR_ARG, "plan is null");
  if (!offset || !bytes) return fail(MOE_ERR_ARG, "offset and bytes must not be null");
  if (p->cfg.act != MOE_ACT_MXFP8)
    return fail(MOE_ERR_ARG, "workspace regions of h exist for MOE_ACT_MXFP8 plans only, got act=%d", p->cfg.act);
  const moe::Layout& L = p->L;
  const size_t R = (size_t)L.Rmax;
  switch (region) {
    case MOE_WS_H_CODES: *offset = L.ws_hq; *bytes = R * L.I; break;
    case MOE_WS_H_SCALES: *offset = L.ws_hs; *bytes = R * (L.I / 32); break;
    default: return fail(MOE_ERR_ARG, "region must be MOE_WS_H_CODES (0) or MOE_WS_H_SCALES (1), got %d", region);
  }
  return ok();
}

moe_status moe_mxfp8_quantize(const uint16_t* x, int32_t rows, int32_t cols, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream) {
  if (rows < 0) return fail(MOE_ERR_ARG, "rows must be >= 0, got %d", rows);
  if (cols <= 0 || cols % 32) return fail(MOE_ERR_SHAPE, "cols must be a positive multiple of 32, got %d", cols);
  if (rows == 0) return ok();
  const void* ptrs[] = {x, codes, scales};
  const char* names[] = {"x", "codes", "scales"};
  for (int i = 0; i < 3; ++i) {
    if (!ptrs[i]) return fail(MOE_ERR_ARG, "%s is null", names[i]);
    if (misaligned(ptrs[i])) return fail(MOE_ERR_ALIGN, "%s must be 16-byte aligned, got %p", names[i], ptrs[i]);
  }
  hipError_t e = moe::launch_quant_bf16(x, rows, cols, codes, scales, stream);
  if (e != hipSuccess) return hip_fail(e, "quant launch");
  return ok();
}

moe_status moe_router_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* ids, float* weights,
                           hipStream_t stream) {
  if (T < 0) return fail(MOE_ERR_ARG, "num_tokens must be >= 0, got %d", T);
  if (E < 1 || E > moe::kRouterMaxExperts)
    return fail(MOE_ERR_SHAPE, "num_experts must be in [1, %d], got %d", moe::kRouterMaxExperts, E);
  if (k < 1 || k > kMaxTopK || k > E)
    return fail(MOE_ERR_SHAPE, "top_k must be in [1, min(%d, num_experts=%d)], got %d", kMaxTopK, E, k);
  if (T == 0) return ok();
  const void* ptrs[] = {logits, ids, weights};
  const char* names[] = {"logits", "topk_ids", "topk_weights"};
  for (int i = 0; i < 3; ++i) {
    if (!ptrs[i]) return fail(MOE_ERR_ARG, "%s is null", names[i]);
    if (misaligned(ptrs[i])) return fail(MOE_ERR_ALIGN, "%s must be 16-byte aligned, got %p", names[i], ptrs[i]);
  }
  hipError_t e = moe::launch_router_topk(logits, T, E, k, ids, weights, stream);
  if (e != hipSuccess) return hip_fail(e, "router launch");
  return ok();
}

moe_status moe_probe_memory(int32_t kind, const void* src, void* dst, size_t bytes, float* sink, int32_t grid,
                            hipStream_t stream) {
  if (kind < MOE_PROBE_READ || kind > MOE_PROBE_COPY)
    return fail(MOE_ERR_ARG, "probe kind must be 0 (read), 1 (non-temporal read) or 2 (copy), got %d", kind);
  if (grid < 1 || grid > moe::kProbeSinkFloats)
    return fail(MOE_ERR_ARG, "grid must be in [1, %d], got %d", moe::kProbeSinkFloats, grid);
  if (bytes == 0 || bytes % 16) return fail(MOE_ERR_SHAPE, "bytes must be a positive multiple of 16, got %zu", bytes);
  if (!src || !sink || (kind == MOE_PROBE_COPY && !dst)) return fail(MOE_ERR_ARG, "a probe buffer is null");
  if (misaligned(src) || (dst && misaligned(dst)))
    return fail(MOE_ERR_ALIGN, "probe buffers must be 16-byte aligned");
  hipError_t e = moe::launch_probe_memory(kind, src, dst, bytes, sink, grid, stream);
  if (e != hipSuccess) return hip_fail(e, "probe launch");
  return ok();
}

moe_status moe_probe_mfma(int32_t kind, int32_t iters, float* sink, int32_t grid, double* flops,
                          hipStream_t stream) {
  if (kind != MOE_PROBE_MFMA_BF16 && kind != MOE_PROBE_MFMA_F8F4)
    return fail(MOE_ERR_ARG, "probe kind must be 0 (bf16) or 1 (f8f6f4), got %d", kind);
  if (grid < 1 || grid > moe::kProbeSinkFloats)
    return fail(MOE_ERR_ARG, "grid must be in [1, %d], got %d", moe::kProbeSinkFloats, grid);
  if (iters < 1) return fail(MOE_ERR_ARG, "iters must be >= 1, got %d", iters);
  if (!sink || !flops) return fail(MOE_ERR_ARG, "sink and flops must not be null");
  hipError_t e = moe::launch_probe_mfma(kind, iters, sink, grid, flops, stream);
  if (e != hipSuccess) return hip_fail(e, "probe launch");
  return ok();
}

moe_status moe_probe_mfma_f8f4_blocks(const uint8_t* a, const uint8_t* b, const uint8_t* sa, const uint8_t* sb,
                                      const float* c, float* d, int32_t n, hipStream_t stream) {
  if (n < 1 || n > 65536) return fail(MOE_ERR_ARG, "n must be in [1, 65536], got %d", n);
  const void* ptrs[] = {a, b, sa, sb, c, d};
  const char* names[] = {"a_lanes", "b_lanes", "a_scales", "b_scales", "c", "d"};
  for (int i = 0; i < 6; ++i) {
    if (!ptrs[i]) return fail(MOE_ERR_ARG, "%s is null", names[i]);
    if (misaligned(ptrs[i])) return fail(MOE_ERR_ALIGN, "%s must be 16-byte aligned, got %p", names[i], ptrs[i]);
  }
  hipError_t e = moe::launch_probe_mfma_blocks(a, b, sa, sb, c, d, n, stream);
  if (e != hipSuccess) return hip_fail(e, "probe launch");
  return ok();
}

moe_status moe_mxfp4_set_stage_events(moe_mxfp4_plan_t p, hipEvent_t* events, int32_t n) {
  if (!p) return fail(MOE_ERR_ARG, "plan is null");
  if (n != 0 && n != 5) return fail(MOE_ERR_ARG, "stage events: n must be 0 or 5, got %d", n);
  if (n && !events) return fail(MOE_ERR_ARG, "stage events array is null");
  for (int i = 0; i < n; ++i) p->events[i] = events[i];
  p->n_events = n;
  return ok();
}

void moe_mxfp4_destroy(moe_mxfp4_plan_t p) { delete p; }

const char* moe_mxfp4_last_error(void) { return g_err.c_str(); }

}  // extern "C"
