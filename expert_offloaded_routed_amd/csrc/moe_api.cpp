// Host side of the libmoe C ABI: argument validation, workspace layout, kernel launches and
// slot refills.  See include/moe.h for the contract of each call.
#include <hip/hip_runtime_api.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>

#include "moe.h"
#include "moe_internal.h"

namespace moe {

static_assert(kScratchBytes == MOE_NOALLOC_SCRATCH_BYTES, "moe.h states the static scratch size");

thread_local std::string g_last_error;

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status ok() {
  g_last_error.clear();
  return MOE_OK;
}

moe_status check_shape(const moe_shape* s) {
  if (!s) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
  if (s->hidden <= 0 || s->inter <= 0 || s->n_experts <= 0 || s->top_k <= 0 || s->n_slots <= 0)
    return fail(MOE_ERR_INVALID_ARG, "shape fields must be positive (H=%d I=%d E=%d k=%d S=%d)",
                s->hidden, s->inter, s->n_experts, s->top_k, s->n_slots);
  if (s->hidden % 64 || s->inter % 32)
    return fail(MOE_ERR_UNSUPPORTED, "need hidden %% 64 == 0 and inter %% 32 == 0 (H=%d I=%d)",
                s->hidden, s->inter);
  if (s->hidden > kMaxHidden)
    return fail(MOE_ERR_UNSUPPORTED, "hidden %d > %d", s->hidden, kMaxHidden);
  if (s->inter > kMaxInter)
    return fail(MOE_ERR_UNSUPPORTED, "inter %d > %d", s->inter, kMaxInter);
  if (s->n_experts > kMaxExperts)
    return fail(MOE_ERR_UNSUPPORTED, "n_experts %d > %d", s->n_experts, kMaxExperts);
  if (s->top_k > kMaxTopK || s->top_k > s->n_experts)
    return fail(MOE_ERR_UNSUPPORTED, "top_k %d must be <= min(n_experts, %d)", s->top_k, kMaxTopK);
  if (s->format < MOE_FORMAT_MXFP4 || s->format > MOE_FORMAT_NVFP4)
    return fail(MOE_ERR_UNSUPPORTED, "unknown expert format %d", s->format);
  return MOE_OK;
}

static moe_status hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Bound on routes per call (one bucketing workgroup walks them all).
constexpr int kMaxRoutesPerCall = 1 << 20;

static moe_status check_ws(const moe_shape* s, int M, void* ws, size_t ws_bytes, WsLayout* W) {
  if (M < 0) return fail(MOE_ERR_INVALID_ARG, "M = %d < 0", M);
  if ((size_t)M * s->top_k > (size_t)kMaxRoutesPerCall)
    return fail(MOE_ERR_UNSUPPORTED, "M * top_k > %d", kMaxRoutesPerCall);
  if (!ws) return fail(MOE_ERR_INVALID_ARG, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0)
    return fail(MOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  *W = ws_layout(s->hidden, s->inter, s->n_experts, s->top_k, M);
  if (ws_bytes < W->total)
    return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed for M=%d", ws_bytes, W->total, M);
  return MOE_OK;
}

template <typename T>
static T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}

static BucketOut bucket_out(void* ws, const WsLayout& W, int32_t* counts, int32_t* offsets,
                            int32_t* perm, int32_t* cold_count, int32_t* cold_routes) {
  BucketOut o;
  o.route_slot = at<int32_t>(ws, W.route_slot);
  o.ws_perm = at<int32_t>(ws, W.perm);
  o.meta = at<int32_t>(ws, W.meta);
  o.dist = at<int4>(ws, W.dist);
  o.items = at<int2>(ws, W.items);
  o.cold_list = at<int32_t>(ws, W.cold_list);
  o.u_counts = counts;
  o.u_offsets = offsets;
  o.u_perm = perm;
  o.u_cold_count = cold_count;
  o.u_cold_routes = cold_routes;
  return o;
}

static moe_status check_map(const moe_shape* s, const int32_t* e2s) {
  if (!e2s && s->n_experts > s->n_slots)
    return fail(MOE_ERR_INVALID_ARG, "identity expert_to_slot needs n_slots >= n_experts");
  return MOE_OK;
}

static moe_status check_x_slots(const uint16_t* x, const uint8_t* slots) {
  if (!x || !slots) return fail(MOE_ERR_INVALID_ARG, "x and slots are required");
  if ((reinterpret_cast<uintptr_t>(x) & 15) || (reinterpret_cast<uintptr_t>(slots) & 255))
    return fail(MOE_ERR_INVALID_ARG, "x must be 16-byte and slots 256-byte aligned");
  return MOE_OK;
}

// Route arguments of a call: top-k from `logits` (or the given ids / weights), the expert map.
static RouteArgs route_args(const moe_shape* sh, int M, const float* logits, const int32_t* ids,
                            const float* w, const int32_t* e2s, int32_t* out_ids, float* out_w,
                            int32_t* cold_count, int32_t* cold_routes) {
  RouteArgs a;
  a.logits = logits;
  a.ids_in = ids;
  a.w_in = w;
  a.e2s = e2s;
  a.M = M;
  a.k = sh->top_k;
  a.E = sh->n_experts;
  a.S = sh->n_slots;
  a.topk_ids = out_ids;
  a.topk_w = out_w;
  a.cold_count = cold_count;
  a.cold_routes = cold_routes;
  return a;
}

static RouteWs route_ws(void* ws, const WsLayout& W) {
  RouteWs r;
  r.meta = at<int32_t>(ws, W.meta);
  r.dist = at<int4>(ws, W.dist);
  r.items = at<int2>(ws, W.items);
  r.perm = at<int32_t>(ws, W.perm);
  r.route_slot = at<int32_t>(ws, W.route_slot);
  return r;
}

// MOE_DECODE_UNFUSED=1: one-token layer calls keep gate/up and down as two launches.
static bool decode_unfused() {
  static const bool v = [] {
    const char* s = getenv("MOE_DECODE_UNFUSED");
    return s != nullptr && s[0] == '1';
  }();
  return v;
}

// Stage mark of moe_layer_forward_marked.
static hipError_t record_mark(hipEvent_t ev, hipStream_t stream) { return hipEventRecord(ev, stream); }

// Where the routes of a call come from.
enum class RouteSrc {
  kLogits,  // router logits in the workspace: top-k still to do
  kIds,     // caller's ids / w
};

// Calls whose route table the one-workgroup kernel builds faster than the top-k / bucketing
// kernel: one token (a single top-k), or at most kRouteTableMaxRoutes routes over at most 64
// experts (its table build is quadratic in the routes and its top-k one wave per token).
static bool route_table_fits(int M, int k, int E) {
  return (size_t)M * k <= (size_t)kRouteTableMaxRoutes && (M == 1 || E <= 64);
}

// The expert stages of a call whose experts are not MXFP4: the route-table kernel (small calls)
// or the top-k / bucketing kernel writes the route table, then the generic gate/up and down
// kernels of the format run.
static moe_status run_experts_fmt(const moe_shape* sh, const uint16_t* x, int M,
                                  const float* logits, int32_t* ids, float* w, const int32_t* e2s,
                                  const uint8_t* slots, float* y, int32_t* cold_count,
                                  int32_t* cold_routes, void* ws, const WsLayout& W, bool do_gateup,
                                  bool do_down, hipStream_t stream, const hipEvent_t* marks,
                                  uint16_t* x_next) {
  const int H = sh->hidden, I = sh->inter, k = sh->top_k, E = sh->n_experts;
  const FmtLayout F = fmt_layout(sh->format, H, I);
  const RouteWs rw = route_ws(ws, W);
  hipError_t e;
  if (do_gateup) {
    if (route_table_fits(M, k, E)) {
      const RouteArgs rt = route_args(sh, M, logits, ids, w, e2s, logits ? ids : nullptr,
                                      logits ? w : nullptr, cold_count, cold_routes);
      e = launch_route_table(rt, rw, stream);
    } else {
      const BucketOut o = bucket_out(ws, W, nullptr, nullptr, nullptr, cold_count, cold_routes);
      e = launch_topk_bucket(logits, M, k, ids, w, true, ids, E, sh->n_slots, e2s, o, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "route table launch");
  }
  if (marks && (e = record_mark(marks[1], stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  const RouteArgs ra = route_args(sh, M, nullptr, ids, w, e2s, nullptr, nullptr, nullptr, nullptr);
  if (do_gateup) {
    const int nd_max = (int)((size_t)M * k < (size_t)E ? (size_t)M * k : (size_t)E);
    e = launch_gateup_fmt(sh->format, x, H, I, slots, F.image_bytes, F, nd_max, ra, rw,
                          at<uint16_t>(ws, W.hq), stream);
    if (e != hipSuccess) return hip_fail(e, "gate/up launch");
  }
  if (marks && (e = record_mark(marks[2], stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if (do_down) {
    e = launch_down_fmt(sh->format, H, I, slots, F.image_bytes, F, ra, rw, at<uint16_t>(ws, W.hq),
                        at<float>(ws, W.pdn), y, Residual{x, x_next}, stream);
    if (e != hipSuccess) return hip_fail(e, "down launch");
  }
  if (marks && (e = record_mark(marks[3], stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  return MOE_OK;
}

// The expert stages of a call.  Small calls (M*k <= 256) rebuild the route table inside every
// gate/up workgroup (top-k from the logits, or the ids); one of them also publishes it to the
// workspace for the down kernel.  Larger calls run the top-k / bucketing kernel first, which
// writes the table.  do_gateup / do_down select the stages.
static moe_status run_experts(const moe_shape* sh, const uint16_t* x, int M, RouteSrc src,
                              const float* logits, int32_t* ids, float* w, const int32_t* e2s,
                              const uint8_t* slots, float* y, int32_t* cold_count,
                              int32_t* cold_routes, void* ws, const WsLayout& W, bool do_gateup,
                              bool do_down, hipStream_t stream, const hipEvent_t* marks = nullptr,
                              uint16_t* x_next = nullptr) {
  if (sh->format != MOE_FORMAT_MXFP4)
    return run_experts_fmt(sh, x, M, src == RouteSrc::kLogits ? logits : nullptr, ids, w, e2s,
                           slots, y, cold_count, cold_routes, ws, W, do_gateup, do_down, stream,
                           marks, x_next);
  const ImageLayout L = image_layout(sh->hidden, sh->inter);
  const ExpertPlan p = plan_experts(L, M, sh->n_experts, sh->top_k);
  const RouteWs rw = route_ws(ws, W);
  if (src != RouteSrc::kLogits) logits = nullptr;
  hipError_t e;
  if (!p.prologue && do_gateup) {
    // one token, or a few routes over few experts: the one-workgroup route table; otherwise
    // (and on the grouped path, which also needs the work list) the top-k / bucketing kernel
    if (!p.grouped && route_table_fits(M, sh->top_k, sh->n_experts)) {
      const RouteArgs rt = route_args(sh, M, logits, ids, w, e2s, logits ? ids : nullptr,
                                      logits ? w : nullptr, cold_count, cold_routes);
      e = launch_route_table(rt, rw, stream);
    } else {
      const BucketOut o = bucket_out(ws, W, nullptr, nullptr, nullptr, cold_count, cold_routes);
      e = launch_topk_bucket(logits, M, sh->top_k, ids, w, true, ids, sh->n_experts, sh->n_slots,
                             e2s, o, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "route table launch");
    logits = nullptr;  // ids / w are final from here on
  }
  if (marks && (e = record_mark(marks[1], stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if (do_gateup) {
    // in the prologue case the writer workgroup publishes top-k results and the cold report
    const RouteArgs ra = route_args(sh, M, logits, ids, w, e2s, logits ? ids : nullptr,
                                    logits ? w : nullptr, p.prologue ? cold_count : nullptr,
                                    p.prologue ? cold_routes : nullptr);
    e = p.grouped ? launch_gateup_grouped(x, sh->hidden, sh->inter, slots, L, p, ra, rw,
                                          at<uint8_t>(ws, W.hq), stream)
                  : launch_gateup(x, M, sh->hidden, sh->inter, slots, L, p, ra, rw,
                                  at<uint16_t>(ws, W.hq), stream);
    if (e != hipSuccess) return hip_fail(e, "gate/up launch");
  }
  if (marks && (e = record_mark(marks[2], stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if (do_down) {
    const RouteArgs ra = route_args(sh, M, nullptr, ids, w, e2s, nullptr, nullptr, nullptr, nullptr);
    const Residual res{x, x_next};
    e = p.grouped ? launch_down_grouped(M, sh->hidden, sh->inter, slots, L, p, ra, rw,
                                        at<uint8_t>(ws, W.hq), at<float>(ws, W.pdn), y, res, stream)
                  : launch_down(M, sh->hidden, sh->inter, slots, L, p, ra, rw,
                                at<uint16_t>(ws, W.hq), at<uint64_t>(ws, W.pw),
                                at<uint32_t>(ws, W.dncall), y, res, stream);
    if (e != hipSuccess) return hip_fail(e, "down launch");
  }
  if (marks && (e = record_mark(marks[3], stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  return MOE_OK;
}

// Cold report of an empty call (M = 0).
static moe_status empty_call(const moe_shape* sh, const int32_t* e2s, int32_t* cold_count,
                             void* ws, const WsLayout& W, hipStream_t stream) {
  if (!cold_count) return MOE_OK;
  const BucketOut o = bucket_out(ws, W, nullptr, nullptr, nullptr, cold_count, nullptr);
  hipError_t e = launch_topk_bucket(nullptr, 0, sh->top_k, nullptr, nullptr, true, nullptr,
                                    sh->n_experts, sh->n_slots, e2s, o, stream);
  if (e != hipSuccess) return hip_fail(e, "bucket launch");
  return MOE_OK;
}

static moe_status layer_forward(const moe_shape* shape, const uint16_t* x, int32_t M,
                                const uint16_t* w_router, const float* router_bias,
                                const int32_t* expert_to_slot, const uint8_t* slots,
                                int32_t* topk_ids, float* topk_w, float* y, int32_t* cold_count,
                             int32_t* cold_routes, void* ws, size_t ws_bytes, hipStream_t stream,
                                const hipEvent_t* marks, uint16_t* x_next) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  WsLayout W;
  st = check_ws(shape, M, ws, ws_bytes, &W);
  if (st != MOE_OK) return st;
  st = check_map(shape, expert_to_slot);
  if (st != MOE_OK) return st;
  if (M == 0) {
    st = empty_call(shape, expert_to_slot, cold_count, ws, W, stream);
    return st != MOE_OK ? st : ok();
  }
  st = check_x_slots(x, slots);
  if (st != MOE_OK) return st;
  if (!w_router || !topk_ids || !topk_w || !y)
    return fail(MOE_ERR_INVALID_ARG,
                "moe_layer_forward: w_router, topk_ids, topk_w and y are required");
  if (reinterpret_cast<uintptr_t>(w_router) & 15)
    return fail(MOE_ERR_INVALID_ARG, "moe_layer_forward: w_router must be 16-byte aligned");
  if (x_next && (reinterpret_cast<uintptr_t>(x_next) & 1))
    return fail(MOE_ERR_INVALID_ARG, "moe_layer_forward_residual: x_next must be 2-byte aligned");
  float* logits = at<float>(ws, W.logits);
  hipError_t e;
  // One token with a fusable shape: the layer after the router (or the whole layer, router
  // included, for small routers) is one launch.  MOE_DECODE_UNFUSED=1 in the environment selects
  // the multi-launch path.
  const ImageLayout L = image_layout(shape->hidden, shape->inter);
  const ExpertPlan p = plan_experts(L, M, shape->n_experts, shape->top_k);
  const bool fused = shape->format == MOE_FORMAT_MXFP4 && !decode_unfused() &&
                     layer_decode_fusable(L, p, M, shape->top_k, shape->n_experts);
  const bool router_inside = fused && layer_decode_router_inside(L, shape->n_experts);
  if (marks && (e = record_mark(marks[0], stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if (!router_inside) {
    e = launch_router(x, M, w_router, router_bias, shape->n_experts, shape->hidden, logits,
                      stream);
    if (e != hipSuccess) return hip_fail(e, "router launch");
  }
  if (fused) {
    if (marks && (e = record_mark(marks[1], stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    const RouteArgs ra = route_args(shape, M, router_inside ? nullptr : logits, topk_ids, topk_w,
                                    expert_to_slot, topk_ids, topk_w, cold_count, cold_routes);
    e = launch_layer_decode(x, w_router, router_bias, M, shape->hidden, shape->inter, slots, L, p,
                            ra, route_ws(ws, W), at<uint64_t>(ws, W.hf), y, Residual{x, x_next},
                            stream);
    if (e != hipSuccess) return hip_fail(e, "fused decode launch");
    for (int i = 2; marks && i < 4; ++i)
      if ((e = record_mark(marks[i], stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    return ok();
  }
  const RouteSrc src = RouteSrc::kLogits;
  st = run_experts(shape, x, M, src, logits, topk_ids, topk_w, expert_to_slot, slots, y,
                   cold_count, cold_routes, ws, W, true, true, stream, marks, x_next);
  return st != MOE_OK ? st : ok();
}

// The GPU part of moe_layer_forward_hybrid: router + top-k, the routes and x staged to the host
// (staging->routed recorded behind them), then the hot experts, all on the stream.
moe_status layer_route_and_hot(const moe_shape* shape, const uint16_t* x, int32_t M,
                               const uint16_t* w_router, const float* router_bias,
                               const int32_t* expert_to_slot, const uint8_t* slots,
                               int32_t* topk_ids, float* topk_w, float* y, void* ws,
                               size_t ws_bytes, hipStream_t stream,
                               const moe_hybrid_staging* staging) {
  WsLayout W;
  moe_status st = check_ws(shape, M, ws, ws_bytes, &W);
  if (st != MOE_OK) return st;
  st = check_x_slots(x, slots);
  if (st != MOE_OK) return st;
  if (!w_router || !topk_ids || !topk_w || !y)
    return fail(MOE_ERR_INVALID_ARG, "moe_layer_forward_hybrid: w_router, topk_ids, topk_w and y are required");
  if (reinterpret_cast<uintptr_t>(w_router) & 15)
    return fail(MOE_ERR_INVALID_ARG, "moe_layer_forward_hybrid: w_router must be 16-byte aligned");
  const int E = shape->n_experts, k = shape->top_k, H = shape->hidden;
  float* logits = at<float>(ws, W.logits);
  hipError_t e = launch_router(x, M, w_router, router_bias, E, H, logits, stream);
  if (e != hipSuccess) return hip_fail(e, "router launch");
  const BucketOut o = bucket_out(ws, W, nullptr, nullptr, nullptr, nullptr, nullptr);
  e = launch_topk_bucket(logits, M, k, topk_ids, topk_w, false, topk_ids, E, shape->n_slots, nullptr,
                         o, stream);
  if (e != hipSuccess) return hip_fail(e, "top-k launch");
  const size_t Mk = (size_t)M * k;
  if ((e = hipMemcpyAsync(staging->x, x, sizeof(uint16_t) * M * H, hipMemcpyDeviceToHost, stream)) != hipSuccess ||
      (e = hipMemcpyAsync(staging->ids, topk_ids, sizeof(int32_t) * Mk, hipMemcpyDeviceToHost, stream)) != hipSuccess ||
      (e = hipMemcpyAsync(staging->w, topk_w, sizeof(float) * Mk, hipMemcpyDeviceToHost, stream)) != hipSuccess)
    return hip_fail(e, "hipMemcpyAsync");
  if ((e = hipEventRecord(staging->routed, stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  return run_experts(shape, x, M, RouteSrc::kIds, nullptr, topk_ids, topk_w, expert_to_slot, slots, y,
                     nullptr, nullptr, ws, W, true, true, stream);
}

// The routing part of moe_layer_forward_staged: router + top-k (as moe_route), then the route
// count of every expert into counts_dev.
moe_status staged_route_and_count(const moe_shape* shape, const uint16_t* x, int32_t M,
                                  const uint16_t* w_router, const float* router_bias,
                                  int32_t* topk_ids, float* topk_w, int32_t* counts_dev, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  WsLayout W;
  moe_status st = check_ws(shape, M, ws, ws_bytes, &W);
  if (st != MOE_OK) return st;
  if (!x || !w_router || !topk_ids || !topk_w)
    return fail(MOE_ERR_INVALID_ARG, "moe_layer_forward_staged: x, w_router, topk_ids and topk_w are required");
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w_router)) & 15)
    return fail(MOE_ERR_INVALID_ARG, "moe_layer_forward_staged: x and w_router must be 16-byte aligned");
  const int E = shape->n_experts, k = shape->top_k;
  float* logits = at<float>(ws, W.logits);
  hipError_t e = launch_router(x, M, w_router, router_bias, E, shape->hidden, logits, stream);
  if (e != hipSuccess) return hip_fail(e, "router launch");
  BucketOut o = bucket_out(ws, W, counts_dev, nullptr, nullptr, nullptr, nullptr);
  e = launch_topk_bucket(logits, M, k, topk_ids, topk_w, false, topk_ids, E, E, nullptr, o, stream);
  if (e != hipSuccess) return hip_fail(e, "top-k launch");
  e = launch_topk_bucket(nullptr, M, k, nullptr, nullptr, true, topk_ids, E, E, nullptr, o, stream);
  if (e != hipSuccess) return hip_fail(e, "bucket launch");
  return MOE_OK;
}

// The expert part of a staged pass: moe_experts_forward on the staging slots with the pass's map.
moe_status staged_experts(const moe_shape* shape, const uint16_t* x, int32_t M,
                          const int32_t* topk_ids, const float* topk_w, const int32_t* e2s,
                          const uint8_t* slots, float* y, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  WsLayout W;
  moe_status st = check_ws(shape, M, ws, ws_bytes, &W);
  if (st != MOE_OK) return st;
  st = check_x_slots(x, slots);
  if (st != MOE_OK) return st;
  return run_experts(shape, x, M, RouteSrc::kIds, nullptr, const_cast<int32_t*>(topk_ids),
                     const_cast<float*>(topk_w), e2s, slots, y, nullptr, nullptr, ws, W, true, true,
                     stream);
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_expert_image_bytes(const moe_shape* shape, size_t* bytes) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = expert_image_bytes(shape);
  return ok();
}

moe_status moe_workspace_size(const moe_shape* shape, int32_t max_M, size_t* bytes) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  if (max_M < 0) return fail(MOE_ERR_INVALID_ARG, "max_M < 0");
  if ((size_t)max_M * shape->top_k > (size_t)kMaxRoutesPerCall)
    return fail(MOE_ERR_UNSUPPORTED, "max_M * top_k > %d", kMaxRoutesPerCall);
  *bytes = ws_layout(shape->hidden, shape->inter, shape->n_experts, shape->top_k, max_M).total;
  return ok();
}

moe_status moe_layer_launches(const moe_shape* shape, int32_t M, int32_t* n) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!n) return fail(MOE_ERR_INVALID_ARG, "n is NULL");
  if (M < 0) return fail(MOE_ERR_INVALID_ARG, "M < 0");
  if (M == 0) {
    *n = 1;  // the cold report of an empty call
    return ok();
  }
  if (shape->format != MOE_FORMAT_MXFP4) {
    *n = 4;  // router, top-k / bucket, gate/up, down + combine
    return ok();
  }
  const ImageLayout L = image_layout(shape->hidden, shape->inter);
  const ExpertPlan p = plan_experts(L, M, shape->n_experts, shape->top_k);
  if (!decode_unfused() && layer_decode_fusable(L, p, M, shape->top_k, shape->n_experts))
    *n = layer_decode_router_inside(L, shape->n_experts) ? 1 : 2;  // [router,] fused layer
  else if (p.grouped)
    *n = 5;                     // router, top-k / bucket, gate/up, down, combine
  else
    *n = p.prologue ? 3 : 4;    // router, [top-k / bucket,] gate/up, down + combine
  return ok();
}

moe_status moe_route(const moe_shape* shape, const uint16_t* x, int32_t M, const uint16_t* w_router,
                     const float* router_bias, int32_t* topk_ids, float* topk_w, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  WsLayout W;
  st = check_ws(shape, M, ws, ws_bytes, &W);
  if (st != MOE_OK) return st;
  if (M == 0) return ok();
  if (!x || !w_router || !topk_ids || !topk_w)
    return fail(MOE_ERR_INVALID_ARG, "moe_route: x, w_router, topk_ids and topk_w are required");
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w_router)) & 15)
    return fail(MOE_ERR_INVALID_ARG, "moe_route: x and w_router must be 16-byte aligned");
  float* logits = at<float>(ws, W.logits);
  hipError_t e = launch_router(x, M, w_router, router_bias, shape->n_experts, shape->hidden, logits,
                               stream);
  if (e != hipSuccess) return hip_fail(e, "router launch");
  const BucketOut o = bucket_out(ws, W, nullptr, nullptr, nullptr, nullptr, nullptr);
  e = launch_topk_bucket(logits, M, shape->top_k, topk_ids, topk_w, false, topk_ids,
                         shape->n_experts, shape->n_slots, nullptr, o, stream);
  if (e != hipSuccess) return hip_fail(e, "top-k launch");
  return ok();
}

moe_status moe_bucket_routes(const moe_shape* shape, const int32_t* topk_ids, int32_t M,
                             const int32_t* expert_to_slot, int32_t* counts, int32_t* offsets,
                             int32_t* perm, int32_t* cold_count, int32_t* cold_routes, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  WsLayout W;
  st = check_ws(shape, M, ws, ws_bytes, &W);
  if (st != MOE_OK) return st;
  if (M > 0 && !topk_ids) return fail(MOE_ERR_INVALID_ARG, "topk_ids is NULL");
  st = check_map(shape, expert_to_slot);
  if (st != MOE_OK) return st;
  const BucketOut o = bucket_out(ws, W, counts, offsets, perm, cold_count, cold_routes);
  hipError_t e = launch_topk_bucket(nullptr, M, shape->top_k, nullptr, nullptr, true, topk_ids,
                                    shape->n_experts, shape->n_slots, expert_to_slot, o, stream);
  if (e != hipSuccess) return hip_fail(e, "bucket launch");
  return ok();
}

moe_status moe_experts_forward(const moe_shape* shape, const uint16_t* x, int32_t M,
                               const int32_t* topk_ids, const float* topk_w,
                               const int32_t* expert_to_slot, const uint8_t* slots, float* y,
                               int32_t* cold_count, int32_t* cold_routes, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  WsLayout W;
  st = check_ws(shape, M, ws, ws_bytes, &W);
  if (st != MOE_OK) return st;
  st = check_map(shape, expert_to_slot);
  if (st != MOE_OK) return st;
  if (M == 0) {
    st = empty_call(shape, expert_to_slot, cold_count, ws, W, stream);
    return st != MOE_OK ? st : ok();
  }
  st = check_x_slots(x, slots);
  if (st != MOE_OK) return st;
  if (!topk_ids || !topk_w || !y)
    return fail(MOE_ERR_INVALID_ARG, "moe_experts_forward: topk_ids, topk_w and y are required");
  st = run_experts(shape, x, M, RouteSrc::kIds, nullptr, const_cast<int32_t*>(topk_ids),
                   const_cast<float*>(topk_w), expert_to_slot, slots, y, cold_count, cold_routes, ws,
                   W, true, true, stream);
  return st != MOE_OK ? st : ok();
}

moe_status moe_layer_forward(const moe_shape* shape, const uint16_t* x, int32_t M,
                             const uint16_t* w_router, const float* router_bias,
                             const int32_t* expert_to_slot, const uint8_t* slots,
                             int32_t* topk_ids, float* topk_w, float* y, int32_t* cold_count,
                             int32_t* cold_routes, void* ws, size_t ws_bytes, hipStream_t stream) {
  return layer_forward(shape, x, M, w_router, router_bias, expert_to_slot, slots, topk_ids, topk_w,
                       y, cold_count, cold_routes, ws, ws_bytes, stream, nullptr, nullptr);
}

moe_status moe_layer_forward_residual(const moe_shape* shape, const uint16_t* x, int32_t M,
                                      const uint16_t* w_router, const float* router_bias,
                                      const int32_t* expert_to_slot, const uint8_t* slots,
                                      int32_t* topk_ids, float* topk_w, float* y,
                                      int32_t* cold_count, int32_t* cold_routes, uint16_t* x_next,
                                      void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!x_next) return fail(MOE_ERR_INVALID_ARG, "moe_layer_forward_residual: x_next is NULL");
  return layer_forward(shape, x, M, w_router, router_bias, expert_to_slot, slots, topk_ids, topk_w,
                       y, cold_count, cold_routes, ws, ws_bytes, stream, nullptr, x_next);
}

moe_status moe_layer_forward_noalloc(const moe_shape* shape, const uint16_t* x, int32_t M,
                                     const uint16_t* w_router, const float* router_bias,
                                     const int32_t* expert_to_slot, const uint8_t* slots,
                                     int32_t* topk_ids, float* topk_w, float* y,
                                     int32_t* cold_count, int32_t* cold_routes, int32_t* errors,
                                     hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (M < 0) return fail(MOE_ERR_INVALID_ARG, "M = %d < 0", M);
  if ((size_t)M * shape->top_k > (size_t)kMaxRoutesPerCall)
    return fail(MOE_ERR_UNSUPPORTED, "M * top_k > %d", kMaxRoutesPerCall);
  const size_t need = ws_layout(shape->hidden, shape->inter, shape->n_experts, shape->top_k, M).total;
  if (need > kScratchBytes)
    return fail(MOE_ERR_WORKSPACE,
                "moe_layer_forward_noalloc: M=%d needs %zu bytes of workspace, more than the %zu of "
                "the static scratch; use moe_layer_forward with a workspace",
                M, need, kScratchBytes);
  if (errors && (reinterpret_cast<uintptr_t>(errors) & 3))
    return fail(MOE_ERR_INVALID_ARG, "moe_layer_forward_noalloc: errors must be 4-byte aligned");
  hipError_t e = hipSuccess;
  void* ws = static_scratch(&e);
  if (ws == nullptr) return hip_fail(e, "static scratch");
  st = layer_forward(shape, x, M, w_router, router_bias, expert_to_slot, slots, topk_ids, topk_w, y,
                     cold_count, cold_routes, ws, kScratchBytes, stream, nullptr, nullptr);
  if (st != MOE_OK) return st;
  if (errors) {
    e = launch_take_errors(static_cast<int32_t*>(ws) + kMetaErr, errors, stream);
    if (e != hipSuccess) return hip_fail(e, "error word launch");
  }
  return ok();
}

moe_status moe_layer_forward_marked(const moe_shape* shape, const uint16_t* x, int32_t M,
                                    const uint16_t* w_router, const float* router_bias,
                                    const int32_t* expert_to_slot, const uint8_t* slots,
                                    int32_t* topk_ids, float* topk_w, float* y,
                                    int32_t* cold_count, int32_t* cold_routes, void* ws,
                                    size_t ws_bytes, hipStream_t stream, const hipEvent_t* marks) {
  if (!marks || !marks[0] || !marks[1] || !marks[2] || !marks[3])
    return fail(MOE_ERR_INVALID_ARG, "moe_layer_forward_marked: four events are required");
  if (M <= 0) return fail(MOE_ERR_INVALID_ARG, "moe_layer_forward_marked: M must be positive");
  return layer_forward(shape, x, M, w_router, router_bias, expert_to_slot, slots, topk_ids, topk_w,
                       y, cold_count, cold_routes, ws, ws_bytes, stream, marks, nullptr);
}

moe_status moe_experts_gateup(const moe_shape* shape, const uint16_t* x, int32_t M,
                              const int32_t* topk_ids, const float* topk_w,
                              const int32_t* expert_to_slot, const uint8_t* slots, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  WsLayout W;
  st = check_ws(shape, M, ws, ws_bytes, &W);
  if (st != MOE_OK) return st;
  st = check_map(shape, expert_to_slot);
  if (st != MOE_OK) return st;
  if (M == 0) return ok();
  st = check_x_slots(x, slots);
  if (st != MOE_OK) return st;
  if (!topk_ids || !topk_w)
    return fail(MOE_ERR_INVALID_ARG, "moe_experts_gateup: topk_ids and topk_w are required");
  st = run_experts(shape, x, M, RouteSrc::kIds, nullptr, const_cast<int32_t*>(topk_ids),
                   const_cast<float*>(topk_w), expert_to_slot, slots, nullptr, nullptr, nullptr, ws,
                   W, true, false, stream);
  return st != MOE_OK ? st : ok();
}

moe_status moe_experts_down(const moe_shape* shape, int32_t M, const int32_t* topk_ids,
                            const float* topk_w, const int32_t* expert_to_slot,
                            const uint8_t* slots, float* y, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  WsLayout W;
  st = check_ws(shape, M, ws, ws_bytes, &W);
  if (st != MOE_OK) return st;
  st = check_map(shape, expert_to_slot);
  if (st != MOE_OK) return st;
  if (M == 0) return ok();
  if (!topk_ids || !topk_w || !y || !slots)
    return fail(MOE_ERR_INVALID_ARG, "moe_experts_down: topk_ids, topk_w, slots and y are required");
  if (reinterpret_cast<uintptr_t>(slots) & 255)
    return fail(MOE_ERR_INVALID_ARG, "slots must be 256-byte aligned");
  st = run_experts(shape, nullptr, M, RouteSrc::kIds, nullptr, const_cast<int32_t*>(topk_ids),
                   const_cast<float*>(topk_w), expert_to_slot, slots, y, nullptr, nullptr, ws, W,
                   false, true, stream);
  return st != MOE_OK ? st : ok();
}

moe_status moe_workspace_errors(void* ws, size_t ws_bytes, int32_t* flags, hipStream_t stream) {
  if (!ws) return fail(MOE_ERR_INVALID_ARG, "moe_workspace_errors: ws is required");
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0)
    return fail(MOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (ws_bytes < align256(4 * (size_t)kMetaWords))
    return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes holds no header", ws_bytes);
  if (reinterpret_cast<uintptr_t>(flags) & 3)
    return fail(MOE_ERR_INVALID_ARG, "moe_workspace_errors: flags must be 4-byte aligned");
  int32_t* word = static_cast<int32_t*>(ws) + kMetaErr;  // the header is at offset 0
  hipError_t e = launch_take_errors(word, flags, stream);
  if (e != hipSuccess) return hip_fail(e, "error word launch");
  return ok();
}

moe_status moe_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!src || !sink) return fail(MOE_ERR_INVALID_ARG, "moe_hbm_read_probe: src and sink are required");
  if ((reinterpret_cast<uintptr_t>(src) & 15) || (bytes & 15) || bytes == 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_hbm_read_probe: src 16-byte aligned, bytes a positive multiple of 16");
  hipError_t e = launch_stream_probe(src, bytes, sink, stream);
  if (e != hipSuccess) return hip_fail(e, "probe launch");
  return ok();
}

moe_status moe_residual_bf16(const uint16_t* x, const float* y, uint16_t* out, size_t n,
                             hipStream_t stream) {
  if (n == 0) return ok();
  if (!x || !y || !out) return fail(MOE_ERR_INVALID_ARG, "moe_residual_bf16: NULL pointer");
  hipError_t e = launch_residual(x, y, out, n, stream);
  if (e != hipSuccess) return hip_fail(e, "residual launch");
  return ok();
}

moe_status moe_slot_refill(const moe_shape* shape, uint8_t* slots, const uint8_t* host_bank,
                           const int32_t* experts, const int32_t* slot_ids, int32_t n,
                           hipStream_t copy_stream, hipEvent_t wait_before, hipEvent_t done) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (n < 0) return fail(MOE_ERR_INVALID_ARG, "n < 0");
  if (n > 0 && (!slots || !host_bank || !experts || !slot_ids))
    return fail(MOE_ERR_INVALID_ARG, "moe_slot_refill: slots, host_bank, experts, slot_ids are required");
  for (int i = 0; i < n; ++i) {
    if (experts[i] < 0 || experts[i] >= shape->n_experts)
      return fail(MOE_ERR_INVALID_ARG, "refill %d: expert %d out of range", i, experts[i]);
    if (slot_ids[i] < 0 || slot_ids[i] >= shape->n_slots)
      return fail(MOE_ERR_INVALID_ARG, "refill %d: slot %d out of range", i, slot_ids[i]);
    for (int j = 0; j < i; ++j)
      if (slot_ids[j] == slot_ids[i])
        return fail(MOE_ERR_INVALID_ARG, "refill: slot %d written twice", slot_ids[i]);
  }
  const size_t img = expert_image_bytes(shape);
  hipError_t e;
  if (wait_before) {
    e = hipStreamWaitEvent(copy_stream, wait_before, 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  }
  for (int i = 0; i < n; ++i) {
    e = hipMemcpyAsync(slots + (size_t)slot_ids[i] * img, host_bank + (size_t)experts[i] * img, img,
                       hipMemcpyHostToDevice, copy_stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
  }
  if (done) {
    e = hipEventRecord(done, copy_stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  return ok();
}

}  // extern "C"
