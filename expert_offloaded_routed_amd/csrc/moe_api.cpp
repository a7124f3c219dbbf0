// Host side of the libmoe C ABI: argument validation, workspace layout, kernel launches,
// expert image packing and slot refills.  See include/moe.h for the contract of each call.
#include <hip/hip_runtime_api.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "moe.h"
#include "moe_internal.h"

namespace moe {
hipError_t launch_fill_u32(unsigned* p, int n, unsigned v, hipStream_t s);
hipError_t launch_router(const uint16_t* x, int M, const uint16_t* wr, const float* bias, int E,
                         int H, int k, float* logits, unsigned* ticket, int32_t* ids, float* w,
                         hipStream_t s);
hipError_t launch_bucket(const int32_t* ids, int Mk, int E, int S, const int32_t* e2s,
                         int32_t* route_slot, int32_t* ws_perm, int32_t* meta, int32_t* dist_expert,
                         int32_t* dist_slot, int32_t* dist_off, int32_t* dist_cnt, int nd_max,
                         int32_t* cold_list, int32_t* u_counts, int32_t* u_offsets,
                         int32_t* u_perm, int32_t* u_cold_count, int32_t* u_cold_routes,
                         hipStream_t s);
hipError_t launch_gateup(const uint16_t* x, int M, int H, int I, int E, int k,
                         const uint8_t* slots, const ImageLayout& L, const int32_t* meta,
                         const int32_t* dist_slot, const int32_t* dist_off, const int32_t* dist_cnt,
                         const int32_t* perm, uint16_t* hbuf, hipStream_t s);
hipError_t launch_down(int M, int H, int I, int E, int k, const uint8_t* slots,
                       const ImageLayout& L, const int32_t* meta, const int32_t* dist_slot,
                       const int32_t* dist_off, const int32_t* dist_cnt, const int32_t* perm,
                       const int32_t* route_slot, const uint16_t* hbuf, const float* topk_w,
                       float* pdn, unsigned* tickets, float* y, hipStream_t s);

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
  if (s->n_experts > kMaxExperts)
    return fail(MOE_ERR_UNSUPPORTED, "n_experts %d > %d", s->n_experts, kMaxExperts);
  if (s->top_k > kMaxTopK || s->top_k > s->n_experts)
    return fail(MOE_ERR_UNSUPPORTED, "top_k %d must be <= min(n_experts, %d)", s->top_k, kMaxTopK);
  return MOE_OK;
}

static moe_status hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

static moe_status check_ws(const moe_shape* s, int M, void* ws, size_t ws_bytes, WsLayout* W) {
  if (M < 0) return fail(MOE_ERR_INVALID_ARG, "M = %d < 0", M);
  if ((size_t)M * s->top_k > (size_t)1 << 24) return fail(MOE_ERR_UNSUPPORTED, "M*k too large");
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

// Large-M token batches reuse the bucketing kernel's single workgroup; bound its work.
constexpr int kMaxRoutesPerCall = 1 << 20;

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_expert_image_bytes(const moe_shape* shape, size_t* bytes) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = image_layout(shape->hidden, shape->inter).image_bytes;
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

moe_status moe_workspace_init(const moe_shape* shape, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  WsLayout W;
  st = check_ws(shape, 0, ws, ws_bytes, &W);
  if (st != MOE_OK) return st;
  hipError_t e = launch_fill_u32(at<unsigned>(ws, 0), (int)(W.counters_end / 4), 0u, stream);
  if (e != hipSuccess) return hip_fail(e, "fill kernel");
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
  hipError_t e = launch_router(x, M, w_router, router_bias, shape->n_experts, shape->hidden,
                               shape->top_k, at<float>(ws, W.logits), at<unsigned>(ws, W.route_ticket),
                               topk_ids, topk_w, stream);
  if (e != hipSuccess) return hip_fail(e, "router launch");
  return ok();
}

static moe_status bucket_common(const moe_shape* shape, const int32_t* topk_ids, int32_t M,
                                const int32_t* e2s, int32_t* counts, int32_t* offsets,
                                int32_t* perm, int32_t* cold_count, int32_t* cold_routes,
                                void* ws, const WsLayout& W, hipStream_t stream) {
  if (!e2s && shape->n_experts > shape->n_slots)
    return fail(MOE_ERR_INVALID_ARG, "identity expert_to_slot needs n_slots >= n_experts");
  const int Mk = M * shape->top_k;
  if (Mk > kMaxRoutesPerCall) return fail(MOE_ERR_UNSUPPORTED, "M * top_k > %d", kMaxRoutesPerCall);
  const int nd_max = Mk < shape->n_experts ? Mk : shape->n_experts;
  hipError_t e = launch_bucket(topk_ids, Mk, shape->n_experts, shape->n_slots, e2s,
                               at<int32_t>(ws, W.route_slot), at<int32_t>(ws, W.perm),
                               at<int32_t>(ws, W.meta), at<int32_t>(ws, W.dist_expert),
                               at<int32_t>(ws, W.dist_slot), at<int32_t>(ws, W.dist_off),
                               at<int32_t>(ws, W.dist_cnt), nd_max, at<int32_t>(ws, W.cold_list),
                               counts, offsets, perm, cold_count, cold_routes, stream);
  if (e != hipSuccess) return hip_fail(e, "bucket launch");
  return MOE_OK;
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
  st = bucket_common(shape, topk_ids, M, expert_to_slot, counts, offsets, perm, cold_count,
                     cold_routes, ws, W, stream);
  if (st != MOE_OK) return st;
  return ok();
}

static moe_status check_expert_args(const moe_shape* shape, const uint16_t* x, int32_t M,
                                    const uint8_t* slots, void* ws, size_t ws_bytes, WsLayout* W) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  st = check_ws(shape, M, ws, ws_bytes, W);
  if (st != MOE_OK) return st;
  if (M > 0 && (!x || !slots)) return fail(MOE_ERR_INVALID_ARG, "x and slots are required");
  if ((reinterpret_cast<uintptr_t>(x) & 15) || (reinterpret_cast<uintptr_t>(slots) & 255))
    return fail(MOE_ERR_INVALID_ARG, "x must be 16-byte and slots 256-byte aligned");
  return MOE_OK;
}

static moe_status gateup_common(const moe_shape* shape, const uint16_t* x, int32_t M,
                                const uint8_t* slots, void* ws, const WsLayout& W,
                                hipStream_t stream) {
  const ImageLayout L = image_layout(shape->hidden, shape->inter);
  hipError_t e = launch_gateup(x, M, shape->hidden, shape->inter, shape->n_experts, shape->top_k,
                               slots, L, at<int32_t>(ws, W.meta), at<int32_t>(ws, W.dist_slot),
                               at<int32_t>(ws, W.dist_off), at<int32_t>(ws, W.dist_cnt),
                               at<int32_t>(ws, W.perm), at<uint16_t>(ws, W.hbuf), stream);
  if (e != hipSuccess) return hip_fail(e, "gate/up launch");
  return MOE_OK;
}

static moe_status down_common(const moe_shape* shape, int32_t M, const float* topk_w,
                              const uint8_t* slots, float* y, void* ws, const WsLayout& W,
                              hipStream_t stream) {
  const ImageLayout L = image_layout(shape->hidden, shape->inter);
  hipError_t e = launch_down(M, shape->hidden, shape->inter, shape->n_experts, shape->top_k, slots, L,
                             at<int32_t>(ws, W.meta), at<int32_t>(ws, W.dist_slot),
                             at<int32_t>(ws, W.dist_off), at<int32_t>(ws, W.dist_cnt),
                             at<int32_t>(ws, W.perm), at<int32_t>(ws, W.route_slot),
                             at<uint16_t>(ws, W.hbuf), topk_w, at<float>(ws, W.pdn),
                             at<unsigned>(ws, W.dn_tickets), y, stream);
  if (e != hipSuccess) return hip_fail(e, "down launch");
  return MOE_OK;
}

moe_status moe_experts_forward(const moe_shape* shape, const uint16_t* x, int32_t M,
                               const int32_t* topk_ids, const float* topk_w,
                               const int32_t* expert_to_slot, const uint8_t* slots, float* y,
                               int32_t* cold_count, int32_t* cold_routes, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  WsLayout W;
  moe_status st = check_expert_args(shape, x, M, slots, ws, ws_bytes, &W);
  if (st != MOE_OK) return st;
  if (M > 0 && (!topk_ids || !topk_w || !y))
    return fail(MOE_ERR_INVALID_ARG, "moe_experts_forward: topk_ids, topk_w and y are required");
  st = bucket_common(shape, topk_ids, M, expert_to_slot, nullptr, nullptr, nullptr, cold_count,
                     cold_routes, ws, W, stream);
  if (st != MOE_OK) return st;
  if (M == 0) return ok();
  st = gateup_common(shape, x, M, slots, ws, W, stream);
  if (st != MOE_OK) return st;
  st = down_common(shape, M, topk_w, slots, y, ws, W, stream);
  if (st != MOE_OK) return st;
  return ok();
}

moe_status moe_experts_gateup(const moe_shape* shape, const uint16_t* x, int32_t M,
                              const uint8_t* slots, void* ws, size_t ws_bytes, hipStream_t stream) {
  WsLayout W;
  moe_status st = check_expert_args(shape, x, M, slots, ws, ws_bytes, &W);
  if (st != MOE_OK) return st;
  if (M == 0) return ok();
  st = gateup_common(shape, x, M, slots, ws, W, stream);
  if (st != MOE_OK) return st;
  return ok();
}

moe_status moe_experts_down(const moe_shape* shape, int32_t M, const float* topk_w,
                            const uint8_t* slots, float* y, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  WsLayout W;
  moe_status st = check_expert_args(shape, nullptr, 0, slots, ws, ws_bytes, &W);
  if (st != MOE_OK) return st;
  st = check_ws(shape, M, ws, ws_bytes, &W);
  if (st != MOE_OK) return st;
  if (M == 0) return ok();
  if (!topk_w || !y || !slots)
    return fail(MOE_ERR_INVALID_ARG, "moe_experts_down: topk_w, slots and y are required");
  st = down_common(shape, M, topk_w, slots, y, ws, W, stream);
  if (st != MOE_OK) return st;
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
  const size_t img = image_layout(shape->hidden, shape->inter).image_bytes;
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
