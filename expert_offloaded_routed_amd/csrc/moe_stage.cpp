// Prefill with staged experts: the experts a call touches are copied into a staging slot array
// and the unchanged expert kernels run on it, in double-buffered passes when they do not all
// fit.  See moe_layer_forward_staged in moe.h.
#include <hip/hip_runtime_api.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "moe.h"
#include "moe_internal.h"

namespace moe {
moe_status fail(moe_status st, const char* fmt, ...);
moe_status ok();
moe_status check_shape(const moe_shape* s);
moe_status staged_route_and_count(const moe_shape* shape, const uint16_t* x, int32_t M,
                                  const uint16_t* w_router, const float* router_bias,
                                  int32_t* topk_ids, float* topk_w, int32_t* counts_dev, void* ws,
                                  size_t ws_bytes, hipStream_t stream);
moe_status staged_experts(const moe_shape* shape, const uint16_t* x, int32_t M,
                          const int32_t* topk_ids, const float* topk_w, const int32_t* e2s,
                          const uint8_t* slots, float* y, void* ws, size_t ws_bytes,
                          hipStream_t stream);

static moe_status hipf(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_layer_forward_staged(const moe_shape* shape, const uint16_t* x, int32_t M,
                                               const uint16_t* w_router, const float* router_bias,
                                               const uint8_t* host_bank, int32_t* topk_ids,
                                               float* topk_w, float* y, moe_prefill_staging* st,
                                               void* ws, size_t ws_bytes, hipStream_t stream,
                                               int32_t* n_touched, int32_t* n_passes) {
  moe_status rs = check_shape(shape);
  if (rs != MOE_OK) return rs;
  if (!st || !st->slots || st->n_slots < 1 || !st->counts_dev || !st->counts_host ||
      !st->maps_dev || !st->maps_host || !st->y_pass || !st->copy_stream || !st->ev_counts ||
      !st->ev_copied[0] || !st->ev_copied[1] || !st->ev_done[0] || !st->ev_done[1])
    return fail(MOE_ERR_INVALID_ARG, "moe_layer_forward_staged: incomplete staging");
  if (!host_bank || !y) return fail(MOE_ERR_INVALID_ARG, "moe_layer_forward_staged: host_bank and y are required");
  if (M < 0 || M > st->max_M)
    return fail(MOE_ERR_INVALID_ARG, "moe_layer_forward_staged: M = %d outside [0, %d]", M, st->max_M);
  if (reinterpret_cast<uintptr_t>(st->slots) & 255)
    return fail(MOE_ERR_INVALID_ARG, "staging slots must be 256-byte aligned");
  if (n_touched) *n_touched = 0;
  if (n_passes) *n_passes = 0;
  if (M == 0) return ok();
  const int E = shape->n_experts, H = shape->hidden;
  const size_t img = expert_image_bytes(shape);
  hipError_t e;
  // 1. routes and the route count of every expert (on the stream), then on the host
  rs = staged_route_and_count(shape, x, M, w_router, router_bias, topk_ids, topk_w, st->counts_dev,
                              ws, ws_bytes, stream);
  if (rs != MOE_OK) return rs;
  if ((e = hipMemcpyAsync(st->counts_host, st->counts_dev, sizeof(int32_t) * E,
                          hipMemcpyDeviceToHost, stream)) != hipSuccess)
    return hipf(e, "hipMemcpyAsync");
  if ((e = hipEventRecord(st->ev_counts, stream)) != hipSuccess) return hipf(e, "hipEventRecord");
  if ((e = hipEventSynchronize(st->ev_counts)) != hipSuccess) return hipf(e, "hipEventSynchronize");
  std::vector<int> touched;
  for (int ex = 0; ex < E; ++ex)
    if (st->counts_host[ex] > 0) touched.push_back(ex);
  const int nt = (int)touched.size();
  // 2. passes: every touched expert staged once, in ascending id.  All of them in one pass when
  // they fit; otherwise passes of half the staging slots, the copies of pass b + 1 (copy stream)
  // overlapping the expert kernels of pass b, each half reused once its pass is done.
  const int per = nt <= st->n_slots ? nt : st->n_slots / 2;
  if (per < 1) return fail(MOE_ERR_INVALID_ARG, "staging needs at least 2 slots for %d experts", nt);
  const int np = (nt + per - 1) / per;
  // the staging's maps of the last call may still be in flight: wait for its passes
  for (int b = 0; b < 2; ++b)
    if (st->pending[b]) {
      if ((e = hipEventSynchronize(st->ev_done[b])) != hipSuccess) return hipf(e, "hipEventSynchronize");
      st->pending[b] = 0;
    }
  for (int p = 0; p < np; ++p) {
    const int buf = np == 1 ? 0 : p & 1;
    const int base = np == 1 ? 0 : buf * per;
    const int lo = p * per, hi = std::min(nt, lo + per);
    if (p >= 2) {  // this half's previous pass must be done before it is overwritten
      if ((e = hipStreamWaitEvent(st->copy_stream, st->ev_done[buf], 0)) != hipSuccess)
        return hipf(e, "hipStreamWaitEvent");
      if ((e = hipEventSynchronize(st->ev_done[buf])) != hipSuccess)  // (its host map too)
        return hipf(e, "hipEventSynchronize");
    }
    int32_t* map_h = st->maps_host + (size_t)buf * E;
    int32_t* map_d = st->maps_dev + (size_t)buf * E;
    for (int ex = 0; ex < E; ++ex) map_h[ex] = -1;
    for (int i = lo; i < hi; ++i) {
      const int ex = touched[i];
      map_h[ex] = base + (i - lo);
      if ((e = hipMemcpyAsync(st->slots + (size_t)(base + i - lo) * img, host_bank + (size_t)ex * img,
                              img, hipMemcpyHostToDevice, st->copy_stream)) != hipSuccess)
        return hipf(e, "hipMemcpyAsync");
    }
    if ((e = hipEventRecord(st->ev_copied[buf], st->copy_stream)) != hipSuccess) return hipf(e, "hipEventRecord");
    if ((e = hipStreamWaitEvent(stream, st->ev_copied[buf], 0)) != hipSuccess) return hipf(e, "hipStreamWaitEvent");
    if ((e = hipMemcpyAsync(map_d, map_h, sizeof(int32_t) * E, hipMemcpyHostToDevice, stream)) != hipSuccess)
      return hipf(e, "hipMemcpyAsync");
    // pass 0 forms y; later passes form their hot-only part and add it
    float* out = p == 0 ? y : st->y_pass;
    moe_shape ss = *shape;
    ss.n_slots = st->n_slots;  // the staging slots
    rs = staged_experts(&ss, x, M, topk_ids, topk_w, map_d, st->slots, out, ws, ws_bytes, stream);
    if (rs != MOE_OK) return rs;
    if (p > 0 && (e = launch_add_f32(y, st->y_pass, (size_t)M * H, stream)) != hipSuccess)
      return hipf(e, "add launch");
    if ((e = hipEventRecord(st->ev_done[buf], stream)) != hipSuccess) return hipf(e, "hipEventRecord");
    st->pending[buf] = 1;
  }
  if (n_touched) *n_touched = nt;
  if (n_passes) *n_passes = np;
  return ok();
}
