// Cold routes on the host cores: the CPU half of the hybrid layer.  Routes whose expert has no
// GPU slot are skipped by the GPU kernels; here they are computed from the pinned host bank (the
// same expert images the slots hold) while the GPU runs the hot experts, and their weighted sum
// is added to the GPU's output.  See moe_cold_forward_host / moe_layer_forward_hybrid in moe.h.
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <thread>
#include <vector>

#include "moe.h"
#include "moe_internal.h"

namespace moe {
moe_status fail(moe_status st, const char* fmt, ...);
moe_status ok();
moe_status check_shape(const moe_shape* s);
moe_status layer_route_and_hot(const moe_shape* shape, const uint16_t* x, int32_t M,
                               const uint16_t* w_router, const float* router_bias,
                               const int32_t* expert_to_slot, const uint8_t* slots,
                               int32_t* topk_ids, float* topk_w, float* y, void* ws,
                               size_t ws_bytes, hipStream_t stream,
                               const moe_hybrid_staging* staging);

namespace {

// E2M1 magnitudes by the 3 low bits of a code (OCP MX v1.0: exponent bits 2..1, mantissa bit 0).
constexpr float kE2M1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

inline float e8m0(uint8_t x) { return x == 255 ? NAN : ldexpf(1.0f, (int)x - 127); }

inline float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// fp32 -> bf16 bits, round to nearest even (NaN -> 0x7FC0).
inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Dot of one 32-element MXFP4 block (16 code bytes, low nibble first) with 32 activations.
inline float block_dot(const uint8_t* codes, const float* a) {
  float s = 0.0f;
  for (int c = 0; c < 16; ++c) {
    const uint8_t v = codes[c];
    const uint8_t lo = v & 0xF, hi = v >> 4;
    const float wl = (lo & 8) ? -kE2M1[lo & 7] : kE2M1[lo & 7];
    const float wh = (hi & 8) ? -kE2M1[hi & 7] : kE2M1[hi & 7];
    s += wl * a[2 * c] + wh * a[2 * c + 1];
  }
  return s;
}

// Row `row` of the gate (up = false) or up matrix, dotted with x [H], from an expert image.
float gu_row_dot(const uint8_t* img, const ImageLayout& L, int row, bool up, const float* x) {
  const int t = row / 32, lane = (row % 32) + (up ? 32 : 0);
  const uint8_t* tb = img + (size_t)t * L.gu_tile_bytes;
  const uint8_t* scl = tb + (size_t)L.nb_h * 1024;
  float acc = 0.0f;
  for (int b = 0; b < L.nb_h; ++b) {
    const float sc = e8m0(scl[(size_t)(b >> 2) * 256 + lane * 4 + (b & 3)]);
    acc += sc * block_dot(tb + (size_t)b * 1024 + lane * 16, x + 32 * b);
  }
  return acc;
}

// Row `row` of the down matrix, dotted with h [I].
float dn_row_dot(const uint8_t* img, const ImageLayout& L, int row, const float* h) {
  const uint8_t* tb = img + L.gu_bytes + (size_t)(row / 16) * L.dn_tile_bytes;
  float acc = 0.0f;
  for (int b = 0; b < L.nb_i; ++b) {
    const int s = b / 4, lane = row % 16 + 16 * (b % 4);
    const uint8_t* codes = tb + (size_t)s * 1024 + lane * 16;  // (a partial last step also starts at s * 1024)
    const float sc = e8m0(tb[L.dn_code_bytes + (size_t)(s >> 2) * 256 + lane * 4 + (s & 3)]);
    acc += sc * block_dot(codes, h + 32 * b);
  }
  return acc;
}

// Runs f(i) for i in [0, n) on up to `threads` threads (the calling thread included).
template <typename F>
void parallel_for(int n, int threads, F f) {
  threads = std::max(1, std::min(threads, n));
  if (threads == 1) {
    for (int i = 0; i < n; ++i) f(i);
    return;
  }
  std::atomic<int> next{0};
  auto work = [&]() {
    for (int i = next.fetch_add(1); i < n; i = next.fetch_add(1)) f(i);
  };
  std::vector<std::thread> pool;
  pool.reserve(threads - 1);
  for (int t = 1; t < threads; ++t) pool.emplace_back(work);
  work();
  for (auto& th : pool) th.join();
}

constexpr int kRowChunk = 64;  // rows per work item

}  // namespace

moe_status cold_forward_host(const moe_shape* shape, const uint8_t* bank, const uint16_t* x,
                             int M, const int32_t* ids, const float* w, const int32_t* e2s,
                             float* y_cold, int n_threads) {
  const int H = shape->hidden, I = shape->inter, E = shape->n_experts, k = shape->top_k;
  const ImageLayout L = image_layout(H, I);
  memset(y_cold, 0, sizeof(float) * (size_t)M * H);
  struct Route {
    int m, j, e;
  };
  std::vector<Route> cold;
  for (int m = 0; m < M; ++m)
    for (int j = 0; j < k; ++j) {
      const int e = ids[m * k + j];
      if (e < 0 || e >= E) continue;  // not a route the GPU computes either (flagged there)
      const int s = e2s ? e2s[e] : e;
      if (s < 0 || s >= shape->n_slots) cold.push_back({m, j, e});
    }
  if (cold.empty()) return ok();
  if (n_threads <= 0) n_threads = (int)std::max(1u, std::thread::hardware_concurrency());
  // activations as fp32 (exact)
  std::vector<float> xf((size_t)M * H);
  for (size_t i = 0; i < xf.size(); ++i) xf[i] = bf16_to_f32(x[i]);
  // 1. h = bf16(silu(g) * u) of every cold route, row chunks in parallel
  const int nr = (int)cold.size();
  const int gchunks = (I + kRowChunk - 1) / kRowChunk;
  std::vector<float> h((size_t)nr * I);
  parallel_for(nr * gchunks, n_threads, [&](int it) {
    const int r = it / gchunks, c = it % gchunks;
    const uint8_t* img = bank + (size_t)cold[r].e * L.image_bytes;
    const float* xr = xf.data() + (size_t)cold[r].m * H;
    for (int i = c * kRowChunk; i < std::min(I, (c + 1) * kRowChunk); ++i) {
      const float g = gu_row_dot(img, L, i, false, xr);
      const float u = gu_row_dot(img, L, i, true, xr);
      const float a = g / (1.0f + expf(-g)) * u;
      h[(size_t)r * I + i] = bf16_to_f32(f32_to_bf16(a));
    }
  });
  // 2. down rows and the weighted sum over each token's cold routes in ascending j
  std::vector<int> first(M + 1, 0);  // cold routes of token m: [first[m], first[m + 1])
  for (const Route& c : cold) first[c.m + 1]++;
  for (int m = 0; m < M; ++m) first[m + 1] += first[m];
  const int dchunks = (H + kRowChunk - 1) / kRowChunk;
  parallel_for(M * dchunks, n_threads, [&](int it) {
    const int m = it / dchunks, c = it % dchunks;
    for (int row = c * kRowChunk; row < std::min(H, (c + 1) * kRowChunk); ++row) {
      float acc = 0.0f;
      for (int r = first[m]; r < first[m + 1]; ++r) {  // (routes were listed by m, then j)
        const uint8_t* img = bank + (size_t)cold[r].e * L.image_bytes;
        acc += w[cold[r].m * k + cold[r].j] * dn_row_dot(img, L, row, h.data() + (size_t)r * I);
      }
      y_cold[(size_t)m * H + row] = acc;
    }
  });
  return ok();
}

}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_cold_forward_host(const moe_shape* shape, const uint8_t* host_bank,
                                 const uint16_t* x, int32_t M, const int32_t* topk_ids,
                                 const float* topk_w, const int32_t* expert_to_slot,
                                 float* y_cold, int32_t n_threads) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (shape->format != MOE_FORMAT_MXFP4)
    return fail(MOE_ERR_UNSUPPORTED, "the host expert path reads MXFP4 images only (format %d)",
                shape->format);
  if (M < 0) return fail(MOE_ERR_INVALID_ARG, "M < 0");
  if (M == 0) return ok();
  if (!host_bank || !x || !topk_ids || !topk_w || !y_cold)
    return fail(MOE_ERR_INVALID_ARG, "moe_cold_forward_host: NULL pointer");
  return cold_forward_host(shape, host_bank, x, M, topk_ids, topk_w, expert_to_slot, y_cold,
                           n_threads);
}

moe_status moe_layer_forward_hybrid(const moe_shape* shape, const uint16_t* x, int32_t M,
                                    const uint16_t* w_router, const float* router_bias,
                                    const int32_t* expert_to_slot,
                                    const int32_t* expert_to_slot_host, const uint8_t* slots,
                                    const uint8_t* host_bank, int32_t* topk_ids, float* topk_w,
                                    float* y, moe_hybrid_staging* staging, int32_t n_threads,
                                    void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (shape->format != MOE_FORMAT_MXFP4)
    return fail(MOE_ERR_UNSUPPORTED, "the host expert path reads MXFP4 images only (format %d)",
                shape->format);
  if (!staging || !staging->x || !staging->ids || !staging->w || !staging->y_cold ||
      !staging->y_cold_dev || !staging->routed || !staging->added)
    return fail(MOE_ERR_INVALID_ARG, "moe_layer_forward_hybrid: incomplete staging");
  if (!expert_to_slot || !expert_to_slot_host || !host_bank)
    return fail(MOE_ERR_INVALID_ARG,
                "moe_layer_forward_hybrid: expert_to_slot (device and host) and host_bank are required");
  if (M < 0 || M > staging->max_M)
    return fail(MOE_ERR_INVALID_ARG, "moe_layer_forward_hybrid: M = %d outside [0, %d]", M,
                staging->max_M);
  if (M == 0) return ok();
  const size_t H = (size_t)shape->hidden, k = (size_t)shape->top_k;
  hipError_t e;
  // the previous call's upload of y_cold has left the staging buffer
  if (staging->pending) {
    e = hipEventSynchronize(staging->added);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipEventSynchronize: %s", hipGetErrorString(e));
    staging->pending = 0;
  }
  // 1. route, stage x, ids and weights to the host, 2. the hot experts (all on the stream)
  st = layer_route_and_hot(shape, x, M, w_router, router_bias, expert_to_slot, slots, topk_ids,
                           topk_w, y, ws, ws_bytes, stream, staging);
  if (st != MOE_OK) return st;
  // 3. the cold routes on the host cores while the GPU runs the hot experts
  e = hipEventSynchronize(staging->routed);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipEventSynchronize: %s", hipGetErrorString(e));
  st = cold_forward_host(shape, host_bank, staging->x, M, staging->ids, staging->w,
                         expert_to_slot_host, staging->y_cold, n_threads);
  if (st != MOE_OK) return st;
  // 4. y += y_cold on the stream, behind the hot experts
  e = hipMemcpyAsync(staging->y_cold_dev, staging->y_cold, sizeof(float) * M * H,
                     hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
  e = launch_add_f32(y, staging->y_cold_dev, (size_t)M * H, stream);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "add launch: %s", hipGetErrorString(e));
  e = hipEventRecord(staging->added, stream);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  staging->pending = 1;
  (void)k;
  return ok();
}

}  // extern "C"
