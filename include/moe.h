/*
 * moe.h -- C ABI of libmoe: one routed Mixture-of-Experts layer whose experts live in a GPU
 * slot cache backed by pinned host memory, for AMD Instinct MI355X (gfx950).
 *
 * The method (page title, section):
 *   [MoE expert offload]  xinfer documentation "MoE expert offload": intro, "How it works",
 *                         "Options", "Supported".
 *   [ninfer v0.4.0]       "NInfer-Offload v0.4.0 -- expert cache: faster Flash-Next decode",
 *                         section "New".
 *   [ORT hybrid PR]       "[CUDA/CPU] Add hybrid GPU/CPU expert offload for MoEPacked
 *                         block-packed weights", sections "Key Changes" and "Table A".
 *   [tinyserve]           "tinyserve -- MoE Expert Offloading for Consumer GPUs", sections
 *                         "How it works" and "Configuration".
 *   [OCP MX v1.0]         OCP Microscaling Formats Specification v1.0 (MXFP4 = 32-element
 *                         blocks of FP4 E2M1 values sharing one E8M0 scale).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked [host].  The caller allocates and owns every
 *     buffer, stream and event; the library allocates no device memory.
 *   - GPU calls only enqueue work on the given stream (asynchronous); none synchronises the
 *     device.  Argument and shape errors are detected on the host before anything is enqueued
 *     and leave every output untouched.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Every call returns a moe_status; moe_last_error() gives a message for the calling thread.
 *   - Supported shapes: hidden % 64 == 0, inter % 32 == 0, 1 <= top_k <= min(n_experts, 32),
 *     n_experts <= 1024, hidden <= 8192, inter <= 4096, n_slots >= 1.  x, w_router: 16-byte aligned;
 *     slot arrays and workspaces: 256-byte aligned.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, bad size, out-of-range value */
  MOE_ERR_UNSUPPORTED = -2, /* shape outside the supported set above */
  MOE_ERR_HIP = -3,         /* a HIP runtime call failed (message has the HIP error) */
  MOE_ERR_WORKSPACE = -4,   /* workspace smaller than moe_workspace_size() */
  MOE_ERR_STATE = -5        /* cache object used inconsistently (e.g. step not increasing) */
} moe_status;

/* Expert weight formats [MoE expert offload, "Supported": besides MXFP4, unquantised bf16,
 * block FP8 and NVFP4 experts run through the same generic slot path].  Readings of the three
 * that the pages name but do not define (the usual published definitions):
 *   MOE_FORMAT_BF16      bf16 weights, no scales;
 *   MOE_FORMAT_FP8_BLOCK OCP FP8 E4M3 weights (bias 7, subnormals, max 448, S.1111.111 = NaN)
 *                        times one fp32 scale per 128 x 128 block of the [N, K] matrix;
 *   MOE_FORMAT_NVFP4     E2M1 weights (as in MXFP4) times one E4M3 scale per 16 elements along
 *                        K, times one fp32 scale of the whole matrix. */
typedef enum {
  MOE_FORMAT_MXFP4 = 0,
  MOE_FORMAT_BF16 = 1,
  MOE_FORMAT_FP8_BLOCK = 2,
  MOE_FORMAT_NVFP4 = 3
} moe_format;

/* Layer shape.  hidden = H, inter = I (per-expert intermediate size), n_experts = E,
 * top_k = k, n_slots = S (GPU slots; S >= E means every expert can be resident), format = the
 * experts' moe_format (0 = MXFP4, so a zero-initialised field keeps MXFP4). */
typedef struct {
  int32_t hidden;
  int32_t inter;
  int32_t n_experts;
  int32_t top_k;
  int32_t n_slots;
  int32_t format;
} moe_shape;

/* ---------------------------------------------------------------------------------------
 * Expert images.  One expert = gate [I,H], up [I,H] and down [H,I] MXFP4 matrices
 * [OCP MX v1.0].  Canonical layout (the caller's): row-major [N,K] with blocks of 32 along K;
 * codes [N][K/2] with element 2c in the low nibble of byte c and 2c+1 in the high nibble;
 * scales [N][K/32] as E8M0 bytes.  The library keeps each expert as one contiguous "image"
 * in its own kernel layout, so that a GPU slot holds exactly one image and a refill from the
 * pinned host bank is one copy [MoE expert offload, "How it works": the GEMMs read
 * [num_slots, N, K] slot tensors].  Slot s of a slot array starts at s * image_bytes.
 * --------------------------------------------------------------------------------------- */

/* Bytes of one expert image (a multiple of 256).  [host] out. */
moe_status moe_expert_image_bytes(const moe_shape* shape, size_t* bytes);

/* Convert one expert from the canonical layout to its image.  All pointers [host]; the
 * image buffer must hold moe_expert_image_bytes() bytes.  Pure host code.
 * For the other formats the six pointers are each matrix's elements and scales, row-major:
 *   MOE_FORMAT_BF16:      *_codes = bf16 [N][K] (uint16 bit patterns); *_scales unused (NULL);
 *   MOE_FORMAT_FP8_BLOCK: *_codes = E4M3 bytes [N][K]; *_scales = fp32 [ceil(N/128)][ceil(K/128)];
 *   MOE_FORMAT_NVFP4:     *_codes = E2M1 [N][K/2] (element 2c in the low nibble of byte c);
 *                         *_scales = 4 + N*K/16 bytes: the fp32 matrix scale, then E4M3 bytes
 *                         [N][K/16].
 * Their image is these six arrays in that order, each at a multiple of 256 bytes. */
moe_status moe_pack_expert(const moe_shape* shape,
                           const uint8_t* gate_codes, const uint8_t* gate_scales,
                           const uint8_t* up_codes, const uint8_t* up_scales,
                           const uint8_t* down_codes, const uint8_t* down_scales,
                           uint8_t* image);

/* Inverse of moe_pack_expert (round-trip check, debugging).  All pointers [host]. */
moe_status moe_unpack_expert(const moe_shape* shape, const uint8_t* image,
                             uint8_t* gate_codes, uint8_t* gate_scales,
                             uint8_t* up_codes, uint8_t* up_scales,
                             uint8_t* down_codes, uint8_t* down_scales);

/* ---------------------------------------------------------------------------------------
 * Workspace.  One device buffer (256-byte aligned) used by moe_route, moe_bucket_routes,
 * moe_experts_forward and moe_layer_forward for calls with M <= max_M.  It carries logits,
 * route buckets, h and partial sums from one kernel of a call to the next, and in a fixed
 * header the device error word (moe_workspace_errors) and the state the one-token fused kernel
 * keeps between calls.  Fill it with zeros once before its first use (any later call keeps the
 * header consistent; the rest needs no initialisation).  Calls sharing a workspace must be
 * ordered on one stream; concurrent calls need separate workspaces.
 * --------------------------------------------------------------------------------------- */
moe_status moe_workspace_size(const moe_shape* shape, int32_t max_M, size_t* bytes /*[host]*/);

/* Device error flags (bits of the workspace error word). */
enum {
  MOE_DEVERR_BAD_ID = 1,   /* a route's expert id lies outside [0, E): the route was treated as cold */
  MOE_DEVERR_BAD_SLOT = 2, /* expert_to_slot maps a routed expert outside [-1, S): treated as cold */
  MOE_DEVERR_HANDOFF = 4   /* a workgroup could not collect what other workgroups of the same
                              launch hand over by value in its bounded wait (the one-token fused
                              kernel's h; the few-token down GEMV's rows when two workgroups share
                              a row tile): the y rows (and x_next rows) it forms are NaN, never
                              silently wrong; when the workgroup that advances the call counter
                              is the one that ran out, the workspace is poisoned (every later
                              call on it flags and writes NaN) until it is zero-filled.  Both rely
                              on all workgroups of the launch being resident together; kernels
                              of other streams that hold compute units can break that */
};

/* Take the device error word of a workspace: copy it to *flags and clear it, asynchronously
 * on stream (one small kernel, so it can be captured in a HIP graph) [ORT hybrid PR, "Key
 * Changes": the hot-expert kernel takes an optional expert_to_slot map and skips routes whose
 * slot is negative].  Routes whose id or slot lies outside that map's contract are skipped like
 * cold ones and reported here instead of being read out of bounds.  The word accumulates: every
 * call on the workspace ORs in the MOE_DEVERR_* flags it raises, so *flags holds those of every
 * call since the last moe_workspace_errors (0 = none).
 * ws: the workspace (256-byte aligned, ws_bytes >= 256); flags: one int32 in device memory or
 * in pinned host memory, 4-byte aligned, or NULL (clear only).  Read it after the stream has
 * passed the call. */
moe_status moe_workspace_errors(void* ws, size_t ws_bytes, int32_t* flags, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Router [ninfer v0.4.0, "New": the router is no longer a single thread block;
 * ORT hybrid PR, "Notes" 2: one fp32-accumulating router contract for any token count].
 *   logits[m,e] = sum_h x[m,h] * W_r[e,h] + bias[e]   (bf16 inputs, fp32 accumulation)
 *   then per token: the k largest logits (ties to the lower expert id), ordered by value
 *   descending, and their softmax, which equals softmax over all E followed by top-k and
 *   renormalisation.
 * x [M,H] bf16; w_router [E,H] bf16 row-major; router_bias [E] fp32 or NULL (zero);
 * topk_ids [M,k] int32 and topk_w [M,k] fp32 are written.  0 <= M <= max_M of the workspace;
 * M = 0 enqueues nothing.
 * --------------------------------------------------------------------------------------- */
moe_status moe_route(const moe_shape* shape, const uint16_t* x, int32_t M,
                     const uint16_t* w_router, const float* router_bias,
                     int32_t* topk_ids, float* topk_w,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Route resolve and bucketing [ORT hybrid PR, "Key Changes": expert_to_slot, slot < 0 is
 * cold; tinyserve, "How it works" item 6: group tokens by expert so that each expert is
 * loaded once per call].
 *   For each route r = m*k + j with expert e = topk_ids[r]:
 *     slot = expert_to_slot ? expert_to_slot[e] : e;  cold iff slot < 0.
 *   counts[e] = routes to e; offsets[e] = sum of counts below e (offsets[E] = M*k);
 *   perm[offsets[e] .. offsets[e+1]) = the routes of e (order inside a bucket unspecified);
 *   cold_count = number of cold routes; cold_routes = their r in ascending order.
 * expert_to_slot [E] int32 or NULL (identity, needs E <= S).  Routes with an id outside
 * [0,E) are cold and not bucketed; routes whose expert maps to a slot outside [-1,S) are
 * cold (and bucketed).  counts [E], offsets [E+1],
 * perm [M*k], cold_count [1], cold_routes [M*k] are written; any of them may be NULL.
 * moe_experts_forward runs this step itself; the entry point exposes it on its own.
 * --------------------------------------------------------------------------------------- */
moe_status moe_bucket_routes(const moe_shape* shape, const int32_t* topk_ids, int32_t M,
                             const int32_t* expert_to_slot,
                             int32_t* counts, int32_t* offsets, int32_t* perm,
                             int32_t* cold_count, int32_t* cold_routes,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Expert FFNs and combine over the slot cache [MoE expert offload, "How it works";
 * ORT hybrid PR, "Key Changes"; tinyserve, "How it works" item 2: fused dequant + matmul
 * on the native quantised weights, no bf16 weight copy].
 *   For every hot route r = (m, j) with expert e in slot s:
 *     g = Wg_e x_m, u = Wu_e x_m (fp32 accumulation over exactly decoded MXFP4 weights),
 *     h = bf16(silu(g) * u), d_r = Wd_e h.
 *   y[m] = sum over j = 0..k-1 of the hot routes, in ascending j, of topk_w[m,j] * d_(m,j).
 *   Cold routes are skipped and reported: y is the hot-only partial output.
 * x [M,H] bf16; topk_ids/topk_w [M,k]; expert_to_slot as in moe_bucket_routes;
 * slots = the device slot array (n_slots images); y [M,H] fp32 is overwritten (zeros for a
 * token whose routes are all cold); cold_count [1] / cold_routes [M*k] may be NULL.
 * Deterministic: the result does not depend on slot numbering, bucket order or timing.
 * Formats other than MXFP4 (shape->format) run generic kernels for every M, after the
 * bucketing kernel: gate/up decodes each 16-byte chunk of a weight row exactly to bf16 pairs,
 * dots them with x in fp32 and applies the chunk's scales to the chunk's sum (FP8 block: the
 * block scale; NVFP4: each 16-element scale times the matrix scale); down does the same over
 * h, then the combine above.  The one-token fused kernel and the grouped GEMM are MXFP4 only.
 * --------------------------------------------------------------------------------------- */
moe_status moe_experts_forward(const moe_shape* shape, const uint16_t* x, int32_t M,
                               const int32_t* topk_ids, const float* topk_w,
                               const int32_t* expert_to_slot, const uint8_t* slots,
                               float* y, int32_t* cold_count, int32_t* cold_routes,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Whole layer in one call: moe_route followed by moe_experts_forward.  For one token, or up to
 * 64 routes over at most 64 experts, the top-k, slot resolve and bucketing run inside the expert
 * kernels (three launches: router GEMV, gate/up, down + combine).  For one token (M = 1, top_k <= 16) of the MXFP4 shapes the
 * fused kernel is built for (moe_layer_launches reports it; GPT-OSS-20B's is one) gate/up and
 * down are one launch of one workgroup per compute unit, h handed from gate/up to down by value
 * through the workspace in words tagged with the call; for routers of at most 32 experts and
 * H <= 4096 the router runs inside that launch too (one launch in all), else before it (two);
 * the environment variable MOE_DECODE_UNFUSED=1, read once per process, keeps three.  Same
 * arguments and outputs as the two calls; the numerics are bitwise theirs, except on the
 * fused path, whose sums over K run in another order (agreement within 1e-4 relative L2);
 * topk_ids [M,k] and topk_w [M,k] are written too (bitwise on every path).
 * --------------------------------------------------------------------------------------- */
moe_status moe_layer_forward(const moe_shape* shape, const uint16_t* x, int32_t M,
                             const uint16_t* w_router, const float* router_bias,
                             const int32_t* expert_to_slot, const uint8_t* slots,
                             int32_t* topk_ids, float* topk_w, float* y,
                             int32_t* cold_count, int32_t* cold_routes,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_layer_forward with an event recorded on `stream` at each stage boundary, for timing the
 * stages of exactly the launches of a layer call: marks[0] before the router, marks[1] after
 * the route stage (router, plus the top-k / bucketing kernel when the call needs it), marks[2]
 * after the gate/up kernel, marks[3] after the down stage.  When gate/up and down are one
 * launch, marks[2] and marks[3] are both recorded after it.  marks: four events created by the
 * caller with timing enabled; M >= 1.  Results equal moe_layer_forward's. */
moe_status moe_layer_forward_marked(const moe_shape* shape, const uint16_t* x, int32_t M,
                                    const uint16_t* w_router, const float* router_bias,
                                    const int32_t* expert_to_slot, const uint8_t* slots,
                                    int32_t* topk_ids, float* topk_w, float* y,
                                    int32_t* cold_count, int32_t* cold_routes,
                                    void* ws, size_t ws_bytes, hipStream_t stream,
                                    const hipEvent_t* marks);

/* moe_layer_forward without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The workspace is a static array inside the library, one per GPU, of MOE_NOALLOC_SCRATCH_BYTES
 * (8 MiB), held until the process ends; the call allocates nothing and calls no allocating
 * routine.  A call whose workspace (moe_workspace_size for its M) exceeds that size is
 * rejected with MOE_ERR_WORKSPACE before anything is enqueued (the one-token decode and the
 * few-token calls fit; large prefills do not).  Every call on a GPU shares that GPU's array and
 * it keeps the last call's contents: calls that overlap on one GPU (other streams, other host
 * threads) race and must be ordered by the caller.  The first call on a device clears the array
 * synchronously, so it must not be made while a stream is being captured.
 * errors: one int32 (device or pinned host memory) or NULL: after the call's kernels the
 * array's device error word (MOE_DEVERR_*, see moe_workspace_errors) is copied there and
 * cleared.  Other arguments and results are those of moe_layer_forward, bitwise. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
moe_status moe_layer_forward_noalloc(const moe_shape* shape, const uint16_t* x, int32_t M,
                                     const uint16_t* w_router, const float* router_bias,
                                     const int32_t* expert_to_slot, const uint8_t* slots,
                                     int32_t* topk_ids, float* topk_w, float* y,
                                     int32_t* cold_count, int32_t* cold_routes, int32_t* errors,
                                     hipStream_t stream);

/* Number of kernel launches moe_layer_forward makes for M tokens of this shape: 1 or 2 when
 * gate/up and down run as one launch (router inside it, or before it), 3 for one token or up to
 * 64 routes over at most 64 experts, 4 for the other calls below 64 tokens and for the formats
 * other than MXFP4, 5 on the grouped-GEMM path (M >= 64), 1 for M = 0.  For callers that budget graph nodes or time stages.  Writes *n; no
 * device work. */
moe_status moe_layer_launches(const moe_shape* shape, int32_t M, int32_t* n);

/* The two kernel stages of moe_experts_forward, on their own (for timing a stage or for
 * callers that interleave other work).  Arguments as in moe_experts_forward.
 *   moe_experts_gateup: h = bf16(silu(Wg x) * (Wu x)) for every hot route, kept in the
 *                       workspace [tinyserve, "How it works" item 2: gate and up fused here].
 *   moe_experts_down:   y = ordered sum over hot routes of topk_w * (Wd h), as in
 *                       moe_experts_forward; needs the h and the route table that the last
 *                       moe_experts_gateup (or moe_experts_forward) with the same routes and
 *                       expert_to_slot left in this workspace.
 * moe_experts_gateup + moe_experts_down == moe_experts_forward (without the cold report). */
moe_status moe_experts_gateup(const moe_shape* shape, const uint16_t* x, int32_t M,
                              const int32_t* topk_ids, const float* topk_w,
                              const int32_t* expert_to_slot, const uint8_t* slots,
                              void* ws, size_t ws_bytes, hipStream_t stream);
moe_status moe_experts_down(const moe_shape* shape, int32_t M, const int32_t* topk_ids,
                            const float* topk_w, const int32_t* expert_to_slot,
                            const uint8_t* slots, float* y, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* moe_layer_forward that also writes x_next = bf16(x + y) (round to nearest even), the input
 * of the next layer of a stack [MoE expert offload, "How it works": the layers of the model run
 * one after another on the same token], from the kernels that form y: no launch of its own.
 * x_next [M,H] bf16, 2-byte aligned, may equal x (then x is overwritten after every use of it
 * in the call).  Equal, bitwise, to moe_layer_forward followed by moe_residual_bf16(x, y,
 * x_next, M*H). */
moe_status moe_layer_forward_residual(const moe_shape* shape, const uint16_t* x, int32_t M,
                                      const uint16_t* w_router, const float* router_bias,
                                      const int32_t* expert_to_slot, const uint8_t* slots,
                                      int32_t* topk_ids, float* topk_w, float* y,
                                      int32_t* cold_count, int32_t* cold_routes,
                                      uint16_t* x_next, void* ws, size_t ws_bytes,
                                      hipStream_t stream);

/* Residual chaining of stacked layers: out[i] = bf16(x[i] + y[i]) (round to nearest even),
 * for feeding one layer's output to the next [MoE expert offload, "How it works": the layers of
 * the model run one after another on the same token].  x, out: bf16 [n] (out may equal x);
 * y: fp32 [n].  n = 0 enqueues nothing. */
moe_status moe_residual_bf16(const uint16_t* x, const float* y, uint16_t* out, size_t n,
                             hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Hybrid GPU-hot / CPU-cold layer [ORT hybrid PR, "Key Changes": routes to cold experts
 * (slot < 0) are skipped on the GPU and accumulated on the CPU, whose worker threads execute the
 * cold experts while the hot-expert kernel runs, through reusable pinned staging buffers and
 * timing-disabled events; ninfer v0.4.0, "New": cold experts run on the CPU].
 *
 * moe_cold_forward_host: the cold routes alone, on the host cores (all pointers [host]):
 *   y_cold[m] = sum over j = 0..k-1 (ascending) of the routes whose expert maps to no slot
 *   (expert_to_slot[e] outside [0, S); NULL = identity, nothing cold) of
 *   topk_w[m,j] * (Wd_e h), h = bf16(silu(Wg_e x_m) * (Wu_e x_m)), fp32 accumulation.
 *   host_bank: E expert images back to back (moe_pack_expert layout, the bytes the slots hold);
 *   x [M,H] bf16; topk_ids / topk_w [M,k]; y_cold [M,H] fp32 is overwritten (zeros for a token
 *   with no cold route); routes with an id outside [0, E) are skipped.  n_threads <= 0: one per
 *   host core.  Synchronous, deterministic (the result does not depend on n_threads).
 *   MXFP4 experts only (other formats: MOE_ERR_UNSUPPORTED, as for moe_layer_forward_hybrid).
 *
 * moe_layer_forward_hybrid: the whole layer with cold routes on the host:
 *   on stream: router + top-k (as moe_route), copies of x, topk_ids and topk_w into the pinned
 *   staging (then staging->routed is recorded), the hot experts (as moe_experts_forward, y =
 *   hot-only output); on the calling thread, once staging->routed has passed: the cold routes
 *   (moe_cold_forward_host) into staging->y_cold while the GPU runs the hot experts; then on
 *   stream: y_cold is uploaded to staging->y_cold_dev and added to y (staging->added is
 *   recorded).  So y = y_hot + y_cold, every route of the layer.  Returns once the host part is
 *   done and the upload is enqueued.  The next call on the same staging first waits for
 *   staging->added.  expert_to_slot (device) and expert_to_slot_host hold the same map.
 * --------------------------------------------------------------------------------------- */
typedef struct {
  int32_t max_M;      /* tokens the buffers hold */
  uint16_t* x;        /* [host, pinned] [max_M, H] */
  int32_t* ids;       /* [host, pinned] [max_M, k] */
  float* w;           /* [host, pinned] [max_M, k] */
  float* y_cold;      /* [host, pinned] [max_M, H] */
  float* y_cold_dev;  /* device [max_M, H] */
  hipEvent_t routed;  /* created by the caller (timing may be disabled) */
  hipEvent_t added;   /* created by the caller */
  int32_t pending;    /* set by the library; 0 before the first call */
} moe_hybrid_staging;

moe_status moe_cold_forward_host(const moe_shape* shape, const uint8_t* host_bank,
                                 const uint16_t* x, int32_t M, const int32_t* topk_ids,
                                 const float* topk_w, const int32_t* expert_to_slot,
                                 float* y_cold, int32_t n_threads);

moe_status moe_layer_forward_hybrid(const moe_shape* shape, const uint16_t* x, int32_t M,
                                    const uint16_t* w_router, const float* router_bias,
                                    const int32_t* expert_to_slot,
                                    const int32_t* expert_to_slot_host, const uint8_t* slots,
                                    const uint8_t* host_bank, int32_t* topk_ids, float* topk_w,
                                    float* y, moe_hybrid_staging* staging, int32_t n_threads,
                                    void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Prefill with staged experts [MoE expert offload, "How it works", Prefill: when a call
 * touches more distinct experts than the layer has slots, the experts are copied into a
 * staging buffer by pinned asynchronous memcpy and the unchanged GEMM runs on it; tinyserve,
 * "How it works" item 6: batched prefill groups tokens by expert and loads each expert once].
 *   On stream: router + top-k (as moe_route), the route count of every expert; the host waits
 *   for the counts (one synchronisation per call), takes the touched experts in ascending id
 *   and copies each once from host_bank (pinned, E images back to back) into the staging slots
 *   with hipMemcpyAsync on staging->copy_stream.  If they all fit (touched <= n_slots) one pass
 *   runs the expert kernels (the grouped GEMMs for M >= 64) on them: y is the whole layer.
 *   Otherwise passes of n_slots / 2 experts alternate between the two halves of the staging
 *   slots: the copies of pass b + 1 overlap the expert kernels of pass b, each pass's output is
 *   added to y on the stream (y = the sum over passes, every route once).  *n_touched and
 *   *n_passes [host] report what was done (may be NULL).  Returns once every pass is enqueued;
 *   the next call on the same staging waits for this one's passes before reusing its buffers.
 * The staging (caller-owned): slots device [n_slots][image] (256-byte aligned), counts_dev [E],
 * counts_host [host, pinned] [E], maps_dev [2][E], maps_host [host, pinned] [2][E], y_pass
 * device [max_M][H], a copy stream and five events created by the caller; pending zeroed.
 * --------------------------------------------------------------------------------------- */
typedef struct {
  int32_t max_M;
  int32_t n_slots;
  uint8_t* slots;
  int32_t* counts_dev;
  int32_t* counts_host;
  int32_t* maps_dev;
  int32_t* maps_host;
  float* y_pass;
  hipStream_t copy_stream;
  hipEvent_t ev_counts, ev_copied[2], ev_done[2];
  int32_t pending[2];
} moe_prefill_staging;

moe_status moe_layer_forward_staged(const moe_shape* shape, const uint16_t* x, int32_t M,
                                   const uint16_t* w_router, const float* router_bias,
                                   const uint8_t* host_bank, int32_t* topk_ids, float* topk_w,
                                   float* y, moe_prefill_staging* staging, void* ws,
                                   size_t ws_bytes, hipStream_t stream, int32_t* n_touched,
                                   int32_t* n_passes);

/* ---------------------------------------------------------------------------------------
 * Slot refill [ninfer v0.4.0, "New": experts are copied to the GPU in the background;
 * MoE expert offload, intro: routed experts stay in pinned host RAM; ORT hybrid PR,
 * "Key Changes": pinned staging ordered by timing-disabled events].
 *   For i < n: copy expert images host_bank[experts[i]] -> slots[slot_ids[i]] with
 *   hipMemcpyAsync on copy_stream.  If wait_before is not NULL, copy_stream first waits for it
 *   (e.g. the event recorded after the last kernels that read those slots); if done is not
 *   NULL it is recorded on copy_stream after the copies (the compute stream waits on it
 *   before the refilled experts become visible).
 * host_bank [host, pinned]: E images back to back; experts, slot_ids [host].
 * --------------------------------------------------------------------------------------- */
moe_status moe_slot_refill(const moe_shape* shape, uint8_t* slots, const uint8_t* host_bank,
                           const int32_t* experts, const int32_t* slot_ids, int32_t n,
                           hipStream_t copy_stream, hipEvent_t wait_before, hipEvent_t done);

/* ---------------------------------------------------------------------------------------
 * Slot-cache policy, host only [MoE expert offload, "How it works": per-layer LRU table,
 * misses take least-recently-used slots; ninfer v0.4.0, "New": at most two refills per
 * layer and call, in the background, replacing the least used; tinyserve, "How it works"
 * item 3 and "Configuration": LFRU eviction].
 * One cache object per layer.  moe_cache_policy_step(step t, observed routes):
 *   1. refills planned with visible_step <= t become resident;
 *   2. for the observed routes: route/hit counters, LFRU frequencies (+1 per route, all
 *      halved every decay_period steps), last_use = t for routed resident experts;
 *   3. routed experts that are cold and not in flight, by (route count desc, id asc), are
 *      admitted while fewer than max_refills_per_step were admitted at t and fewer than
 *      max_pending are in flight: victim = lowest empty slot, else among resident slots not
 *      in flight and not routed at t the smallest (last_use, slot) [LRU] or
 *      (freq, last_use, slot) [LFRU]; the old expert is cold at once, the slot's last_use
 *      becomes t and the new expert becomes visible at t + lag_steps;
 *   4. the map expert -> slot (or -1) for step t is written to expert_to_slot [host, E].
 * topk_ids [host] [M,k] are the routes the caller observed (M = 0 or NULL: none).
 * plan [host] receives up to max_refills_per_step entries; *n_plan their number.
 * Steps must strictly increase.  Pure host code, deterministic.
 * --------------------------------------------------------------------------------------- */
typedef struct moe_cache moe_cache;

enum { MOE_POLICY_LRU = 0, MOE_POLICY_LFRU = 1 };

typedef struct {
  int32_t policy;               /* MOE_POLICY_LRU or MOE_POLICY_LFRU */
  int32_t max_refills_per_step; /* >= 0 (0 = static placement) */
  int32_t lag_steps;            /* >= 1 */
  int32_t max_pending;          /* >= 1 */
  int32_t decay_period;         /* LFRU halving period in steps, 0 = never */
} moe_cache_config;

typedef struct {
  int32_t expert;       /* expert to copy in */
  int32_t slot;         /* destination slot */
  int32_t evicted;      /* expert that held the slot, or -1 */
  int32_t reserved;     /* 0 */
  int64_t visible_step; /* first step whose map contains the new expert */
} moe_refill;

typedef struct {
  int64_t steps, routes, hits, refills, evictions;
} moe_cache_stats;

/* initial_slot_expert [host] [S]: expert held by each slot, -1 = empty (NULL = all empty). */
moe_status moe_cache_create(const moe_shape* shape, const moe_cache_config* config,
                            const int32_t* initial_slot_expert, moe_cache** out);
moe_status moe_cache_policy_step(moe_cache* cache, int64_t step, const int32_t* topk_ids,
                                 int32_t M, moe_refill* plan, int32_t* n_plan,
                                 int32_t* expert_to_slot, moe_cache_stats* stats);
void moe_cache_destroy(moe_cache* cache);

/* Checkpoint and replay of a cache: moe_cache_save writes the whole state (configuration, step
 * index, both maps, recency, LFRU frequencies, refills in flight, counters) as plain data into
 * buf [host], moe_cache_state_bytes(cache) bytes; moe_cache_restore loads such a state into a
 * cache created for the same (E, S, k), replacing its state and configuration, so that the
 * steps that follow plan exactly what the saved cache would have planned.  A buffer that is not
 * a saved state, or an inconsistent one, is rejected with MOE_ERR_INVALID_ARG and leaves the
 * cache unchanged; a state of another shape gives MOE_ERR_STATE.  The device cache's state is
 * plain device memory with no pointers: copying its state_bytes out and back is its
 * checkpoint. */
moe_status moe_cache_state_bytes(const moe_cache* cache, size_t* bytes);
moe_status moe_cache_save(const moe_cache* cache, void* buf, size_t bytes);
moe_status moe_cache_restore(moe_cache* cache, const void* buf, size_t bytes);

/* ---------------------------------------------------------------------------------------
 * GPU-resident slot cache [MoE expert offload, "How it works", Decode: the per-layer LRU table
 * is kept on the GPU, a kernel looks routed experts up and assigns least-recently-used slots to
 * misses, a second kernel copies the missing experts straight from device-mapped pinned host
 * memory into their slots; both have fixed launch shapes and read the miss count from device
 * memory, so decode stays inside graphs with no host sync; ninfer v0.4.0, "New": at most two
 * refills per layer and call].  The policy is moe_cache_policy_step's, step for step, over state
 * that lives in device memory, so a decode loop (policy, layer, copy) can be captured whole in
 * a HIP graph.  Step t observes the routes the caller passes (e.g. those of step t - 1).
 *
 * moe_device_cache_size: bytes of the device state of one layer's cache.  [host] out.
 * moe_device_cache_init: writes the state (config, initial placement [host] [S] or NULL, step
 *   index of the first step) into `state` (device, 256-byte aligned); returns once written.
 *   R and Q at most 16.
 * moe_device_cache_step: one step, enqueued on stream: observed_ids [n_observed] (device; ids
 *   outside [0, E) are not observed, so a buffer of -1 stands for "nothing observed"),
 *   expert_to_slot [E] (device, out: the map of this step, as moe_cache_policy_step publishes
 *   it), plan [<= R] and n_plan [1] (device, out: this step's refills).  The state's step index
 *   advances by one.
 * moe_device_cache_copy: the planned refills, enqueued on stream: n_plan and plan as written by
 *   moe_device_cache_step; images from host_bank (pinned host memory, device-mapped: allocated
 *   with hipHostMalloc, E images back to back) into slots.  One kernel of a fixed shape; with
 *   n_plan = 0 it does nothing.  The caller orders it after the last kernels that read the
 *   victim slots and before the first that reads a refilled slot (visible_step), e.g. on a side
 *   stream with events.
 * moe_device_cache_stats: copies the state's counters to *stats (device or pinned host
 *   memory), on stream.
 * --------------------------------------------------------------------------------------- */
moe_status moe_device_cache_size(const moe_shape* shape, size_t* bytes);
moe_status moe_device_cache_init(const moe_shape* shape, const moe_cache_config* config,
                                 const int32_t* initial_slot_expert, int64_t first_step,
                                 void* state, size_t state_bytes, hipStream_t stream);
moe_status moe_device_cache_step(const moe_shape* shape, void* state, size_t state_bytes,
                                 const int32_t* observed_ids, int32_t n_observed,
                                 int32_t* expert_to_slot, moe_refill* plan, int32_t* n_plan,
                                 hipStream_t stream);
moe_status moe_device_cache_copy(const moe_shape* shape, const int32_t* n_plan,
                                 const moe_refill* plan, const uint8_t* host_bank, uint8_t* slots,
                                 hipStream_t stream);
moe_status moe_device_cache_stats(const moe_shape* shape, const void* state, size_t state_bytes,
                                  moe_cache_stats* stats, hipStream_t stream);

/* Measurement aid (not part of the layer): reads `bytes` of device memory at src once, in
 * 16-byte loads, with the launch shape of the fused one-token kernel (one workgroup of 16 waves
 * per compute unit, every load of a thread issued before any is used).  Its duration is the
 * device's read-streaming ceiling for a weight stream of that size, against which the fused
 * kernel's rate is reported next to the published HBM peak.  sink: one uint32 of device memory
 * (written only in a case that cannot occur).  src 16-byte aligned; bytes a positive multiple
 * of 16. */
moe_status moe_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

/* Message describing the last failure of a call on this thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
