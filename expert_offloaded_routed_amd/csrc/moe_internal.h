// Internal definitions shared by the host API and the kernels of libmoe (not installed).
//
// Expert image layout (kernel layout, produced by moe_pack_expert):
//
//   [ gate/up section | down section ]  padded to a multiple of 256 bytes.
//
//   gate/up section: I/32 tiles.  Tile t covers gate rows and up rows 32t..32t+31 over the
//   whole input dimension K = H (nb = H/32 blocks, ng = ceil(nb/4) groups of 4 blocks):
//     codes : nb blocks x 64 lanes x 16 B.  Lane l < 32 holds gate row 32t+l, lane l >= 32
//             holds up row 32t+(l-32); the 16 bytes are that row's block b (32 E2M1 codes,
//             canonical nibble order).  One wave-wide 16-byte load = 1 KiB contiguous.
//     scales: ng groups x 64 lanes x 4 B; byte i of a lane's word in group q is the E8M0
//             scale of block 4q+i of that lane's row (127 = 1.0 past the last block).
//   down section: H/16 tiles of 16 rows over K = I (nb = I/32 blocks), in K steps of 4 blocks
//   (128 elements), each step one operand of the block-scaled MFMA (16 rows x 128 K, E2M1):
//     codes : lane l holds row l%16, block 4s + l/16 of step s (16 B).  Full steps are 1 KiB
//             (lane-major); a final partial step (nb % 4 blocks) stores only its lanes
//             l < 16*(nb % 4), also lane-major.
//     scales: ceil(steps/4) words per lane: byte j of word q is the E8M0 scale of the lane's
//             block at step 4q+j (127 past the last block).
//
// In the gate/up section every lane of a wave owns one output row and all lanes walk the same
// input block at the same time, so the activation block is uniform across the wave.  The down
// section feeds the matrix cores directly (no decode): h enters as the other operand, split
// into two E4M3 terms per element under a shared per-block scale (see the workspace below).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kMaxHidden = 8192;
constexpr int kMaxInter = 4096;      // at most 32 down K steps
constexpr int kBucketThreads = 1024; // threads of the top-k / bucketing workgroup
constexpr int kTopkThreads = 128;    // threads of a workgroup of the multi-workgroup top-k
constexpr int kDnRows = 16;          // rows of a down tile (one MFMA operand)

inline size_t align256(size_t v) { return (v + 255) / 256 * 256; }

struct ImageLayout {
  int H, I;
  int nb_h, ng_h;  // gate/up: blocks and groups along K = H
  int nb_i;        // down: blocks along K = I
  int dn_ks;       // down: K steps of 4 blocks
  int dn_full, dn_rem;  // full K steps; blocks of the final partial step (0: none)
  int dn_scale_words;   // ceil(dn_ks / 4) scale words per lane
  int gu_tiles, dn_tiles;
  size_t gu_tile_bytes, dn_code_bytes, dn_tile_bytes;
  size_t gu_bytes, dn_bytes, image_bytes;
  int h_pad;        // I rounded up to whole K steps (128 elements)
  size_t h_stride;  // workspace bytes of one route's split h: hi[h_pad], lo[h_pad], scales[4*dn_ks]
};

inline ImageLayout image_layout(int H, int I) {
  ImageLayout L;
  L.H = H;
  L.I = I;
  L.nb_h = H / 32;
  L.ng_h = (L.nb_h + 3) / 4;
  L.nb_i = I / 32;
  L.dn_ks = (L.nb_i + 3) / 4;
  L.dn_full = L.nb_i / 4;
  L.dn_rem = L.nb_i % 4;
  L.dn_scale_words = (L.dn_ks + 3) / 4;
  L.gu_tiles = I / 32;
  L.dn_tiles = H / kDnRows;
  L.gu_tile_bytes = (size_t)L.nb_h * 1024 + (size_t)L.ng_h * 256;
  L.dn_code_bytes = (size_t)L.dn_full * 1024 + (size_t)L.dn_rem * 256;
  L.dn_tile_bytes = L.dn_code_bytes + (size_t)L.dn_scale_words * 256;
  L.h_pad = L.dn_ks * 128;
  L.h_stride = ((size_t)2 * L.h_pad + (size_t)4 * L.dn_ks + 15) / 16 * 16;
  L.gu_bytes = L.gu_tile_bytes * L.gu_tiles;
  L.dn_bytes = L.dn_tile_bytes * L.dn_tiles;
  L.image_bytes = (L.gu_bytes + L.dn_bytes + 255) / 256 * 256;
  return L;
}

// Expert images of the other formats (MOE_FORMAT_BF16, MOE_FORMAT_FP8_BLOCK, MOE_FORMAT_NVFP4):
// the six canonical tensors of moe_pack_expert, each row-major and starting at a multiple of
// 256 bytes, in the order [gate | gate scales | up | up scales | down | down scales]; the image is
// padded to a multiple of 256 bytes.  Element bytes of a matrix [N][K]: bf16 2NK, E4M3 NK,
// E2M1 NK/2.  Scale bytes: none (bf16); fp32 [ceil(N/128)][ceil(K/128)] (FP8 block); one fp32
// global scale followed by E4M3 bytes [N][K/16] (NVFP4).
struct FmtLayout {
  size_t gate, gate_s, up, up_s, down, down_s, image_bytes;
};
inline size_t fmt_elem_bytes(int fmt, int N, int K) {
  const size_t nk = (size_t)N * K;
  return fmt == MOE_FORMAT_BF16 ? 2 * nk : fmt == MOE_FORMAT_FP8_BLOCK ? nk : nk / 2;
}
inline size_t fmt_scale_bytes(int fmt, int N, int K) {
  if (fmt == MOE_FORMAT_FP8_BLOCK) return 4 * (size_t)((N + 127) / 128) * ((K + 127) / 128);
  if (fmt == MOE_FORMAT_NVFP4) return 4 + (size_t)N * (K / 16);
  return 0;
}
inline FmtLayout fmt_layout(int fmt, int H, int I) {
  FmtLayout F;
  size_t o = 0;
  F.gate = o;    o = align256(o + fmt_elem_bytes(fmt, I, H));
  F.gate_s = o;  o = align256(o + fmt_scale_bytes(fmt, I, H));
  F.up = o;      o = align256(o + fmt_elem_bytes(fmt, I, H));
  F.up_s = o;    o = align256(o + fmt_scale_bytes(fmt, I, H));
  F.down = o;    o = align256(o + fmt_elem_bytes(fmt, H, I));
  F.down_s = o;  o = align256(o + fmt_scale_bytes(fmt, H, I));
  F.image_bytes = o;
  return F;
}
// Bytes of one expert image of the shape's format.
inline size_t expert_image_bytes(const moe_shape* s) {
  return s->format == MOE_FORMAT_MXFP4 ? image_layout(s->hidden, s->inter).image_bytes
                                       : fmt_layout(s->format, s->hidden, s->inter).image_bytes;
}

// Calls with at least this many tokens take the grouped GEMM path (and the MFMA router).
constexpr int kGroupedMinTokens = 64;
// The MFMA router splits K over this many workgroups (for at most kRouterMaxE experts); the
// logit row of a token is then held as that many partial sums M*E floats apart (the first
// with the bias), summed in ascending order by the top-k.
constexpr int kRouterParts = 4;
constexpr int kRouterMaxE = 512;
__host__ __device__ inline int router_parts(int M, int E) {
  return M >= kGroupedMinTokens && E <= kRouterMaxE ? kRouterParts : 1;
}

// Workspace: a fixed header, then per-call arrays sized for M tokens.
//
// Header (offset 0, the same for every M, so that the error word can be read without knowing
// the last call's size), int32 meta[kMetaWords]:
//   [0] distinct hot experts of the call, [1] its cold routes, [2] the device error flags
//   (kErr* bits) that the calls on this workspace raised since moe_workspace_errors last took
//   them (kernels only OR bits in), [3] length of the grouped work list, [6] the fused
//   one-token launches' call id and [7] their poison word (both zero in a zero-filled
//   workspace; see k_layer_decode).
// Then, also at a fixed offset, the tagged h words of the fused one-token kernel (no other
// kernel writes there, so a stale word can only carry an older call's tag).
struct WsLayout {
  size_t meta;           // i32 [kMetaWords], offset 0
  size_t hf;             // u64 [kFusedMaxK][kMaxInter / 2]: {h pair, call tag}, fixed offset
  size_t dncall;         // u32 [kMaxHidden / 16]: split down GEMV, call id per row tile, fixed offset
  size_t pw;             // u64 [16*k][2048]: the split down GEMV's {row value, tag} words, at an
                         // offset fixed by the shape (only when the shape can split)
  size_t logits;         // f32 [router_parts(M, E)][M][E]
  size_t route_slot;     // i32 [M*k]
  size_t counts;         // i32 [E]
  size_t offsets;        // i32 [E+1]
  size_t perm;           // i32 [M*k]
  size_t dist;           // i32x4 [nd_max]: distinct hot experts {slot, bucket offset, count, id}
  size_t cold_list;      // i32 [M*k]
  size_t items;          // i32x2 [n_items_max]: grouped GEMM work list {distinct expert, first route}
  size_t hq;             // h of every route: bf16 [I] (GEMV paths, M < 64) or, on the grouped
                         // path, split for the block-scaled MFMA (ImageLayout::h_stride bytes)
  size_t pdn;            // f32 [M*k][H]: down partial sums of the grouped path
  size_t total;
};

constexpr int kMetaWords = 16;  // int32 words of the workspace header
constexpr int kMetaErr = 2;     // index of the error word
constexpr int kMetaCall = 6;    // fused one-token kernel: call id (8-byte aligned with ...)
constexpr int kMetaPoison = 7;  // ... the poison word: a launch lost its hand-over of h
constexpr size_t kFusedHBytes = (size_t)16 * kMaxInter * 4;  // tagged h of up to 16 routes
// The fused one-token kernel computes the router itself for at most this many experts of at
// most 8 chunks of 8 per lane (H <= 4096); larger routers run as their own kernel first.
constexpr int kFusedRouterMaxE = 32;
constexpr int kFusedRouterMaxCPL = 8;

// Grouped GEMM work items: (distinct hot expert, pass of up to kItemRoutes of its routes).
// sum over experts of ceil(c_e / kItemRoutes) <= (number of experts) + M*k / kItemRoutes.
constexpr int kItemRoutes = 64;
inline int n_items_max(int Mk, int E) {
  const int nd = Mk < E ? Mk : E;
  return nd + Mk / kItemRoutes;
}

// Shapes whose few-token down GEMV may share each row tile between two workgroups: one K part
// (I <= 1024) and at most kSplitMaxTiles row tiles (H <= 2048); calls of at most kSplitMaxTokens
// tokens, whose handed-over rows fit the workspace's fixed word region.
constexpr int kSplitMaxTiles = 128;
constexpr int kSplitMaxTokens = 16;
// Words of one route in that region: a row's word sits at route * kSplitRowStride + row, the
// same place for every shape, so that a word another shape left behind belongs to the same row
// tile (whose call id has moved past its tag) and is never taken for this call's.
constexpr int kSplitRowStride = kSplitMaxTiles * 16;
inline bool down_split_possible(const ImageLayout& L) {
  return L.dn_ks <= 8 && L.dn_tiles <= kSplitMaxTiles;
}

inline WsLayout ws_layout(int H, int I, int E, int k, int M) {
  WsLayout W;
  const ImageLayout L = image_layout(H, I);
  const size_t Mk = (size_t)M * k;
  const size_t nd = Mk < (size_t)E ? Mk : (size_t)E;
  size_t o = 0;
  W.meta = o;        o = align256(o + 4 * (size_t)kMetaWords);
  W.hf = o;          o = align256(o + kFusedHBytes);
  W.dncall = o;      o = align256(o + 4 * (size_t)(kMaxHidden / 16));
  W.pw = o;          o = align256(o + (down_split_possible(L) ? 8 * (size_t)kSplitMaxTokens * k * kSplitRowStride : 0));
  W.logits = o;      o = align256(o + 4 * (size_t)router_parts(M, E) * M * E);
  W.route_slot = o;  o = align256(o + 4 * Mk);
  W.counts = o;      o = align256(o + 4 * (size_t)E);
  W.offsets = o;     o = align256(o + 4 * ((size_t)E + 1));
  W.perm = o;        o = align256(o + 4 * Mk);
  W.dist = o;        o = align256(o + 16 * nd);
  W.cold_list = o;   o = align256(o + 4 * Mk);
  W.items = o;       o = align256(o + 8 * (size_t)n_items_max((int)Mk, E));
  W.hq = o;          o = align256(o + Mk * (L.h_stride > 2 * (size_t)I ? L.h_stride : 2 * (size_t)I));
  W.pdn = o;         o = align256(o + 4 * Mk * (size_t)H);
  W.total = o;
  return W;
}

// Error flags raised by the device in meta[kMetaErr] (the values of MOE_DEVERR_* in moe.h).
enum : int32_t { kErrBadId = 1, kErrBadSlot = 2, kErrHandoff = 4 };

// Outputs of the resolve / bucketing stage (workspace arrays, then optional caller arrays).
struct BucketOut {
  int32_t *route_slot, *ws_perm, *meta;
  int4* dist;
  int2* items;
  int32_t *cold_list, *u_counts, *u_offsets, *u_perm, *u_cold_count, *u_cold_routes;
};

// Launch shape of the expert kernels for one call.
struct ExpertPlan {
  int nd_max;        // upper bound of distinct hot experts (gate/up grid.y)
  bool grouped;      // many tokens: grouped GEMM on MFMA (route table from the bucketing kernel)
  int n_items_max;   // bound of the grouped GEMM work list (grid.y)
  bool prologue;     // every expert workgroup rebuilds the route table (M*k <= kProMaxRoutes)
  int gu_waves;      // waves per gate/up workgroup
  int gu_groups;     // most K groups (of 4 blocks) any gate/up wave holds
  int gu_dgrid;      // gate/up grid.y: hot experts in flight at once (looped past it)
};

// Routes of a call as the expert kernels see them (kernel arguments, passed by value).
struct RouteArgs {
  const float* logits;      // top-k from these (NULL: use ids_in / w_in)
  const int32_t* ids_in;    // [M*k]
  const float* w_in;        // [M*k]
  const int32_t* e2s;       // [E] or NULL (identity)
  int M, k, E, S;
  int32_t* topk_ids;        // outputs of the writer workgroup, [M*k] or NULL
  float* topk_w;
  int32_t* cold_count;      // [1] or NULL
  int32_t* cold_routes;     // [M*k] or NULL
};

// Route table in the workspace: written by the route kernel, the bucketing kernel or the writer
// workgroup of a gate/up launch that builds it itself; read by the expert kernels.
struct RouteWs {
  int32_t* meta;        // [0] distinct hot experts, [1] cold routes, [2] error flags
  int4* dist;           // {slot, offset into perm, count, expert id}, ascending expert id
  int2* items;          // grouped GEMM work list, meta[3] entries
  int32_t* perm;        // hot routes grouped by expert
  int32_t* route_slot;  // slot of every route, -1 = cold
};

// Residual chaining by the kernels that produce y: out[m][h] = bf16(x[m][h] + y[m][h]) (out may
// equal x; out == NULL: nothing).
struct Residual {
  const uint16_t* x;
  uint16_t* out;
};

// GPU-resident slot cache (moe_dcache.hip): state in device memory, one header then arrays.
constexpr int kDcacheMaxQ = 16;        // refills per step and in flight, at most
constexpr int kDcacheCopyGroups = 128; // workgroups of the copy kernel (fixed launch shape)
struct DevCacheHdr {
  int64_t step;      // the next step's index
  int64_t stats[5];  // steps, routes, hits, refills, evictions (the order of moe_cache_stats)
  int32_t E, S, R, L, Q, policy, decay, n_pending;
  int32_t pend_e[kDcacheMaxQ], pend_s[kDcacheMaxQ];
  int64_t pend_vis[kDcacheMaxQ];
};
struct DevCacheLayout {
  size_t slot_expert, expert_slot, last_use, freq, total;  // i32 [S], i32 [E], i64 [S], i64 [E]
};
__host__ __device__ inline DevCacheLayout dcache_layout(int E, int S) {
  DevCacheLayout D;
  size_t o = (sizeof(DevCacheHdr) + 255) / 256 * 256;
  D.last_use = o;     o += 8 * (size_t)S;
  D.freq = o;         o += 8 * (size_t)E;
  D.slot_expert = o;  o += 4 * (size_t)S;
  D.expert_slot = o;  o += 4 * (size_t)E;
  D.total = (o + 255) / 256 * 256;
  return D;
}
hipError_t launch_dcache_step(uint8_t* state, int E, int S, const int32_t* obs, int n_obs,
                              int32_t* map_out, moe_refill* plan, int32_t* n_plan, hipStream_t s);
hipError_t launch_dcache_copy(const int32_t* n_plan, const moe_refill* plan, const uint8_t* bank,
                              uint8_t* slots, size_t image_bytes, int E, int S, int R,
                              hipStream_t s);

// Kernel launchers (moe_kernels.hip).
hipError_t launch_router(const uint16_t* x, int M, const uint16_t* wr, const float* bias, int E,
                         int H, float* logits, hipStream_t s);
// Reads `bytes` (a multiple of 16) of src once with the fused decode kernel's launch shape.
hipError_t launch_stream_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);
// y[i] += add[i] for i < n.
hipError_t launch_add_f32(float* y, const float* add, size_t n, hipStream_t s);
// Copies the error word to *out (device or pinned host memory; NULL: nowhere) and clears it.
hipError_t launch_take_errors(int32_t* word, int32_t* out, hipStream_t s);
// The static scratch of the current device (the workspace of moe_layer_forward_noalloc):
// kScratchBytes, 256-byte aligned, zero-filled at its first use; NULL and *err set on failure.
constexpr size_t kScratchBytes = (size_t)8 << 20;
void* static_scratch(hipError_t* err);
bool layer_decode_fusable(const ImageLayout& L, const ExpertPlan& p, int M, int k, int E);
// The fused one-token kernel computes the router itself (no router launch before it).
bool layer_decode_router_inside(const ImageLayout& L, int E);
// wr / bias: the router, used when layer_decode_router_inside (else ra.logits holds the logits);
// hf: the workspace's tagged h region.
hipError_t launch_layer_decode(const uint16_t* x, const uint16_t* wr, const float* bias, int M,
                               int H, int I, const uint8_t* slots, const ImageLayout& L,
                               const ExpertPlan& p, const RouteArgs& ra, const RouteWs& rw,
                               uint64_t* hf, float* y, Residual res, hipStream_t s);
// The route table of a call of at most kRouteTableMaxRoutes routes (M >= 1) in one workgroup:
// top-k from ra.logits (or ra.ids_in / ra.w_in), then the table in the workspace, the top-k
// results (ra.topk_ids / topk_w, when the logits are given) and the cold report (ra.cold_count /
// cold_routes), all optional outputs.
constexpr int kRouteTableMaxRoutes = 256;
hipError_t launch_route_table(const RouteArgs& ra, const RouteWs& rw, hipStream_t s);
// logits: router_parts(M, E) partial rows per token (see kRouterParts).
hipError_t launch_topk_bucket(const float* logits, int M, int k, int32_t* topk_ids, float* topk_w,
                              bool do_bucket, const int32_t* ids, int E, int S,
                              const int32_t* e2s, const BucketOut& o, hipStream_t s);
ExpertPlan plan_experts(const ImageLayout& L, int M, int E, int k);
hipError_t launch_gateup(const uint16_t* x, int M, int H, int I, const uint8_t* slots,
                         const ImageLayout& L, const ExpertPlan& p, const RouteArgs& ra,
                         const RouteWs& rw, uint16_t* hbuf, hipStream_t s);
// Workgroups per tile of the down GEMV (1, or 2 handing rows over through the workspace).
int down_split(const ImageLayout& L, int M, int k, int E);
hipError_t launch_down(int M, int H, int I, const uint8_t* slots, const ImageLayout& L,
                       const ExpertPlan& p, const RouteArgs& ra, const RouteWs& rw,
                       const uint16_t* hbuf, uint64_t* pw, uint32_t* dncall, float* y, Residual res, hipStream_t s);
// The expert kernels of the other formats (moe_formats.hip), after the bucketing kernel:
// gate/up + SiLU into hbuf (bf16 [M*k][I]); down, route partials in pdn ([M*k][H] fp32) and the
// ordered combine into y (and the residual).
hipError_t launch_gateup_fmt(int fmt, const uint16_t* x, int H, int I, const uint8_t* slots,
                             size_t image_bytes, const FmtLayout& F, int nd_max,
                             const RouteArgs& ra, const RouteWs& rw, uint16_t* hbuf,
                             hipStream_t s);
hipError_t launch_down_fmt(int fmt, int H, int I, const uint8_t* slots, size_t image_bytes,
                           const FmtLayout& F, const RouteArgs& ra, const RouteWs& rw,
                           const uint16_t* hbuf, float* pdn, float* y, Residual res,
                           hipStream_t s);
hipError_t launch_residual(const uint16_t* x, const float* y, uint16_t* out, size_t n,
                           hipStream_t s);
hipError_t launch_gateup_grouped(const uint16_t* x, int H, int I, const uint8_t* slots,
                                 const ImageLayout& L, const ExpertPlan& p, const RouteArgs& ra,
                                 const RouteWs& rw, uint8_t* hq, hipStream_t s);
hipError_t launch_down_grouped(int M, int H, int I, const uint8_t* slots, const ImageLayout& L,
                               const ExpertPlan& p, const RouteArgs& ra, const RouteWs& rw,
                               const uint8_t* hq, float* pdn, float* y, Residual res,
                               hipStream_t s);

}  // namespace moe
