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
//   down section: H/RD tiles of RD = 64/S rows over K = I (nb = I/32 blocks), S chosen per
//   shape (dn_segments below).  Lane l = r*S + s owns row r of the tile and K segment s; at
//   step t it holds block t*S + s of its row.  Steps with all lanes active are 1 KiB each
//   (lane-major, 16 B per lane); the final partial step (when S does not divide nb) stores
//   only its active lanes, row by row (index r*(nb % S) + s).  Then ceil(T/4) words per lane
//   of scale bytes: byte i of word q is the scale of the lane's block at step 4q+i (127 past
//   the end).
//
// In the gate/up section every lane of a wave owns one output row and all lanes walk the same
// input block at the same time, so the activation block is uniform across the wave and is read
// through the scalar unit.  The down section trades that for more, smaller tiles so that one
// workgroup can own a few output rows for every routed expert and combine them on its own.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kMaxHidden = 8192;
constexpr int kMaxInter = 4096;      // down steps per lane stay <= 16 with S = 8
constexpr int kBucketThreads = 1024; // threads of the top-k / bucketing workgroup
constexpr size_t kDownLdsBudget = 48 * 1024;  // dynamic LDS of the down kernel (h + row sums)

struct ImageLayout {
  int H, I;
  int nb_h, ng_h;  // gate/up: blocks and groups along K = H
  int nb_i;        // down: blocks along K = I
  int dn_seg;      // S: lanes (K segments) per down row
  int dn_rows;     // RD = 64 / S rows per down tile
  int dn_steps;    // T = ceil(nb_i / S) steps per lane
  int dn_scale_words;  // ceil(T / 4) scale words per lane
  int gu_tiles, dn_tiles;
  size_t gu_tile_bytes, dn_code_bytes, dn_tile_bytes;
  size_t gu_bytes, dn_bytes, image_bytes;
};

// S for the down tiles: the fewest padding scale bytes with at most 16 steps per lane, ties to
// the larger S (more, smaller tiles).
inline int dn_segments(int nb) {
  int best = 1;
  long best_pad = -1;
  for (int S = 8; S >= 1; S /= 2) {
    const int T = (nb + S - 1) / S;
    if (T > 16) continue;
    const long pad = (long)((T + 3) / 4) * 256 - (long)nb * (64 / S);
    if (best_pad < 0 || pad < best_pad) {
      best = S;
      best_pad = pad;
    }
  }
  return best;
}

inline ImageLayout image_layout(int H, int I) {
  ImageLayout L;
  L.H = H;
  L.I = I;
  L.nb_h = H / 32;
  L.ng_h = (L.nb_h + 3) / 4;
  L.nb_i = I / 32;
  L.dn_seg = dn_segments(L.nb_i);
  L.dn_rows = 64 / L.dn_seg;
  L.dn_steps = (L.nb_i + L.dn_seg - 1) / L.dn_seg;
  L.dn_scale_words = (L.dn_steps + 3) / 4;
  L.gu_tiles = I / 32;
  L.dn_tiles = H / L.dn_rows;
  L.gu_tile_bytes = (size_t)L.nb_h * 1024 + (size_t)L.ng_h * 256;
  const int full = L.nb_i / L.dn_seg, rem = L.nb_i % L.dn_seg;
  L.dn_code_bytes = ((size_t)full * 64 + (size_t)L.dn_rows * rem) * 16;
  L.dn_tile_bytes = L.dn_code_bytes + (size_t)L.dn_scale_words * 256;
  L.gu_bytes = L.gu_tile_bytes * L.gu_tiles;
  L.dn_bytes = L.dn_tile_bytes * L.dn_tiles;
  L.image_bytes = (L.gu_bytes + L.dn_bytes + 255) / 256 * 256;
  return L;
}

// Workspace: per-call arrays sized for M tokens (nothing survives between calls).
struct WsLayout {
  size_t logits;         // f32 [M][E]
  size_t route_slot;     // i32 [M*k]
  size_t counts;         // i32 [E]
  size_t offsets;        // i32 [E+1]
  size_t perm;           // i32 [M*k]
  size_t meta;           // i32 [8]: n_dist, cold_count, error flags
  size_t dist;           // i32x4 [nd_max]: distinct hot experts {slot, bucket offset, count, id}
  size_t cold_list;      // i32 [M*k]
  size_t items;          // i32x2 [n_items_max]: grouped GEMM work list {distinct expert, first route}
  size_t hbuf;           // bf16 [M*k][I]
  size_t pdn;            // f32 [M*k][H]: down partial sums when they do not fit in LDS
  size_t hand;           // u32 counters of the fused decode kernel, one per 64 bytes
  size_t total;
};

inline size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// Fused decode kernel handoff: kHandSub arrival counters per distinct hot expert (gate/up tile t
// counts on counter t % kHandSub), each on its own 64-byte line.
constexpr int kHandSub = 8;
constexpr int kHandStride = 16;  // 32-bit words between counters

// Grouped GEMM work items: (distinct hot expert, pass of up to kItemRoutes of its routes).
// sum over experts of ceil(c_e / kItemRoutes) <= (number of experts) + M*k / kItemRoutes.
constexpr int kItemRoutes = 64;
inline int n_items_max(int Mk, int E) {
  const int nd = Mk < E ? Mk : E;
  return nd + Mk / kItemRoutes;
}

inline WsLayout ws_layout(int H, int I, int E, int k, int M) {
  WsLayout W;
  const ImageLayout L = image_layout(H, I);
  const size_t Mk = (size_t)M * k;
  const size_t nd = Mk < (size_t)E ? Mk : (size_t)E;
  (void)L;
  size_t o = 0;
  W.logits = o;      o = align256(o + 4 * (size_t)M * E);
  W.route_slot = o;  o = align256(o + 4 * Mk);
  W.counts = o;      o = align256(o + 4 * (size_t)E);
  W.offsets = o;     o = align256(o + 4 * ((size_t)E + 1));
  W.perm = o;        o = align256(o + 4 * Mk);
  W.meta = o;        o = align256(o + 4 * 8);
  W.dist = o;        o = align256(o + 16 * nd);
  W.cold_list = o;   o = align256(o + 4 * Mk);
  W.items = o;       o = align256(o + 8 * (size_t)n_items_max((int)Mk, E));
  W.hbuf = o;        o = align256(o + 2 * Mk * I);
  W.pdn = o;         o = align256(o + 4 * Mk * (size_t)H);
  W.hand = o;        o = align256(o + 64 * (size_t)nd * kHandSub);
  W.total = o;
  return W;
}

// Error flags raised by the device in meta[2]; meta[3] holds the length of the work list.
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
  bool h_in_lds;     // down: h of every route staged in LDS
  bool part_in_lds;  // down: per-route row sums in LDS (else in the workspace)
  size_t dn_lds;     // down: dynamic LDS bytes
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

// Kernel launchers (moe_kernels.hip).
hipError_t launch_router(const uint16_t* x, int M, const uint16_t* wr, const float* bias, int E,
                         int H, float* logits, uint32_t* zero, int n_zero, hipStream_t s);
bool layer_decode_fusable(const ImageLayout& L, const ExpertPlan& p, int M);
hipError_t launch_layer_decode(const uint16_t* x, int M, int H, int I, const uint8_t* slots,
                               const ImageLayout& L, const ExpertPlan& p, const RouteArgs& ra,
                               const RouteWs& rw, uint16_t* hbuf, float* y, uint32_t* hand,
                               hipStream_t s);
hipError_t launch_topk_bucket(const float* logits, int M, int k, int32_t* topk_ids, float* topk_w,
                              bool do_bucket, const int32_t* ids, int E, int S,
                              const int32_t* e2s, const BucketOut& o, hipStream_t s);
ExpertPlan plan_experts(const ImageLayout& L, int M, int E, int k);
hipError_t launch_gateup(const uint16_t* x, int M, int H, int I, const uint8_t* slots,
                         const ImageLayout& L, const ExpertPlan& p, const RouteArgs& ra,
                         const RouteWs& rw, uint16_t* hbuf, hipStream_t s);
hipError_t launch_down(int M, int H, int I, const uint8_t* slots, const ImageLayout& L,
                       const ExpertPlan& p, const RouteArgs& ra, const RouteWs& rw,
                       const uint16_t* hbuf, float* pdn, float* y, hipStream_t s);
hipError_t launch_residual(const uint16_t* x, const float* y, uint16_t* out, size_t n,
                           hipStream_t s);
hipError_t launch_gateup_grouped(const uint16_t* x, int H, int I, const uint8_t* slots,
                                 const ImageLayout& L, const ExpertPlan& p, const RouteArgs& ra,
                                 const RouteWs& rw, uint16_t* hbuf, hipStream_t s);
hipError_t launch_down_grouped(int M, int H, int I, const uint8_t* slots, const ImageLayout& L,
                               const ExpertPlan& p, const RouteArgs& ra, const RouteWs& rw,
                               const uint16_t* hbuf, float* pdn, float* y, hipStream_t s);

}  // namespace moe
