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
//   down section: H/64 tiles.  Tile t covers down rows 64t..64t+63 over K = I, same scheme
//   with lane l holding row 64t+l.
//
// Every lane of a wave works on its own output row and all lanes of a wave walk the same
// input block at the same time, so the activation block is uniform across the wave and is
// read through the scalar unit (no LDS and no vector-memory traffic for activations).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kMaxHidden = 8192;
constexpr int kMaxKC = 4;            // max K-chunks (workgroups) per down tile
constexpr int kWavesPerGroup = 4;    // waves per workgroup in the expert kernels
constexpr int kRouterWaves = 4;      // waves per workgroup in the router
constexpr int kBucketThreads = 1024; // threads of the single bucketing workgroup

struct ImageLayout {
  int H, I;
  int nb_h, ng_h;  // gate/up: blocks and groups along K = H
  int nb_i, ng_i;  // down: blocks and groups along K = I
  int gu_tiles, dn_tiles;
  size_t gu_tile_bytes, dn_tile_bytes;
  size_t gu_bytes, dn_bytes, image_bytes;
};

inline ImageLayout image_layout(int H, int I) {
  ImageLayout L;
  L.H = H;
  L.I = I;
  L.nb_h = H / 32;
  L.ng_h = (L.nb_h + 3) / 4;
  L.nb_i = I / 32;
  L.ng_i = (L.nb_i + 3) / 4;
  L.gu_tiles = I / 32;
  L.dn_tiles = H / 64;
  L.gu_tile_bytes = (size_t)L.nb_h * 1024 + (size_t)L.ng_h * 256;
  L.dn_tile_bytes = (size_t)L.nb_i * 1024 + (size_t)L.ng_i * 256;
  L.gu_bytes = L.gu_tile_bytes * L.gu_tiles;
  L.dn_bytes = L.dn_tile_bytes * L.dn_tiles;
  L.image_bytes = (L.gu_bytes + L.dn_bytes + 255) / 256 * 256;
  return L;
}

// Workspace: a fixed counter block, then per-call arrays sized for M tokens.
struct WsLayout {
  size_t route_ticket;   // uint32 [1]
  size_t dn_tickets;     // uint32 [dn_tiles]
  size_t counters_end;
  size_t logits;         // f32 [M][E]
  size_t route_slot;     // i32 [M*k]
  size_t counts;         // i32 [E]
  size_t offsets;        // i32 [E+1]
  size_t perm;           // i32 [M*k]
  size_t meta;           // i32 [8]: n_dist, cold_count, error flags
  size_t dist_expert;    // i32 [nd_max]
  size_t dist_slot;      // i32 [nd_max]
  size_t dist_off;       // i32 [nd_max]
  size_t dist_cnt;       // i32 [nd_max]
  size_t cold_list;      // i32 [M*k]
  size_t hbuf;           // bf16 [M*k][I]
  size_t pdn;            // f32 [M*k][kMaxKC][H]
  size_t total;
};

inline size_t align256(size_t v) { return (v + 255) / 256 * 256; }

inline WsLayout ws_layout(int H, int I, int E, int k, int M) {
  WsLayout W;
  const ImageLayout L = image_layout(H, I);
  const size_t Mk = (size_t)M * k;
  const size_t nd = Mk < (size_t)E ? Mk : (size_t)E;
  size_t o = 0;
  W.route_ticket = o;
  o += 4;
  W.dn_tickets = o;
  o += 4 * (size_t)L.dn_tiles;
  o = align256(o);
  W.counters_end = o;
  W.logits = o;      o = align256(o + 4 * (size_t)M * E);
  W.route_slot = o;  o = align256(o + 4 * Mk);
  W.counts = o;      o = align256(o + 4 * (size_t)E);
  W.offsets = o;     o = align256(o + 4 * ((size_t)E + 1));
  W.perm = o;        o = align256(o + 4 * Mk);
  W.meta = o;        o = align256(o + 4 * 8);
  W.dist_expert = o; o = align256(o + 4 * nd);
  W.dist_slot = o;   o = align256(o + 4 * nd);
  W.dist_off = o;    o = align256(o + 4 * nd);
  W.dist_cnt = o;    o = align256(o + 4 * nd);
  W.cold_list = o;   o = align256(o + 4 * Mk);
  W.hbuf = o;        o = align256(o + 2 * Mk * I);
  W.pdn = o;         o = align256(o + 4 * Mk * kMaxKC * (size_t)H);
  W.total = o;
  return W;
}

// Error flags raised by the device in meta[2].
enum : int32_t { kErrBadId = 1, kErrBadSlot = 2 };

}  // namespace moe
