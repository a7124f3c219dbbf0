// HIP kernels of libmoe for gfx950 (CDNA4, wave64).
//
//   k_router        bf16 router GEMV + bias, one wave per expert row (logits to the workspace).
//   k_topk_bucket   softmax / top-k / renormalise (one wave per token), then in one workgroup:
//                   route -> slot resolve, cold report, per-expert counts, DPP prefix scans,
//                   bucket permutation, list of distinct hot experts.
//   k_gateup        fused MXFP4 gate/up GEMV + SiLU(g)*u -> h (bf16) per route.  One workgroup
//                   per (distinct hot expert, 32-row tile), its waves split K.  For small
//                   calls each workgroup first rebuilds the route table (top-k, resolve,
//                   buckets) in LDS, which replaces the top-k / bucketing kernel.
//   k_down_combine  MXFP4 down GEMV of every hot route for a few output rows per workgroup,
//                   then y = ordered (ascending j) weighted sum of those routes.
// Dependencies between stages go through kernel boundaries only: a device-scope fence or a
// shared arrival counter per workgroup costs tens of nanoseconds each, serialised, on MI355X.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// =============================================================================================
// Router GEMV
// =============================================================================================
// grid.x = E (one wave per expert row); the wave keeps its row of W_r in registers (H/8 chunks
// of 8 bf16, chunk c = lane + 64*i) and reads the same chunks of every token's x.
constexpr int kRouterMaxChunksPerLane = kMaxHidden / 8 / 64;  // 16

__global__ __launch_bounds__(64) void k_router(const uint16_t* __restrict__ x, int M,
                                               const uint16_t* __restrict__ wr,
                                               const float* __restrict__ bias, int E, int H,
                                               float* __restrict__ logits) {
  const int lane = threadIdx.x;
  const int e = blockIdx.x;
  const int nch = H / 8;
  uint4 wrow[kRouterMaxChunksPerLane];
#pragma unroll
  for (int i = 0; i < kRouterMaxChunksPerLane; ++i) {
    const int c = lane + 64 * i;
    wrow[i] = c < nch ? reinterpret_cast<const uint4*>(wr + (size_t)e * H)[c] : make_uint4(0, 0, 0, 0);
  }
  const float b = bias != nullptr ? bias[e] : 0.0f;
  for (int m = 0; m < M; ++m) {
    const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)m * H);
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < kRouterMaxChunksPerLane; ++i) {
      const int c = lane + 64 * i;
      if (c < nch) {
        const uint4 xv = xr[c];
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wrow[i].x), as_bf16x2(xv.x), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wrow[i].y), as_bf16x2(xv.y), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wrow[i].z), as_bf16x2(xv.z), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wrow[i].w), as_bf16x2(xv.w), acc, false);
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) logits[(size_t)m * E + e] = acc + b;
  }
}

// Softmax / top-k / renormalise of one token by one wave: the k largest logits (ties to the
// lower id) in descending order and their softmax.
__device__ void topk_token(const float* __restrict__ lrow, int E, int k, int32_t* __restrict__ ids,
                           float* __restrict__ w) {
  constexpr int kMaxPerLane = kMaxExperts / 64;  // 16
  const int lane = threadIdx.x & 63;
  float v[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int ee = lane + 64 * i;
    v[i] = ee < E ? lrow[ee] : -INFINITY;
  }
  float my_v = -INFINITY, top = 0.0f;
  int my_i = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) argmax_step(bv, bi, v[i], lane + 64 * i);
    wave_argmax(bv, bi);  // uniform winner
    if (j == 0) top = bv;
    if (lane == j) {
      my_v = bv;
      my_i = bi;
    }
    if ((bi & 63) == lane) {
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i)
        if (i == (bi >> 6)) v[i] = -INFINITY;
    }
  }
  const float ex = lane < k ? expf(my_v - top) : 0.0f;
  const float den = wave_sum(ex);
  if (lane < k) {
    ids[lane] = my_i;
    w[lane] = ex / den;
  }
}

// =============================================================================================
// Route resolve + bucketing (one workgroup of kBucketThreads)
// =============================================================================================
// Exclusive scan of one value per thread over the whole workgroup; returns the total.
__device__ int block_exclusive_scan(int v, int* s_wave, int& total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int incl = wave_inclusive_scan(v);
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int t = lane < nw ? s_wave[lane] : 0;
    const int ti = wave_inclusive_scan(t);
    if (lane < nw) s_wave[lane] = ti - t;  // exclusive prefix of wave totals
    if (lane == nw - 1) s_wave[kBucketThreads / 64] = ti;
  }
  __syncthreads();
  const int out = s_wave[wave] + incl - v;
  total = s_wave[kBucketThreads / 64];
  __syncthreads();
  return out;
}

// Route resolve + bucketing by one workgroup (any multiple of 64 threads up to kBucketThreads):
// route -> slot, per-expert counts (LDS atomics), exclusive scans (DPP wave scans), bucket
// permutation, distinct hot experts in ascending id, cold routes in ascending order.
struct BucketSmem {
  int cnt[kMaxExperts];
  int off[kMaxExperts];
  int wave[kBucketThreads / 64 + 1];
  int err;
};

__device__ void bucket_stage(BucketSmem& sm, const int32_t* __restrict__ ids, int Mk, int E, int S,
                             const int32_t* __restrict__ e2s, int32_t* __restrict__ route_slot,
                             int32_t* __restrict__ ws_perm, int32_t* __restrict__ meta,
                             int32_t* __restrict__ dist_expert, int32_t* __restrict__ dist_slot,
                             int32_t* __restrict__ dist_off, int32_t* __restrict__ dist_cnt,
                             int nd_max, int32_t* __restrict__ cold_list,
                             int32_t* __restrict__ u_counts, int32_t* __restrict__ u_offsets,
                             int32_t* __restrict__ u_perm, int32_t* __restrict__ u_cold_count,
                             int32_t* __restrict__ u_cold_routes) {
  int* s_cnt = sm.cnt;
  int* s_off = sm.off;
  int* s_wave = sm.wave;
  int& s_err = sm.err;
  const int tid = threadIdx.x;
  if (tid == 0) s_err = 0;
  for (int e = tid; e < E; e += blockDim.x) s_cnt[e] = 0;
  __syncthreads();

  // resolve + count
  for (int r = tid; r < Mk; r += blockDim.x) {
    const int e = ids[r];
    int slot = -1;
    if (e >= 0 && e < E) {
      slot = e2s ? e2s[e] : e;
      if (slot < -1 || slot >= S) {
        atomicOr(&s_err, kErrBadSlot);
        slot = -1;
      }
      atomicAdd(&s_cnt[e], 1);
    } else {
      atomicOr(&s_err, kErrBadId);
    }
    route_slot[r] = slot;
  }
  __syncthreads();

  // offsets (exclusive scan over experts) and distinct hot experts (scan of flags)
  int running = 0, running_d = 0;
  for (int e0 = 0; e0 < E; e0 += blockDim.x) {
    const int e = e0 + tid;
    const int c = e < E ? s_cnt[e] : 0;
    int slot = -1;
    if (e < E && c > 0) {
      slot = e2s ? e2s[e] : e;
      if (slot < 0 || slot >= S) slot = -1;
    }
    const int hot = (c > 0 && slot >= 0) ? 1 : 0;
    int tot, tot_d;
    const int off = running + block_exclusive_scan(c, s_wave, tot);
    const int di = running_d + block_exclusive_scan(hot, s_wave, tot_d);
    if (e < E) {
      s_off[e] = off;
      if (u_counts) u_counts[e] = c;
      if (u_offsets) u_offsets[e] = off;
      if (hot && di < nd_max) {
        dist_expert[di] = e;
        dist_slot[di] = slot;
        dist_off[di] = off;
        dist_cnt[di] = c;
      }
    }
    running += tot;
    running_d += tot_d;
  }
  if (tid == 0) {
    if (u_offsets) u_offsets[E] = running;
    meta[0] = running_d < nd_max ? running_d : nd_max;
  }
  __syncthreads();

  // permutation: each route takes the next place of its expert's bucket
  for (int r = tid; r < Mk; r += blockDim.x) {
    const int e = ids[r];
    if (e >= 0 && e < E) {
      const int pos = atomicAdd(&s_off[e], 1);
      if (pos >= 0 && pos < Mk) {
        ws_perm[pos] = r;
        if (u_perm) u_perm[pos] = r;
      }
    }
  }

  // cold routes in ascending order
  int running_c = 0;
  for (int r0 = 0; r0 < Mk; r0 += blockDim.x) {
    const int r = r0 + tid;
    const int cold = (r < Mk && route_slot[r] < 0) ? 1 : 0;
    int tot;
    const int ci = running_c + block_exclusive_scan(cold, s_wave, tot);
    if (cold && ci < Mk) {
      cold_list[ci] = r;
      if (u_cold_routes) u_cold_routes[ci] = r;
    }
    running_c += tot;
  }
  if (tid == 0) {
    meta[1] = running_c;
    meta[2] = s_err;
    if (u_cold_count) *u_cold_count = running_c;
  }
}

// grid = ceil(M / 16) workgroups of kBucketThreads.  Stage 1 (logits != NULL): wave w of
// workgroup b does the top-k of tokens b*16 + w, b*16 + w + 16*gridDim.x, ...  Stage 2
// (do_bucket, single workgroup only): resolve and bucketing.
__global__ __launch_bounds__(kBucketThreads) void k_topk_bucket(
    const float* __restrict__ logits, int M, int k, int32_t* __restrict__ topk_ids,
    float* __restrict__ topk_w, int do_bucket,
    const int32_t* __restrict__ ids, int Mk, int E, int S, const int32_t* __restrict__ e2s,
    int32_t* __restrict__ route_slot, int32_t* __restrict__ ws_perm, int32_t* __restrict__ meta,
    int32_t* __restrict__ dist_expert, int32_t* __restrict__ dist_slot,
    int32_t* __restrict__ dist_off, int32_t* __restrict__ dist_cnt, int nd_max,
    int32_t* __restrict__ cold_list, int32_t* __restrict__ u_counts,
    int32_t* __restrict__ u_offsets, int32_t* __restrict__ u_perm,
    int32_t* __restrict__ u_cold_count, int32_t* __restrict__ u_cold_routes) {
  __shared__ BucketSmem sm;
  if (logits != nullptr) {
    const int nw = blockDim.x >> 6;
    for (int m = blockIdx.x * nw + (threadIdx.x >> 6); m < M; m += nw * gridDim.x)
      topk_token(logits + (size_t)m * E, E, k, topk_ids + (size_t)m * k, topk_w + (size_t)m * k);
    if (!do_bucket) return;
    __syncthreads();  // this workgroup's ids are visible to it from here on
  }
  if (blockIdx.x != 0) return;
  bucket_stage(sm, ids, Mk, E, S, e2s, route_slot, ws_perm, meta, dist_expert, dist_slot, dist_off,
               dist_cnt, nd_max, cold_list, u_counts, u_offsets, u_perm, u_cold_count,
               u_cold_routes);
}

// =============================================================================================
// Expert GEMVs
// =============================================================================================
// Both expert kernels stream one expert image tile per workgroup: 64 lanes x one 16-byte code
// chunk per K block (1 KiB per wave-wide load), 4 blocks per group, up to kMaxGroups groups
// per wave all loaded before any arithmetic so that every wave keeps up to 16 loads in flight.
// Each lane owns one output row; the activation block of the current token is uniform across
// the wave and comes through scalar loads.  The waves of a workgroup split K; their partial
// sums meet in LDS in a fixed order.
constexpr int kMaxGroups = 4;
constexpr int kMaxWaves = 16;
constexpr int kTokPerPass = 8;  // routes of one expert handled per pass (LDS rows)

// Loads the wave's K range: groups g0 .. g0+ngw-1 (ngw <= kMaxGroups, wave-uniform).  Blocks
// past the last one (nb % 4 != 0) re-read block nb-1 and are later weighted by zero.
template <int G>
__device__ __forceinline__ void load_tile_range(const uint4* __restrict__ codes,
                                                const uint32_t* __restrict__ scl, int nb, int g0,
                                                int ngw, int lane, uint32_t (&s4)[G],
                                                uint4 (&c)[4 * G]) {
#pragma unroll
  for (int q = 0; q < G; ++q) {
    if (q < ngw) {
      const int g = g0 + q;
      s4[q] = scl[g * 64 + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) c[4 * q + i] = codes[min(4 * g + i, nb - 1) * 64 + lane];
    }
  }
}

// Keeps the compiler from hoisting the decode of the loaded codes out of a token loop (which
// would need 16 VGPRs per block for every block at once).
template <int G>
__device__ __forceinline__ void opaque(uint4 (&c)[4 * G]) {
#pragma unroll
  for (int j = 0; j < 4 * G; ++j)
    asm volatile("" : "+v"(c[j].x), "+v"(c[j].y), "+v"(c[j].z), "+v"(c[j].w));
}

// Sum over the loaded blocks of scale * (codes . act block); act is uniform across the wave.
// Activations are fetched through the scalar unit two blocks (128 bytes, 32 SGPRs) at a time.
template <int G>
__device__ __forceinline__ float dot_tile_range(const uint4 (&c)[4 * G], const uint32_t (&s4)[G],
                                                int nb, int g0, int ngw,
                                                const uint16_t* __restrict__ act) {
  float acc = 0.0f;
#pragma unroll
  for (int q = 0; q < G; ++q) {
    if (q < ngw) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int b0 = 4 * (g0 + q) + 2 * p;
        const uint4* ag = reinterpret_cast<const uint4*>(act + 32 * b0);
        uint4 a[8];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const bool ok = b0 + i < nb;
#pragma unroll
          for (int j = 0; j < 4; ++j) a[4 * i + j] = ok ? ag[4 * i + j] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if (b0 + i < nb) {
            const float sc = e8m0_to_f32((s4[q] >> (8 * (2 * p + i))) & 0xFFu);
            acc = fmaf(sc, block_dot(c[4 * q + 2 * p + i], a[4 * i], a[4 * i + 1], a[4 * i + 2], a[4 * i + 3]), acc);
          }
        }
      }
    }
  }
  return acc;
}

// ---- routes of one call, as seen by an expert workgroup ---------------------------------------
// For up to kProMaxRoutes routes every expert workgroup rebuilds the route table itself in LDS
// (top-k from the logits or the given ids, slot resolve, distinct hot experts in ascending id,
// deterministic bucket order); larger calls read the table the bucketing kernel left in the
// workspace.  Rebuilding it costs a few hundred cycles and saves a kernel boundary.
constexpr int kProMaxRoutes = 256;

struct RouteLds {
  int ids[kProMaxRoutes];
  float w[kProMaxRoutes];
  int slot[kProMaxRoutes];
  int perm[kProMaxRoutes];
  int first[kProMaxRoutes];  // route is the first of its expert
  int cnt[kProMaxRoutes];    // routes of the route's expert
  int dist_slot[kProMaxRoutes];
  int dist_off[kProMaxRoutes];
  int dist_cnt[kProMaxRoutes];
  int nd;
};

__device__ void route_prologue(RouteLds& rt, const RouteArgs& a, bool writer) {
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int nw = nthr >> 6;
  const int Mk = a.M * a.k;
  if (tid == 0) rt.nd = 0;
  if (a.logits != nullptr) {
    for (int m = tid >> 6; m < a.M; m += nw)
      topk_token(a.logits + (size_t)m * a.E, a.E, a.k, rt.ids + m * a.k, rt.w + m * a.k);
  } else {
    for (int r = tid; r < Mk; r += nthr) {
      rt.ids[r] = a.ids_in[r];
      rt.w[r] = a.w_in[r];
    }
  }
  __syncthreads();
  for (int r = tid; r < Mk; r += nthr) {
    const int e = rt.ids[r];
    int slot = -1;
    if (e >= 0 && e < a.E) {
      slot = a.e2s ? a.e2s[e] : e;
      if (slot < 0 || slot >= a.S) slot = -1;
    }
    rt.slot[r] = slot;
    int c = 0, before = 0;
    for (int r2 = 0; r2 < Mk; ++r2) {
      if (rt.ids[r2] == e) {
        ++c;
        before += r2 < r;
      }
    }
    rt.cnt[r] = c;
    rt.first[r] = before == 0;
    if (writer && a.topk_ids != nullptr) {
      a.topk_ids[r] = e;
      a.topk_w[r] = rt.w[r];
    }
  }
  __syncthreads();
  for (int r = tid; r < Mk; r += nthr) {
    const int e = rt.ids[r];
    if (rt.slot[r] >= 0) {
      int di = 0, off = 0, pos = 0;
      for (int r2 = 0; r2 < Mk; ++r2) {
        const int e2 = rt.ids[r2];
        if (rt.slot[r2] >= 0 && rt.first[r2] && e2 < e) {
          ++di;
          off += rt.cnt[r2];
        }
        pos += (e2 == e && r2 < r);
      }
      rt.perm[off + pos] = r;
      if (rt.first[r]) {
        rt.dist_slot[di] = rt.slot[r];
        rt.dist_off[di] = off;
        rt.dist_cnt[di] = rt.cnt[r];
        atomicAdd(&rt.nd, 1);
      }
    } else if (writer && a.cold_routes != nullptr) {
      int ci = 0;
      for (int r2 = 0; r2 < r; ++r2) ci += rt.slot[r2] < 0;
      a.cold_routes[ci] = r;
    }
  }
  if (writer && a.cold_count != nullptr && tid < 64) {
    int c = 0;
    for (int r = tid; r < Mk; r += 64) c += rt.slot[r] < 0;
    c = (int)wave_sum((float)c);
    if (tid == 0) *a.cold_count = c;
  }
  __syncthreads();
}

// ---- gate/up + SiLU*up ----------------------------------------------------------------------
// grid = (I/32 tiles, nd_max); block = nw waves.  Lane l < 32 accumulates gate row 32*tile + l,
// lane l >= 32 the matching up row; wave w covers groups [w*ng/nw, (w+1)*ng/nw).
template <bool SINGLE, int G, bool PRO>
__global__ __launch_bounds__(kMaxWaves * 64) void k_gateup(
    const uint16_t* __restrict__ x, int H, int I, const uint8_t* __restrict__ slots,
    size_t image_bytes, size_t gu_tile_bytes, int nb, int ng, RouteArgs ra, RouteWs rw,
    uint16_t* __restrict__ hbuf) {
  __shared__ float red[kMaxWaves][SINGLE ? 1 : kTokPerPass][64];
  __shared__ RouteLds rt;
  const int tile = blockIdx.x;
  const int d = blockIdx.y;
  const int Mk = ra.M * ra.k;
  int slot, cnt, off;
  const int* perm;
  if (PRO) {
    route_prologue(rt, ra, tile == 0 && d == 0);
    if (d >= rt.nd) return;
    slot = rt.dist_slot[d];
    cnt = rt.dist_cnt[d];
    off = rt.dist_off[d];
    perm = rt.perm;
  } else {
    if (d >= rw.meta[0]) return;
    slot = rw.dist_slot[d];
    cnt = rw.dist_cnt[d];
    off = rw.dist_off[d];
    perm = rw.perm;
  }
  if (cnt <= 0 || off < 0 || off + cnt > Mk) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;

  const uint8_t* tbase = slots + (size_t)slot * image_bytes + (size_t)tile * gu_tile_bytes;
  const uint4* codes = reinterpret_cast<const uint4*>(tbase);
  const uint32_t* scl = reinterpret_cast<const uint32_t*>(tbase + (size_t)nb * 1024);
  const int g0 = wave * ng / nw;
  const int ngw = (wave + 1) * ng / nw - g0;
  uint32_t s4[G];
  uint4 c[4 * G];
  load_tile_range<G>(codes, scl, nb, g0, ngw, lane, s4, c);

  for (int base = 0; base < cnt; base += kTokPerPass) {
    const int nt = min(kTokPerPass, cnt - base);
    if (SINGLE) {  // one token per call: one route per expert, arithmetic overlaps the loads
      const int r = __builtin_amdgcn_readfirstlane(perm[off]);
      red[wave][0][lane] = dot_tile_range<G>(c, s4, nb, g0, ngw, x + (size_t)(r / ra.k) * H);
    } else {
#pragma unroll 1
      for (int t = 0; t < nt; ++t) {
        opaque<G>(c);
        const int r = __builtin_amdgcn_readfirstlane(perm[off + base + t]);
        red[wave][t][lane] = dot_tile_range<G>(c, s4, nb, g0, ngw, x + (size_t)(r / ra.k) * H);
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < nt * 32; idx += blockDim.x) {
      const int t = idx >> 5;
      const int row = idx & 31;
      float g = 0.0f, u = 0.0f;
      for (int w = 0; w < nw; ++w) {
        g += red[w][t][row];
        u += red[w][t][row + 32];
      }
      const int r = perm[off + base + t];
      hbuf[(size_t)r * I + tile * 32 + row] = (uint16_t)f32_to_bf16_bits(silu_f32(g) * u);
    }
    __syncthreads();
  }
}

// ---- down + ordered combine -----------------------------------------------------------------
// The down section of an image holds tiles of RD = 64/S rows.  Lane l = r*S + s of a wave owns
// row r of the tile and K segment s: at step t it holds block t*S + s of its row (steps past
// the last block hold nothing).  Steps with every lane active are 1 KiB each; the final,
// partial step stores only its active lanes, row by row.  Scale bytes follow the codes, four
// steps per lane word.
//
// grid = H/RD tiles; block = 4 waves.  A workgroup owns RD output rows for every hot route:
// wave w takes distinct experts w, w+4, ...; for each route of an expert the S lanes of a row
// add their segment sums (DPP), and the row result goes to `part`.  After a barrier the
// workgroup forms y[m][row] = sum over j ascending (hot routes) of w[m,j] * part[(m,j)][row]:
// no other workgroup is involved, so the combine needs no cross-workgroup synchronisation.
// h comes from LDS when every route fits (hp = 80-byte pitch per block, 64 used: the padding
// spreads the S segments of a row over distinct LDS banks), else straight from the workspace.
template <int S>
__device__ __forceinline__ float seg_sum(float v) {
  if (S >= 2) v += dpp_f<0xB1>(v);
  if (S >= 4) v += dpp_f<0x4E>(v);
  if (S >= 8) v += dpp_f<0x141>(v);
  return v;
}

constexpr int kDownWaves = 4;
constexpr int kDownMaxSteps = 16;

template <int S, bool PRO>
__global__ __launch_bounds__(kDownWaves * 64) void k_down_combine(
    int H, int I, const uint8_t* __restrict__ slots, size_t image_bytes, size_t gu_bytes,
    size_t dn_tile_bytes, int nb, int T, int tq, RouteArgs ra, RouteWs rw,
    const uint16_t* __restrict__ hbuf, int h_in_lds, int part_in_lds, float* __restrict__ pdn,
    float* __restrict__ y) {
  constexpr int RD = 64 / S;
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ RouteLds rt;
  const int tile = blockIdx.x;
  const int Mk = ra.M * ra.k;
  int nd;
  if (PRO) {
    route_prologue(rt, ra, false);
    nd = rt.nd;
  } else {
    nd = rw.meta[0];
  }
  const int* route_slot = PRO ? rt.slot : rw.route_slot;
  const float* wts = PRO ? rt.w : ra.w_in;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane / S;
  const int sg = lane % S;
  const int full = nb / S;      // steps with all lanes active
  const int rem = nb - full * S;  // active segments in the final partial step

  // The first expert's weights are requested before h is staged, so that both latencies overlap.
  const uint8_t* sec = slots + gu_bytes + (size_t)tile * dn_tile_bytes;
  const size_t code_bytes = ((size_t)full * 64 + (size_t)RD * rem) * 16;
  uint4 c[kDownMaxSteps];
  uint32_t s4[kDownMaxSteps / 4];
  auto load_expert = [&](int d) {
    const int slot = PRO ? rt.dist_slot[d] : rw.dist_slot[d];
    const uint8_t* tb = sec + (size_t)slot * image_bytes;
    const uint4* codes = reinterpret_cast<const uint4*>(tb);
#pragma unroll
    for (int t = 0; t < kDownMaxSteps; ++t) {
      if (t < full) c[t] = codes[t * 64 + lane];
      else if (t == full && sg < rem) c[t] = codes[full * 64 + r * rem + sg];
      else c[t] = make_uint4(0, 0, 0, 0);
    }
    const uint32_t* scl = reinterpret_cast<const uint32_t*>(tb + code_bytes);
#pragma unroll
    for (int q = 0; q < kDownMaxSteps / 4; ++q) s4[q] = q < tq ? scl[q * 64 + lane] : 0u;
  };
  if (wave < nd) load_expert(wave);

  // h of every hot route: LDS copy (pitch 80 B per block) or the workspace (pitch 64 B)
  const uint8_t* hsrc;
  int hpitch;
  if (h_in_lds) {
    uint8_t* hs = smem;
    for (int idx = threadIdx.x; idx < Mk * nb * 4; idx += blockDim.x) {
      const int route = idx / (nb * 4);
      const int rb = idx - route * nb * 4;
      if (route_slot[route] >= 0)
        *reinterpret_cast<uint4*>(hs + ((size_t)route * nb + (rb >> 2)) * 80 + (rb & 3) * 16) =
            *reinterpret_cast<const uint4*>(hbuf + (size_t)route * I + (rb >> 2) * 32 + (rb & 3) * 8);
    }
    hsrc = hs;
    hpitch = 80;
  } else {
    hsrc = reinterpret_cast<const uint8_t*>(hbuf);
    hpitch = 64;
  }
  float* part = part_in_lds ? reinterpret_cast<float*>(smem + (h_in_lds ? (size_t)Mk * nb * 80 : 0))
                            : pdn + (size_t)tile * Mk * RD;
  __syncthreads();

  for (int d = wave; d < nd; d += kDownWaves) {
    const int cnt = PRO ? rt.dist_cnt[d] : rw.dist_cnt[d];
    const int off = PRO ? rt.dist_off[d] : rw.dist_off[d];
    const int* perm = PRO ? rt.perm : rw.perm;
    if (d != wave) load_expert(d);
    if (cnt <= 0 || off < 0 || off + cnt > Mk) continue;
#pragma unroll 1
    for (int j = 0; j < cnt; ++j) {
      const int route = perm[off + j];
      const uint8_t* hr = hsrc + (size_t)route * nb * hpitch;
      float acc = 0.0f;
#pragma unroll
      for (int t = 0; t < kDownMaxSteps; ++t) {
        const int b = t * S + sg;
        if (t < T && b < nb) {
          const uint4* a = reinterpret_cast<const uint4*>(hr + (size_t)b * hpitch);
          const float sc = e8m0_to_f32((s4[t >> 2] >> (8 * (t & 3))) & 0xFFu);
          acc = fmaf(sc, block_dot(c[t], a[0], a[1], a[2], a[3]), acc);
        }
      }
      acc = seg_sum<S>(acc);
      if (sg == 0) part[route * RD + r] = acc;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < ra.M * RD; idx += blockDim.x) {
    const int m = idx / RD;
    const int rr = idx - m * RD;
    float acc = 0.0f;
    for (int j = 0; j < ra.k; ++j) {
      const int route = m * ra.k + j;
      if (route_slot[route] >= 0) acc = fmaf(wts[route], part[route * RD + rr], acc);
    }
    y[(size_t)m * H + tile * RD + rr] = acc;
  }
}


// =============================================================================================
// Launchers (called from the host API after every argument has been validated)
// =============================================================================================
hipError_t launch_router(const uint16_t* x, int M, const uint16_t* wr, const float* bias, int E,
                         int H, float* logits, hipStream_t s) {
  hipLaunchKernelGGL(k_router, dim3(E), dim3(64), 0, s, x, M, wr, bias, E, H, logits);
  return hipGetLastError();
}

hipError_t launch_topk_bucket(const float* logits, int M, int k, int32_t* topk_ids, float* topk_w,
                              bool do_bucket, const int32_t* ids, int E, int S,
                              const int32_t* e2s, const BucketOut& o, hipStream_t s) {
  const int Mk = M * k;
  const int nd_max = Mk < E ? Mk : E;
  const int per_wg = kBucketThreads / 64;
  if (logits != nullptr && do_bucket && M > per_wg) {
    // many tokens: a multi-workgroup top-k, then the single-workgroup bucketing
    hipError_t e = launch_topk_bucket(logits, M, k, topk_ids, topk_w, false, ids, E, S, e2s, o, s);
    if (e != hipSuccess) return e;
    return launch_topk_bucket(nullptr, M, k, nullptr, nullptr, true, ids, E, S, e2s, o, s);
  }
  const int grid = (logits != nullptr && !do_bucket) ? (M + per_wg - 1) / per_wg : 1;
  hipLaunchKernelGGL(k_topk_bucket, dim3(grid > 0 ? grid : 1), dim3(kBucketThreads), 0, s, logits,
                     M, k, topk_ids, topk_w, do_bucket ? 1 : 0, ids, Mk, E, S, e2s, o.route_slot,
                     o.ws_perm, o.meta, o.dist_expert, o.dist_slot, o.dist_off, o.dist_cnt, nd_max,
                     o.cold_list, o.u_counts, o.u_offsets, o.u_perm, o.u_cold_count,
                     o.u_cold_routes);
  return hipGetLastError();
}


constexpr int kNumCUs = 256;      // MI355X compute units
constexpr int kWavesPerCU = 16;   // resident waves per CU for a kernel of <= 128 VGPRs

ExpertPlan plan_experts(const ImageLayout& L, int M, int E, int k) {
  ExpertPlan p;
  const int Mk = M * k;
  p.nd_max = Mk < E ? Mk : E;
  p.prologue = Mk <= kProMaxRoutes;
  // gate/up waves per workgroup: each wave holds at most kMaxGroups groups of its tile's K;
  // the kernels are built for <= 128 VGPRs, so a CU holds kWavesPerCU waves.  Pick the widest
  // workgroup that still lets every workgroup of the grid be resident at once.
  const int units = L.gu_tiles * p.nd_max;
  const int lo = (L.ng_h + kMaxGroups - 1) / kMaxGroups;
  const int hi = L.ng_h < kMaxWaves ? L.ng_h : kMaxWaves;
  int best = lo < hi ? lo : hi, best_rounds = 1 << 30;
  for (int w = (lo < hi ? lo : hi); w <= hi; ++w) {
    const int per_cu = kWavesPerCU / w > 0 ? kWavesPerCU / w : 1;
    const int rounds = (units + kNumCUs * per_cu - 1) / (kNumCUs * per_cu);
    if (rounds < best_rounds || (rounds == best_rounds && w > best)) {
      best = w;
      best_rounds = rounds;
    }
  }
  p.gu_waves = best < 1 ? 1 : best;
  p.gu_groups = (L.ng_h + p.gu_waves - 1) / p.gu_waves;
  // down: h in LDS when every route's h fits, partial sums in LDS when they fit
  const size_t h_lds = (size_t)Mk * L.nb_i * 80;
  const size_t part = (size_t)Mk * L.dn_rows * 4;
  p.h_in_lds = h_lds + part <= kDownLdsBudget;
  p.part_in_lds = (p.h_in_lds ? h_lds : 0) + part <= kDownLdsBudget;
  p.dn_lds = (p.h_in_lds ? h_lds : 0) + (p.part_in_lds ? part : 0);
  return p;
}

hipError_t launch_gateup(const uint16_t* x, int M, int H, int I, const uint8_t* slots,
                         const ImageLayout& L, const ExpertPlan& p, const RouteArgs& ra,
                         const RouteWs& rw, uint16_t* hbuf, hipStream_t s) {
  const dim3 g(L.gu_tiles, p.nd_max), b(p.gu_waves * 64);
#define MOE_GU(SINGLE, G, PRO)                                                                     \
  hipLaunchKernelGGL((k_gateup<SINGLE, G, PRO>), g, b, 0, s, x, H, I, slots, L.image_bytes,      \
                     L.gu_tile_bytes, L.nb_h, L.ng_h, ra, rw, hbuf)
  // the single-token variant lets arithmetic overlap the loads but holds more registers, so
  // it is only used with at most 3 groups per wave
  const bool single = M == 1 && p.gu_groups <= 3;
  if (p.prologue) {
    if (single) {
      if (p.gu_groups <= 1) MOE_GU(true, 1, true);
      else if (p.gu_groups == 2) MOE_GU(true, 2, true);
      else MOE_GU(true, 3, true);
    } else {
      if (p.gu_groups <= 2) MOE_GU(false, 2, true);
      else MOE_GU(false, 4, true);
    }
  } else {
    if (p.gu_groups <= 2) MOE_GU(false, 2, false);
    else MOE_GU(false, 4, false);
  }
#undef MOE_GU
  return hipGetLastError();
}

hipError_t launch_down(int M, int H, int I, const uint8_t* slots, const ImageLayout& L,
                       const ExpertPlan& p, const RouteArgs& ra, const RouteWs& rw,
                       const uint16_t* hbuf, float* pdn, float* y, hipStream_t s) {
  const dim3 g(L.dn_tiles), b(kDownWaves * 64);
#define MOE_DN(SEG, PRO)                                                                          \
  hipLaunchKernelGGL((k_down_combine<SEG, PRO>), g, b, p.dn_lds, s, H, I, slots, L.image_bytes, \
                     L.gu_bytes, L.dn_tile_bytes, L.nb_i, L.dn_steps, L.dn_scale_words, ra, rw,  \
                     hbuf, p.h_in_lds ? 1 : 0, p.part_in_lds ? 1 : 0, pdn, y)
  switch (L.dn_seg * 2 + (p.prologue ? 1 : 0)) {
    case 2 * 8 + 1: MOE_DN(8, true); break;
    case 2 * 8: MOE_DN(8, false); break;
    case 2 * 4 + 1: MOE_DN(4, true); break;
    case 2 * 4: MOE_DN(4, false); break;
    case 2 * 2 + 1: MOE_DN(2, true); break;
    case 2 * 2: MOE_DN(2, false); break;
    case 2 * 1 + 1: MOE_DN(1, true); break;
    default: MOE_DN(1, false); break;
  }
#undef MOE_DN
  return hipGetLastError();
}

}  // namespace moe
