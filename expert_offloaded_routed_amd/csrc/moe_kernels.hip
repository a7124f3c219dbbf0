// HIP kernels of libmoe for gfx950 (CDNA4, wave64).
//
//   k_router        bf16 router GEMV + bias, one wave per expert row (logits to the workspace).
//   k_topk_bucket   softmax / top-k / renormalise (one wave per token), then in one workgroup:
//                   route -> slot resolve, cold report, per-expert counts, DPP prefix scans,
//                   bucket permutation, list of distinct hot experts, grouped work list.
//   k_gateup        fused MXFP4 gate/up GEMV + SiLU(g)*u -> h per route (split for the matrix
//                   cores).  One workgroup per (distinct hot expert, 32-row tile), its waves
//                   split K.  For small calls each workgroup first rebuilds the route table
//                   (top-k, resolve, buckets) in LDS, which replaces the top-k / bucketing kernel.
//   k_down_mx       down projection of every hot route on the block-scaled MFMA (E2M1 weights,
//                   h as two E4M3 terms), per (expert, routes) item -> fp32 partial rows;
//   k_combine       then y = ordered (ascending j) weighted sum of those rows.
//   k_layer_decode  one token: gate/up and down (with the combine) in one launch.
//   k_gateup_grouped / k_router_grouped: bf16 MFMA GEMMs for many tokens.
// Dependencies between stages go through kernel boundaries, except inside k_layer_decode, which
// hands h over by value (see there): a device-scope fence per workgroup costs tens of
// nanoseconds, serialised, on MI355X.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// =============================================================================================
// Router GEMV
// =============================================================================================
// grid.x = E (one wave per expert row); the wave keeps its row of W_r in registers (H/8 chunks
// of 8 bf16, chunk c = lane + 64*i) and reads the same chunks of every token's x.

// CPL = ceil(H/8/64) chunks per lane.  Every load is issued unconditionally (chunk index
// clamped, the product of a chunk past the row selected away), so that no load waits alone in
// a branch.  The x rows of TG tokens are requested together (one cache round trip for the group
// instead of one a token); each token's sum is formed exactly as alone.
template <int CPL, int TG>
__device__ __forceinline__ void router_tokens(const uint16_t* __restrict__ x, int m0, int nch,
                                              int H, int E, int e, float b,
                                              const uint4 (&wrow)[CPL], float* __restrict__ logits) {
  const int lane = threadIdx.x;
  uint4 xv[TG][CPL];
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)(m0 + t) * H);
#pragma unroll
    for (int i = 0; i < CPL; ++i) xv[t][i] = xr[min(lane + 64 * i, nch - 1)];
  }
  float acc[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    acc[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const float v = dot8_bf16(wrow[i], xv[t][i], acc[t]);
      acc[t] = lane + 64 * i < nch ? v : acc[t];
    }
  }
#pragma unroll
  for (int t = 0; t < TG; ++t) acc[t] = wave_sum(acc[t]);
  if (lane == 0)
#pragma unroll
    for (int t = 0; t < TG; ++t) logits[(size_t)(m0 + t) * E + e] = acc[t] + b;
}

template <int CPL>
__global__ __launch_bounds__(64) void k_router(const uint16_t* __restrict__ x, int M,
                                               const uint16_t* __restrict__ wr,
                                               const float* __restrict__ bias, int E, int H,
                                               float* __restrict__ logits) {
  const int lane = threadIdx.x;
  const int e = blockIdx.x;
  const int nch = H / 8;
  const uint4* wsrc = reinterpret_cast<const uint4*>(wr + (size_t)e * H);
  uint4 wrow[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) wrow[i] = ld_nt(wsrc + min(lane + 64 * i, nch - 1));
  const float b = bias != nullptr ? bias[e] : 0.0f;
  // groups of tokens whose x rows fit beside the row in registers (at most 32 chunks a lane)
  constexpr int TG = 32 / CPL >= 8 ? 8 : (32 / CPL >= 4 ? 4 : (32 / CPL >= 2 ? 2 : 1));
  int m = 0;
  for (; m + TG <= M; m += TG) router_tokens<CPL, TG>(x, m, nch, H, E, e, b, wrow, logits);
  if constexpr (TG > 4)
    if (m + 4 <= M) {
      router_tokens<CPL, 4>(x, m, nch, H, E, e, b, wrow, logits);
      m += 4;
    }
  if constexpr (TG > 2)
    if (m + 2 <= M) {
      router_tokens<CPL, 2>(x, m, nch, H, E, e, b, wrow, logits);
      m += 2;
    }
  if (m < M) router_tokens<CPL, 1>(x, m, nch, H, E, e, b, wrow, logits);
}

// Softmax / top-k / renormalise of one token by one wave: the k largest logits in descending
// order (ties to the lower id; NaN ranks below every number) and their softmax, which equals
// the full softmax renormalised over the k routes.
//
// E <= 64: lane e holds logit e and counts the logits that rank above it (k independent of the
// cost).  Larger E: k rounds of a wave argmax over PL logits per lane.
__device__ __forceinline__ float rank_key(float v) { return v != v ? -INFINITY : v; }

// A logit's value key: a monotone 32-bit image of the value (NaN as -inf, -0 as +0), never
// zero.  The 64-bit rank key adds the bitwise complement of the id in the low word, so that
// ties go to the lower id.
__device__ __forceinline__ uint32_t value_key(float v) {
  v = rank_key(v);
  if (v == 0.0f) v = 0.0f;
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t rank_key64(float v, int id) {
  return ((uint64_t)value_key(v) << 32) | (uint32_t)~(uint32_t)id;
}
// Number of lanes j < E (E <= 64) whose key is larger than this lane's (keys are distinct):
// the lane's rank.  One 64-bit compare per lane j on a broadcast key, all in the vector unit.
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int j) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, j);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), j);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ int key_rank(uint64_t key, int E) {
  int rank = 0;
  for (int j = 0; j < E; ++j) rank += readlane_u64(key, j) > key ? 1 : 0;
  return rank;
}

// Logit e of a row held as P partial sums P_STRIDE floats apart, summed in ascending order.
template <int P>
__device__ __forceinline__ float logit_at(const float* __restrict__ lrow, size_t pstride, int e) {
  float v = lrow[e];
#pragma unroll
  for (int z = 1; z < P; ++z) v += lrow[z * pstride + e];
  return v;
}

template <int P>
__device__ void topk_rank(const float* __restrict__ lrow, size_t pstride, int E, int k,
                          int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  // unconditional loads (a load in a branch is waited for alone)
  const float lv = logit_at<P>(lrow, pstride, min(lane, E - 1));
  const float v = lane < E ? rank_key(lv) : -INFINITY;
  const int rank = key_rank(rank_key64(lv, lane), E);
  const bool sel = lane < E && rank < k;
  const uint64_t first = __ballot(lane < E && rank == 0);
  const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), (int)__ffsll((long long)first) - 1));
  const float ex = sel ? expf(v - top) : 0.0f;
  const float den = wave_sum(ex);
  if (sel) {
    ids[rank] = lane;
    w[rank] = ex / den;
  }
}

__device__ __forceinline__ float key_value32(uint32_t h) {
  return __uint_as_float((h & 0x80000000u) ? (h ^ 0x80000000u) : ~h);
}
__device__ __forceinline__ float key_value(uint64_t key) { return key_value32((uint32_t)(key >> 32)); }
__device__ __forceinline__ int key_id(uint64_t key) { return (int)~(uint32_t)key; }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)dpp_i<0xB1>((int)v));
  v = max(v, (uint32_t)dpp_i<0x4E>((int)v));
  v = max(v, (uint32_t)dpp_i<0x141>((int)v));
  v = max(v, (uint32_t)dpp_i<0x140>((int)v));
  v = max(v, (uint32_t)swz_xor16_i((int)v));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  return max(a, b);
}

// 64 < E: lane l holds the value keys of experts l, l + 64, ... (PL of them); then k rounds of:
// the wave's largest value key (each lane's best, then DPP / swizzle / readlane on 32 bits),
// the lowest expert id holding it (one ballot per register, lowest register first: ids in
// register i are 64 i .. 64 i + 63), and that key cleared.  Ties thus go to the lower id, as
// with the 64-bit rank keys.  All branch-free; the id search runs on the scalar unit.
template <int PL, int P>
__device__ void topk_argmax(const float* __restrict__ lrow, size_t pstride, int E, int k,
                            int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  float lv[PL];
  uint32_t key[PL];
  // every load issued before any is used (clamped in range; loads in a branch would each be
  // waited for alone); slots past E get key 0, below every real key
#pragma unroll
  for (int i = 0; i < PL; ++i) lv[i] = logit_at<P>(lrow, pstride, min(lane + 64 * i, E - 1));
#pragma unroll
  for (int i = 0; i < PL; ++i) key[i] = lane + 64 * i < E ? value_key(lv[i]) : 0u;
  uint32_t mine = 0u;  // lane j < k: the j-th value key and its id
  int mine_id = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t best = key[0];
#pragma unroll
    for (int i = 1; i < PL; ++i) best = max(best, key[i]);
    best = wave_max_u32(best);  // uniform
    int id = 0;
#pragma unroll
    for (int i = PL - 1; i >= 0; --i) {
      const uint64_t b = __ballot(key[i] == best);
      id = b != 0 ? 64 * i + (int)__ffsll((long long)b) - 1 : id;
    }
    id = __builtin_amdgcn_readfirstlane(id);
    mine = lane == j ? best : mine;
    mine_id = lane == j ? id : mine_id;
#pragma unroll
    for (int i = 0; i < PL; ++i) key[i] = lane + 64 * i == id ? 0u : key[i];
  }
  const float v = key_value32(mine);
  const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float ex = lane < k ? expf(v - top) : 0.0f;
  const float den = wave_sum(ex);
  if (lane < k) {
    ids[lane] = mine_id;
    w[lane] = ex / den;
  }
}

// The logit row may be held as P partial sums pstride floats apart (the K-split router GEMM).
// (Split rows are produced for at most kRouterMaxE experts.)
template <int P>
__device__ void topk_token_p(const float* __restrict__ lrow, size_t pstride, int E, int k,
                             int32_t* __restrict__ ids, float* __restrict__ w) {
  if (E <= 64) topk_rank<P>(lrow, pstride, E, k, ids, w);
  else if (E <= 128) topk_argmax<2, P>(lrow, pstride, E, k, ids, w);
  else if (E <= 256) topk_argmax<4, P>(lrow, pstride, E, k, ids, w);
  else if (P > 1 || E <= 512) topk_argmax<8, P>(lrow, pstride, E, k, ids, w);
  else topk_argmax<16, P>(lrow, pstride, E, k, ids, w);
}
__device__ void topk_token(const float* __restrict__ lrow, int E, int k, int32_t* __restrict__ ids,
                           float* __restrict__ w, int parts = 1, size_t pstride = 0) {
  if (parts == kRouterParts) topk_token_p<kRouterParts>(lrow, pstride, E, k, ids, w);
  else topk_token_p<1>(lrow, pstride, E, k, ids, w);
}

// =============================================================================================
// Route resolve + bucketing (one workgroup of kBucketThreads)
// =============================================================================================
// Workgroup barrier ordering LDS only: global loads in flight stay in flight across it, and
// global stores are not waited for (a full barrier waits for every store to complete).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Exclusive scan of one value per thread over the whole workgroup; returns the total.  Its
// barriers order LDS only.
__device__ int block_exclusive_scan(int v, int* s_wave, int& total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int incl = wave_inclusive_scan(v);
  if (lane == 63) s_wave[wave] = incl;
  lds_barrier();
  if (wave == 0) {
    const int t = lane < nw ? s_wave[lane] : 0;
    const int ti = wave_inclusive_scan(t);
    if (lane < nw) s_wave[lane] = ti - t;  // exclusive prefix of wave totals
    if (lane == nw - 1) s_wave[kBucketThreads / 64] = ti;
  }
  lds_barrier();
  const int out = s_wave[wave] + incl - v;
  total = s_wave[kBucketThreads / 64];
  lds_barrier();
  return out;
}

// Exclusive scans of three values per thread over the whole workgroup at once (one set of
// barriers for the three): out[c] = the prefix of value c, total[c] = its sum.
__device__ void block_exclusive_scan3(const int (&v)[3], int (*s_wave)[kBucketThreads / 64 + 1],
                                      int (&out)[3], int (&total)[3]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  int incl[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) incl[c] = wave_inclusive_scan(v[c]);
  if (lane == 63)
#pragma unroll
    for (int c = 0; c < 3; ++c) s_wave[c][wave] = incl[c];
  lds_barrier();
  if (wave == 0) {
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      const int t = lane < nw ? s_wave[c][lane] : 0;
      const int ti = wave_inclusive_scan(t);
      if (lane < nw) s_wave[c][lane] = ti - t;  // exclusive prefix of wave totals
      if (lane == nw - 1) s_wave[c][kBucketThreads / 64] = ti;
    }
  }
  lds_barrier();
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    out[c] = s_wave[c][wave] + incl[c] - v[c];
    total[c] = s_wave[c][kBucketThreads / 64];
  }
  lds_barrier();
}

// Route resolve + bucketing by one workgroup (any multiple of 64 threads up to kBucketThreads):
// route -> slot, per-expert counts (LDS atomics), exclusive scans (DPP wave scans), bucket
// permutation, distinct hot experts in ascending id, cold routes in ascending order.
// Routes r = tid + j*blockDim.x with j < kBucketRegRoutes keep their expert and slot in
// registers across the stages below (each stage would otherwise wait on its own global reads).
constexpr int kBucketRegRoutes = 8;

struct BucketSmem {
  int cnt[kMaxExperts];
  int off[kMaxExperts];
  int slot[kMaxExperts];  // resolved slot of every expert that has a route (-1: cold)
  int wave[kBucketThreads / 64 + 1];
  int wave3[3][kBucketThreads / 64 + 1];
  int err;
  // the top-k of the single-workgroup call (at most one token a wave), handed to the bucketing
  // in LDS
  int32_t tk_ids[kBucketThreads / 64 * kMaxTopK];
  float tk_w[kBucketThreads / 64 * kMaxTopK];
  int32_t e2s[kMaxExperts];  // the expert map, copied while the top-k runs (same call)
};

__device__ void bucket_stage(BucketSmem& sm, const int32_t* __restrict__ ids, int Mk, int E, int S,
                             const int32_t* __restrict__ e2s, int32_t* __restrict__ route_slot,
                             int32_t* __restrict__ ws_perm, int32_t* __restrict__ meta,
                             int4* __restrict__ dist, int nd_max, int2* __restrict__ items,
                             int n_items_max, int32_t* __restrict__ cold_list,
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
  lds_barrier();

  // resolve + count (every expert with a route also records its slot: equal writes)
  const int bd = blockDim.x;
  const int nreg = min(kBucketRegRoutes, (Mk + bd - 1) / bd);  // uniform: passes that have routes
  int e_r[kBucketRegRoutes], s_r[kBucketRegRoutes];
#pragma unroll
  for (int j = 0; j < kBucketRegRoutes; ++j) {
    const int r = tid + j * bd;
    e_r[j] = j < nreg && r < Mk ? ids[r] : 0;
    s_r[j] = 0;
  }
#pragma unroll
  for (int j = 0; j < kBucketRegRoutes; ++j) {
    if (j >= nreg) break;
    const bool ok = tid + j * bd < Mk && e_r[j] >= 0 && e_r[j] < E;
    s_r[j] = e2s && ok ? e2s[e_r[j]] : e_r[j];
  }
  auto resolve = [&](int r, int e, int slot) {
    if (e >= 0 && e < E) {
      if (slot < -1 || slot >= S) {
        atomicOr(&s_err, kErrBadSlot);
        slot = -1;
      }
      atomicAdd(&s_cnt[e], 1);
      sm.slot[e] = slot;
    } else {
      atomicOr(&s_err, kErrBadId);
      slot = -1;
    }
    route_slot[r] = slot;
    return slot;
  };
#pragma unroll
  for (int j = 0; j < kBucketRegRoutes; ++j) {
    if (j >= nreg) break;
    const int r = tid + j * bd;
    if (r < Mk) s_r[j] = resolve(r, e_r[j], s_r[j]);
  }
  for (int r = tid + kBucketRegRoutes * bd; r < Mk; r += bd) {
    const int e = ids[r];
    resolve(r, e, e >= 0 && e < E ? (e2s ? e2s[e] : e) : -1);
  }
  // (the cold list reads route_slot back when a thread has more than one route: then the
  // barrier also waits for those stores)
  if (Mk > bd)
    __syncthreads();
  else
    lds_barrier();

  // offsets (exclusive scan over experts), distinct hot experts (scan of flags) and the work
  // list of the grouped GEMM: one item per (distinct hot expert, pass of kItemRoutes routes)
  int running = 0, running_d = 0, running_i = 0;
  for (int e0 = 0; e0 < E; e0 += blockDim.x) {
    const int e = e0 + tid;
    const int c = e < E ? s_cnt[e] : 0;
    const int slot = e < E && c > 0 ? sm.slot[e] : -1;
    const int hot = (c > 0 && slot >= 0) ? 1 : 0;
    const int np = hot ? (c + kItemRoutes - 1) / kItemRoutes : 0;
    int ex[3], tt[3];
    block_exclusive_scan3({c, hot, np}, sm.wave3, ex, tt);
    const int off = running + ex[0], di = running_d + ex[1], ii = running_i + ex[2];
    const int tot = tt[0], tot_d = tt[1], tot_i = tt[2];
    if (e < E) {
      s_off[e] = off;
      if (u_counts) u_counts[e] = c;
      if (u_offsets) u_offsets[e] = off;
      if (hot && di < nd_max) {
        dist[di] = make_int4(slot, off, c, e);
        if (items != nullptr)
          for (int p = 0; p < np && ii + p < n_items_max; ++p) items[ii + p] = make_int2(di, p * kItemRoutes);
      }
    }
    running += tot;
    running_d += tot_d;
    running_i += tot_i;
  }
  if (tid == 0) {
    if (u_offsets) u_offsets[E] = running;
    meta[0] = running_d < nd_max ? running_d : nd_max;
    meta[3] = running_i < n_items_max ? running_i : n_items_max;
  }
  lds_barrier();

  // permutation: each route takes the next place of its expert's bucket
  auto place = [&](int r, int e) {
    if (e >= 0 && e < E) {
      const int pos = atomicAdd(&s_off[e], 1);
      if (pos >= 0 && pos < Mk) {
        ws_perm[pos] = r;
        if (u_perm) u_perm[pos] = r;
      }
    }
  };
#pragma unroll
  for (int j = 0; j < kBucketRegRoutes; ++j) {
    if (j >= nreg) break;
    if (tid + j * bd < Mk) place(tid + j * bd, e_r[j]);
  }
  for (int r = tid + kBucketRegRoutes * bd; r < Mk; r += bd) place(r, ids[r]);

  // cold routes in ascending order.  One route a thread: its slot is in registers.  Up to
  // kBucketRegRoutes a thread: thread t takes the consecutive routes [t*per, t*per + per), their
  // slots read back together (written by the resolve above, before a barrier), so that one scan
  // orders all of them.  Beyond that, one scan per pass of blockDim.x routes.
  int running_c = 0;
  const int per = (Mk + bd - 1) / bd;
  if (per <= 1) {
    const int cold = tid < Mk && s_r[0] < 0 ? 1 : 0;
    int tot;
    const int ci = block_exclusive_scan(cold, s_wave, tot);
    if (cold && ci < Mk) {
      cold_list[ci] = tid;
      if (u_cold_routes) u_cold_routes[ci] = tid;
    }
    running_c = tot;
  } else if (per <= kBucketRegRoutes) {
    const int r0 = tid * per;
    int sv[kBucketRegRoutes];
#pragma unroll
    for (int q = 0; q < kBucketRegRoutes; ++q) sv[q] = q < per && r0 + q < Mk ? route_slot[r0 + q] : 0;
    int nc = 0;
#pragma unroll
    for (int q = 0; q < kBucketRegRoutes; ++q) nc += sv[q] < 0 ? 1 : 0;
    int tot;
    int ci = block_exclusive_scan(nc, s_wave, tot);
#pragma unroll
    for (int q = 0; q < kBucketRegRoutes; ++q)
      if (sv[q] < 0 && ci < Mk) {
        cold_list[ci] = r0 + q;
        if (u_cold_routes) u_cold_routes[ci] = r0 + q;
        ++ci;
      }
    running_c = tot;
  } else {
    for (int r0 = 0; r0 < Mk; r0 += blockDim.x) {
      const int r = r0 + tid;
      const int j = r0 / bd;
      int sl = 0;
#pragma unroll
      for (int i = 0; i < kBucketRegRoutes; ++i) sl = i == j ? s_r[i] : sl;
      const int cold = r < Mk && (j < kBucketRegRoutes ? sl : route_slot[r]) < 0 ? 1 : 0;
      int tot;
      const int ci = running_c + block_exclusive_scan(cold, s_wave, tot);
      if (cold && ci < Mk) {
        cold_list[ci] = r;
        if (u_cold_routes) u_cold_routes[ci] = r;
      }
      running_c += tot;
    }
  }
  if (tid == 0) {
    meta[1] = running_c;
    if (s_err != 0) atomicOr(&meta[kMetaErr], s_err);  // the error word only accumulates
    if (u_cold_count) *u_cold_count = running_c;
  }
}

// Stage 1 (logits != NULL): wave w of workgroup b does the top-k of tokens b*nw + w,
// b*nw + w + nw*gridDim.x, ... (nw waves per workgroup: kTopkThreads / 64 when the top-k runs
// alone, else kBucketThreads / 64).  Stage 2 (do_bucket, single workgroup of kBucketThreads
// only): resolve and bucketing.
__global__ __launch_bounds__(kBucketThreads) void k_topk_bucket(
    const float* __restrict__ logits, int M, int k, int32_t* __restrict__ topk_ids,
    float* __restrict__ topk_w, int do_bucket,
    const int32_t* __restrict__ ids, int Mk, int E, int S, const int32_t* __restrict__ e2s,
    int32_t* __restrict__ route_slot, int32_t* __restrict__ ws_perm, int32_t* __restrict__ meta,
    int4* __restrict__ dist, int nd_max, int2* __restrict__ items, int n_items_max,
    int32_t* __restrict__ cold_list, int32_t* __restrict__ u_counts,
    int32_t* __restrict__ u_offsets, int32_t* __restrict__ u_perm,
    int32_t* __restrict__ u_cold_count, int32_t* __restrict__ u_cold_routes) {
  __shared__ BucketSmem sm;
  if (logits != nullptr) {
    const int nw = blockDim.x >> 6;
    // one workgroup doing both stages with the bucketing reading the top-k's ids: the top-k
    // goes to LDS (no global round trip), then to the outputs
    const bool lds = do_bucket && gridDim.x == 1 && M <= nw && k <= kMaxTopK && ids == topk_ids;
    int32_t* oid = lds ? sm.tk_ids : topk_ids;
    float* ow = lds ? sm.tk_w : topk_w;
    // ... and the expert map to LDS: requested before the top-k (one entry a thread), stored
    // after it, so that its latency overlaps the top-k
    const bool map_lds = lds && e2s != nullptr && E <= (int)blockDim.x;
    const int e2v = map_lds && (int)threadIdx.x < E ? e2s[threadIdx.x] : 0;
    for (int m = blockIdx.x * nw + (threadIdx.x >> 6); m < M; m += nw * gridDim.x)
      topk_token(logits + (size_t)m * E, E, k, oid + (size_t)m * k, ow + (size_t)m * k,
                 router_parts(M, E), (size_t)M * E);
    if (!do_bucket) return;
    if (map_lds && (int)threadIdx.x < E) sm.e2s[threadIdx.x] = e2v;
    // this workgroup's ids are visible to it from here on (in LDS, or in global memory: then the
    // barrier waits for the stores)
    if (lds)
      lds_barrier();
    else
      __syncthreads();
    if (lds) {
      for (int i = threadIdx.x; i < Mk; i += blockDim.x) {
        topk_ids[i] = sm.tk_ids[i];
        topk_w[i] = sm.tk_w[i];
      }
      ids = sm.tk_ids;
      if (map_lds) e2s = sm.e2s;
    }
  }
  if (blockIdx.x != 0) return;
  bucket_stage(sm, ids, Mk, E, S, e2s, route_slot, ws_perm, meta, dist, nd_max, items, n_items_max,
               cold_list, u_counts, u_offsets, u_perm, u_cold_count,
               u_cold_routes);
}

// =============================================================================================
// Expert GEMVs
// =============================================================================================
// Both expert kernels stream one expert image tile per workgroup: 64 lanes x one 16-byte code
// chunk per K block (1 KiB per wave-wide load), 4 blocks per group, up to kMaxGroups groups
// per wave all loaded before any arithmetic so that every wave keeps up to 16 loads in flight.
// Each lane owns one output row; the activation block of the current token is uniform across
// the wave: it is read from an LDS copy of the tokens' activations (broadcast reads) when they
// fit, else through scalar loads.  The waves of a workgroup split K; their partial sums meet in
// LDS in a fixed order.
//
// Memory operations of a wave complete in issue order, so the issue order is chosen: inputs that
// are needed first (activations, the route table, scale words) are requested before the bulk of
// the weight codes, and every load of a phase is unconditional (addresses clamped in range)
// so that no load sits in a divergent branch that must drain before the next one issues.
constexpr int kMaxGroups = 4;
constexpr int kMaxWaves = 16;
constexpr int kTokPerPass = 8;   // routes of one expert handled per pass (LDS rows)
constexpr int kXLdsBytes = 20480;  // activations of a call staged in LDS up to this size

// Loads the wave's K range: groups g0 .. g0+ngw-1 (ngw <= G, wave-uniform).  Every load is
// issued unconditionally, so that the compiler can count outstanding loads exactly and let the
// arithmetic on each block wait for that block alone: groups past ngw re-read the wave's last
// group and blocks past nb re-read block nb-1 (both weighted by zero or skipped later).  The
// scale words come first: their decode is needed before the first block's arithmetic.
template <int G>
__device__ __forceinline__ void load_tile_range(const uint4* __restrict__ codes,
                                                const uint32_t* __restrict__ scl, int nb, int g0,
                                                int ngw, int lane, uint32_t (&s4)[G],
                                                uint4 (&c)[4 * G]) {
  // (the scheduling barriers keep the issue order of the source)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < G; ++q) s4[q] = ld_nt32(scl + (g0 + min(q, ngw - 1)) * 64 + lane);
#pragma unroll
  for (int q = 0; q < G; ++q) {
    const int g = g0 + min(q, ngw - 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) c[4 * q + i] = ld_nt(codes + min(4 * g + i, nb - 1) * 64 + lane);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Same sum as dot_tile_range with the activation row in LDS (every lane reads the same
// address: broadcast).  Straight-line over all 4*G blocks: blocks of groups past ngw or past nb
// read a valid activation block (index clamped) and add nothing (a select), so no weight load
// is used only inside a branch (the compiler would sink such a load behind the others and make
// the first block wait for all of them).
template <int G>
__device__ __forceinline__ float dot_tile_lds(const uint4 (&c)[4 * G], const uint32_t (&s4)[G],
                                              int nb, int g0, int ngw,
                                              const uint16_t* act) {
  float acc = 0.0f;
#pragma unroll
  for (int q = 0; q < G; ++q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = 4 * (g0 + q) + i;
      const bool live = q < ngw && b < nb;
      const uint4* a = reinterpret_cast<const uint4*>(act + 32 * min(b, nb - 1));
      const float sc = e8m0_to_f32((s4[q] >> (8 * i)) & 0xFFu);
      const float v = fmaf(sc, block_dot(c[4 * q + i], a[0], a[1], a[2], a[3]), acc);
      acc = live ? v : acc;
      // one block's activations live at a time: keeps the LDS reads from being hoisted
      // ahead of all blocks (which would need 16 VGPRs per block)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  return acc;
}

// Keeps the compiler from hoisting the decode of the loaded codes out of a token loop (which
// would need 16 VGPRs per block for every block at once).
template <int G>
__device__ __forceinline__ void opaque(uint4 (&c)[4 * G]) {
#pragma unroll
  for (int j = 0; j < 4 * G; ++j)
    asm volatile("" : "+v"(c[j].x), "+v"(c[j].y), "+v"(c[j].z), "+v"(c[j].w));
}

// One 32-element block (16 code bytes) as 16 bf16 pairs, the block scale folded in (exact).
__device__ __forceinline__ void block_to_bf16(const uint4 c, float sc, bf16x2_t (&w)[16]) {
  const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    w[4 * j + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], sc, 0);
    w[4 * j + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], sc, 1);
    w[4 * j + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], sc, 2);
    w[4 * j + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], sc, 3);
  }
}
// ... and its dot with 32 bf16 activations, on two accumulation chains (even / odd pairs).
__device__ __forceinline__ void block_dot_bf16(const bf16x2_t (&w)[16], const uint4 a0, const uint4 a1,
                                               const uint4 a2, const uint4 a3, float& s0, float& s1) {
  const uint32_t aw[16] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w,
                           a2.x, a2.y, a2.z, a2.w, a3.x, a3.y, a3.z, a3.w};
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    s0 = __builtin_amdgcn_fdot2_f32_bf16(w[i], as_bf16x2(aw[i]), s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(w[i + 1], as_bf16x2(aw[i + 1]), s1, false);
  }
}

// dot_tile_lds for kGuNR routes at once (activation rows act + tok[r] * H in LDS): each code
// word is converted to a bf16 pair once (scale 1) and the pair feeds every route's chain, in
// block_dot's pair order and accumulation chains, so each sum is bitwise dot_tile_lds's.
constexpr int kGuNR = 2;
template <int G>
__device__ __forceinline__ void dot_tile_lds_nr(const uint4 (&c)[4 * G], const uint32_t (&s4)[G],
                                                int nb, int g0, int ngw, const uint16_t* xs,
                                                int H, const int (&tok)[kGuNR],
                                                float (&acc)[kGuNR]) {
#pragma unroll
  for (int r = 0; r < kGuNR; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int q = 0; q < G; ++q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = 4 * (g0 + q) + i;
      const bool live = q < ngw && b < nb;
      const float sc = e8m0_to_f32((s4[q] >> (8 * i)) & 0xFFu);
      uint4 a[kGuNR][4];
#pragma unroll
      for (int r = 0; r < kGuNR; ++r) {
        const uint4* ar = reinterpret_cast<const uint4*>(xs + (size_t)tok[r] * H + 32 * min(b, nb - 1));
#pragma unroll
        for (int j = 0; j < 4; ++j) a[r][j] = ar[j];
      }
      const uint4 cb = c[4 * q + i];
      const uint32_t cw[4] = {cb.x, cb.y, cb.z, cb.w};
      // the conversions' scale (1.0) comes out of an empty asm that takes the previous block's
      // sums, so this block is converted after them (the compiler would otherwise convert every
      // block up front and hold all the pairs); the codes themselves are read in place
      float one;
      asm volatile("v_mov_b32 %0, 1.0" : "=v"(one) : "v"(acc[0]), "v"(acc[kGuNR - 1]));
      float s0[kGuNR], s1[kGuNR];
#pragma unroll
      for (int r = 0; r < kGuNR; ++r) s0[r] = s1[r] = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x2_t w0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], one, 0);
        const bf16x2_t w1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], one, 1);
        const bf16x2_t w2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], one, 2);
        const bf16x2_t w3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], one, 3);
#pragma unroll
        for (int r = 0; r < kGuNR; ++r) {
          s0[r] = __builtin_amdgcn_fdot2_f32_bf16(w0, as_bf16x2(a[r][j].x), s0[r], false);
          s1[r] = __builtin_amdgcn_fdot2_f32_bf16(w1, as_bf16x2(a[r][j].y), s1[r], false);
          s0[r] = __builtin_amdgcn_fdot2_f32_bf16(w2, as_bf16x2(a[r][j].z), s0[r], false);
          s1[r] = __builtin_amdgcn_fdot2_f32_bf16(w3, as_bf16x2(a[r][j].w), s1[r], false);
        }
      }
#pragma unroll
      for (int r = 0; r < kGuNR; ++r) {
        const float v = fmaf(sc, s0[r] + s1[r], acc[r]);
        acc[r] = live ? v : acc[r];
      }
      __builtin_amdgcn_sched_barrier(0);  // one block's activations live at a time
    }
  }
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

// ---- route table in LDS -----------------------------------------------------------------------
// For up to kProMaxRoutes routes one workgroup builds the whole route table in LDS: slot of
// every route, the distinct hot experts in ascending id with their bucket offset and count,
// and the permutation that groups hot routes by expert (ascending route index inside a group).
// The expert kernels do this themselves when a call starts from ids or logits (it replaces the
// top-k / bucketing kernel); the route kernel does it once and leaves the table in the workspace.
constexpr int kProMaxRoutes = 256;

struct __align__(16) RouteLds {
  int ids[kProMaxRoutes];
  float w[kProMaxRoutes];
  int slot[kProMaxRoutes];
  int perm[kProMaxRoutes];
  int first[kProMaxRoutes];  // route is the first of its expert
  int cnt[kProMaxRoutes];    // routes of the route's expert (one token: rank of each expert)
  int dist_slot[kProMaxRoutes];
  int dist_off[kProMaxRoutes];
  int dist_cnt[kProMaxRoutes];
  int dist_e[kProMaxRoutes];
  int nd;
  int err;  // kErr* flags of the table: routes with an id outside [0, E) or a slot outside [-1, S)
};
constexpr size_t kRouteLdsBytes = (sizeof(RouteLds) + 15) / 16 * 16;
constexpr size_t kGuLdsBytes = 64 * 1024;  // LDS of a gate/up workgroup at most

// One token over at most kFastE experts (the decode case), by every wave of the workgroup:
// wave w ranks experts w, w + waves, ... (the number of keys above the expert's key, by a
// ballot), the ranks meet in LDS (rt.cnt, unused by one-token tables otherwise), then wave 0
// forms the route table and wave 1 the weights, in registers.  The keys are those of rank_key64, the
// weights use the arithmetic of topk_rank, so the results are bitwise those of moe_route.  The
// distinct hot experts of one token are its selected ids; their ascending order is a ballot
// prefix count.  Contains a workgroup barrier (every thread calls it).
constexpr int kFastE = 64;

// The table from this lane's logit `own` (expert lane, lanes < E) and expert map entry `e2v`.
__device__ __forceinline__ void route_token_small_v(RouteLds& rt, const RouteArgs& a, float own,
                                                    int e2v) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int E = a.E;
  const int lc = lane < E ? lane : 0;
  const uint64_t key = lane < E ? rank_key64(own, lane) : 0ull;  // 0 is below every key
  for (int i = wave; i < E; i += nw) {
    const int r = (int)__popcll(__ballot(key > readlane_u64(key, i)));
    if (lane == 0) rt.cnt[i] = r;
  }
  __syncthreads();
  // the weights by wave 1 (wave 0 without it), beside wave 0's table
  const int ww = nw > 1 ? 1 : 0;
  if (wave != 0 && wave != ww) return;
  const int rank = rt.cnt[lc];
  const bool sel = lane < E && rank < a.k;
  if (wave == ww) {
    const float v = lane < E ? rank_key(own) : -INFINITY;
    const uint64_t first = __ballot(lane < E && rank == 0);
    const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), (int)__ffsll((long long)first) - 1));
    const float ex = sel ? expf(v - top) : 0.0f;
    const float den = wave_sum(ex);
    if (sel) {
      rt.ids[rank] = lane;
      rt.w[rank] = ex / den;
    }
    if (wave != 0) return;
  }
  const int slot_of = a.e2s != nullptr ? e2v : lane;
  int slot = -1;
  if (sel && slot_of >= 0 && slot_of < a.S) slot = slot_of;
  const bool bad = __ballot(sel && (slot_of < -1 || slot_of >= a.S)) != 0ull;
  const bool hot = slot >= 0;
  const uint64_t hm = __ballot(hot);
  const int pos = __popcll(hm & ((1ull << lane) - 1ull));
  if (sel) rt.slot[rank] = slot;
  if (hot) {
    rt.dist_slot[pos] = slot;
    rt.dist_off[pos] = pos;
    rt.dist_cnt[pos] = 1;
    rt.dist_e[pos] = lane;
    rt.perm[pos] = rank;
  }
  if (lane == 0) {
    rt.nd = __popcll(hm);
    rt.err = bad ? kErrBadSlot : 0;
  }
}

__device__ __forceinline__ void route_token_small(RouteLds& rt, const RouteArgs& a) {
  const int lane = threadIdx.x & 63;
  const float* lrow = a.logits;  // row 0; the workspace holds at least 256 bytes of logits
  // Every load is issued before any value is used, and unconditionally (the expert map read
  // falls back to a dummy read of the logits), so that they share one round trip.
  const int lc = lane < a.E ? lane : 0;
  const float own = lrow[lc];
  const int32_t* e2p = a.e2s != nullptr ? a.e2s : reinterpret_cast<const int32_t*>(lrow);
  const int e2v = e2p[lc];
  route_token_small_v(rt, a, own, e2v);
}

// One token over any number of experts: top-k by wave 0 (topk_token), then the route table in
// registers as in route_token_small: the token's ids are distinct, so every hot route is its
// own distinct expert, placed in ascending expert id by a count over the k routes.
__device__ __forceinline__ void route_token_wave(RouteLds& rt, const RouteArgs& a) {
  const int lane = threadIdx.x & 63;
  topk_token_p<1>(a.logits, 0, a.E, a.k, rt.ids, rt.w);
  const bool route = lane < a.k;
  const int e = route ? rt.ids[lane] : 0;
  const int ec = min(max(e, 0), a.E - 1);
  const int s_of = a.e2s != nullptr ? a.e2s[ec] : ec;  // issued for every lane (clamped)
  int slot = -1;
  if (route && e >= 0 && e < a.E && s_of >= 0 && s_of < a.S) slot = s_of;
  const bool bad = __ballot(route && e >= 0 && e < a.E && (s_of < -1 || s_of >= a.S)) != 0ull;
  if (route) rt.slot[lane] = slot;
  const bool hot = slot >= 0;
  const uint64_t hm = __ballot(hot);
  int pos = 0;
  for (int j = 0; j < a.k; ++j) {
    const int ej = __builtin_amdgcn_readlane(e, j);
    pos += (((hm >> j) & 1ull) != 0ull && ej < e) ? 1 : 0;
  }
  if (hot) {
    rt.dist_slot[pos] = slot;
    rt.dist_off[pos] = pos;
    rt.dist_cnt[pos] = 1;
    rt.dist_e[pos] = e;
    rt.perm[pos] = lane;
  }
  if (lane == 0) {
    rt.nd = __popcll(hm);
    rt.err = bad ? kErrBadSlot : 0;
  }
}

// One token over 64 < E <= min(threads, 512) experts (k <= 16), by every wave: wave w ranks its
// 64 keys among themselves (each lane compares its key with the wave's keys, read back from LDS
// as broadcasts), its k best become candidates in LDS; every candidate is then ranked among the
// candidates (four threads a candidate), which for the k best is its rank among all keys (every
// key above one of them is itself a candidate), and wave 0 forms the weights from the k best in
// rank order with the arithmetic of topk_argmax, so ids and weights are bitwise those of
// moe_route.  Threads past E carry small distinct keys below every real key (real keys have a
// nonzero high word).  LDS: the keys over rt.ids .. rt.perm (4 KiB), the candidates' keys over
// rt.first / rt.cnt and their slots in rt.dist_off, the k best in rt.perm / rt.dist_e.
// Contains two workgroup barriers (every thread calls it).
constexpr int kManyMaxK = 16;
constexpr int kManyMaxE = 512;

__device__ __forceinline__ void route_token_many(RouteLds& rt, const RouteArgs& a) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int E = a.E, k = a.k;
  const int tc = min(t, E - 1);
  // every load issued before any value is used (the expert map read falls back to a dummy read)
  const float lv = a.logits[tc];
  const int32_t* e2p = a.e2s != nullptr ? a.e2s : reinterpret_cast<const int32_t*>(a.logits);
  const int e2v = e2p[tc];
  const uint64_t key = t < E ? rank_key64(lv, t) : (uint64_t)(lane + 1);
  const int nwv = (E + 63) / 64;  // waves holding experts
  const int nc = nwv * k, ncp = (nc + 15) & ~15;  // candidates, padded with zero keys
  uint64_t* all_key = reinterpret_cast<uint64_t*>(rt.ids);     // [nwv * 64]
  uint64_t* cand_key = reinterpret_cast<uint64_t*>(rt.first);  // [ncp]
  int* cand_slot = rt.dist_off;                                // [nc]
  if (wave < nwv) {  // uniform; the wave reads back only its own keys
    all_key[t] = key;
    const uint4* wk = reinterpret_cast<const uint4*>(all_key + wave * 64);
    int r = 0;
#pragma unroll
    for (int j = 0; j < 32; j += 8) {
      uint4 p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = wk[j + i];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        r += ((((uint64_t)p[i].y << 32) | p[i].x) > key ? 1 : 0) + ((((uint64_t)p[i].w << 32) | p[i].z) > key ? 1 : 0);
    }
    if (r < k) {
      cand_key[wave * k + r] = key;
      cand_slot[wave * k + r] = a.e2s != nullptr ? e2v : t;
    }
  }
  if (t >= nc && t < ncp) cand_key[t] = 0ull;
  __syncthreads();
  uint64_t* sel_key = reinterpret_cast<uint64_t*>(rt.perm);  // [k], by rank
  int* sel_slot = rt.dist_e;                                   // [k]
  {
    // candidate t / 4 against a quarter of the candidates; the quad's counts summed by DPP
    const int c = min(t >> 2, ncp - 1), part = t & 3, q = ncp / 4;
    const uint64_t ck = cand_key[c];
    const uint4* pk = reinterpret_cast<const uint4*>(cand_key + part * q);
    int r = 0;
    for (int j = 0; j < q / 2; j += 2) {
      const uint4 p0 = pk[j], p1 = pk[j + 1];
      r += ((((uint64_t)p0.y << 32) | p0.x) > ck ? 1 : 0) + ((((uint64_t)p0.w << 32) | p0.z) > ck ? 1 : 0) +
           ((((uint64_t)p1.y << 32) | p1.x) > ck ? 1 : 0) + ((((uint64_t)p1.w << 32) | p1.z) > ck ? 1 : 0);
    }
    r += dpp_i<0xB1>(r);  // quad_perm [1,0,3,2]
    r += dpp_i<0x4E>(r);  // quad_perm [2,3,0,1]
    if (part == 0 && (t >> 2) < nc && r < k && (ck >> 32) != 0ull) {
      sel_key[r] = ck;
      sel_slot[r] = cand_slot[t >> 2];
    }
  }
  __syncthreads();
  if (wave != 0) return;
  // (read before the table below overwrites these arrays; one wave's LDS accesses are ordered)
  const uint64_t mine = lane < k ? sel_key[lane] : 0ull;
  const int s_of = lane < k ? sel_slot[lane] : -1;
  const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(key_value(mine)), 0));
  const float ex = lane < k ? expf(key_value(mine) - top) : 0.0f;
  const float den = wave_sum(ex);
  const bool route = lane < k;
  const int e = route ? key_id(mine) : 0;
  int slot = -1;
  if (route && s_of >= 0 && s_of < a.S) slot = s_of;
  const bool bad = __ballot(route && (s_of < -1 || s_of >= a.S)) != 0ull;
  if (route) {
    rt.ids[lane] = e;
    rt.w[lane] = ex / den;
    rt.slot[lane] = slot;
  }
  const bool hot = slot >= 0;
  const uint64_t hm = __ballot(hot);
  int pos = 0;
  for (int j = 0; j < k; ++j) {
    const int ej = __builtin_amdgcn_readlane(e, j);
    pos += (((hm >> j) & 1ull) != 0ull && ej < e) ? 1 : 0;
  }
  if (hot) {
    rt.dist_slot[pos] = slot;
    rt.dist_off[pos] = pos;
    rt.dist_cnt[pos] = 1;
    rt.dist_e[pos] = e;
    rt.perm[pos] = lane;
  }
  if (lane == 0) {
    rt.nd = __popcll(hm);
    rt.err = bad ? kErrBadSlot : 0;
  }
}

// rt.ids / rt.w [0, Mk) must be in place and rt.err cleared (visible after a barrier).  e2s may
// point to LDS.  Routes with an id outside [0, E) or a slot outside [-1, S) are cold and flagged.
__device__ void build_table(RouteLds& rt, int Mk, int E, int S, const int32_t* e2s) {
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  if (tid == 0) rt.nd = 0;
  for (int r = tid; r < Mk; r += nthr) {
    const int e = rt.ids[r];
    int slot = -1;
    if (e >= 0 && e < E) {
      slot = e2s ? e2s[e] : e;
      if (slot < -1 || slot >= S) atomicOr(&rt.err, kErrBadSlot);
      if (slot < 0 || slot >= S) slot = -1;
    } else {
      atomicOr(&rt.err, kErrBadId);
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
        rt.dist_e[di] = e;
        atomicAdd(&rt.nd, 1);
      }
    }
  }
  __syncthreads();
}

// Caller-visible results of a table: top-k ids / weights and the cold report (any may be NULL).
__device__ void write_routes(const RouteLds& rt, int Mk, int32_t* topk_ids, float* topk_w,
                             int32_t* cold_count, int32_t* cold_routes, int32_t* cold_list) {
  for (int r = threadIdx.x; r < Mk; r += blockDim.x) {
    if (topk_ids != nullptr) {
      topk_ids[r] = rt.ids[r];
      topk_w[r] = rt.w[r];
    }
    if (rt.slot[r] < 0 && (cold_routes != nullptr || cold_list != nullptr)) {
      int ci = 0;
      for (int r2 = 0; r2 < r; ++r2) ci += rt.slot[r2] < 0;
      if (cold_routes != nullptr) cold_routes[ci] = r;
      if (cold_list != nullptr) cold_list[ci] = r;
    }
  }
  if (cold_count != nullptr && threadIdx.x < 64) {
    int c = 0;
    for (int r = threadIdx.x; r < Mk; r += 64) c += rt.slot[r] < 0;
    c = (int)wave_sum((float)c);
    if (threadIdx.x == 0) *cold_count = c;
  }
}

// The table of rt, as the expert kernels read it from the workspace; its error flags are added
// to the workspace's error word.
__device__ void write_table(const RouteLds& rt, int Mk, const RouteWs& w) {
  for (int r = threadIdx.x; r < Mk; r += blockDim.x) {
    w.route_slot[r] = rt.slot[r];
    w.perm[r] = rt.perm[r];  // entries past the hot routes are never read
  }
  for (int d = threadIdx.x; d < rt.nd; d += blockDim.x)
    w.dist[d] = make_int4(rt.dist_slot[d], rt.dist_off[d], rt.dist_cnt[d], rt.dist_e[d]);
  if (threadIdx.x == 0) {
    int c = 0;
    for (int r = 0; r < Mk; ++r) c += rt.slot[r] < 0;
    w.meta[0] = rt.nd;
    w.meta[1] = c;
    if (rt.err != 0) atomicOr(&w.meta[kMetaErr], rt.err);
  }
}

// Route table of an expert workgroup: top-k from the logits or the given ids, then the table.
// The writer workgroup also publishes the top-k results, the cold report and the table.
__device__ void route_prologue(RouteLds& rt, const RouteArgs& a, const RouteWs& w, bool writer) {
  const int tid = threadIdx.x;
  const int nw = blockDim.x >> 6;
  const int Mk = a.M * a.k;
  if (a.logits != nullptr && a.M == 1) {
    if (a.E <= kFastE)
      route_token_small(rt, a);
    else if (a.E <= (int)blockDim.x && a.E <= kManyMaxE && a.k <= kManyMaxK)
      route_token_many(rt, a);
    else if (tid < 64)
      route_token_wave(rt, a);
    __syncthreads();
  } else {
    if (a.logits != nullptr) {
      for (int m = tid >> 6; m < a.M; m += nw)
        topk_token_p<1>(a.logits + (size_t)m * a.E, 0, a.E, a.k, rt.ids + m * a.k, rt.w + m * a.k);
    } else {
      for (int r = tid; r < Mk; r += blockDim.x) {
        rt.ids[r] = a.ids_in[r];
        rt.w[r] = a.w_in[r];
      }
    }
    if (tid == 0) rt.err = 0;
    __syncthreads();
    build_table(rt, Mk, a.E, a.S, a.e2s);
  }
  if (writer) {
    write_routes(rt, Mk, a.topk_ids, a.topk_w, a.cold_count, a.cold_routes, nullptr);
    write_table(rt, Mk, w);
  }
}

// ---- h in the workspace -----------------------------------------------------------------------
// The GEMV paths (M < 64) keep h in bf16, [route][I].  The grouped path keeps it split for the
// down projection's block-scaled MFMA (see mx_pair): per route (h_stride bytes) hi[h_pad] and
// lo[h_pad] E4M3 codes, then one E8M0 scale byte per 32-element block.  Elements past I, and
// scale bytes past the last block, are never written: k_down_mx substitutes zeros and 127.

// out[i] = bf16(x[i] + v) (round to nearest even), the residual chaining of stacked layers.
__device__ __forceinline__ void residual_store(const Residual& res, size_t i, float v) {
  if (res.out != nullptr)
    res.out[i] = (uint16_t)f32_to_bf16_bits(__uint_as_float((uint32_t)res.x[i] << 16) + v);
}

// bf16(silu(g) * u), returned as the fp32 value of that bf16.
__device__ __forceinline__ float swiglu_bf16(float g, float u) {
  return __uint_as_float(f32_to_bf16_bits(silu_f32(g) * u) << 16);
}

// ---- gate/up + SiLU*up ----------------------------------------------------------------------
// grid = (I/32 tiles, nd_max); block = nw waves.  Lane l < 32 accumulates gate row 32*tile + l,
// lane l >= 32 the matching up row; wave w covers groups [w*ng/nw, (w+1)*ng/nw).
// SINGLE: one token per call (M = 1), one route per expert.  XLDS: the M activation rows are
// staged in LDS (when they fit beside the sums and the route table), requested before anything
// else.
template <bool SINGLE, int G, bool PRO, bool XLDS>
__global__ __launch_bounds__(kMaxWaves * 64) void k_gateup(
    const uint16_t* __restrict__ x, int H, int I, const uint8_t* __restrict__ slots,
    size_t image_bytes, size_t gu_tile_bytes, int nb, int ng, RouteArgs ra, RouteWs rw,
    uint16_t* __restrict__ hbuf) {
  // dynamic LDS, sized by the launcher: [red: nw x RP x 64 floats][rt (PRO)][xs: M x H (XLDS)]
  extern __shared__ __align__(16) uint8_t gsm[];
  constexpr int RP = SINGLE ? 1 : kTokPerPass;
  const int tile = blockIdx.x;
  const int d = blockIdx.y;
  const int Mk = ra.M * ra.k;
  const int nthr = blockDim.x;
  const size_t red_bytes = (size_t)(nthr >> 6) * RP * 64 * 4;
  float (*red)[RP][64] = reinterpret_cast<float (*)[RP][64]>(gsm);
  RouteLds& rt = *reinterpret_cast<RouteLds*>(gsm + red_bytes);
  uint16_t* xs = reinterpret_cast<uint16_t*>(gsm + red_bytes + (PRO ? kRouteLdsBytes : 0));

  // Activations to LDS, requested before anything else so that their latency overlaps the
  // route-table reads.
  //  - Route table from the workspace: through registers, 4 chunks per thread (clamped; a
  //    duplicate stores the same value as its owner), loads and stores in this one basic block
  //    (the compiler would otherwise sink the loads to their use, behind the weight loads).
  //    The compute then waits for each weight block as it arrives.
  //  - Table built here (prologue): global-to-LDS copies, one 1 KiB run of 64 chunks per wave
  //    instruction, left in flight across the prologue.  (After such copies the compiler waits
  //    for every outstanding load before the first LDS read, so the compute starts once all
  //    weights have landed.)
  const int n_x = XLDS ? ra.M * H / 8 : 0;
  if (XLDS && !PRO) {
    const uint4* xg = reinterpret_cast<const uint4*>(x);
    uint4* xl = reinterpret_cast<uint4*>(xs);
    uint4 xv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[i] = xg[min(i * nthr + (int)threadIdx.x, n_x - 1)];
#pragma unroll
    for (int i = 0; i < 4; ++i) xl[min(i * nthr + (int)threadIdx.x, n_x - 1)] = xv[i];
    for (int idx = 4 * nthr + (int)threadIdx.x; idx < n_x; idx += nthr) xl[idx] = xg[idx];
  }
  if (XLDS && PRO) {
    typedef __attribute__((address_space(3))) void lds_void;
    const int runs = (n_x + 63) / 64;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int run = wv; run < runs; run += nthr >> 6) {
      const int p = min(run * 64 + (int)(threadIdx.x & 63), n_x - 1);
      __builtin_amdgcn_global_load_lds(x + (size_t)p * 8, (lds_void*)(xs + (size_t)run * 512), 16, 0, 0);
    }
  }

  int slot, cnt, off;
  const int* perm;
  if (PRO) {
    route_prologue(rt, ra, rw, tile == 0 && d == 0);
    if (d >= rt.nd) {
      if (XLDS) __builtin_amdgcn_s_waitcnt(0);  // no copy into LDS outlives the workgroup
      return;
    }
    slot = rt.dist_slot[d];
    cnt = rt.dist_cnt[d];
    off = rt.dist_off[d];
    perm = rt.perm;
  } else {
    // both table reads are consumed by the test, so they are issued together (a load used
    // only past a branch is moved behind it); d < nd_max keeps dist[d] in bounds
    const int nd = rw.meta[0];
    const int4 dd = rw.dist[d];
    asm volatile("" : "+s"(image_bytes), "+s"(gu_tile_bytes));  // fetched now, not after the test
    if (d >= nd || dd.z <= 0) return;  // the whole workgroup leaves together
    slot = dd.x;
    off = dd.y;
    cnt = dd.z;
    perm = rw.perm;
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = nthr >> 6;
  // Without the prologue (at most 2 K groups a wave: the register budget of the loop) the grid
  // holds gridDim.y hot experts at a time, sized so that the grid is resident at once, and
  // workgroup (tile, d) takes experts d, d + gridDim.y, ...; otherwise gridDim.y = nd_max and
  // each workgroup takes one.
  constexpr bool LOOP = !PRO && !SINGLE && G <= 2;
  for (int dcur = d;;) {
  if (cnt > 0 && off >= 0 && off + cnt <= Mk) {

  const uint8_t* tbase = slots + (size_t)slot * image_bytes + (size_t)tile * gu_tile_bytes;
  const uint4* codes = reinterpret_cast<const uint4*>(tbase);
  const uint32_t* scl = reinterpret_cast<const uint32_t*>(tbase + (size_t)nb * 1024);
  const int g0 = wave * ng / nw;
  const int ngw = (wave + 1) * ng / nw - g0;
  uint32_t s4[G];
  uint4 c[4 * G];
  if (XLDS && PRO) {
    // the copies into LDS have landed (long since: they were requested before the route table)
    // and are visible to every wave before any weight is requested, so the compute below waits
    // for each weight block alone (with copies still pending, the compiler would make it wait
    // for every outstanding load)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  // lane j: route j of this expert (the multi-route loop below reads it by readlane)
  const int myr = (!SINGLE && XLDS && G <= 2) ? perm[off + min(lane, cnt - 1)] : 0;
  load_tile_range<G>(codes, scl, nb, g0, ngw, lane, s4, c);
  if (XLDS && !PRO) __syncthreads();  // activations in LDS for every wave

  if (SINGLE) {
    // M = 1: the only route of this expert belongs to token 0.  No loop around the dot, so the
    // decode of the codes cannot be hoisted ahead of it.
    red[wave][0][lane] = dot_tile_lds<G>(c, s4, nb, g0, ngw, xs);
    __syncthreads();
    if (threadIdx.x < 32) {
      const int row = threadIdx.x;
      float g = 0.0f, u = 0.0f;
      for (int w = 0; w < nw; ++w) {
        g += red[w][0][row];
        u += red[w][0][row + 32];
      }
      hbuf[(size_t)perm[off] * I + tile * 32 + row] = (uint16_t)f32_to_bf16_bits(silu_f32(g) * u);
    }
    return;
  }
  for (int base = 0; base < cnt; base += kTokPerPass) {
    const int nt = min(kTokPerPass, cnt - base);
    if (XLDS && G <= 2) {
      // kGuNR routes per decode of the weights (the last group padded with the pass's last
      // route, whose sums are not stored twice); with 4 groups a wave the extra activation
      // registers would spill.  The tokens of the expert's routes come from lane registers
      // (myr), read before the weights, so no load waits inside this loop.
#pragma unroll 1
      for (int t0 = 0; t0 < nt; t0 += kGuNR) {
        // (no opaque() here: the conversions already wait for an asm inside this loop)
        int tok[kGuNR];
#pragma unroll
        for (int u = 0; u < kGuNR; ++u) {
          const int j = base + min(t0 + u, nt - 1);
          tok[u] = (j < 64 ? __builtin_amdgcn_readlane(myr, j)
                           : __builtin_amdgcn_readfirstlane(perm[off + j])) / ra.k;
        }
        float acc[kGuNR];
        dot_tile_lds_nr<G>(c, s4, nb, g0, ngw, xs, H, tok, acc);
#pragma unroll
        for (int u = 0; u < kGuNR; ++u)
          if (t0 + u < nt) red[wave][t0 + u][lane] = acc[u];
      }
    } else {
#pragma unroll 1
      for (int t = 0; t < nt; ++t) {
        opaque<G>(c);
        const int r = __builtin_amdgcn_readfirstlane(perm[off + base + t]);
        const int tok = r / ra.k;
        red[wave][t][lane] = XLDS ? dot_tile_lds<G>(c, s4, nb, g0, ngw, xs + (size_t)tok * H)
                                  : dot_tile_range<G>(c, s4, nb, g0, ngw, x + (size_t)tok * H);
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < nt * 32; idx += nthr) {
      const int t = idx >> 5;
      const int row = idx & 31;
      float g = 0.0f, u = 0.0f;
      for (int w = 0; w < nw; ++w) {
        g += red[w][t][row];
        u += red[w][t][row + 32];
      }
      hbuf[(size_t)perm[off + base + t] * I + tile * 32 + row] =
          (uint16_t)f32_to_bf16_bits(silu_f32(g) * u);
    }
    __syncthreads();
  }

  }  // (a valid table entry)
  if (!LOOP) return;
  dcur += gridDim.y;
  if (dcur >= rw.meta[0]) return;  // (uniform)
  const int4 dn = rw.dist[dcur];
  slot = dn.x;
  off = dn.y;
  cnt = dn.z;
  }  // experts of this workgroup
}

// ---- down projection on the matrix cores --------------------------------------------------------
// A down tile (16 rows of one expert) is streamed one K step (4 blocks = 128 elements) per MFMA
// operand: a wave-wide 16-byte load is 1 KiB, and nothing is decoded (the block-scaled MFMA
// takes the E2M1 codes with their E8M0 scales).  h enters as the other operand: a column is one
// route's hi or lo codes (see mx_pair) with the block scales.

// This lane's A operand of down step s (clamped to the last step; lanes past the stored part
// of a partial step re-read a stored lane and meet zero h).
__device__ __forceinline__ uint4 dn_a(const uint8_t* __restrict__ tb, int s, int ks, int full,
                                      int rem, int lane) {
  s = min(s, ks - 1);
  const int idx = s < full ? s * 64 + lane : full * 64 + min(lane, 16 * rem - 1);
  return ld_nt(reinterpret_cast<const uint4*>(tb) + idx);
}

// Scale word q of this lane (byte j: step 4q + j), clamped to the last word.
__device__ __forceinline__ uint32_t dn_sw(const uint8_t* __restrict__ tb, size_t code_bytes, int q,
                                          int nsw, int lane) {
  return ld_nt32(reinterpret_cast<const uint32_t*>(tb + code_bytes) + min(q, nsw - 1) * 64 + lane);
}

// The block-scaled MFMA with the A scale byte chosen at run time among constants (j & 3 is a
// constant once the step loop is unrolled).
__device__ __forceinline__ f32x4_t mfma_mx_j(int j, const uint4& a, const uint4& b0,
                                             const uint4& b1, f32x4_t c, uint32_t sa,
                                             uint32_t sb) {
  switch (j & 3) {
    case 0: return mfma_mx<0>(a, b0, b1, c, sa, sb);
    case 1: return mfma_mx<1>(a, b0, b1, c, sa, sb);
    case 2: return mfma_mx<2>(a, b0, b1, c, sa, sb);
    default: return mfma_mx<3>(a, b0, b1, c, sa, sb);
  }
}

// Scale word of a route's h for down step s (bytes: blocks 4s .. 4s+3); bytes of blocks past
// the last one are never written, so they read as 127 (1.0, against zero codes).
__device__ __forceinline__ uint32_t h_scale_word(uint32_t w, int s, int nb_i) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (4 * s + j >= nb_i) w = (w & ~(0xFFu << (8 * j))) | (127u << (8 * j));
  return w;
}

// ---- down GEMV (VALU) ----------------------------------------------------------------------------
// For one or a few tokens the down projection is a GEMV over the same tiles: lane l of a wave
// holds, at each K step s, row l%16's block 4s + l/16 (16 code bytes) and takes its dot with
// that block of h (bf16; the 16 lanes of a lane group read the same 64 bytes, an LDS broadcast),
// decoded on the fly by the packed FP4 converter; the 4 lanes of a row (l, l^16, l^32, l^48)
// meet at the end.  A wave holds TM steps of one expert's tile (a K part of it); the waves of a
// workgroup split the hot experts and K.

// This lane's TM steps from s0 (a multiple of 4), scale words first.
template <int TM>
__device__ __forceinline__ void dn_load_steps(const uint8_t* __restrict__ tb, size_t code_bytes,
                                              int s0, int ks, int full, int rem, int nsw, int lane,
                                              uint4 (&c)[TM], uint32_t (&sw)[TM / 4]) {
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < TM / 4; ++q) sw[q] = dn_sw(tb, code_bytes, s0 / 4 + q, nsw, lane);
#pragma unroll
  for (int j = 0; j < TM; ++j) c[j] = dn_a(tb, s0 + j, ks, full, rem, lane);
  __builtin_amdgcn_sched_barrier(0);
}

// h of step s0 of the route whose h row is hr, for this lane (the 64 bytes of its block).
__device__ __forceinline__ void dn_h_first(const uint16_t* hr, int s0, int nb, int g, uint4 (&a)[4]) {
  const uint4* hb = reinterpret_cast<const uint4*>(hr + 32 * min(4 * s0 + g, nb - 1));
  a[0] = hb[0];
  a[1] = hb[1];
  a[2] = hb[2];
  a[3] = hb[3];
}

// One route's partial sum for this lane over steps s0 .. s0+n-1 (n <= TM); hr = the route's h
// (bf16 [I], in LDS or the workspace), its first step already in `an`.  Software-pipelined by
// hand: the h block of step j+1 is read before step j's arithmetic, its address passing through
// an empty asm together with the sum so far, which keeps the compiler from issuing every read
// up front (16 VGPRs per step); during the last step the next route's first step (h row hn) is
// requested into `an`, so that consecutive routes of an expert do not each wait for their h.
// Steps past n or ks, and blocks past nb, read a valid block and add nothing (a select, not a
// product, so whatever that block holds cannot leak in).
template <int TM>
__device__ __forceinline__ float dn_route_dot_pf(const uint4 (&c)[TM], const uint32_t (&sw)[TM / 4],
                                                 int s0, int n, int ks, int nb, int g,
                                                 const uint16_t* hr, const uint16_t* hn,
                                                 uint4 (&an)[4]) {
  float acc = 0.0f;
  int hoff = 0;
  auto read_h = [&](const uint16_t* row, int j, uint4 (&a)[4]) {
    const uint4* hb = reinterpret_cast<const uint4*>(row + hoff + 32 * min(4 * (s0 + j) + g, nb - 1));
    a[0] = hb[0];
    a[1] = hb[1];
    a[2] = hb[2];
    a[3] = hb[3];
  };
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    uint4 ac[4] = {an[0], an[1], an[2], an[3]};
    asm volatile("" : "+v"(acc), "+v"(hoff));
    if (j + 1 < TM)
      read_h(hr, j + 1, an);
    else
      read_h(hn, 0, an);
    const bool live = j < n && s0 + j < ks && 4 * (s0 + j) + g < nb;
    const float sc = e8m0_to_f32((sw[j >> 2] >> (8 * (j & 3))) & 0xFFu);
    const float v = fmaf(sc, block_dot(c[j], ac[0], ac[1], ac[2], ac[3]), acc);
    acc = live ? v : acc;
    __builtin_amdgcn_sched_barrier(0);
  }
  return acc;
}

// Every step of a route's h for this lane (TM x 64 bytes), requested together.
template <int TM>
__device__ __forceinline__ void dn_route_h(const uint16_t* hr, int s0, int nb, int g,
                                           uint4 (&a)[TM][4]) {
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const uint4* hb = reinterpret_cast<const uint4*>(hr + 32 * min(4 * (s0 + j) + g, nb - 1));
    a[j][0] = hb[0];
    a[j][1] = hb[1];
    a[j][2] = hb[2];
    a[j][3] = hb[3];
  }
}

// The route's partial sum from h already in registers (the arithmetic of dn_route_dot_pf).
template <int TM>
__device__ __forceinline__ float dn_route_dot_h(const uint4 (&c)[TM], const uint32_t (&sw)[TM / 4],
                                                int s0, int n, int ks, int nb, int g,
                                                const uint4 (&a)[TM][4]) {
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const bool live = j < n && s0 + j < ks && 4 * (s0 + j) + g < nb;
    const float sc = e8m0_to_f32((sw[j >> 2] >> (8 * (j & 3))) & 0xFFu);
    const float v = fmaf(sc, block_dot(c[j], a[j][0], a[j][1], a[j][2], a[j][3]), acc);
    acc = live ? v : acc;
  }
  return acc;
}

// Sum over the 4 lanes of a row (l, l^16, l^32, l^48); every one of them gets it.
__device__ __forceinline__ float dn_row_sum(float v) { return pair_sum32(pair_sum16(v)); }

// Rounds of a gather of words handed over by value at most (each about a load round trip).
constexpr int kHandSpins = 1 << 13;
constexpr int kDnNR = 2;   // routes of an expert the down GEMV forms together (h in LDS)
constexpr int kDnAll = 4;  // hot experts of a wave whose weights it requests all at once

// Steps of a K part: K split over kparts, rounded up to whole scale words.
__host__ __device__ __forceinline__ int dn_part_steps(int ks, int kparts) {
  return ((ks + kparts - 1) / kparts + 3) & ~3;
}

// grid = (H/16 tiles, S), 8 waves.  Workgroup (tile, p) takes the hot experts p, p + S, ...;
// its waves own (expert, K part) pairs: with kparts K parts, 8/kparts of its experts per pass,
// wave w taking the experts of its list at w % (8/kparts) + (8/kparts)*i and K part
// w / (8/kparts).  Each route's partial rows go to LDS; workgroup (tile, 0) then forms
// y[m][rows] = sum over j ascending (hot routes) of w[m,j] * (its K parts, in order).  With
// S = 2 (one K part; the grid is resident at once, one workgroup per compute unit) workgroup
// (tile, 1) hands its routes' rows to (tile, 0) by value: 64-bit words {row value, tag} with
// device-scope stores at route * kSplitRowStride + row (the same place for every shape), the
// tag being the tile's call id + 1 from the workspace; (tile, 0) polls
// the words of its partner's routes (bounded, like the fused kernel's gather of h) into its
// LDS, forms y, and then advances the tile's call id (its partner has read it: its words carry
// it).  A gather that runs out flags MOE_DEVERR_HANDOFF, writes NaN rows and poisons the
// workspace (the poison word is the fused kernel's).  h comes from an LDS copy when every
// route's h fits (h_lds), else straight from the workspace.  The route table comes from the
// workspace.
template <int TM>
__global__ __launch_bounds__(512) void k_down_gemv(
    int H, int I, const uint8_t* __restrict__ slots, size_t image_bytes, size_t gu_bytes,
    size_t dn_tile_bytes, size_t dn_code_bytes, int ks, int full, int rem, int nsw, int nb,
    int kparts, int h_lds, RouteArgs ra, RouteWs rw, const uint16_t* __restrict__ hbuf,
    float* __restrict__ y, Residual res, uint64_t* __restrict__ pw, uint32_t* __restrict__ dncall) {
  extern __shared__ __align__(16) uint8_t smem[];  // [h copy (h_lds)] [parts: Mk x kparts x 16]
  __shared__ uint32_t s_dcall;                     // split: this tile's call id
  __shared__ int s_dlate;                          // split: the gather ran out, or a poisoned workspace
  const int tile = blockIdx.x;
  const int Mk = ra.M * ra.k;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int sl = 8 / kparts;
  const int kh = wave / sl;
  // this wave's experts: es0, es0 + sl_all, ... (the first and the stride in the hot list)
  const bool split = gridDim.y > 1;  // (then kparts == 1)
  const bool helper = split && blockIdx.y != 0;
  if (split && threadIdx.x == 0) {  // (requested first: its latency overlaps the h copy's)
    const uint32_t c0 = __hip_atomic_load(&dncall[tile], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t pz = __hip_atomic_load(reinterpret_cast<uint32_t*>(&rw.meta[kMetaPoison]),
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_dcall = c0;
    s_dlate = pz != 0u ? 1 : 0;
  }
  const int es0 = (int)blockIdx.y + (int)gridDim.y * (wave % sl);
  const int sl_all = (int)gridDim.y * sl;
  const int spw = dn_part_steps(ks, kparts);
  const int s0 = kh * spw;
  const uint8_t* sec = slots + gu_bytes + (size_t)tile * dn_tile_bytes;
  const int nd_max = Mk < ra.E ? Mk : ra.E;
  const int nd = rw.meta[0];
  const int sw0 = rw.dist[es0 < nd_max ? es0 : nd_max - 1].x;
  const int sd0 = rw.dist[0].x;
  const int slot0 = nd == 0 ? 0 : (es0 < nd ? sw0 : sd0);  // no expert: any valid slot
  const int n_h = h_lds ? Mk * I / 8 : 0;  // 16-byte chunks of h
  if (h_lds) {
    // h straight from the workspace to LDS, one 1 KiB run per wave instruction (runs past n_h
    // re-read the last chunk into padding)
    typedef __attribute__((address_space(3))) void lds_void;
    const int runs = (n_h + 63) / 64;
    for (int run = wave; run < runs; run += 8) {
      const int p = min(run * 64 + lane, n_h - 1);
      __builtin_amdgcn_global_load_lds(hbuf + (size_t)p * 8, (lds_void*)(smem + (size_t)run * 1024), 16, 0, 0);
    }
  }
  // weights of the next expert in flight while this one's routes are formed (not at 16 steps a
  // wave: two sets would not fit the register file)
  constexpr bool PF = TM <= 12;
  uint4 c[TM], cn[PF ? TM : 1];
  uint32_t sw[TM / 4], swn[PF ? TM / 4 : 1];
  dn_load_steps<TM>(sec + (size_t)slot0 * image_bytes, dn_code_bytes, s0, ks, full, rem, nsw, lane, c, sw);
  const uint16_t* hsrc = h_lds ? reinterpret_cast<const uint16_t*>(smem) : hbuf;
  float* parts = reinterpret_cast<float*>(smem + (h_lds ? (size_t)(n_h + 63) / 64 * 1024 : 0));
  __syncthreads();
  const uint32_t tag = s_dcall + 1u;  // (split)
  // a route's partial rows (lanes < 16): to LDS, or from the helper workgroup to its partner
  auto put = [&](int route, float acc) {
    if (helper)
      __hip_atomic_store(&pw[(size_t)route * kSplitRowStride + tile * kDnRows + lane],
                         (uint64_t)__float_as_uint(acc) | ((uint64_t)tag << 32), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    else
      parts[((size_t)route * kparts + kh) * kDnRows + lane] = acc;
  };
  bool fast = false;
  if constexpr (TM <= 4) {
    // A short K part and at most 64 hot experts for this wave: no route-table read on the way
    // from one expert to the next.  Lane i holds the table entry of the wave's i-th expert (one
    // read for all of them); the next expert's weights and route list are requested when an
    // expert starts.
    const int nde = es0 < nd ? (nd - es0 + sl_all - 1) / sl_all : 0;
    if (nde <= 64) {
      fast = true;
      const int4 md = rw.dist[min(es0 + min(lane, max(nde - 1, 0)) * sl_all, nd_max - 1)];
      auto entry = [&](int i, int& slot, int& off, int& cnt) {  // (i uniform)
        slot = __builtin_amdgcn_readlane(md.x, i);
        off = __builtin_amdgcn_readlane(md.y, i);
        const int z = __builtin_amdgcn_readlane(md.z, i);
        cnt = off >= 0 && z > 0 && off + z <= Mk ? z : 0;
      };
      auto routes_of = [&](int off, int cnt) {  // lane j: route j of the expert (j < 64)
        return rw.perm[max(min(off + min(lane, max(cnt - 1, 0)), Mk - 1), 0)];
      };
      if (nde > 0 && h_lds) {
        // h in LDS: each expert's weights are decoded to bf16 once (the block scale folded in,
        // exact; zero for blocks past K, which re-read a valid block) and serve every route of
        // the expert, kDnNR routes at a time with their accumulation chains interleaved (one
        // wave a SIMD has nothing else to hide a chain's latency behind).  With at most kDnAll
        // experts the weights of all of them are requested at once, into registers of their
        // own (a rotation of buffers would wait for each load at the move); otherwise the next
        // expert's as an expert starts.
        auto expert = [&](const uint4 (&cw)[TM], const uint32_t (&swq)[TM / 4], int off, int cnt,
                          int myr) {
          bf16x2_t wd[TM][16];
#pragma unroll
          for (int t = 0; t < TM; ++t) {
            const bool live = t < spw && s0 + t < ks && 4 * (s0 + t) + g < nb;
            const float f = e8m0_to_f32((swq[t >> 2] >> (8 * (t & 3))) & 0xFFu);
            block_to_bf16(cw[t], __uint_as_float(__float_as_uint(f) & (live ? 0xFFFFFFFFu : 0u)), wd[t]);
          }
#pragma unroll 1
          for (int j = 0; j < cnt; j += kDnNR) {
            int rr[kDnNR];
#pragma unroll
            for (int u = 0; u < kDnNR; ++u) {
              const int jj = min(j + u, cnt - 1);
              rr[u] = jj < 64 ? __builtin_amdgcn_readlane(myr, jj) : rw.perm[off + jj];
            }
            float e0[kDnNR], e1[kDnNR];
#pragma unroll
            for (int u = 0; u < kDnNR; ++u) e0[u] = e1[u] = 0.0f;
#pragma unroll
            for (int t = 0; t < TM; ++t) {
#pragma unroll
              for (int u = 0; u < kDnNR; ++u) {
                const uint4* hb = reinterpret_cast<const uint4*>(
                    hsrc + (size_t)rr[u] * I + 32 * min(4 * (s0 + t) + g, nb - 1));
                block_dot_bf16(wd[t], hb[0], hb[1], hb[2], hb[3], e0[u], e1[u]);
              }
              __builtin_amdgcn_sched_barrier(0);  // one step's h at a time in registers
            }
#pragma unroll
            for (int u = 0; u < kDnNR; ++u) {
              const float acc = dn_row_sum(e0[u] + e1[u]);
              if (j + u < cnt && lane < kDnRows) put(rr[u], acc);
            }
          }
        };
        if (nde <= kDnAll) {
          uint4 ca[kDnAll][TM];
          uint32_t swa[kDnAll][TM / 4];
          int offa[kDnAll], cnta[kDnAll], myra[kDnAll];
#pragma unroll
          for (int q = 0; q < kDnAll; ++q) {
            int sq;
            entry(min(q, nde - 1), sq, offa[q], cnta[q]);
            if (q == 0) {  // (requested before the loop)
#pragma unroll
              for (int t = 0; t < TM; ++t) ca[0][t] = c[t];
#pragma unroll
              for (int w4 = 0; w4 < TM / 4; ++w4) swa[0][w4] = sw[w4];
            } else {
              dn_load_steps<TM>(sec + (size_t)sq * image_bytes, dn_code_bytes, s0, ks, full, rem,
                                nsw, lane, ca[q], swa[q]);
            }
            myra[q] = routes_of(offa[q], cnta[q]);
          }
#pragma unroll
          for (int q = 0; q < kDnAll; ++q)
            if (q < nde) expert(ca[q], swa[q], offa[q], cnta[q], myra[q]);
        } else {
          int slot_c, off, cnt;
          entry(0, slot_c, off, cnt);
          int myr = routes_of(off, cnt);
#pragma unroll 1
          for (int i = 0; i < nde; ++i) {
            int slot_n, off_n, cnt_n;
            entry(min(i + 1, nde - 1), slot_n, off_n, cnt_n);
            dn_load_steps<TM>(sec + (size_t)slot_n * image_bytes, dn_code_bytes, s0, ks, full, rem,
                              nsw, lane, cn, swn);
            const int myr_n = routes_of(off_n, cnt_n);
            expert(c, sw, off, cnt, myr);
#pragma unroll
            for (int t = 0; t < TM; ++t) c[t] = cn[t];
#pragma unroll
            for (int q = 0; q < TM / 4; ++q) sw[q] = swn[q];
            myr = myr_n;
            off = off_n;
            cnt = cnt_n;
          }
        }
      } else if (nde > 0) {
        // h in the workspace: every step of the next route's h is requested while a route is
        // formed (the next expert's first route after an expert's last), 2 x TM x 16 VGPRs
        int slot_c, off, cnt;
        entry(0, slot_c, off, cnt);
        int myr = routes_of(off, cnt);
        uint4 hc[TM][4], hn[TM][4];
        dn_route_h<TM>(hsrc + (size_t)__builtin_amdgcn_readfirstlane(myr) * I, s0, nb, g, hc);
#pragma unroll 1
        for (int i = 0; i < nde; ++i) {
          int slot_n, off_n, cnt_n;
          entry(min(i + 1, nde - 1), slot_n, off_n, cnt_n);
          dn_load_steps<TM>(sec + (size_t)slot_n * image_bytes, dn_code_bytes, s0, ks, full, rem,
                            nsw, lane, cn, swn);
          const int myr_n = routes_of(off_n, cnt_n);
          const bool more = i + 1 < nde && cnt_n > 0;
#pragma unroll 1
          for (int j = 0; j < cnt; ++j) {
#pragma unroll
            for (int t = 0; t < TM; ++t) asm volatile("" : "+v"(c[t].x), "+v"(c[t].y), "+v"(c[t].z), "+v"(c[t].w));
            const int route = j < 64 ? __builtin_amdgcn_readlane(myr, j) : rw.perm[off + j];
            int rnext = route;
            if (j + 1 < cnt)
              rnext = j + 1 < 64 ? __builtin_amdgcn_readlane(myr, j + 1) : rw.perm[off + j + 1];
            else if (more)
              rnext = __builtin_amdgcn_readfirstlane(myr_n);
            __builtin_amdgcn_sched_barrier(0);
            dn_route_h<TM>(hsrc + (size_t)rnext * I, s0, nb, g, hn);
            __builtin_amdgcn_sched_barrier(0);
            float acc = dn_route_dot_h<TM>(c, sw, s0, spw, ks, nb, g, hc);
            acc = dn_row_sum(acc);
            if (lane < kDnRows) put(route, acc);
#pragma unroll
            for (int t = 0; t < TM; ++t)
#pragma unroll
              for (int q = 0; q < 4; ++q) hc[t][q] = hn[t][q];
          }
          // (an expert with no valid route left hc alone: the next one's first route now)
          if (cnt == 0 && more)
            dn_route_h<TM>(hsrc + (size_t)__builtin_amdgcn_readfirstlane(myr_n) * I, s0, nb, g, hc);
#pragma unroll
          for (int t = 0; t < TM; ++t) c[t] = cn[t];
#pragma unroll
          for (int q = 0; q < TM / 4; ++q) sw[q] = swn[q];
          myr = myr_n;
          off = off_n;
          cnt = cnt_n;
        }
      }
    }
  }
  for (int d = es0; !fast && d < nd; d += sl_all) {
    const int4 dd = rw.dist[d];
    if constexpr (PF) {
      // the last pass re-requests its own weights, unused
      const int dn = d + sl_all < nd ? d + sl_all : d;
      dn_load_steps<TM>(sec + (size_t)rw.dist[dn].x * image_bytes, dn_code_bytes, s0, ks, full,
                        rem, nsw, lane, cn, swn);
    } else if (d != es0) {
      dn_load_steps<TM>(sec + (size_t)dd.x * image_bytes, dn_code_bytes, s0, ks, full, rem, nsw,
                        lane, c, sw);
    }
    const int off = dd.y;
    const int cnt = off >= 0 && dd.z > 0 && off + dd.z <= Mk ? dd.z : 0;
    // the expert's routes, lane j holding route j0 + j (read together, not one per route), and
    // each route's first step of h requested during the previous route's last step
    for (int j0 = 0; j0 < cnt; j0 += 64) {
      const int nj = min(64, cnt - j0);
      const int myr = rw.perm[off + j0 + min(lane, nj - 1)];
      int route = __builtin_amdgcn_readfirstlane(myr);
      if constexpr (TM <= 4) {
        // a short K part: every step of the next route's h is requested while the current route
        // is formed (2 x TM x 16 VGPRs), so a route waits for at most one round trip
        uint4 hc[TM][4], hn[TM][4];
        dn_route_h<TM>(hsrc + (size_t)route * I, s0, nb, g, hc);
#pragma unroll 1
        for (int j = 0; j < nj; ++j) {
#pragma unroll
          for (int t = 0; t < TM; ++t) asm volatile("" : "+v"(c[t].x), "+v"(c[t].y), "+v"(c[t].z), "+v"(c[t].w));
          const int rnext = __builtin_amdgcn_readlane(myr, min(j + 1, nj - 1));
          __builtin_amdgcn_sched_barrier(0);
          dn_route_h<TM>(hsrc + (size_t)rnext * I, s0, nb, g, hn);
          __builtin_amdgcn_sched_barrier(0);
          float acc = dn_route_dot_h<TM>(c, sw, s0, spw, ks, nb, g, hc);
          acc = dn_row_sum(acc);
          if (lane < kDnRows) put(route, acc);
#pragma unroll
          for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) hc[t][q] = hn[t][q];
          route = rnext;
        }
      } else {
        uint4 an[4];
        dn_h_first(hsrc + (size_t)route * I, s0, nb, g, an);
#pragma unroll 1
        for (int j = 0; j < nj; ++j) {
          // keeps the decode of the codes inside this loop (hoisted, it would hold 16 VGPRs per
          // step)
#pragma unroll
          for (int t = 0; t < TM; ++t) asm volatile("" : "+v"(c[t].x), "+v"(c[t].y), "+v"(c[t].z), "+v"(c[t].w));
          const int rnext = __builtin_amdgcn_readlane(myr, min(j + 1, nj - 1));
          float acc = dn_route_dot_pf<TM>(c, sw, s0, spw, ks, nb, g, hsrc + (size_t)route * I,
                                          hsrc + (size_t)rnext * I, an);
          acc = dn_row_sum(acc);
          if (lane < kDnRows) put(route, acc);
          route = rnext;
        }
      }
    }
    if constexpr (PF) {
#pragma unroll
      for (int t = 0; t < TM; ++t) c[t] = cn[t];
#pragma unroll
      for (int q = 0; q < TM / 4; ++q) sw[q] = swn[q];
    }
  }
  if (helper) return;  // (its stores complete before the workgroup ends)
  if (split) {
    // the partner's experts are the odd entries of the hot list: wave w takes entries
    // 1 + 2w, 1 + 2w + 16, ..., four routes at a time (lane: route lane / 16, row lane % 16)
    bool late = false;
    if (s_dlate == 0) {
      const int lr = lane & 15, lj = lane >> 4;
      for (int dh = 1 + 2 * wave; dh < nd && !late; dh += 16) {
        const int4 dd = rw.dist[dh];
        const int off = dd.y;
        const int cnt = off >= 0 && dd.z > 0 && off + dd.z <= Mk ? dd.z : 0;
        for (int j0 = 0; j0 < cnt && !late; j0 += 4) {
          const int j = j0 + lj;
          const int route = rw.perm[off + min(j, cnt - 1)];
          const uint64_t* src = pw + (size_t)route * kSplitRowStride + tile * kDnRows + lr;
          bool ok = j >= cnt;
          uint64_t v = 0;
          for (int spins = 0;; ++spins) {
            if (!ok) {
              v = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              ok = (uint32_t)(v >> 32) == tag;
            }
            if (__ballot(!ok) == 0ull) break;
            if (spins + 1 >= kHandSpins) {
              late = true;
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
          if (j < cnt) parts[(size_t)route * kDnRows + lr] = __uint_as_float((uint32_t)v);
        }
      }
    }
    if (late && lane == 0) s_dlate = 2;
  }
  __syncthreads();
  if (split && threadIdx.x == 0) {
    // every word of the partner carried this call's id: advance it for the next call; after a
    // lost gather, poison the workspace instead (the partner may not have read the id yet)
    if (s_dlate != 0) atomicOr(&rw.meta[kMetaErr], kErrHandoff);
    if (s_dlate == 2)
      __hip_atomic_store(reinterpret_cast<uint32_t*>(&rw.meta[kMetaPoison]), 1u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    else if (s_dlate == 0)
      __hip_atomic_store(&dncall[tile], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const bool lost = split && s_dlate != 0;
  for (int idx = threadIdx.x; idx < ra.M * kDnRows; idx += blockDim.x) {
    const int m = idx / kDnRows;
    const int r = idx - m * kDnRows;
    float acc = 0.0f;
    // 8 routes at a time: the slots and weights of a batch are requested together (one route
    // at a time, each would wait for its own round trip), then the sum in ascending j
    for (int j0 = 0; j0 < ra.k; j0 += 8) {
      bool hot[8];
      float wv[8], pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int route = m * ra.k + min(j0 + u, ra.k - 1);
        hot[u] = j0 + u < ra.k && rw.route_slot[route] >= 0;
        wv[u] = ra.w_in[route];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int route = m * ra.k + min(j0 + u, ra.k - 1);
        float p = 0.0f;
        for (int h = 0; h < kparts; ++h) p += parts[((size_t)route * kparts + h) * kDnRows + r];
        pv[u] = p;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (hot[u]) acc = fmaf(wv[u], pv[u], acc);
    }
    if (lost) acc = __uint_as_float(0x7FC00000u);  // never a silently wrong value
    y[(size_t)m * H + tile * kDnRows + r] = acc;
    residual_store(res, (size_t)m * H + tile * kDnRows + r, acc);
  }
}

// ---- down + partial sums for the combine --------------------------------------------------------
// grid = (ceil(H/16 / (4*kDnRW)), work items), 256 threads.  An item is one distinct hot expert
// and up to kItemRoutes of its routes (the bucketing work list), or, without a work list, one
// distinct hot expert with all its routes (then fewer than kItemRoutes).  Wave w owns down tiles
// kDnRW*(4*blockIdx.x + w) + q; the item's routes go through in passes of 16 (one MFMA column
// each), the h of a pass staged in LDS 4 K steps at a time, double buffered, the next stage's
// weights and h requested before the current stage's MFMAs.  Each route's rows go to
// pdn[route][row] in fp32; k_combine forms y in the fixed route order.
constexpr int kDnRW = 2;                                // down tiles per wave
constexpr size_t kDownLdsBytes = 150 * 1024;            // dynamic LDS of k_down_gemv (gfx950: 160 KiB a workgroup)
constexpr int kDnSub = 16;                              // routes per pass
constexpr int kDnRoutePitch = 4 * 256 + 16;             // 4 steps of hi|lo (+16: bank spread)

struct DnStage {
  uint8_t b[kDnSub][kDnRoutePitch];  // [route][step * 256 + (lo ? 128 : 0) + k]
  uint32_t sc[kDnSub][4];            // [route][step]: scale bytes of the step's 4 blocks
};

__global__ __launch_bounds__(256) void k_down_mx(
    int H, const uint8_t* __restrict__ slots, size_t image_bytes, size_t gu_bytes,
    size_t dn_tile_bytes, size_t dn_code_bytes, int dn_tiles, int ks, int full, int rem, int nsw,
    int I, int nb_i, int h_pad, int h_stride, RouteArgs ra, RouteWs rw, int use_items,
    const uint8_t* __restrict__ hq, float* __restrict__ pdn) {
  __shared__ __align__(16) DnStage st[2];
  __shared__ int route_of[kItemRoutes];
  const int Mk = ra.M * ra.k;
  int d, base;
  if (use_items) {
    if ((int)blockIdx.y >= rw.meta[3]) return;
    const int2 it = rw.items[blockIdx.y];
    d = it.x;
    base = it.y;
  } else {
    if ((int)blockIdx.y >= rw.meta[0]) return;
    d = blockIdx.y;
    base = 0;
  }
  const int4 dd = rw.dist[d];
  const int slot = dd.x, off = dd.y, cnt = dd.z;
  if (cnt <= 0 || off < 0 || off + cnt > Mk || base < 0 || base >= cnt) return;
  const int nt = min(kItemRoutes, cnt - base);
  const int tid = threadIdx.x;
  for (int i = tid; i < kItemRoutes; i += blockDim.x) route_of[i] = rw.perm[off + base + min(i, nt - 1)];
  __syncthreads();
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int T0 = ((int)blockIdx.x * 4 + w) * kDnRW;
  const uint8_t* tb[kDnRW];
#pragma unroll
  for (int q = 0; q < kDnRW; ++q)
    tb[q] = slots + (size_t)slot * image_bytes + gu_bytes + (size_t)min(T0 + q, dn_tiles - 1) * dn_tile_bytes;
  const int ngrp = (ks + 3) / 4;
  // staging of a 4-step group: thread tid moves chunks tid + 256*k (route ci >> 6, step
  // (ci >> 4) & 3, 16-byte piece ci & 15: hi for pieces 0-7, lo for 8-15) and, as thread
  // tid & 63, the scale word of route (tid & 63) >> 2, step tid & 3.  Every load is issued
  // (addresses clamped); chunks past I or past the last step are replaced by zeros.
  for (int sub = 0; sub < nt; sub += kDnSub) {
    const int ns = min(kDnSub, nt - sub);
    uint4 an[kDnRW][4], bvn[4];
    uint32_t swn[kDnRW], svn;
#define MOE_DN_LOAD(GRP)                                                                         \
  do {                                                                                           \
    _Pragma("unroll") for (int q = 0; q < kDnRW; ++q) {                                          \
      swn[q] = dn_sw(tb[q], dn_code_bytes, (GRP), nsw, lane);                                    \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) an[q][j] = dn_a(tb[q], 4 * (GRP) + j, ks, full, rem, lane); \
    }                                                                                            \
    _Pragma("unroll") for (int k2 = 0; k2 < 4; ++k2) {                                           \
      const int ci = tid + 256 * k2;                                                             \
      const int s_ = 4 * (GRP) + ((ci >> 4) & 3);                                                \
      const int pc = ci & 15;                                                                    \
      const int kpos = 128 * s_ + 16 * (pc & 7);                                                 \
      const uint8_t* src = hq + (size_t)route_of[sub + min(ci >> 6, ns - 1)] * h_stride +      \
                           (pc < 8 ? 0 : h_pad) + 128 * min(s_, ks - 1) + 16 * (pc & 7);         \
      const uint4 v_ = *reinterpret_cast<const uint4*>(src);                                     \
      bvn[k2] = (s_ < ks && kpos < I) ? v_ : make_uint4(0, 0, 0, 0);                             \
    }                                                                                            \
    {                                                                                            \
      const int s_ = 4 * (GRP) + (tid & 3);                                                      \
      const uint8_t* src = hq + (size_t)route_of[sub + min((tid & 63) >> 2, ns - 1)] * h_stride + \
                           2 * h_pad + 4 * min(s_, ks - 1);                                      \
      const uint32_t v_ = *reinterpret_cast<const uint32_t*>(src);                               \
      svn = s_ < ks ? h_scale_word(v_, s_, nb_i) : 0x7F7F7F7Fu;                                  \
    }                                                                                            \
  } while (0)
    MOE_DN_LOAD(0);
    f32x4_t acc[kDnRW];
#pragma unroll
    for (int q = 0; q < kDnRW; ++q) acc[q] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int grp = 0; grp < ngrp; ++grp) {
      DnStage& S = st[grp & 1];
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        const int ci = tid + 256 * k2;
        const int pc = ci & 15;
        *reinterpret_cast<uint4*>(&S.b[ci >> 6][((ci >> 4) & 3) * 256 + (pc < 8 ? 0 : 128) + 16 * (pc & 7)]) = bvn[k2];
      }
      if (tid < 64) S.sc[tid >> 2][tid & 3] = svn;
      uint4 ac[kDnRW][4];
      uint32_t sw[kDnRW];
#pragma unroll
      for (int q = 0; q < kDnRW; ++q) {
        sw[q] = swn[q];
#pragma unroll
        for (int j = 0; j < 4; ++j) ac[q][j] = an[q][j];
      }
      if (grp + 1 < ngrp) MOE_DN_LOAD(grp + 1);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool live = 4 * grp + j < ks;
        const uint8_t* bp = &S.b[c][j * 256 + 16 * g];
        const uint4 h0 = *reinterpret_cast<const uint4*>(bp);
        const uint4 h1 = *reinterpret_cast<const uint4*>(bp + 64);
        const uint4 l0 = *reinterpret_cast<const uint4*>(bp + 128);
        const uint4 l1 = *reinterpret_cast<const uint4*>(bp + 192);
        const uint32_t sb = (S.sc[c][j] >> (8 * g)) & 0xFFu;
#pragma unroll
        for (int q = 0; q < kDnRW; ++q) {
          f32x4_t v = mfma_mx_j(j, ac[q][j], h0, h1, acc[q], sw[q], sb);
          v = mfma_mx_j(j, ac[q][j], l0, l1, v, sw[q], sb);
          acc[q] = live ? v : acc[q];
        }
      }
    }
#undef MOE_DN_LOAD
    // lane (g, c), register i: row 4g + i of the tile, route c of the pass
    if (c < ns) {
      float* pr = pdn + (size_t)route_of[sub + c] * H;
#pragma unroll
      for (int q = 0; q < kDnRW; ++q)
        if (T0 + q < dn_tiles)
#pragma unroll
          for (int i = 0; i < 4; ++i) pr[(T0 + q) * kDnRows + 4 * g + i] = acc[q][i];
    }
    __syncthreads();  // the next pass restages st
  }
}

// =============================================================================================
// Fused decode: one token's layer in one launch, h handed over by value
// =============================================================================================
// One workgroup of 16 waves per compute unit, the grid at most the CU count (so it is resident
// at once, one workgroup per CU).  Every workgroup first computes the router itself when it is
// small (E <= 32 rows of H <= 4096: each wave two rows, with the arithmetic of k_router, from
// L2) or reads the logits of a router kernel, and builds the route table in LDS.  The work is cut
// into units: a gate/up unit is 16 h values of one hot expert (their 16 gate and 16 up rows over
// all of K: image lanes 16f..16f+15 and 32+16f..32+16f+15 of gate/up tile t), a down unit is 8
// output rows (rows 8f..8f+7 of a 16-row down tile) over every hot expert.  At H = I the two
// kinds weigh the same bytes.  Workgroup w takes an equal contiguous share of each kind (the down
// shares in reverse workgroup order, so that shares which round up rarely meet in one workgroup)
// and requests every weight byte of its units at once, the 16 waves splitting each unit's K.
// Then it
//   1. forms its gate/up units: per-lane block dots, the lane pair of a row and the waves summed
//      in a fixed order, h = bf16(silu(g)*u), two values per 64-bit word whose high half is the
//      call's tag, stored write-through (device-scope relaxed stores);
//   2. each wave gathers the h its down entries read into LDS by polling those words (loads
//      that bypass the non-coherent caches) until their tag is the call's: a 64-bit store is
//      seen whole or not at all, so a word with the right tag holds this call's values;
//   3. forms its down units (each wave its entries as soon as its h is in) and y for their
//      rows, hot routes in ascending order (+ residual).
// The tag is the call id + 1.  The call id lives in the workspace header: every workgroup reads
// it at its start, and workgroup 0 advances it once its gather has seen every h word with this
// call's tag (so every h writer has read it).  A zero-filled workspace starts at call 0 with
// every h word tagged 0.  The tagged words have a region of the workspace of their own, at a
// fixed offset, that no other kernel writes.  No atomic read-modify-write is involved.  The
// gather is bounded: a workgroup that runs out of it flags kErrHandoff and writes NaN instead of
// its y rows (it cannot happen with the grid resident); if that is workgroup 0, it poisons the
// workspace and every later launch on it flags and writes NaN until it is zero-filled again.
constexpr int kFusedWaves = 16;
constexpr int kFusedThreads = kFusedWaves * 64;
constexpr int kFusedMaxK = 16;      // routes (hot experts) of the token at most
static_assert(kFusedMaxK * kMaxInter * 4 == kFusedHBytes, "tagged h region of the workspace");

// n / d by a multiply: m = floor((2^32 - 1) / d) + 1 (0 for d = 1) gives floor(n * m / 2^32) =
// n / d exactly while n * (d - 1) < 2^32 (the launcher checks the bounds of every use).
struct FusedDivs {
  uint32_t g, ugpe, np2;  // multipliers of: the grid, gate/up units per expert, step pairs
};
__device__ __forceinline__ int div_m(int n, uint32_t m) {
  return m == 0u ? n : (int)__umulhi((uint32_t)n, m);
}
// Share of workgroup w of U units over G workgroups: [lo, lo + n).
__device__ __forceinline__ void unit_share(int w, uint32_t mg, int U, int& lo, int& n) {
  lo = div_m(w * U, mg);
  n = div_m((w + 1) * U, mg) - lo;
}
// v clamped to [lo, hi]; lo when the range is empty
__device__ __forceinline__ int clampi(int v, int lo, int hi) { return max(min(v, hi), lo); }

// Scale byte j of word w as a float, or zero when !keep.  Branch-free (a mask, not a
// conditional): a conditional use lets the compiler sink the word's load into the branch and
// wait there for every load in flight.
__device__ __forceinline__ float scale_or_zero(uint32_t w, int j, bool keep) {
  const float f = e8m0_to_f32((w >> (8 * j)) & 0xFFu);
  return __uint_as_float(__float_as_uint(f) & (keep ? 0xFFFFFFFFu : 0u));
}

// Adds the dot of one 32-element block (16 code bytes, the block scale sc folded into the
// scaled converter) with 32 bf16 activations to two accumulation chains (even / odd pairs).
__device__ __forceinline__ void block_dot_scaled(const uint4 c, const uint4 a0, const uint4 a1,
                                                 const uint4 a2, const uint4 a3, float sc,
                                                 float& s0, float& s1) {
  const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
  const uint32_t aw[16] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w,
                           a2.x, a2.y, a2.z, a2.w, a3.x, a3.y, a3.z, a3.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], sc, 0),
                                         as_bf16x2(aw[4 * j + 0]), s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], sc, 1),
                                         as_bf16x2(aw[4 * j + 1]), s1, false);
    s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], sc, 2),
                                         as_bf16x2(aw[4 * j + 2]), s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], sc, 3),
                                         as_bf16x2(aw[4 * j + 3]), s1, false);
  }
}

// LDS of the kernel past the route table: x runs (1 KiB each), h rows of the k routes, the
// gate/up sums [NUG][waves][32], the down sums [NUD][k][waves][8] and their wave totals
// [NUD][k][8].
__host__ __device__ __forceinline__ size_t fused_x_bytes(int H) { return (size_t)((H / 8 + 63) / 64) * 1024; }
__host__ __device__ __forceinline__ size_t fused_lds_bytes(int H, int I, int k, int nug, int nud) {
  return fused_x_bytes(H) + (size_t)k * I * 2 + (size_t)nug * kFusedWaves * 32 * 4 +
         (size_t)nud * k * (kFusedWaves + 1) * 8 * 4;
}

// ---- the router inside the fused kernel ----------------------------------------------------
// Each wave computes the logits of two experts with the arithmetic of k_router<CPL> (lane l sums
// the bf16 dot products of chunks l, l + 64, ... in that order, then the wave sum, then the
// bias), so the logits are bitwise those of moe_route.  Every workgroup reads all the rows (from
// L2); the rows a wave takes rotate with the workgroup index, so that the compute units of an
// XCD do not all ask the same L2 channel for the same row at once.  The rows are requested
// first; then this thread's chunk of x (xr, already requested) goes to LDS and a barrier
// publishes it; the products read x from there.  Rows past E re-read the last row and are
// dropped.  Contains a workgroup barrier (every thread calls it).
template <int CPL>
__device__ __forceinline__ void fused_router(const uint16_t* __restrict__ wr,
                                             const float* __restrict__ bias, int E, int H,
                                             uint16_t* xs, const uint4& xr, float* s_logit) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nch = H / 8;
  const int rot = (wave + (int)blockIdx.x) & (kFusedWaves - 1);
  const int e0 = rot, e1 = rot + kFusedWaves;
  const uint4* r0 = reinterpret_cast<const uint4*>(wr + (size_t)min(e0, E - 1) * H);
  const uint4* r1 = reinterpret_cast<const uint4*>(wr + (size_t)min(e1, E - 1) * H);
  uint4 w0[CPL], w1[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) w0[i] = r0[min(lane + 64 * i, nch - 1)];
#pragma unroll
  for (int i = 0; i < CPL; ++i) w1[i] = r1[min(lane + 64 * i, nch - 1)];
  const float* bp = bias != nullptr ? bias : reinterpret_cast<const float*>(wr);  // (a valid address)
  const float b0 = bp[min(e0, E - 1)], b1 = bp[min(e1, E - 1)];
  if ((int)threadIdx.x < nch) reinterpret_cast<uint4*>(xs)[threadIdx.x] = xr;
  lds_barrier();  // x in LDS; the row loads stay in flight
  const uint4* xv = reinterpret_cast<const uint4*>(xs);
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const uint4 xc = xv[min(lane + 64 * i, nch - 1)];
    const float v0 = dot8_bf16(w0[i], xc, a0);
    const float v1 = dot8_bf16(w1[i], xc, a1);
    a0 = lane + 64 * i < nch ? v0 : a0;
    a1 = lane + 64 * i < nch ? v1 : a1;
  }
  a0 = wave_sum(a0);
  a1 = wave_sum(a1);
  if (lane == 0) {
    if (e0 < E) s_logit[e0] = a0 + (bias != nullptr ? b0 : 0.0f);
    if (e1 < E) s_logit[e1] = a1 + (bias != nullptr ? b1 : 0.0f);
  }
}

// ROUTER: the router runs inside (wr, bias, rcpl = H/8/64 chunks per lane); else the logits of a
// router kernel are in the workspace (ra.logits).
template <int NUG, int NEG, int NUD, int NED, bool ROUTER>
__global__ __launch_bounds__(kFusedThreads) void k_layer_decode(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, const float* __restrict__ bias,
    int rcpl, int H, int I, const uint8_t* __restrict__ slots,
    size_t image_bytes, size_t gu_tile_bytes, int nb, size_t gu_bytes, size_t dn_tile_bytes,
    size_t dn_code_bytes, int ks, int full, int rem, int nb_i, RouteArgs ra, RouteWs rw,
    uint64_t* __restrict__ hf, float* __restrict__ y, Residual res, FusedDivs dv) {
  __shared__ RouteLds rt;
  __shared__ int s_dist_of_route[kFusedMaxK];  // one token: route j -> its hot expert index
  __shared__ int s_late;                       // a wave's gather of h ran out of rounds
  __shared__ uint32_t s_tag;                   // this call's tag of the h words
  __shared__ float s_logit[ROUTER ? kFusedRouterMaxE : 1];
  extern __shared__ __align__(16) uint8_t fsm[];
  const int lane = threadIdx.x & 63;
  uint32_t* hdr = reinterpret_cast<uint32_t*>(rw.meta);
  if (threadIdx.x == 0) s_late = 0;  // (the barriers below publish it)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = gridDim.x, wg = blockIdx.x;
  const int K = ra.k;
  uint16_t* xs = reinterpret_cast<uint16_t*>(fsm);
  uint16_t* hs = reinterpret_cast<uint16_t*>(fsm + fused_x_bytes(H));
  float* red_gu = reinterpret_cast<float*>(fsm + fused_x_bytes(H) + (size_t)K * I * 2);
  float* red_dn = red_gu + NUG * kFusedWaves * 32;       // [NUD][K][waves][8]
  float* sum_dn = red_dn + NUD * K * kFusedWaves * 8;    // [NUD][K][8]

  // x: one 16-byte chunk per thread (H / 8 <= threads), requested first; it lands with the
  // router rows (ROUTER) or the route table's loads and goes to LDS
  const int n_x = H / 8;
  const uint4 xr = reinterpret_cast<const uint4*>(x)[min((int)threadIdx.x, n_x - 1)];
  if constexpr (ROUTER) {
    const int lc = lane < ra.E ? lane : 0;
    const int32_t* e2p = ra.e2s != nullptr ? ra.e2s : reinterpret_cast<const int32_t*>(wr);
    const int e2v = e2p[lc];  // (with no map: a dummy read, unused)
    switch (rcpl) {  // (uniform)
      case 1: fused_router<1>(wr, bias, ra.E, H, xs, xr, s_logit); break;
      case 2: fused_router<2>(wr, bias, ra.E, H, xs, xr, s_logit); break;
      case 3: fused_router<3>(wr, bias, ra.E, H, xs, xr, s_logit); break;
      case 4: fused_router<4>(wr, bias, ra.E, H, xs, xr, s_logit); break;
      case 5: fused_router<5>(wr, bias, ra.E, H, xs, xr, s_logit); break;
      case 6: fused_router<6>(wr, bias, ra.E, H, xs, xr, s_logit); break;
      case 7: fused_router<7>(wr, bias, ra.E, H, xs, xr, s_logit); break;
      default: fused_router<8>(wr, bias, ra.E, H, xs, xr, s_logit); break;
    }
    __syncthreads();  // the logits
    route_token_small_v(rt, ra, s_logit[lc], ra.e2s != nullptr ? e2v : lc);
    __syncthreads();
  } else {
    route_prologue(rt, ra, rw, false);
    if ((int)threadIdx.x < n_x) reinterpret_cast<uint4*>(xs)[threadIdx.x] = xr;
  }
  const int nd = rt.nd;
  const int ugpe = I / 16;  // gate/up units per hot expert
  const int Ug = nd * ugpe;
  int gu_lo, ngu, dn_lo, ndn;
  unit_share(wg, dv.g, Ug, gu_lo, ngu);
  unit_share(G - 1 - wg, dv.g, H / 8, dn_lo, ndn);
  // this wave's part of a unit: block pairs [gp0, gp0 + ngp) of a gate/up unit, (expert, step
  // pair) entries [dq0, dq0 + ndq) of a down unit
  const int np = (nb + 1) / 2;
  const int gp0 = wave * np / kFusedWaves, ngp = (wave + 1) * np / kFusedWaves - gp0;
  const int np2 = (ks + 1) / 2;
  const int Ld = (nd > 0 ? nd : 1) * np2;
  const int dq0 = wave * Ld / kFusedWaves, ndq = (wave + 1) * Ld / kFusedWaves - dq0;
  const int half = lane >> 5;                          // gate/up: block 2p + half
  const int ll = lane & 31;
  const int gil = ll < 16 ? ll : ll + 16;              // + 16f: image lane (gate ll / up ll-16)
  const int blk = (lane >> 3) & 3, r8 = lane & 7;      // down: step 2p + half, block 4s + blk
  auto slot_of = [&](int d) {  // (the LDS read is unconditional: no wait inside a branch)
    const int sl = rt.dist_slot[clampi(d, 0, max(nd - 1, 0))];
    return nd > 0 ? sl : 0;
  };

  uint32_t sg[NUG][NEG], sd[NUD][NED];
  uint4 cg[NUG][NEG], cd[NUD][NED];
  // the hot experts of this wave's units and entries, then their slots: every LDS read issued
  // before any is used
  int dg[NUG], t2g[NUG], exq[NED], slg[NUG], sle[NED];
#pragma unroll
  for (int ug = 0; ug < NUG; ++ug) {
    const int u = clampi(gu_lo + clampi(ug, 0, ngu - 1), 0, max(Ug - 1, 0));
    dg[ug] = div_m(u, dv.ugpe);
    t2g[ug] = u - dg[ug] * ugpe;
  }
#pragma unroll
  for (int e = 0; e < NED; ++e) exq[e] = div_m(dq0 + clampi(e, 0, ndq - 1), dv.np2);
#pragma unroll
  for (int ug = 0; ug < NUG; ++ug) slg[ug] = slot_of(dg[ug]);
#pragma unroll
  for (int e = 0; e < NED; ++e) sle[e] = slot_of(exq[e]);
  // (each is the same for the whole wave: in scalar registers, the image bases are formed on
  // the scalar unit)
#pragma unroll
  for (int ug = 0; ug < NUG; ++ug) slg[ug] = __builtin_amdgcn_readfirstlane(slg[ug]);
#pragma unroll
  for (int e = 0; e < NED; ++e) sle[e] = __builtin_amdgcn_readfirstlane(sle[e]);
  const uint8_t* gtb[NUG];
  int gilf[NUG];
#pragma unroll
  for (int ug = 0; ug < NUG; ++ug) {
    gtb[ug] = slots + (size_t)slg[ug] * image_bytes + (size_t)(t2g[ug] >> 1) * gu_tile_bytes;
    gilf[ug] = 16 * (t2g[ug] & 1) + gil;
  }
  const uint8_t* dtb[NUD][NED];
  int dix[NUD][NED], dsw[NUD][NED];
#pragma unroll
  for (int ud = 0; ud < NUD; ++ud) {
    const int u = clampi(dn_lo + clampi(ud, 0, ndn - 1), 0, H / 8 - 1);
    const int il = 16 * blk + 8 * (u & 1) + r8;
#pragma unroll
    for (int e = 0; e < NED; ++e) {
      const int q = dq0 + clampi(e, 0, ndq - 1);
      const int s = min(2 * (q - exq[e] * np2) + half, ks - 1);
      dtb[ud][e] = slots + (size_t)sle[e] * image_bytes + gu_bytes + (size_t)(u >> 1) * dn_tile_bytes;
      dix[ud][e] = s < full ? s * 64 + il : full * 64 + min(il, 16 * rem - 1);
      dsw[ud][e] = (s >> 2) * 64 + il;
    }
  }
  // The gate/up bytes are needed first, and requests compete in the memory system: the gate/up
  // scale words and codes are requested now, the down ones by each wave once its gate/up
  // arithmetic is done (their stream then overlaps the rest of gate/up and the hand-over).
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int e = 0; e < NEG; ++e)
#pragma unroll
    for (int ug = 0; ug < NUG; ++ug) {
      const int b = min(2 * (gp0 + clampi(e, 0, ngp - 1)) + half, nb - 1);
      sg[ug][e] = ld_nt32(reinterpret_cast<const uint32_t*>(gtb[ug] + (size_t)nb * 1024) + (b >> 2) * 64 + gilf[ug]);
    }
#pragma unroll
  for (int e = 0; e < NEG; ++e)
#pragma unroll
    for (int ug = 0; ug < NUG; ++ug) {
      const int b = min(2 * (gp0 + clampi(e, 0, ngp - 1)) + half, nb - 1);
      cg[ug][e] = ld_nt(reinterpret_cast<const uint4*>(gtb[ug]) + b * 64 + gilf[ug]);
    }
  // Workgroup 0 publishes the routes, the cold report and the table (from its LDS copy) only
  // now: stores count with the loads in flight, so before the gate/up requests they would hold
  // those back until they had completed.
  if (wg == 0) {
    write_routes(rt, ra.k, ra.topk_ids, ra.topk_w, ra.cold_count, ra.cold_routes, nullptr);
    write_table(rt, ra.k, rw);
  }
  // The call id and the poison word (thread 0), needed only when h is stored: requested behind
  // the gate/up weights, so that nothing waits for them before.
  uint64_t callw = 0;
  if (threadIdx.x == 0)
    callw = __hip_atomic_load(reinterpret_cast<uint64_t*>(&hdr[kMetaCall]), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_sched_barrier(0);
  // x in LDS for every wave (the gate/up loads stay in flight); with the router inside, the
  // router's own barrier has published it, so each wave starts on its gate/up bytes as soon as
  // they land
  if constexpr (!ROUTER) lds_barrier();
  // The gate/up block scales as floats for the scaled converter (while the codes are in
  // flight); zero for lanes whose block lies past K, which re-read a valid block and must add
  // nothing.
  float fg[NUG][NEG];
#pragma unroll
  for (int ug = 0; ug < NUG; ++ug)
#pragma unroll
    for (int e = 0; e < NEG; ++e) {
      const int b = 2 * (gp0 + clampi(e, 0, ngp - 1)) + half;
      fg[ug][e] = scale_or_zero(sg[ug][e], b & 3, b < nb);
    }
  // hot expert t (< nd) -> its route (one token: every hot route is its own expert), and back
  if ((int)threadIdx.x < nd) s_dist_of_route[rt.perm[rt.dist_off[threadIdx.x]]] = threadIdx.x;

  // ---- 1. gate/up units ----
  // block pair by block pair (the order in which they were requested), one read of the x block
  // serving every unit
  float s0[NUG], s1[NUG];
#pragma unroll
  for (int ug = 0; ug < NUG; ++ug) s0[ug] = s1[ug] = 0.0f;
#pragma unroll
  for (int e = 0; e < NEG; ++e) {
    if (e < ngp) {  // uniform
      const int b = 2 * (gp0 + e) + half;
      const uint4* a = reinterpret_cast<const uint4*>(xs + 32 * min(b, nb - 1));
      const uint4 a0 = a[0], a1 = a[1], a2 = a[2], a3 = a[3];
#pragma unroll
      for (int ug = 0; ug < NUG; ++ug)
        if (ug < ngu)  // uniform
          block_dot_scaled(cg[ug][e], a0, a1, a2, a3, fg[ug][e], s0[ug], s1[ug]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int ug = 0; ug < NUG; ++ug) {
    const float v = pair_sum32(s0[ug] + s1[ug]);  // the other block of each pair
    if (lane < 32) red_gu[(ug * kFusedWaves + wave) * 32 + lane] = v;
  }
  // this wave's gate/up bytes have all landed: its down bytes are requested now (the requests
  // of the waves still waiting for gate/up bytes were issued before them)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ud = 0; ud < NUD; ++ud)
#pragma unroll
    for (int e = 0; e < NED; ++e)
      sd[ud][e] = ld_nt32(reinterpret_cast<const uint32_t*>(dtb[ud][e] + dn_code_bytes) + dsw[ud][e]);
#pragma unroll
  for (int ud = 0; ud < NUD; ++ud)
#pragma unroll
    for (int e = 0; e < NED; ++e) cd[ud][e] = ld_nt(reinterpret_cast<const uint4*>(dtb[ud][e]) + dix[ud][e]);
  __builtin_amdgcn_sched_barrier(0);
  // this call's tag; a poisoned workspace (an earlier launch lost its hand-over) makes this
  // workgroup's rows NaN
  const uint32_t call = (uint32_t)callw;
  if (threadIdx.x == 0) {
    s_tag = call + 1u;
    if ((uint32_t)(callw >> 32) != 0u) {
      s_late = 1;
      atomicOr(&rw.meta[kMetaErr], kErrHandoff);
    }
  }
  __syncthreads();
  const uint32_t tag = s_tag;
  if ((int)threadIdx.x < NUG * 16) {
    const int ug = threadIdx.x >> 4, r = threadIdx.x & 15;
    if (ug < ngu) {  // (the same for both lanes of a pair)
      // (unrolled: the 32 LDS reads issue back to back)
      float g = 0.0f, u = 0.0f;
#pragma unroll
      for (int w = 0; w < kFusedWaves; ++w) {
        g += red_gu[(ug * kFusedWaves + w) * 32 + r];
        u += red_gu[(ug * kFusedWaves + w) * 32 + 16 + r];
      }
      const int uu = gu_lo + ug;
      const int d = div_m(uu, dv.ugpe), t2 = uu - d * ugpe;
      const int route = rt.perm[rt.dist_off[d]];
      const uint32_t hv = f32_to_bf16_bits(silu_f32(g) * u);
      const uint32_t hn = (uint32_t)__shfl_down((int)hv, 1);  // the pair's odd element
      if ((r & 1) == 0) {
        const size_t pos = (size_t)route * I + (t2 >> 1) * 32 + 16 * (t2 & 1) + r;  // even
        __hip_atomic_store(&hf[pos >> 1], (uint64_t)(hv | (hn << 16)) | ((uint64_t)tag << 32),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (ndn == 0) {  // no down unit here: the down loads (dummies) drain before the exit
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }

  // The down weights (in flight since this wave's gate/up arithmetic) are decoded to bf16 while
  // h is still being formed elsewhere, so that only the products remain after the gather.
  bf16x2_t wd[NUD][NED][16];
#pragma unroll
  for (int ud = 0; ud < NUD; ++ud)
#pragma unroll
    for (int e = 0; e < NED; ++e) {
      const int q = dq0 + clampi(e, 0, ndq - 1);
      const int ex = div_m(q, dv.np2);
      const int st = 2 * (q - ex * np2) + half;
      block_to_bf16(cd[ud][e], scale_or_zero(sd[ud][e], st & 3, st < ks && 4 * st + blk < nb_i), wd[ud][e]);
      // (here, not sunk into the products after the gather)
#pragma unroll
      for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(wd[ud][e][i]));
    }

  // ---- 2. this wave's h into LDS ----
  // Entry (hot expert ex, step pair p) reads h[ex][256p, 256p + 256) (clamped to I): 64 chunks
  // of 4 values (two tagged words, 16 bytes).  Each wave polls the chunks of its own entries
  // only, lane l taking chunk l of each, and a lane re-requests a chunk only until both its
  // words carry the call's tag.  No other wave reads these LDS bytes (a wave's own LDS
  // operations complete in order), so the products of a wave start as soon as its own h has
  // landed, with no workgroup barrier.
  {
    constexpr int PC = NED;
    const uint64_t* src[PC];
    int dst[PC];
    bool need[PC];
#pragma unroll
    for (int i = 0; i < PC; ++i) {
      const int q = dq0 + clampi(i, 0, ndq - 1);
      const int ex = div_m(q, dv.np2);
      const int exc = clampi(ex, 0, max(nd - 1, 0));
      const int route = nd > 0 ? rt.perm[rt.dist_off[exc]] : 0;
      const int off = min(256 * (q - ex * np2) + 4 * lane, I - 4);
      need[i] = i < ndq && ex < nd;
      src[i] = hf + (((size_t)route * I + off) >> 1);
      dst[i] = exc * I + off;
    }
    bool late = false;
    for (int spins = 0;; ++spins) {
      uint64_t v[PC][2];
#pragma unroll
      for (int i = 0; i < PC; ++i)
        if (need[i]) {
          v[i][0] = __hip_atomic_load(src[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          v[i][1] = __hip_atomic_load(src[i] + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      bool left = false;
#pragma unroll
      for (int i = 0; i < PC; ++i)
        if (need[i]) {
          if ((uint32_t)(v[i][0] >> 32) == tag && (uint32_t)(v[i][1] >> 32) == tag) {
            reinterpret_cast<uint2*>(hs)[dst[i] / 4] = make_uint2((uint32_t)v[i][0], (uint32_t)v[i][1]);
            need[i] = false;
          } else {
            left = true;
          }
        }
      if (__ballot(left) == 0ull) break;
      if (spins + 1 >= kHandSpins) {
        late = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (late && lane == 0) {
      atomicOr(&rw.meta[kMetaErr], kErrHandoff);
      s_late = 1;  // this workgroup's y rows become NaN
    }
    // (the products below read LDS written by other lanes of this wave)
    asm volatile("" ::: "memory");
  }

  // ---- 3. down units and y ----
  // Entry by entry (one h block read serves every unit); a wave's entries are consecutive
  // (expert, step pair)s, so they cover at most two hot experts: ex0 and ex0 + 1.
  const int ex0 = div_m(dq0, dv.np2);
  float accA[NUD], accB[NUD];
#pragma unroll
  for (int ud = 0; ud < NUD; ++ud) accA[ud] = accB[ud] = 0.0f;
#pragma unroll
  for (int e = 0; e < NED; ++e) {
    const int q = dq0 + e;
    const int ex = div_m(q, dv.np2);
    if (e < ndq && ex < nd) {  // uniform
      const int st = 2 * (q - ex * np2) + half;
      const uint4* hb = reinterpret_cast<const uint4*>(hs + (size_t)ex * I + 32 * min(4 * st + blk, nb_i - 1));
      const uint4 h0 = hb[0], h1 = hb[1], h2 = hb[2], h3 = hb[3];
#pragma unroll
      for (int ud = 0; ud < NUD; ++ud) {
        if (ud < ndn) {  // uniform
          float t0 = 0.0f, t1 = 0.0f;
          block_dot_bf16(wd[ud][e], h0, h1, h2, h3, t0, t1);
          if (ex == ex0)
            accA[ud] += t0 + t1;
          else
            accB[ud] += t0 + t1;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // rows of each unit: the lanes of a row summed (8 per row), written per hot expert slot
  // (zero for the slots this wave has no entry of)
#pragma unroll
  for (int ud = 0; ud < NUD; ++ud) {
    if (ud < ndn) {
      const float va = pair_sum32(pair_sum16(pair_sum8(accA[ud])));
      const float vb = pair_sum32(pair_sum16(pair_sum8(accB[ud])));
      if (lane < 8)
        for (int j = 0; j < K; ++j)
          red_dn[((ud * K + j) * kFusedWaves + wave) * 8 + lane] = j == ex0 ? va : (j == ex0 + 1 ? vb : 0.0f);
    }
  }
  __syncthreads();
  // y for every row: each hot expert's row over the waves, then the routes in ascending order
  // (one token: route j = rank j).  With few routes one wave does it all, lane (unit, row,
  // slot); otherwise the sums over the waves come first, from every thread, then the routes.
  constexpr int T = 64 / (NUD * 8);  // slots per row in the one-wave form
  const int row0 = 8 * dn_lo;
  const bool late_wg = s_late != 0;  // (written before the barrier above)
  // Workgroup 0 (which always has a down unit) has now seen every h word of every hot expert
  // with this call's tag, so every workgroup that stores h has read the call id: it advances the
  // id for the next launch.  (A workgroup with no gate/up unit that started even later reads the
  // advanced id, finds no word with its tag and flags the call; none of its words exist.)  If
  // its gather ran out of rounds, some workgroup may not have read the id yet: the id stays and
  // the workspace is poisoned instead, so that no later launch can take a word of this one.
  if (wg == 0 && threadIdx.x == 0) {
    if (late_wg)
      __hip_atomic_store(&hdr[kMetaPoison], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      __hip_atomic_store(&hdr[kMetaCall], call + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  auto store_y = [&](int row, float acc_y) {
    if (late_wg) acc_y = __uint_as_float(0x7FC00000u);  // never a silently wrong value
    y[row] = acc_y;
    // the residual reads x from its LDS copy
    if (res.out != nullptr)
      res.out[row] = (uint16_t)f32_to_bf16_bits(__uint_as_float((uint32_t)xs[row] << 16) + acc_y);
  };
  if (K <= 4 && NUD * 8 <= kFusedWaves) {
    // one row per wave (wave = unit * 8 + row): lane (slot t, wave w) takes that wave's sum of
    // the row for hot expert slot t; the rows of 16 lanes sum over the waves; then the routes
    // in ascending order
    const int ud = wave >> 3, r = wave & 7;
    if (ud < ndn) {  // (uniform)
      const int t = lane >> 4, w = lane & 15;
      float p = red_dn[((ud * K + min(t, K - 1)) * kFusedWaves + w) * 8 + r];
      p = row_sum16(p);
      float pt[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pt[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), 16 * i));
      float acc_y = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j < K) {
          const int dj = s_dist_of_route[j];
          float pj = 0.0f;
#pragma unroll
          for (int i = 0; i < 4; ++i) pj = dj == i ? pt[i] : pj;
          if (rt.slot[j] >= 0) acc_y = fmaf(rt.w[j], pj, acc_y);
        }
      }
      if (lane == 0) store_y(row0 + wave, acc_y);
    }
  } else if (K <= T) {
    if (wave == 0) {
      const int t = lane % T;
      const int rr = lane / T;  // unit * 8 + row
      const int ud = rr >> 3, r = rr & 7;
      float p = 0.0f;
      if (t < K)
#pragma unroll
        for (int w = 0; w < kFusedWaves; ++w) p += red_dn[((ud * K + t) * kFusedWaves + w) * 8 + r];
      float pt[T];
#pragma unroll
      for (int i = 0; i < T; ++i) pt[i] = __shfl(p, rr * T + i);
      if (t == 0 && ud < ndn) {
        // (unrolled over the K <= T routes: their LDS reads issue together)
        float acc_y = 0.0f;
#pragma unroll
        for (int j = 0; j < T; ++j) {
          if (j < K) {
            const int dj = s_dist_of_route[j];
            float pj = 0.0f;
#pragma unroll
            for (int i = 0; i < T; ++i) pj = dj == i ? pt[i] : pj;
            if (rt.slot[j] >= 0) acc_y = fmaf(rt.w[j], pj, acc_y);
          }
        }
        store_y(row0 + rr, acc_y);
      }
    }
  } else {
    for (int i = threadIdx.x; i < NUD * K * 8; i += kFusedThreads) {
      const int r = i & 7, uj = i >> 3;  // uj = unit * K + hot expert
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < kFusedWaves; ++w) v += red_dn[(uj * kFusedWaves + w) * 8 + r];
      sum_dn[i] = v;
    }
    __syncthreads();
    if ((int)threadIdx.x < NUD * 8) {
      const int ud = threadIdx.x >> 3, r = threadIdx.x & 7;
      if (ud < ndn) {
        // (unrolled over the routes: every LDS read issues before the ordered sum; cold routes
        // have no hot expert index, so theirs is clamped and the term skipped)
        float pj[kFusedMaxK], wj[kFusedMaxK];
        bool hj[kFusedMaxK];
#pragma unroll
        for (int j = 0; j < kFusedMaxK; ++j) {
          const int jc = min(j, K - 1);
          hj[j] = j < K && rt.slot[jc] >= 0;
          wj[j] = rt.w[jc];
          pj[j] = sum_dn[(ud * K + min(max(s_dist_of_route[jc], 0), K - 1)) * 8 + r];
        }
        float acc_y = 0.0f;
#pragma unroll
        for (int j = 0; j < kFusedMaxK; ++j)
          if (hj[j]) acc_y = fmaf(wj[j], pj[j], acc_y);
        store_y(row0 + threadIdx.x, acc_y);
      }
    }
  }
}

// =============================================================================================
// Grouped GEMM path (many tokens per expert): bf16 MFMA on dequantised MXFP4 weights
// =============================================================================================
// With tens of routes per expert the weights are worth decoding once and reusing for every
// route, which is a dense contraction: v_mfma_f32_16x16x32_bf16.  Its operands (gfx950):
//   A (routes x K):   lane l holds A[l % 16][8*(l/16) .. +8]   (8 bf16)
//   B (weights x K):  lane l holds B[l % 16][8*(l/16) .. +8]
//   C (routes x rows): lane l, register i holds C[4*(l/16) + i][l % 16].
// One K step of 32 is one MXFP4 block, so a lane's B fragment is one code dword (8 E2M1 values)
// converted with the block scale by the gfx950 scaled converter, which is exact.  The B
// fragments come straight from the expert image: in the gate/up layout wave w, lane l reads
// dword l/16 of image lane 16w + l%16 (wave 0/1 = gate rows 0-15/16-31, wave 2/3 = up rows),
// so a wave's read of one block is 256 contiguous bytes.  The routes' activation rows (A) are
// gathered through the bucket permutation into LDS, KC blocks at a time, double buffered; the
// next chunk's weights and activations are requested before the current chunk's MFMAs.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// staged activation rows: a native vector type (an array of the HIP uint4 struct stayed in
// scratch memory across the chunk loop)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGemmTok = 64;                 // routes per pass: 4 MFMA tiles of 16
static_assert(kGemmTok == kItemRoutes, "one work item is one pass of a grouped GEMM workgroup");
constexpr int kGemmKC = 4;                   // K blocks (of 32) per chunk
constexpr int kGemmPitch = kGemmKC * 32 + 8;  // bf16 per LDS row: 272 bytes, 16 tokens hit 16 bank groups
constexpr int kGemmXPerThread = kGemmTok * kGemmKC * 4 / 256;  // 16-byte chunks staged per thread

__device__ __forceinline__ bf16x8_t fp4x8_to_bf16(uint32_t w, float scale) {
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  bf16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Activation rows of one pass: 64 rows x KC blocks, 16 bytes per chunk, rows clamped to the pass
// (rows past it are never stored back) and K clamped to the row (blocks past it meet zero weights).
struct GemmRows {
  int tok[kGemmTok];  // (token indices, not pointers: a pointer read back from LDS would make the
                      // loads flat ones, which the waits for LDS reads also wait for)
  int route[kGemmTok];
};

__device__ __forceinline__ void gemm_load_rows(const uint16_t* __restrict__ x, const GemmRows& gr,
                                               int kc, int K,
                                               u32x4_t (&xv)[kGemmXPerThread]) {
#pragma unroll
  for (int i = 0; i < kGemmXPerThread; ++i) {
    const int c = (int)threadIdx.x + 256 * i;
    const int tok = c >> 4;
    const int q = c & 15;  // block q>>2, quarter q&3
    const int e = min(kc * kGemmKC * 32 + q * 8, K - 8);
    xv[i] = *reinterpret_cast<const u32x4_t*>(x + (size_t)gr.tok[tok] * K + e);
  }
}

__device__ __forceinline__ void gemm_store_rows(uint16_t (*xb)[kGemmPitch],
                                                const u32x4_t (&xv)[kGemmXPerThread]) {
#pragma unroll
  for (int i = 0; i < kGemmXPerThread; ++i) {
    const int c = (int)threadIdx.x + 256 * i;
    *reinterpret_cast<u32x4_t*>(&xb[c >> 4][(c & 15) * 8]) = xv[i];
  }
}

// Loads of one K chunk (kGemmKC = 4 blocks) for the gate/up tile of one wave: per row tile q (16
// rows: image lanes 16q .. 16q+15, q = 0, 1 gate and 2, 3 up) lane (n, g) takes the whole 16-byte
// code chunk of row n in block g of the chunk (one dwordx4 load) and the scale word of the
// chunk's group (byte g is the block's scale).  The MFMA K steps then run over the chunk in a
// permuted order: step j, lane group g = elements 8j .. 8j+7 of block g (the activations are read
// from LDS in the same order).  Blocks past nb re-read block nb-1 and get scale 0.
static_assert(kGemmKC == 4, "one chunk = one scale word per row");
struct GuChunk {
  uint4 code[4];
  uint32_t scale[4];
};

__device__ __forceinline__ void gu_load_chunk(const uint8_t* tb, int nb, int kc, int n, int g,
                                              GuChunk& ch) {
  const uint32_t* sbase = reinterpret_cast<const uint32_t*>(tb + (size_t)nb * 1024);
  const int b = min(kc * kGemmKC + g, nb - 1);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    ch.code[q] = *reinterpret_cast<const uint4*>(tb + (size_t)b * 1024 + (size_t)(16 * q + n) * 16);
    ch.scale[q] = sbase[(size_t)min(kc, (nb - 1) / 4) * 64 + 16 * q + n];
  }
}

// grid = (ceil(I/32 / 4), work items), 256 threads.  One item = one distinct hot expert and up to
// 64 of its routes (busy experts are split over several items, so that one popular expert does
// not serialise the call).  Wave w owns gate/up image tile 4*blockIdx.x + w (32 gate + 32 up
// rows) for the item's routes: 4 route tiles x 4 row tiles of MFMA accumulators, and a lane
// ends up holding gate row r and up row r of the same route, so h = bf16(silu(g) * u) needs no
// exchange.  The routes' activations are staged once per 4 image tiles.
__global__ __launch_bounds__(256) void k_gateup_grouped(
    const uint16_t* __restrict__ x, int H, int I, const uint8_t* __restrict__ slots,
    size_t image_bytes, size_t gu_tile_bytes, int nb, int n_tiles, int h_pad, int h_stride,
    RouteArgs ra, RouteWs rw, uint8_t* __restrict__ hq) {
  __shared__ __align__(16) uint16_t xb[2][kGemmTok][kGemmPitch];
  __shared__ GemmRows gr;
  const int Mk = ra.M * ra.k;
  if ((int)blockIdx.y >= rw.meta[3]) return;
  const int2 item = rw.items[blockIdx.y];  // (distinct expert, first route of the pass)
  const int4 dd = rw.dist[item.x];
  const int slot = dd.x, off = dd.y, cnt = dd.z;
  if (cnt <= 0 || off < 0 || off + cnt > Mk || item.y < 0 || item.y >= cnt) return;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int tile = min(4 * (int)blockIdx.x + w, n_tiles - 1);  // waves past the last tile idle
  const bool tile_ok = 4 * (int)blockIdx.x + w < n_tiles;
  const uint8_t* tb = slots + (size_t)slot * image_bytes + (size_t)tile * gu_tile_bytes;
  const int nkc = (nb + kGemmKC - 1) / kGemmKC;
  const int base = item.y;
  const int nt = min(kGemmTok, cnt - base);
  const int ntt = (nt + 15) >> 4;
  for (int i = threadIdx.x; i < kGemmTok; i += blockDim.x) {
    const int r = rw.perm[off + base + min(i, nt - 1)];
    gr.route[i] = r;
    gr.tok[i] = r / ra.k;
  }
  __syncthreads();
  f32x4_t acc[4][4];  // [route tile][row tile]
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[t][q] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  u32x4_t xv[kGemmXPerThread];
  GuChunk nxt;
  gemm_load_rows(x, gr, 0, H, xv);
  gu_load_chunk(tb, nb, 0, n, g, nxt);
  for (int kc = 0; kc < nkc; ++kc) {
    const int buf = kc & 1;
    gemm_store_rows(xb[buf], xv);
    const GuChunk cur = nxt;
    if (kc + 1 < nkc) {
      gemm_load_rows(x, gr, kc + 1, H, xv);
      gu_load_chunk(tb, nb, kc + 1, n, g, nxt);
    }
    __syncthreads();
    // this lane's block of the chunk: g (scale 0 past K)
    float sq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) sq[q] = scale_or_zero(cur.scale[q], g, kc * kGemmKC + g < nb);
#pragma unroll
    for (int j = 0; j < kGemmKC; ++j) {
      bf16x8_t av[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        av[t] = *reinterpret_cast<const bf16x8_t*>(&xb[buf][t * 16 + n][g * 32 + j * 8]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t cw = j == 0 ? cur.code[q].x : j == 1 ? cur.code[q].y : j == 2 ? cur.code[q].z : cur.code[q].w;
        const bf16x8_t bw = fp4x8_to_bf16(cw, sq[q]);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (t < ntt) acc[t][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[t], bw, acc[t][q], 0, 0, 0);
      }
    }
  }
  // lane (n, g), register i of row tile q: route t*16 + 4g + i, row 16q + n of the image tile;
  // the 16 lanes of DPP row g hold that route's whole block of h (elements n and 16 + n)
  if (tile_ok) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t * 16 + g * 4 + i;
        if (tok < nt) {  // the same for the whole row
          const float h0 = swiglu_bf16(acc[t][0][i], acc[t][2][i]);
          const float h1 = swiglu_bf16(acc[t][1][i], acc[t][3][i]);
          const int sh = mx_shift(row_max_i(max(f32_exp(h0), f32_exp(h1))));
          uint32_t hi0, lo0, hi1, lo1;
          mx_pair(h0, sh, &hi0, &lo0);
          mx_pair(h1, sh, &hi1, &lo1);
          uint8_t* hr = hq + (size_t)gr.route[tok] * h_stride;
          hr[tile * 32 + n] = (uint8_t)hi0;
          hr[tile * 32 + 16 + n] = (uint8_t)hi1;
          hr[h_pad + tile * 32 + n] = (uint8_t)lo0;
          hr[h_pad + tile * 32 + 16 + n] = (uint8_t)lo1;
          if (n == 0) hr[2 * h_pad + tile] = (uint8_t)(sh + 127);
        }
      }
  }
  (void)I;
}

// ---- router GEMM for many tokens ---------------------------------------------------------------
// grid = (ceil(M/64), ceil(E/64)), 256 threads: logits for 64 tokens x 64 experts, wave w owns
// experts 16w .. +16 of the block.  A = the tokens' activations (staged in LDS, as above), B =
// router rows read straight from memory (a lane's 8 K elements are 16 contiguous bytes).  Same
// fp32 accumulation of bf16 products as k_router, in another order.
__global__ __launch_bounds__(256) void k_router_grouped(const uint16_t* __restrict__ x, int M,
                                                        const uint16_t* __restrict__ wr,
                                                        const float* __restrict__ bias, int E,
                                                        int H, float* __restrict__ logits) {
  __shared__ __align__(16) uint16_t xb[2][kGemmTok][kGemmPitch];
  __shared__ GemmRows gr;
  const int tok0 = blockIdx.x * kGemmTok;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int e = blockIdx.y * 64 + 16 * w + n;
  const uint16_t* brow = wr + (size_t)min(e, E - 1) * H + g * 8;
  for (int i = threadIdx.x; i < kGemmTok; i += blockDim.x) gr.tok[i] = min(tok0 + i, M - 1);
  __syncthreads();
  const int ntt = (min(kGemmTok, M - tok0) + 15) >> 4;
  // this workgroup's share of K: chunks [kc0, kc1) of kGemmKC blocks
  const int nkc_all = (H / 32 + kGemmKC - 1) / kGemmKC;
  const int kc0 = blockIdx.z * nkc_all / gridDim.z, kc1 = (blockIdx.z + 1) * nkc_all / gridDim.z;
  const int nkc = kc1 - kc0;
  logits += (size_t)blockIdx.z * M * E;
  f32x4_t acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  u32x4_t xv[kGemmXPerThread];
  uint4 bn[kGemmKC];
  auto load_b = [&](int kc) {
#pragma unroll
    for (int j = 0; j < kGemmKC; ++j)
      bn[j] = *reinterpret_cast<const uint4*>(brow + min((kc * kGemmKC + j) * 32, H - 32));
  };
  gemm_load_rows(x, gr, kc0, H, xv);
  load_b(kc0);
  for (int kc = kc0; kc < kc1; ++kc) {
    const int buf = (kc - kc0) & 1;
    gemm_store_rows(xb[buf], xv);
    uint4 bc[kGemmKC];
#pragma unroll
    for (int j = 0; j < kGemmKC; ++j) bc[j] = bn[j];
    if (kc + 1 < kc1) {
      gemm_load_rows(x, gr, kc + 1, H, xv);
      load_b(kc + 1);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kGemmKC; ++j) {
      bf16x8_t bw = __builtin_bit_cast(bf16x8_t, bc[j]);
      if ((kc * kGemmKC + j) * 32 >= H) bw = bf16x8_t{};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t < ntt) {
          const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(&xb[buf][t * 16 + n][j * 32 + g * 8]);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bw, acc[t], 0, 0, 0);
        }
      }
    }
  }
  (void)nkc;
  if (e < E) {
    const float b = bias != nullptr && blockIdx.z == 0 ? bias[e] : 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = tok0 + t * 16 + g * 4 + i;
        if (m < M) logits[(size_t)m * E + e] = acc[t][i] + b;
      }
  }
}

// y[m][h] = sum over j ascending of the hot routes m*k+j of w * pdn[m*k+j][h] (cold routes add
// nothing).  One thread per (token, 4 rows).  KB routes at a time, every load of a batch
// requested before the first is used (the rows of a cold route are read and left unused), then
// the sum in ascending j (KB = 4: registers, occupancy).
template <int KB>
__global__ __launch_bounds__(256) void k_combine(int M, int k, int H, RouteArgs ra, RouteWs rw,
                                                 const float* __restrict__ pdn,
                                                 float* __restrict__ y, Residual res) {
  const int q = blockIdx.x * blockDim.x + threadIdx.x;
  const int per = H / 4;
  if (q >= M * per) return;
  const int m = q / per;
  const int h = (q - m * per) * 4;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int j0 = 0; j0 < k; j0 += KB) {
    bool hot[KB];
    float wt[KB];
    float4 v[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int r = m * k + min(j0 + u, k - 1);
      hot[u] = j0 + u < k && rw.route_slot[r] >= 0;
      wt[u] = ra.w_in[r];
      v[u] = *reinterpret_cast<const float4*>(pdn + (size_t)r * H + h);
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (hot[u]) {
        acc.x = fmaf(wt[u], v[u].x, acc.x);
        acc.y = fmaf(wt[u], v[u].y, acc.y);
        acc.z = fmaf(wt[u], v[u].z, acc.z);
        acc.w = fmaf(wt[u], v[u].w, acc.w);
      }
    }
  }
  float* yo = y + (size_t)m * H + h;  // the caller's y need not be 16-byte aligned
  yo[0] = acc.x;
  yo[1] = acc.y;
  yo[2] = acc.z;
  yo[3] = acc.w;
  const size_t i = (size_t)m * H + h;
  residual_store(res, i, acc.x);
  residual_store(res, i + 1, acc.y);
  residual_store(res, i + 2, acc.z);
  residual_store(res, i + 3, acc.w);
}

// =============================================================================================
// The route table of a call in one workgroup: top-k from the logits (or the given ids), slot
// resolve and buckets in LDS, then the table, the top-k results and the cold report written
// out, as the writer workgroup of a gate/up launch with the prologue does.  It does the
// bucketing kernel's work for calls of at most kProMaxRoutes routes in fewer dependent steps.
// =============================================================================================
static_assert(kProMaxRoutes == kRouteTableMaxRoutes, "route table bound");
__global__ __launch_bounds__(512) void k_route_table(RouteArgs ra, RouteWs rw) {
  __shared__ RouteLds rt;
  route_prologue(rt, ra, rw, true);
}

hipError_t launch_route_table(const RouteArgs& ra, const RouteWs& rw, hipStream_t s) {
  if (ra.M < 1 || ra.M * ra.k > kProMaxRoutes) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_route_table, dim3(1), dim3(512), 0, s, ra, rw);
  return hipGetLastError();
}

// =============================================================================================
// The workspace's error word, taken by the caller: copied out, then cleared (in stream order)
// =============================================================================================
__global__ __launch_bounds__(64) void k_take_errors(int32_t* __restrict__ word,
                                                    int32_t* __restrict__ out) {
  if (threadIdx.x == 0) {
    const int32_t v = __hip_atomic_exchange(word, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (out != nullptr) *out = v;
  }
}

// y += add (the cold routes' sum onto the hot output of the hybrid layer), 4 elements a thread.
__global__ __launch_bounds__(256) void k_add_f32(float* __restrict__ y, const float* __restrict__ add,
                                                 size_t n) {
  const size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  for (size_t j = i; j < i + 4 && j < n; ++j) y[j] += add[j];
}

hipError_t launch_add_f32(float* y, const float* add, size_t n, hipStream_t s) {
  const size_t threads = (n + 3) / 4;
  hipLaunchKernelGGL(k_add_f32, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, y, add, n);
  return hipGetLastError();
}

// Read-streaming probe: `bytes` of src read once in non-temporal 16-byte loads (as the weight
// streams are read) by a grid of one workgroup of
// 16 waves per compute unit (the fused decode kernel's launch shape), every load of a thread
// issued before any is used; the values are folded into one word that is stored only if it
// equals an impossible pattern (so that the loads cannot be dropped).
__global__ __launch_bounds__(1024) void k_stream_probe(const uint4* __restrict__ src, size_t n16,
                                                       uint32_t* __restrict__ sink) {
  constexpr int U = 8;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (size_t c0 = t; c0 < n16; c0 += stride * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld_nt(src + min(c0 + (size_t)u * stride, n16 - 1));
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u && t == stride) sink[0] = acc;  // (t never equals stride)
}

hipError_t launch_take_errors(int32_t* word, int32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(k_take_errors, dim3(1), dim3(64), 0, s, word, out);
  return hipGetLastError();
}

// =============================================================================================
// Static scratch: the workspace of moe_layer_forward_noalloc, for callers that cannot allocate
// =============================================================================================
// One array per GPU, held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address is taken once per device with
// hipGetSymbolAddress (with that device current) and only that address is ever used.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

void* static_scratch(hipError_t* err) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    // the header (error word, the fused kernel's call counter) must start at zero: cleared once
    // here, synchronously (not in a stream a caller might be capturing)
    if (e == hipSuccess) e = hipMemset(p, 0, kScratchBytes);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
      *err = e;
      return nullptr;
    }
    addr[dev] = p;
  }
  *err = hipSuccess;
  return addr[dev];
}

// =============================================================================================
// Residual chaining between stacked layers: out = bf16(x + y), one thread per 2 elements
// =============================================================================================
__global__ __launch_bounds__(256) void k_residual(const uint16_t* __restrict__ x,
                                                  const float* __restrict__ y,
                                                  uint16_t* __restrict__ out, size_t n) {
  const size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 2;
  if (i >= n) return;
  for (size_t j = i; j < i + 2 && j < n; ++j) {
    const float xv = __uint_as_float((uint32_t)x[j] << 16);
    out[j] = (uint16_t)f32_to_bf16_bits(xv + y[j]);
  }
}

// =============================================================================================
// Launchers (called from the host API after every argument has been validated)
// =============================================================================================
hipError_t launch_router(const uint16_t* x, int M, const uint16_t* wr, const float* bias, int E,
                         int H, float* logits, hipStream_t s) {
  if (M >= kGroupedMinTokens)  // a dense GEMM: MFMA
    hipLaunchKernelGGL(k_router_grouped, dim3((M + kGemmTok - 1) / kGemmTok, (E + 63) / 64, router_parts(M, E)), dim3(256),
                       0, s, x, M, wr, bias, E, H, logits);
  else {
    const int cpl = (H / 8 + 63) / 64;
    switch (cpl) {
#define MOE_RT(C)                                                                                  \
  case C:                                                                                          \
    hipLaunchKernelGGL((k_router<C>), dim3(E), dim3(64), 0, s, x, M, wr, bias, E, H, logits);     \
    break;
      MOE_RT(1) MOE_RT(2) MOE_RT(3) MOE_RT(4) MOE_RT(5) MOE_RT(6) MOE_RT(7) MOE_RT(8)
      MOE_RT(9) MOE_RT(10) MOE_RT(11) MOE_RT(12) MOE_RT(13) MOE_RT(14) MOE_RT(15) MOE_RT(16)
#undef MOE_RT
      default: return hipErrorInvalidValue;
    }
  }
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
  // The top-k alone runs one wave per token on two-wave workgroups, spread over the compute
  // units: sixteen waves of one workgroup would share a CU's four SIMDs, and this stage is a
  // chain of dependent wave reductions.
  const bool topk_only = logits != nullptr && !do_bucket;
  const int threads = topk_only ? kTopkThreads : kBucketThreads;
  const int grid = topk_only ? (M + threads / 64 - 1) / (threads / 64) : 1;
  hipLaunchKernelGGL(k_topk_bucket, dim3(grid > 0 ? grid : 1), dim3(threads), 0, s, logits,
                     M, k, topk_ids, topk_w, do_bucket ? 1 : 0, ids, Mk, E, S, e2s, o.route_slot,
                     o.ws_perm, o.meta, o.dist, nd_max, o.items, o.items ? n_items_max(Mk, E) : 0,
                     o.cold_list, o.u_counts, o.u_offsets, o.u_perm, o.u_cold_count,
                     o.u_cold_routes);
  return hipGetLastError();
}


constexpr int kNumCUs = 256;      // MI355X compute units (when the device cannot be queried)
constexpr int kWavesPerCU = 16;   // resident waves per CU for a kernel of <= 128 VGPRs

static int device_cus();

ExpertPlan plan_experts(const ImageLayout& L, int M, int E, int k) {
  ExpertPlan p;
  const int Mk = M * k;
  p.nd_max = Mk < E ? Mk : E;
  // M >= kGroupedMinTokens: the grouped GEMM (it needs H a multiple of 64 for its row tiles,
  // which every supported shape is) with the route table from the bucketing kernel
  // (also when the GEMV down kernel could not hold the partial rows of every route in LDS)
  const int dn_kparts = L.dn_ks > 8 ? 2 : 1;
  p.grouped = M >= kGroupedMinTokens || (size_t)Mk * dn_kparts * kDnRows * 4 > kDownLdsBytes;
  p.n_items_max = n_items_max(Mk, E);
  // every gate/up workgroup rebuilding the route table pays a top-k per token: worth it for one
  // token, or for a few routes over few experts; otherwise the top-k / bucketing kernel does it
  // once
  p.prologue = !p.grouped && Mk <= kProMaxRoutes && (M == 1 || (E <= 64 && Mk <= 64));
  // gate/up waves per workgroup: each wave holds at most kMaxGroups groups of its tile's K;
  // the kernels are built for <= 128 VGPRs, so a CU holds kWavesPerCU waves.  Pick the widest
  // workgroup that still lets every workgroup of the grid be resident at once.
  const int units = L.gu_tiles * p.nd_max;
  const int cus_q = device_cus();
  const int cus = cus_q > 0 ? cus_q : kNumCUs;
  const int lo = (L.ng_h + kMaxGroups - 1) / kMaxGroups;
  const int hi = L.ng_h < kMaxWaves ? L.ng_h : kMaxWaves;
  int best = lo < hi ? lo : hi, best_rounds = 1 << 30;
  for (int w = (lo < hi ? lo : hi); w <= hi; ++w) {
    const int per_cu = kWavesPerCU / w > 0 ? kWavesPerCU / w : 1;
    const int rounds = (units + cus * per_cu - 1) / (cus * per_cu);
    if (rounds < best_rounds || (rounds == best_rounds && w > best)) {
      best = w;
      best_rounds = rounds;
    }
  }
  p.gu_waves = best < 1 ? 1 : best;
  p.gu_groups = (L.ng_h + p.gu_waves - 1) / p.gu_waves;
  // Without the prologue (the table comes from the workspace) the gate/up workgroups loop over
  // the hot experts, gu_dgrid at a time: as many as the compute units hold at once, so that the
  // workgroups of experts that are not hot (nd_max bounds the distinct experts, the call usually
  // has fewer) do not take a second round of the grid.
  // The looping kernel holds at most 2 K groups a wave: as many waves as that takes.
  p.gu_dgrid = p.nd_max;
  if (!p.prologue && !p.grouped && (L.ng_h + 1) / 2 <= kMaxWaves) {
    p.gu_waves = (L.ng_h + 1) / 2 > p.gu_waves ? (L.ng_h + 1) / 2 : p.gu_waves;
    p.gu_groups = (L.ng_h + p.gu_waves - 1) / p.gu_waves;
    const int per_cu = kWavesPerCU / p.gu_waves > 0 ? kWavesPerCU / p.gu_waves : 1;
    const int fit = cus * per_cu / (L.gu_tiles > 0 ? L.gu_tiles : 1);
    p.gu_dgrid = fit < 1 ? 1 : (fit < p.nd_max ? fit : p.nd_max);
  }
  return p;
}

hipError_t launch_gateup(const uint16_t* x, int M, int H, int I, const uint8_t* slots,
                         const ImageLayout& L, const ExpertPlan& p, const RouteArgs& ra,
                         const RouteWs& rw, uint16_t* hbuf, hipStream_t s) {
  // (the looping variants, G = 2 without the prologue, take gu_dgrid experts at a time)
  const dim3 g(L.gu_tiles, !p.prologue && p.gu_groups <= 2 ? p.gu_dgrid : p.nd_max),
      b(p.gu_waves * 64);
  // the single-token variant lets arithmetic overlap the loads but holds more registers, so
  // it is only used with at most 3 groups per wave; M == 1 always fits the LDS copy of x
  const bool single = M == 1 && p.gu_groups <= 3;
  const size_t red = (size_t)p.gu_waves * (single ? 1 : kTokPerPass) * 64 * 4;
  const size_t fixed = red + (p.prologue ? kRouteLdsBytes : 0);
  const size_t xb = (size_t)M * H * 2;
  const bool xlds = fixed + xb <= kGuLdsBytes;
  const size_t lds = fixed + (xlds ? xb : 0);
#define MOE_GU(SINGLE, G, PRO, XLDS)                                                               \
  hipLaunchKernelGGL((k_gateup<SINGLE, G, PRO, XLDS>), g, b, lds, s, x, H, I, slots,              \
                     L.image_bytes, L.gu_tile_bytes, L.nb_h, L.ng_h, ra, rw, hbuf)
  if (single) {
    if (p.prologue) {
      if (p.gu_groups <= 1) MOE_GU(true, 1, true, true);
      else if (p.gu_groups == 2) MOE_GU(true, 2, true, true);
      else MOE_GU(true, 3, true, true);
    } else {
      if (p.gu_groups <= 1) MOE_GU(true, 1, false, true);
      else if (p.gu_groups == 2) MOE_GU(true, 2, false, true);
      else MOE_GU(true, 3, false, true);
    }
  } else if (p.prologue) {
    if (xlds) {
      if (p.gu_groups <= 2) MOE_GU(false, 2, true, true);
      else MOE_GU(false, 4, true, true);
    } else {
      if (p.gu_groups <= 2) MOE_GU(false, 2, true, false);
      else MOE_GU(false, 4, true, false);
    }
  } else {
    if (xlds) {
      if (p.gu_groups <= 2) MOE_GU(false, 2, false, true);
      else MOE_GU(false, 4, false, true);
    } else {
      if (p.gu_groups <= 2) MOE_GU(false, 2, false, false);
      else MOE_GU(false, 4, false, false);
    }
  }
#undef MOE_GU
  return hipGetLastError();
}

// Down for the work items (use_items) or the distinct hot experts, then the ordered combine.
static hipError_t launch_down_mx(int M, int H, int I, const uint8_t* slots, const ImageLayout& L,
                                 int n_items, bool use_items, const RouteArgs& ra,
                                 const RouteWs& rw, const uint8_t* hq, float* pdn, float* y,
                                 Residual res, hipStream_t s) {
  const int per_wg = 4 * kDnRW;
  hipLaunchKernelGGL(k_down_mx, dim3((L.dn_tiles + per_wg - 1) / per_wg, n_items), dim3(256), 0, s,
                     H, slots, L.image_bytes, L.gu_bytes, L.dn_tile_bytes, L.dn_code_bytes,
                     L.dn_tiles, L.dn_ks, L.dn_full, L.dn_rem, L.dn_scale_words, I, L.nb_i, L.h_pad,
                     (int)L.h_stride, ra, rw, use_items ? 1 : 0, hq, pdn);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int threads = M * (H / 4);
  hipLaunchKernelGGL(k_combine<4>, dim3((threads + 255) / 256), dim3(256), 0, s, M, ra.k, H, ra,
                     rw, pdn, y, res);
  return hipGetLastError();
}

// Workgroups per down tile of the GEMV path: 2 (the hot experts split between them, one handing
// its rows to the other) when the tiles fill at most half of the compute units (the grid is
// then resident at once: one workgroup per compute unit), K is one part and there are enough
// hot experts to share, else 1.
constexpr int kDnSplitMinExperts = 16;
int down_split(const ImageLayout& L, int M, int k, int E) {
  const int cus = device_cus();
  const int nd_max = M * k < E ? M * k : E;
  // (one K part and at most kSplitMaxTiles tiles; the row words of a split call live in a
  // region sized for kSplitMaxTokens tokens)
  return down_split_possible(L) && M <= kSplitMaxTokens && nd_max >= kDnSplitMinExperts &&
                 cus > 0 && 2 * L.dn_tiles <= cus
             ? 2
             : 1;
}

hipError_t launch_down(int M, int H, int I, const uint8_t* slots, const ImageLayout& L,
                       const ExpertPlan& p, const RouteArgs& ra, const RouteWs& rw,
                       const uint16_t* hbuf, uint64_t* pw, uint32_t* dncall, float* y, Residual res,
                       hipStream_t s) {
  (void)p;
  const int Mk = M * ra.k;
  // long K in two parts (4 experts per pass, half the steps per wave), short K in one (8
  // experts per pass); a wave holds at most 16 steps
  const int kparts = L.dn_ks > 8 ? 2 : 1;
  const int spw = dn_part_steps(L.dn_ks, kparts);
  const int S = down_split(L, M, ra.k, ra.E);
  const size_t parts = (size_t)Mk * kparts * kDnRows * 4;
  const size_t hcopy = ((size_t)Mk * I / 8 + 63) / 64 * 1024;
  const bool h_lds = hcopy + parts <= kDownLdsBytes;
  const size_t lds = (h_lds ? hcopy : 0) + parts;
  if (lds > kDownLdsBytes || spw > 16 || (S > 1 && (pw == nullptr || dncall == nullptr)))
    return hipErrorInvalidValue;
#define MOE_DG(TM)                                                                                 \
  hipLaunchKernelGGL((k_down_gemv<TM>), dim3(L.dn_tiles, S), dim3(512), lds, s, H, I, slots,        \
                     L.image_bytes, L.gu_bytes, L.dn_tile_bytes, L.dn_code_bytes, L.dn_ks,          \
                     L.dn_full, L.dn_rem, L.dn_scale_words, L.nb_i, kparts, h_lds ? 1 : 0, ra, rw,  \
                     hbuf, y, res, pw, dncall)
  if (spw <= 4) MOE_DG(4);
  else if (spw <= 8) MOE_DG(8);
  else if (spw <= 12) MOE_DG(12);
  else MOE_DG(16);
#undef MOE_DG
  return hipGetLastError();
}

hipError_t launch_gateup_grouped(const uint16_t* x, int H, int I, const uint8_t* slots,
                                 const ImageLayout& L, const ExpertPlan& p, const RouteArgs& ra,
                                 const RouteWs& rw, uint8_t* hq, hipStream_t s) {
  hipLaunchKernelGGL(k_gateup_grouped, dim3((L.gu_tiles + 3) / 4, p.n_items_max), dim3(256), 0, s, x,
                     H, I, slots, L.image_bytes, L.gu_tile_bytes, L.nb_h, L.gu_tiles, L.h_pad,
                     (int)L.h_stride, ra, rw, hq);
  return hipGetLastError();
}

hipError_t launch_down_grouped(int M, int H, int I, const uint8_t* slots, const ImageLayout& L,
                               const ExpertPlan& p, const RouteArgs& ra, const RouteWs& rw,
                               const uint8_t* hq, float* pdn, float* y, Residual res,
                               hipStream_t s) {
  return launch_down_mx(M, H, I, slots, L, p.n_items_max, true, ra, rw, hq, pdn, y, res, s);
}

hipError_t launch_residual(const uint16_t* x, const float* y, uint16_t* out, size_t n,
                           hipStream_t s) {
  const size_t threads = (n + 1) / 2;
  hipLaunchKernelGGL(k_residual, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, x, y, out, n);
  return hipGetLastError();
}

// Launch shape of k_layer_decode for a layer: grid, unit bounds per workgroup and wave, LDS.
struct FusedCfg {
  int G = 0, nug = 0, neg = 0, nud = 0, ned = 0;
  size_t lds = 0;
};

static int fused_key(const FusedCfg& c) { return ((c.nug * 10 + c.neg) * 10 + c.nud) * 10 + c.ned; }

#define MOE_LD_SWITCH(KEY, CALL)                                                                   \
  switch (KEY) {                                                                                   \
    case 1111: CALL(1, 1, 1, 1); break;                                                            \
    case 2212: CALL(2, 2, 1, 2); break;                                                            \
    case 2222: CALL(2, 2, 2, 2); break;                                                            \
    case 3323: CALL(3, 3, 2, 3); break;                                                            \
    default: break;                                                                                \
  }

// Compute units of the current device (0 without one: the fused path is then never chosen) and
// whether k_layer_decode<key> fits one workgroup per compute unit; cached per device.
static int device_cus() {
  static std::atomic<int> cache[16];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    v = cus > 0 ? cus : -1;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v > 0 ? v : 0;
}

// The answer depends on the dynamic LDS of the launch (it varies with H, I and k), so the cache
// holds the LDS size it was asked for with it: {lds, 1 fits / -1 does not} per device.
template <int NUG, int NEG, int NUD, int NED, bool ROUTER>
static bool fused_resident(size_t lds) {
  static std::atomic<int64_t> cache[16];  // [device]: lds << 2 | (1 fits, 2 does not); 0 unknown
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return false;
  const int64_t v = cache[dev].load(std::memory_order_relaxed);
  if (v != 0 && (size_t)(v >> 2) == lds) return (v & 3) == 1;
  int per_cu = 0;
  const bool fits = hipOccupancyMaxActiveBlocksPerMultiprocessor(
                        &per_cu, k_layer_decode<NUG, NEG, NUD, NED, ROUTER>, kFusedThreads, lds) == hipSuccess &&
                    per_cu >= 1;
  cache[dev].store(((int64_t)lds << 2) | (fits ? 1 : 2), std::memory_order_relaxed);
  return fits;
}

static uint32_t div_magic(uint32_t d) { return d <= 1 ? 0u : (uint32_t)(0xFFFFFFFFull / d + 1); }
// div_m is exact for numerators up to n_max with divisor d
static bool div_exact(uint64_t n_max, uint64_t d) { return d >= 1 && n_max * (d - 1) < (1ull << 32); }

static int router_cpl(const ImageLayout& L) { return (L.H / 8 + 63) / 64; }

bool layer_decode_router_inside(const ImageLayout& L, int E) {
  return E <= kFusedRouterMaxE && router_cpl(L) <= kFusedRouterMaxCPL;
}

static bool fused_config(const ImageLayout& L, const ExpertPlan& p, int k, bool router, FusedCfg& c) {
  if (k < 1 || k > kFusedMaxK || p.grouped || !p.prologue) return false;
  const int cus = device_cus();
  const int ug_max = k * (L.I / 16), ud = L.H / 8;
  c.G = std::min(cus, std::max(ug_max, ud));
  if (c.G < 1) return false;
  c.nug = (ug_max + c.G - 1) / c.G;
  c.nud = (ud + c.G - 1) / c.G;
  c.neg = ((L.nb_h + 1) / 2 + kFusedWaves - 1) / kFusedWaves;
  c.ned = (k * ((L.dn_ks + 1) / 2) + kFusedWaves - 1) / kFusedWaves;
  c.lds = fused_lds_bytes(L.H, L.I, k, c.nug, c.nud);
  // a wave's down entries (consecutive (expert, step pair)s) cover at most two hot experts
  if (c.ned > (L.dn_ks + 1) / 2) return false;
  if (c.lds + sizeof(RouteLds) > 64 * 1024) return false;
  if (L.H / 8 > kFusedThreads) return false;  // x: one chunk per thread
  // the divisions by multiply: unit shares (w * U over the grid), units per expert, step pairs
  const uint64_t ugpe = (uint64_t)(L.I / 16), np2 = (uint64_t)((L.dn_ks + 1) / 2);
  if (!div_exact((uint64_t)c.G * (uint64_t)std::max(ug_max, ud), (uint64_t)c.G) ||
      !div_exact((uint64_t)k * ugpe + kFusedWaves, ugpe) ||
      !div_exact((uint64_t)k * np2 + kFusedWaves, np2))
    return false;
  // the smallest instantiation that holds the bounds
  const int keys[][4] = {{1, 1, 1, 1}, {2, 2, 1, 2}, {2, 2, 2, 2}, {3, 3, 2, 3}};
  for (const auto& kk : keys)
    if (c.nug <= kk[0] && c.neg <= kk[1] && c.nud <= kk[2] && c.ned <= kk[3]) {
      c.nug = kk[0];
      c.neg = kk[1];
      c.nud = kk[2];
      c.ned = kk[3];
      c.lds = fused_lds_bytes(L.H, L.I, k, c.nug, c.nud);
      bool fits = false;
#define MOE_LD_FIT(A, B, C, D)                                              \
  fits = router ? fused_resident<A, B, C, D, true>(c.lds)                  \
                : fused_resident<A, B, C, D, false>(c.lds)
      MOE_LD_SWITCH(fused_key(c), MOE_LD_FIT)
#undef MOE_LD_FIT
      return fits;
    }
  return false;
}

bool layer_decode_fusable(const ImageLayout& L, const ExpertPlan& p, int M, int k, int E) {
  FusedCfg c;
  return M == 1 && fused_config(L, p, k, layer_decode_router_inside(L, E), c);
}

hipError_t launch_layer_decode(const uint16_t* x, const uint16_t* wr, const float* bias, int M,
                               int H, int I, const uint8_t* slots, const ImageLayout& L,
                               const ExpertPlan& p, const RouteArgs& ra, const RouteWs& rw,
                               uint64_t* hf, float* y, Residual res, hipStream_t s) {
  FusedCfg c;
  const bool router = layer_decode_router_inside(L, ra.E);
  if (M != 1 || !fused_config(L, p, ra.k, router, c)) return hipErrorInvalidValue;
  if (!router && ra.logits == nullptr) return hipErrorInvalidValue;
  const FusedDivs dv = {div_magic((uint32_t)c.G), div_magic((uint32_t)(I / 16)),
                        div_magic((uint32_t)((L.dn_ks + 1) / 2))};
  hipError_t e = hipErrorInvalidValue;
#define MOE_LD_R(A, B, C, D, R)                                                                    \
  hipLaunchKernelGGL((k_layer_decode<A, B, C, D, R>), dim3(c.G), dim3(kFusedThreads), c.lds, s, x, \
                     wr, bias, router_cpl(L), H, I, slots, L.image_bytes, L.gu_tile_bytes, L.nb_h, \
                     L.gu_bytes, L.dn_tile_bytes, L.dn_code_bytes, L.dn_ks, L.dn_full, L.dn_rem,   \
                     L.nb_i, ra, rw, hf, y, res, dv)
#define MOE_LD(A, B, C, D)                                                                         \
  do {                                                                                             \
    if (router)                                                                                    \
      MOE_LD_R(A, B, C, D, true);                                                                  \
    else                                                                                           \
      MOE_LD_R(A, B, C, D, false);                                                                 \
    e = hipGetLastError();                                                                         \
  } while (0)
  MOE_LD_SWITCH(fused_key(c), MOE_LD)
#undef MOE_LD
#undef MOE_LD_R
  return e;
}
#undef MOE_LD_SWITCH

hipError_t launch_stream_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t s) {
  const int cus = device_cus();
  hipLaunchKernelGGL(k_stream_probe, dim3(cus > 0 ? cus : kNumCUs), dim3(1024), 0, s,
                     reinterpret_cast<const uint4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace moe
