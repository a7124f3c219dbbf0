// HIP kernels of libmoe for gfx950 (CDNA4, wave64).
//
//   k_router    multi-workgroup bf16 router GEMV/GEMM + bias; the last workgroup to finish
//               (device-scope arrival counter) does softmax/top-k/renormalise per token.
//   k_bucket    one workgroup: route -> slot resolve, cold report, per-expert counts, prefix
//               scans (DPP), bucket permutation, list of distinct hot experts.
//   k_gateup    fused MXFP4 gate/up GEMV + SiLU(g)*u -> h (bf16) per route.  One workgroup
//               per (distinct hot expert, 32-row tile), its waves split K.
//   k_down      MXFP4 down GEMV per route into fp32 partials, then the last workgroup of each
//               64-row tile (arrival counter) adds the routes of every token in ascending j.
//   k_fill_u32  fill kernel for the workspace counters.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// =============================================================================================
// Router
// =============================================================================================
// grid.x = ceil(E / kRouterWaves); block = kRouterWaves * 64.  Wave w owns expert row
// e = blockIdx.x * kRouterWaves + w and keeps that row of W_r in registers (H/8 chunks of
// 8 bf16 spread over the lanes); tokens are staged in LDS `tok_chunk` at a time.
constexpr int kRouterMaxChunksPerLane = kMaxHidden / 8 / 64;  // 16

__global__ __launch_bounds__(kRouterWaves * 64) void k_router(
    const uint16_t* __restrict__ x, int M, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int E, int H, int k, int tok_chunk,
    float* __restrict__ logits, unsigned* __restrict__ ticket, int32_t* __restrict__ topk_ids,
    float* __restrict__ topk_w) {
  extern __shared__ uint4 xs[];  // [tok_chunk][H/8]
  __shared__ int s_last;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int e = blockIdx.x * kRouterWaves + wave;
  const int nch = H / 8;  // 16-byte chunks per row
  const bool has_row = e < E;

  uint4 wrow[kRouterMaxChunksPerLane];
#pragma unroll
  for (int i = 0; i < kRouterMaxChunksPerLane; ++i) {
    const int c = lane + 64 * i;
    wrow[i] = (has_row && c < nch) ? reinterpret_cast<const uint4*>(wr + (size_t)e * H)[c]
                                   : make_uint4(0, 0, 0, 0);
  }
  const float b = (has_row && bias != nullptr) ? bias[e] : 0.0f;

  for (int m0 = 0; m0 < M; m0 += tok_chunk) {
    const int nt = min(tok_chunk, M - m0);
    __syncthreads();
    for (int idx = threadIdx.x; idx < nt * nch; idx += blockDim.x)
      xs[idx] = reinterpret_cast<const uint4*>(x + (size_t)m0 * H)[idx];
    __syncthreads();
    if (has_row) {
      for (int t = 0; t < nt; ++t) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < kRouterMaxChunksPerLane; ++i) {
          const int c = lane + 64 * i;
          if (c < nch) {
            const uint4 xv = xs[t * nch + c];
            acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wrow[i].x), as_bf16x2(xv.x), acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wrow[i].y), as_bf16x2(xv.y), acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wrow[i].z), as_bf16x2(xv.z), acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wrow[i].w), as_bf16x2(xv.w), acc, false);
          }
        }
        acc = wave_sum(acc);
        if (lane == 0) logits[(size_t)(m0 + t) * E + e] = acc + b;
      }
    }
  }

  // Arrival: the last workgroup sees every logit.
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(ticket, 1u) == gridDim.x - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  constexpr int kMaxPerLane = kMaxExperts / 64;  // 16
  for (int m = wave; m < M; m += kRouterWaves) {
    float v[kMaxPerLane];
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int ee = lane + 64 * i;
      v[i] = ee < E ? __builtin_nontemporal_load(logits + (size_t)m * E + ee) : -INFINITY;
    }
    float my_v = -INFINITY;
    int my_i = 0;
    float top = 0.0f;
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
      topk_ids[(size_t)m * k + lane] = my_i;
      topk_w[(size_t)m * k + lane] = ex / den;
    }
  }
  if (threadIdx.x == 0) *ticket = 0u;  // ready for the next call
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

__global__ __launch_bounds__(kBucketThreads) void k_bucket(
    const int32_t* __restrict__ ids, int Mk, int E, int S, const int32_t* __restrict__ e2s,
    int32_t* __restrict__ route_slot, int32_t* __restrict__ ws_perm, int32_t* __restrict__ meta,
    int32_t* __restrict__ dist_expert, int32_t* __restrict__ dist_slot,
    int32_t* __restrict__ dist_off, int32_t* __restrict__ dist_cnt, int nd_max,
    int32_t* __restrict__ cold_list, int32_t* __restrict__ u_counts,
    int32_t* __restrict__ u_offsets, int32_t* __restrict__ u_perm,
    int32_t* __restrict__ u_cold_count, int32_t* __restrict__ u_cold_routes) {
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_off[kMaxExperts];
  __shared__ int s_wave[kBucketThreads / 64 + 1];
  __shared__ int s_err;
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

// =============================================================================================
// Gate/up + SiLU*up
// =============================================================================================
// grid = (gu_tiles, nd_max); block = kWavesPerGroup * 64.  Lane l < 32 accumulates gate row
// 32*tile + l, lane l >= 32 the matching up row; wave w walks groups [g0, g1) of the K blocks.
// The activation block of the current token is uniform across the wave (scalar loads).
template <int NT>
__global__ __launch_bounds__(kWavesPerGroup * 64) void k_gateup(
    const uint16_t* __restrict__ x, int H, int I, int k, const uint8_t* __restrict__ slots,
    size_t image_bytes, size_t gu_tile_bytes, int nb, int ng, const int32_t* __restrict__ meta,
    const int32_t* __restrict__ dist_slot, const int32_t* __restrict__ dist_off,
    const int32_t* __restrict__ dist_cnt, const int32_t* __restrict__ perm, int Mk,
    uint16_t* __restrict__ hbuf) {
  __shared__ float red[kWavesPerGroup][NT][64];
  const int tile = blockIdx.x;
  const int d = blockIdx.y;
  if (d >= meta[0]) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = dist_slot[d];
  const int cnt = dist_cnt[d];
  const int off = dist_off[d];
  if (cnt <= 0 || off < 0 || off + cnt > Mk) return;

  const uint8_t* tbase = slots + (size_t)slot * image_bytes + (size_t)tile * gu_tile_bytes;
  const uint4* codes = reinterpret_cast<const uint4*>(tbase);
  const uint32_t* scl = reinterpret_cast<const uint32_t*>(tbase + (size_t)nb * 1024);
  const int g0 = wave * ng / kWavesPerGroup;
  const int g1 = (wave + 1) * ng / kWavesPerGroup;

  for (int base = 0; base < cnt; base += NT) {
    const int nt = min(NT, cnt - base);
    int tok[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int r = perm[off + base + (t < nt ? t : 0)];
      tok[t] = __builtin_amdgcn_readfirstlane(r / k);
    }
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.0f;

    for (int q = g0; q < g1; ++q) {
      const uint32_t s4 = scl[q * 64 + lane];
      uint4 c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = 4 * q + i;
        c[i] = b < nb ? codes[b * 64 + lane] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = 4 * q + i;
        if (b < nb) {
          const float sc = e8m0_to_f32((s4 >> (8 * i)) & 0xFFu);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            if (t < nt) {
              const uint4* xa = reinterpret_cast<const uint4*>(x + (size_t)tok[t] * H + 32 * b);
              const float p = block_dot(c[i], xa[0], xa[1], xa[2], xa[3]);
              acc[t] = fmaf(sc, p, acc[t]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();
    for (int idx = threadIdx.x; idx < nt * 32; idx += blockDim.x) {
      const int t = idx >> 5;
      const int row = idx & 31;
      float g = 0.0f, u = 0.0f;
#pragma unroll
      for (int w = 0; w < kWavesPerGroup; ++w) {
        g += red[w][t][row];
        u += red[w][t][row + 32];
      }
      const int r = perm[off + base + t];
      hbuf[(size_t)r * I + tile * 32 + row] = (uint16_t)f32_to_bf16_bits(silu_f32(g) * u);
    }
    __syncthreads();
  }
}

// =============================================================================================
// Down + ordered combine
// =============================================================================================
// grid = (dn_tiles, nd_max, KC); block = kWavesPerGroup * 64.  Lane l accumulates down row
// 64*tile + l of expert d over K-chunk kc (further split over the waves).  Partials go to
// pdn[route][kc][row]; the last workgroup to arrive for the tile forms
// y[m][row] = sum_j (hot, ascending j) w[m,j] * sum_kc pdn[(m,j)][kc][row].
template <int NT>
__global__ __launch_bounds__(kWavesPerGroup * 64) void k_down(
    int M, int H, int I, int k, const uint8_t* __restrict__ slots, size_t image_bytes,
    size_t gu_bytes, size_t dn_tile_bytes, int nb, int ng, int KC,
    const int32_t* __restrict__ meta, const int32_t* __restrict__ dist_slot,
    const int32_t* __restrict__ dist_off, const int32_t* __restrict__ dist_cnt,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ route_slot, int Mk,
    const uint16_t* __restrict__ hbuf, const float* __restrict__ topk_w, float* __restrict__ pdn,
    unsigned* __restrict__ tickets, float* __restrict__ y) {
  __shared__ float red[kWavesPerGroup][NT][64];
  __shared__ int s_last;
  const int tile = blockIdx.x;
  const int d = blockIdx.y;
  const int kc = blockIdx.z;
  const int nd = meta[0];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (d >= nd) {
    if (nd == 0 && d == 0 && kc == 0) {  // every route cold: the output is zero
      for (int idx = threadIdx.x; idx < M * 64; idx += blockDim.x)
        y[(size_t)(idx >> 6) * H + tile * 64 + (idx & 63)] = 0.0f;
    }
    return;
  }
  const int slot = dist_slot[d];
  const int cnt = dist_cnt[d];
  const int off = dist_off[d];
  const bool ok = cnt > 0 && off >= 0 && off + cnt <= Mk;

  if (ok) {
    const uint8_t* tbase =
        slots + (size_t)slot * image_bytes + gu_bytes + (size_t)tile * dn_tile_bytes;
    const uint4* codes = reinterpret_cast<const uint4*>(tbase);
    const uint32_t* scl = reinterpret_cast<const uint32_t*>(tbase + (size_t)nb * 1024);
    const int c0 = kc * ng / KC, c1 = (kc + 1) * ng / KC;
    const int g0 = c0 + wave * (c1 - c0) / kWavesPerGroup;
    const int g1 = c0 + (wave + 1) * (c1 - c0) / kWavesPerGroup;

    for (int base = 0; base < cnt; base += NT) {
      const int nt = min(NT, cnt - base);
      int rt[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t)
        rt[t] = __builtin_amdgcn_readfirstlane(perm[off + base + (t < nt ? t : 0)]);
      float acc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = 0.0f;

      for (int q = g0; q < g1; ++q) {
        const uint32_t s4 = scl[q * 64 + lane];
        uint4 c[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int b = 4 * q + i;
          c[i] = b < nb ? codes[b * 64 + lane] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int b = 4 * q + i;
          if (b < nb) {
            const float sc = e8m0_to_f32((s4 >> (8 * i)) & 0xFFu);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              if (t < nt) {
                const uint4* ha = reinterpret_cast<const uint4*>(hbuf + (size_t)rt[t] * I + 32 * b);
                const float p = block_dot(c[i], ha[0], ha[1], ha[2], ha[3]);
                acc[t] = fmaf(sc, p, acc[t]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) red[wave][t][lane] = acc[t];
      __syncthreads();
      for (int idx = threadIdx.x; idx < nt * 64; idx += blockDim.x) {
        const int t = idx >> 6;
        const int row = idx & 63;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < kWavesPerGroup; ++w) s += red[w][t][row];
        const int r = perm[off + base + t];
        pdn[((size_t)r * KC + kc) * H + tile * 64 + row] = s;
      }
      __syncthreads();
    }
  }

  // Arrival: the last of the nd*KC workgroups of this tile forms the ordered combine.
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(&tickets[tile], 1u) == (unsigned)(nd * KC - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int idx = threadIdx.x; idx < M * 64; idx += blockDim.x) {
    const int m = idx >> 6;
    const int row = tile * 64 + (idx & 63);
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int r = m * k + j;
      if (route_slot[r] >= 0) {
        float s = 0.0f;
        for (int c = 0; c < KC; ++c)
          s += __builtin_nontemporal_load(pdn + ((size_t)r * KC + c) * H + row);
        acc = fmaf(topk_w[r], s, acc);
      }
    }
    y[(size_t)m * H + row] = acc;
  }
  if (threadIdx.x == 0) tickets[tile] = 0u;
}

__global__ void k_fill_u32(unsigned* __restrict__ p, int n, unsigned v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// =============================================================================================
// Launchers (called from the host API after every argument has been validated)
// =============================================================================================
hipError_t launch_fill_u32(unsigned* p, int n, unsigned v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u32, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_router(const uint16_t* x, int M, const uint16_t* wr, const float* bias, int E,
                         int H, int k, float* logits, unsigned* ticket, int32_t* ids, float* w,
                         hipStream_t s) {
  const int row_bytes = H * 2;
  int tok_chunk = 49152 / row_bytes;
  tok_chunk = tok_chunk < 1 ? 1 : (tok_chunk > 8 ? 8 : tok_chunk);
  if (tok_chunk > M) tok_chunk = M;
  const size_t lds = (size_t)tok_chunk * row_bytes;
  const int grid = (E + kRouterWaves - 1) / kRouterWaves;
  hipLaunchKernelGGL(k_router, dim3(grid), dim3(kRouterWaves * 64), lds, s, x, M, wr, bias, E, H,
                     k, tok_chunk, logits, ticket, ids, w);
  return hipGetLastError();
}

hipError_t launch_bucket(const int32_t* ids, int Mk, int E, int S, const int32_t* e2s,
                         int32_t* route_slot, int32_t* ws_perm, int32_t* meta, int32_t* dist_expert,
                         int32_t* dist_slot, int32_t* dist_off, int32_t* dist_cnt, int nd_max,
                         int32_t* cold_list, int32_t* u_counts, int32_t* u_offsets,
                         int32_t* u_perm, int32_t* u_cold_count, int32_t* u_cold_routes,
                         hipStream_t s) {
  hipLaunchKernelGGL(k_bucket, dim3(1), dim3(kBucketThreads), 0, s, ids, Mk, E, S, e2s, route_slot,
                     ws_perm, meta, dist_expert, dist_slot, dist_off, dist_cnt, nd_max, cold_list,
                     u_counts, u_offsets, u_perm, u_cold_count, u_cold_routes);
  return hipGetLastError();
}

template <int NT>
static void gateup_nt(dim3 g, hipStream_t s, const uint16_t* x, int H, int I, int k,
                      const uint8_t* slots, const ImageLayout& L, const int32_t* meta,
                      const int32_t* dist_slot, const int32_t* dist_off, const int32_t* dist_cnt,
                      const int32_t* perm, int Mk, uint16_t* hbuf) {
  hipLaunchKernelGGL(k_gateup<NT>, g, dim3(kWavesPerGroup * 64), 0, s, x, H, I, k, slots,
                     L.image_bytes, L.gu_tile_bytes, L.nb_h, L.ng_h, meta, dist_slot, dist_off,
                     dist_cnt, perm, Mk, hbuf);
}

template <int NT>
static void down_nt(dim3 g, hipStream_t s, int M, int H, int I, int k, const uint8_t* slots,
                    const ImageLayout& L, int KC, const int32_t* meta, const int32_t* dist_slot,
                    const int32_t* dist_off, const int32_t* dist_cnt, const int32_t* perm,
                    const int32_t* route_slot, int Mk, const uint16_t* hbuf, const float* topk_w,
                    float* pdn, unsigned* tickets, float* y) {
  hipLaunchKernelGGL(k_down<NT>, g, dim3(kWavesPerGroup * 64), 0, s, M, H, I, k, slots,
                     L.image_bytes, L.gu_bytes, L.dn_tile_bytes, L.nb_i, L.ng_i, KC, meta,
                     dist_slot, dist_off, dist_cnt, perm, route_slot, Mk, hbuf, topk_w, pdn,
                     tickets, y);
}

static int tokens_per_pass(int M) { return M >= 8 ? 8 : (M >= 4 ? 4 : (M >= 2 ? 2 : 1)); }

int down_kchunks(const ImageLayout& L, int nd_max) {
  // K-chunks: enough workgroups to cover the chip at least twice, at least one group of
  // 4 blocks per wave.
  const int units = L.dn_tiles * nd_max;
  int KC = (512 + units - 1) / units;
  const int kc_cap = L.ng_i / kWavesPerGroup > 0 ? L.ng_i / kWavesPerGroup : 1;
  if (KC > kc_cap) KC = kc_cap;
  if (KC > kMaxKC) KC = kMaxKC;
  if (KC < 1) KC = 1;
  return KC;
}

hipError_t launch_gateup(const uint16_t* x, int M, int H, int I, int E, int k,
                         const uint8_t* slots, const ImageLayout& L, const int32_t* meta,
                         const int32_t* dist_slot, const int32_t* dist_off, const int32_t* dist_cnt,
                         const int32_t* perm, uint16_t* hbuf, hipStream_t s) {
  const int Mk = M * k;
  const int nd_max = Mk < E ? Mk : E;
  const dim3 g(L.gu_tiles, nd_max);
  switch (tokens_per_pass(M)) {
    case 1: gateup_nt<1>(g, s, x, H, I, k, slots, L, meta, dist_slot, dist_off, dist_cnt, perm, Mk, hbuf); break;
    case 2: gateup_nt<2>(g, s, x, H, I, k, slots, L, meta, dist_slot, dist_off, dist_cnt, perm, Mk, hbuf); break;
    case 4: gateup_nt<4>(g, s, x, H, I, k, slots, L, meta, dist_slot, dist_off, dist_cnt, perm, Mk, hbuf); break;
    default: gateup_nt<8>(g, s, x, H, I, k, slots, L, meta, dist_slot, dist_off, dist_cnt, perm, Mk, hbuf); break;
  }
  return hipGetLastError();
}

hipError_t launch_down(int M, int H, int I, int E, int k, const uint8_t* slots,
                       const ImageLayout& L, const int32_t* meta, const int32_t* dist_slot,
                       const int32_t* dist_off, const int32_t* dist_cnt, const int32_t* perm,
                       const int32_t* route_slot, const uint16_t* hbuf, const float* topk_w,
                       float* pdn, unsigned* tickets, float* y, hipStream_t s) {
  const int Mk = M * k;
  const int nd_max = Mk < E ? Mk : E;
  const int KC = down_kchunks(L, nd_max);
  const dim3 g(L.dn_tiles, nd_max, KC);
  switch (tokens_per_pass(M)) {
    case 1: down_nt<1>(g, s, M, H, I, k, slots, L, KC, meta, dist_slot, dist_off, dist_cnt, perm, route_slot, Mk, hbuf, topk_w, pdn, tickets, y); break;
    case 2: down_nt<2>(g, s, M, H, I, k, slots, L, KC, meta, dist_slot, dist_off, dist_cnt, perm, route_slot, Mk, hbuf, topk_w, pdn, tickets, y); break;
    case 4: down_nt<4>(g, s, M, H, I, k, slots, L, KC, meta, dist_slot, dist_off, dist_cnt, perm, route_slot, Mk, hbuf, topk_w, pdn, tickets, y); break;
    default: down_nt<8>(g, s, M, H, I, k, slots, L, KC, meta, dist_slot, dist_off, dist_cnt, perm, route_slot, Mk, hbuf, topk_w, pdn, tickets, y); break;
  }
  return hipGetLastError();
}

}  // namespace moe
