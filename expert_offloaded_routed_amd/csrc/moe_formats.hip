// The generic expert path: expert formats other than MXFP4 through the same slot cache and route
// table [MoE expert offload, "Supported": bf16, block FP8, NVFP4 and MXFP4 experts share one
// generic path that keeps every expert tensor, weights and scales, in host RAM].
//
// The image of such an expert is its six tensors row-major (FmtLayout in moe_internal.h), so a
// refill is still one copy of one image.  A lane takes a weight row 16 bytes at a time (bf16: 8
// elements, E4M3: 16, E2M1: 32), turns them exactly into bf16 pairs on the gfx950 converters and
// dots them with the activations in fp32; the chunk's scale factors multiply the chunk's sum:
//   bf16       none;
//   FP8 block  E4M3 elements (OCP, bias 7), one fp32 scale per 128 x 128 block of the matrix
//              (a 16-element chunk never straddles two blocks);
//   NVFP4      E2M1 elements (element 2c in the low nibble of byte c), one E4M3 scale per 16
//              elements of a row times one fp32 scale of the matrix (a chunk spans two scales).
//
// A lane requests U chunks of its row (chunk_unroll) before it uses any of them.
// k_gateup_fmt: one wave per row index i of one hot expert: gate row i and up row i against
// every route of the expert, kFmtTok routes per pass; h = bf16(silu(g) * u) per route.
// k_down_fmt: one wave per output row r over every hot expert and its routes; each route's sum is
// kept in the workspace by the lane that later combines that route's token (lane m % 64 of the
// wave: it reads back only what it wrote itself), then y[m][r] = sum over ascending j of the hot
// routes of w[m][j] * d, plus the residual.  Both read the route table that the route-table or
// the bucketing kernel wrote.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kFmtWaves = 8;  // waves per workgroup (one row each)
constexpr int kFmtTok = 8;    // routes of an expert per pass (accumulators per lane)

// OCP E4M3 code -> fp32, exactly (subnormals m * 2^-9; S.1111.111 is NaN).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 24, e = (c >> 3) & 0xFu, m = c & 7u;
  float v;
  if (e == 0)
    v = (float)m * 0.001953125f;
  else
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  v = __uint_as_float(__float_as_uint(v) | s);
  return (e == 15u && m == 7u) ? __uint_as_float(0x7FC00000u) : v;
}

template <int FMT>
__host__ __device__ constexpr int chunk_elems() {
  return FMT == MOE_FORMAT_BF16 ? 8 : FMT == MOE_FORMAT_FP8_BLOCK ? 16 : 32;
}

// Byte offset of element k of row r of a matrix [.][K].
template <int FMT>
__device__ __forceinline__ size_t elem_off(int r, int k, int K) {
  const size_t i = (size_t)r * K + k;
  return FMT == MOE_FORMAT_BF16 ? 2 * i : FMT == MOE_FORMAT_FP8_BLOCK ? i : i / 2;
}

// The matrix scale of an NVFP4 scale section (1 for the other formats).
template <int FMT>
__device__ __forceinline__ float matrix_scale(const uint8_t* __restrict__ sc) {
  if constexpr (FMT == MOE_FORMAT_NVFP4) return *reinterpret_cast<const float*>(sc);
  return 1.0f;
}

// Scales of the chunk at element k of row r of a matrix [.][K] whose scale section is sc:
// s0 for its (first) 16 elements, s1 for the next 16 (NVFP4 only: the two E4M3 bytes, one
// 16-bit load, each times the matrix scale g).
template <int FMT>
__device__ __forceinline__ void chunk_scales(const uint8_t* __restrict__ sc, int r, int k, int K,
                                             float g, float& s0, float& s1) {
  if constexpr (FMT == MOE_FORMAT_FP8_BLOCK) {
    s0 = reinterpret_cast<const float*>(sc)[(size_t)(r / 128) * ((K + 127) / 128) + k / 128];
    s1 = 0.0f;
  } else if constexpr (FMT == MOE_FORMAT_NVFP4) {
    // 4 + r * (K / 16) + k / 16 is even: K / 16 and k / 16 are
    const uint32_t b = *reinterpret_cast<const uint16_t*>(sc + 4 + (size_t)r * (K / 16) + k / 16);
    s0 = e4m3_to_f32(b & 0xFFu) * g;
    s1 = e4m3_to_f32(b >> 8) * g;
  } else {
    s0 = s1 = 1.0f;
  }
}

// Chunks a lane has in flight per matrix (requested together before any is used).
template <int FMT>
__host__ __device__ constexpr int chunk_unroll() {
  return FMT == MOE_FORMAT_NVFP4 ? 2 : 4;
}

// acc + the dot of the 8 E2M1 values of word w (byte p: elements 2p, 2p + 1) with 4 bf16 pairs.
__device__ __forceinline__ float fp4_word_dot(uint32_t w, const uint32_t* a, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0),
                                        as_bf16x2(a[0]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1),
                                        as_bf16x2(a[1]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2),
                                        as_bf16x2(a[2]), acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3),
                                         as_bf16x2(a[3]), acc, false);
}

// Sum of the products of one 16-byte weight chunk c with the activations at a (bf16, 16-byte
// aligned), the chunk's scales applied.
template <int FMT>
__device__ __forceinline__ float chunk_dot(const uint4 c, const uint16_t* __restrict__ a, float s0,
                                           float s1) {
  const uint4* a4 = reinterpret_cast<const uint4*>(a);
  if constexpr (FMT == MOE_FORMAT_BF16) {
    return dot8_bf16(c, a4[0], 0.0f);
  } else if constexpr (FMT == MOE_FORMAT_FP8_BLOCK) {
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    const uint4 a0 = a4[0], a1 = a4[1];
    const uint32_t aw[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // word j: elements 4j .. 4j+3, two bf16 pairs
      acc = __builtin_amdgcn_fdot2_f32_bf16(
          __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[j], 1.0f, false), as_bf16x2(aw[2 * j]), acc,
          false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(
          __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[j], 1.0f, true), as_bf16x2(aw[2 * j + 1]),
          acc, false);
    }
    return acc * s0;
  } else {
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    const uint4 a0 = a4[0], a1 = a4[1], a2 = a4[2], a3 = a4[3];
    const uint32_t aw[16] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w,
                             a2.x, a2.y, a2.z, a2.w, a3.x, a3.y, a3.z, a3.w};
    // elements 0..15 (words 0-1) and 16..31 (words 2-3)
    float b0 = fp4_word_dot(cw[0], aw, 0.0f);
    b0 = fp4_word_dot(cw[1], aw + 4, b0);
    float b1 = fp4_word_dot(cw[2], aw + 8, 0.0f);
    b1 = fp4_word_dot(cw[3], aw + 12, b1);
    return b0 * s0 + b1 * s1;
  }
}

__device__ __forceinline__ float bf16_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

}  // namespace

// grid = (I / kFmtWaves, nd_max): wave w of workgroup x takes row i = x * kFmtWaves + w of the
// gate and up matrices of hot expert blockIdx.y (I % 32 == 0, so every wave has a row).
template <int FMT>
__global__ __launch_bounds__(kFmtWaves * 64) void k_gateup_fmt(
    const uint16_t* __restrict__ x, int H, int I, const uint8_t* __restrict__ slots,
    size_t image_bytes, FmtLayout F, RouteArgs ra, RouteWs rw, uint16_t* __restrict__ hbuf) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * kFmtWaves + (threadIdx.x >> 6);
  const int d = blockIdx.y;
  if (d >= rw.meta[0] || i >= I) return;
  const int4 dd = rw.dist[d];
  const int slot = dd.x, off = dd.y, cnt = dd.z;
  const int Mk = ra.M * ra.k;
  if (cnt <= 0 || off < 0 || off + cnt > Mk || slot < 0 || slot >= ra.S) return;
  const uint8_t* img = slots + (size_t)slot * image_bytes;
  constexpr int EPC = chunk_elems<FMT>();
  constexpr int U = chunk_unroll<FMT>();
  const int nch = H / EPC;
  const float gs = matrix_scale<FMT>(img + F.gate_s), us = matrix_scale<FMT>(img + F.up_s);
  for (int base = 0; base < cnt; base += kFmtTok) {
    const int nt = min(kFmtTok, cnt - base);
    int route[kFmtTok];
    size_t xo[kFmtTok];
#pragma unroll
    for (int t = 0; t < kFmtTok; ++t) {
      route[t] = t < nt ? rw.perm[off + base + t] : 0;
      xo[t] = (size_t)(route[t] / ra.k) * H;
    }
    float ag[kFmtTok], au[kFmtTok];
#pragma unroll
    for (int t = 0; t < kFmtTok; ++t) ag[t] = au[t] = 0.0f;
    for (int c0 = lane; c0 < nch; c0 += 64 * U) {
      uint4 cg[U], cu[U];
      float g0[U], g1[U], u0[U], u1[U];
      int kk[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {  // (past the row: the last chunk again, unused)
        kk[u] = min(c0 + 64 * u, nch - 1) * EPC;
        cg[u] = ld_nt(reinterpret_cast<const uint4*>(img + F.gate + elem_off<FMT>(i, kk[u], H)));
        cu[u] = ld_nt(reinterpret_cast<const uint4*>(img + F.up + elem_off<FMT>(i, kk[u], H)));
        chunk_scales<FMT>(img + F.gate_s, i, kk[u], H, gs, g0[u], g1[u]);
        chunk_scales<FMT>(img + F.up_s, i, kk[u], H, us, u0[u], u1[u]);
      }
#pragma unroll
      for (int t = 0; t < kFmtTok; ++t) {
        if (t < nt) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            if (c0 + 64 * u < nch) {
              ag[t] += chunk_dot<FMT>(cg[u], x + xo[t] + kk[u], g0[u], g1[u]);
              au[t] += chunk_dot<FMT>(cu[u], x + xo[t] + kk[u], u0[u], u1[u]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kFmtTok; ++t) {
      if (t < nt) {
        const float g = wave_sum(ag[t]), u = wave_sum(au[t]);
        if (lane == 0) hbuf[(size_t)route[t] * I + i] = (uint16_t)f32_to_bf16_bits(silu_f32(g) * u);
      }
    }
  }
}

// grid = H / kFmtWaves: wave w of workgroup x takes output row r = x * kFmtWaves + w
// (H % 64 == 0, so every wave has a row).  pdn [M*k][H]: the route sums of the call.
template <int FMT>
__global__ __launch_bounds__(kFmtWaves * 64) void k_down_fmt(
    int H, int I, const uint8_t* __restrict__ slots, size_t image_bytes, FmtLayout F, RouteArgs ra,
    RouteWs rw, const uint16_t* __restrict__ hbuf, float* __restrict__ pdn, float* __restrict__ y,
    Residual res) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * kFmtWaves + (threadIdx.x >> 6);
  if (r >= H) return;
  const int Mk = ra.M * ra.k;
  const int nd = rw.meta[0];
  constexpr int EPC = chunk_elems<FMT>();
  constexpr int U = chunk_unroll<FMT>();
  const int nch = I / EPC;
  for (int d = 0; d < nd; ++d) {
    const int4 dd = rw.dist[d];
    const int slot = dd.x, off = dd.y, cnt = dd.z;
    if (cnt <= 0 || off < 0 || off + cnt > Mk || slot < 0 || slot >= ra.S) continue;
    const uint8_t* img = slots + (size_t)slot * image_bytes;
    for (int base = 0; base < cnt; base += kFmtTok) {
      const int nt = min(kFmtTok, cnt - base);
      int route[kFmtTok];
#pragma unroll
      for (int t = 0; t < kFmtTok; ++t) route[t] = t < nt ? rw.perm[off + base + t] : 0;
      float acc[kFmtTok];
#pragma unroll
      for (int t = 0; t < kFmtTok; ++t) acc[t] = 0.0f;
      const float ds = matrix_scale<FMT>(img + F.down_s);
      for (int c0 = lane; c0 < nch; c0 += 64 * U) {
        uint4 cd[U];
        float s0[U], s1[U];
        int kk[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {  // (past the row: the last chunk again, unused)
          kk[u] = min(c0 + 64 * u, nch - 1) * EPC;
          cd[u] = ld_nt(reinterpret_cast<const uint4*>(img + F.down + elem_off<FMT>(r, kk[u], I)));
          chunk_scales<FMT>(img + F.down_s, r, kk[u], I, ds, s0[u], s1[u]);
        }
#pragma unroll
        for (int t = 0; t < kFmtTok; ++t) {
          if (t < nt) {
#pragma unroll
            for (int u = 0; u < U; ++u)
              if (c0 + 64 * u < nch)
                acc[t] += chunk_dot<FMT>(cd[u], hbuf + (size_t)route[t] * I + kk[u], s0[u], s1[u]);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < kFmtTok; ++t) {
        if (t < nt) {
          const float v = wave_sum(acc[t]);
          if (lane == ((route[t] / ra.k) & 63)) pdn[(size_t)route[t] * H + r] = v;
        }
      }
    }
  }
  // y for this row: lane m % 64 combines token m from the sums it stored itself
  for (int m = lane; m < ra.M; m += 64) {
    float acc = 0.0f;
    // 8 routes at a time: every load of a batch requested before the first is used (a cold
    // route's word is read and left unused), then the sum in ascending j
    for (int j0 = 0; j0 < ra.k; j0 += 8) {
      bool hot[8];
      float wv[8], pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = m * ra.k + min(j0 + u, ra.k - 1);
        hot[u] = j0 + u < ra.k && rw.route_slot[q] >= 0;
        wv[u] = ra.w_in[q];
        pv[u] = pdn[(size_t)q * H + r];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (hot[u]) acc = fmaf(wv[u], pv[u], acc);
    }
    const size_t o = (size_t)m * H + r;
    y[o] = acc;
    if (res.out) res.out[o] = (uint16_t)f32_to_bf16_bits(bf16_f32(res.x[o]) + acc);
  }
}

hipError_t launch_gateup_fmt(int fmt, const uint16_t* x, int H, int I, const uint8_t* slots,
                             size_t image_bytes, const FmtLayout& F, int nd_max,
                             const RouteArgs& ra, const RouteWs& rw, uint16_t* hbuf,
                             hipStream_t s) {
  if (nd_max <= 0) return hipSuccess;
  const dim3 g(I / kFmtWaves, nd_max), b(kFmtWaves * 64);
  switch (fmt) {
    case MOE_FORMAT_BF16:
      hipLaunchKernelGGL(k_gateup_fmt<MOE_FORMAT_BF16>, g, b, 0, s, x, H, I, slots, image_bytes,
                         F, ra, rw, hbuf);
      break;
    case MOE_FORMAT_FP8_BLOCK:
      hipLaunchKernelGGL(k_gateup_fmt<MOE_FORMAT_FP8_BLOCK>, g, b, 0, s, x, H, I, slots,
                         image_bytes, F, ra, rw, hbuf);
      break;
    case MOE_FORMAT_NVFP4:
      hipLaunchKernelGGL(k_gateup_fmt<MOE_FORMAT_NVFP4>, g, b, 0, s, x, H, I, slots, image_bytes,
                         F, ra, rw, hbuf);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_down_fmt(int fmt, int H, int I, const uint8_t* slots, size_t image_bytes,
                           const FmtLayout& F, const RouteArgs& ra, const RouteWs& rw,
                           const uint16_t* hbuf, float* pdn, float* y, Residual res,
                           hipStream_t s) {
  const dim3 g(H / kFmtWaves), b(kFmtWaves * 64);
  switch (fmt) {
    case MOE_FORMAT_BF16:
      hipLaunchKernelGGL(k_down_fmt<MOE_FORMAT_BF16>, g, b, 0, s, H, I, slots, image_bytes, F, ra,
                         rw, hbuf, pdn, y, res);
      break;
    case MOE_FORMAT_FP8_BLOCK:
      hipLaunchKernelGGL(k_down_fmt<MOE_FORMAT_FP8_BLOCK>, g, b, 0, s, H, I, slots, image_bytes, F,
                         ra, rw, hbuf, pdn, y, res);
      break;
    case MOE_FORMAT_NVFP4:
      hipLaunchKernelGGL(k_down_fmt<MOE_FORMAT_NVFP4>, g, b, 0, s, H, I, slots, image_bytes, F, ra,
                         rw, hbuf, pdn, y, res);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
