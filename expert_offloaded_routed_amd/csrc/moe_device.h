// Device helpers for gfx950: wave64 reductions with DPP / ds_swizzle, MXFP4 decode via the
// CDNA4 packed FP4->bf16 converter, bf16 dot products with fp32 accumulation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ---- DPP / swizzle lane exchange ------------------------------------------------------------
// dpp_ctrl values (GFX9 encoding): quad_perm [1,0,3,2] = 0xB1 (lane ^ 1), [2,3,0,1] = 0x4E
// (lane ^ 2), row_half_mirror = 0x141, row_mirror = 0x140, row_shr:n = 0x110 + n,
// row_bcast:15 = 0x142, row_bcast:31 = 0x143.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
// ds_swizzle bit mode: and_mask 0x1F, xor_mask 0x10 -> exchange with lane ^ 16 (within 32).
__device__ __forceinline__ int swz_xor16_i(int v) { return __builtin_amdgcn_ds_swizzle(v, 0x401F); }
__device__ __forceinline__ float swz_xor16_f(float v) {
  return __int_as_float(swz_xor16_i(__float_as_int(v)));
}

// Sums over the lane pairs (l, l^8), (l, l^16) and (l, l^32), on the VALU: a DPP rotate by 8
// within rows of 16, and the gfx950 permlane swaps, whose two results hold the lower and the
// upper lane of each pair.  Both lanes of a pair get the same bits.
__device__ __forceinline__ float pair_sum8(float v) { return v + dpp_f<0x128>(v); }
__device__ __forceinline__ float pair_sum16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float pair_sum32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Sum over each row of 16 lanes (quad swaps, then the half-row and row mirrors); a lane's
// result is deterministic, though lanes of a row may differ in the last bits.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return v;
}

// Sum over the 64 lanes; every lane gets the same (deterministically ordered) total.
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  v += swz_xor16_f(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
}

// (value, index) argmax over the wave: larger value wins, equal values -> lower index.
__device__ __forceinline__ void argmax_step(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(float& v, int& i) {
  float ov = dpp_f<CTRL>(v);
  int oi = dpp_i<CTRL>(i);
  argmax_step(v, i, ov, oi);
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_dpp<0xB1>(v, i);
  argmax_dpp<0x4E>(v, i);
  argmax_dpp<0x141>(v, i);
  argmax_dpp<0x140>(v, i);
  argmax_step(v, i, swz_xor16_f(v), swz_xor16_i(i));
  float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  int i0 = __builtin_amdgcn_readlane(i, 0);
  float v1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  int i1 = __builtin_amdgcn_readlane(i, 32);
  v = v0;
  i = i0;
  argmax_step(v, i, v1, i1);
}

// Inclusive prefix sum over the 64 lanes (row shifts inside rows of 16, then row broadcasts).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += dpp_i<0x111>(v);
  v += dpp_i<0x112>(v);
  v += dpp_i<0x114>(v);
  v += dpp_i<0x118>(v);
  v += dpp_i<0x142, 0xA>(v);
  v += dpp_i<0x143, 0xC>(v);
  return v;
}

// ---- weight loads ------------------------------------------------------------------------------
// A 16-byte load of weight bytes that a call reads once, marked non-temporal: the stream of expert
// weights then does not displace what is reused from the caches (activations, h, route tables),
// and on MI355X it streams faster (the one-token layer: 20.2 -> 19.0 us a step).
typedef uint32_t nt_u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  const nt_u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
// The same for a 4-byte word (scale words of the weight streams).
__device__ __forceinline__ uint32_t ld_nt32(const uint32_t* p) { return __builtin_nontemporal_load(p); }

// ---- number formats ---------------------------------------------------------------------------
// E8M0 scale byte -> fp32: 2^(x-127) (x = 0 gives the fp32 subnormal 2^-127); x = 255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t x) {
  const float v = __builtin_amdgcn_ldexpf(1.0f, (int)x - 127);
  return x == 255 ? __uint_as_float(0x7FC00000u) : v;
}

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }

// Dot product of 8 bf16 pairs (one 16-byte chunk each), accumulated in fp32 pair by pair.
__device__ __forceinline__ float dot8_bf16(const uint4& w, const uint4& x, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.x), as_bf16x2(x.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.y), as_bf16x2(x.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.z), as_bf16x2(x.z), acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.w), as_bf16x2(x.w), acc, false);
}

// Sum over one 32-element MXFP4 block (codes c, unscaled) times 32 bf16 activations a:
// each code byte holds two E2M1 values (low nibble first) that the gfx950 converter turns into
// an exact bf16 pair, dotted with the matching activation pair in fp32.
__device__ __forceinline__ float block_dot(const uint4 c, const uint4 a0, const uint4 a1,
                                           const uint4 a2, const uint4 a3) {
  const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
  const uint32_t aw[16] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w,
                           a2.x, a2.y, a2.z, a2.w, a3.x, a3.y, a3.z, a3.w};
  // two independent accumulation chains (even and odd element pairs), summed at the end
  float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], 1.0f, 0),
                                         as_bf16x2(aw[4 * j + 0]), s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], 1.0f, 1),
                                         as_bf16x2(aw[4 * j + 1]), s1, false);
    s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], 1.0f, 2),
                                         as_bf16x2(aw[4 * j + 2]), s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], 1.0f, 3),
                                         as_bf16x2(aw[4 * j + 3]), s1, false);
  }
  return s0 + s1;
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

// ---- h for the block-scaled matrix cores ------------------------------------------------------
// A block of 32 bf16 values h (one MXFP4 block of the down projection's K) enters the
// gfx950 block-scaled MFMA as 2^s * (hi + lo): s = (largest binary exponent in the block) - 7,
// so that |h| * 2^-s < 2^8; hi = h * 2^-s rounded to E4M3 (OCP: bias 7, with subnormals, max
// 448), lo = the remainder rounded to E4M3 again.  A bf16 value has 8 significant bits, hi
// takes the top 4 and the remainder (at most 4 more) is exact in E4M3 as long as it is not
// below E4M3's smallest subnormal: every element within 2^-9 of the block's largest
// magnitude is represented exactly, smaller ones to within 2^-10 * 2^s (2^-17 of the block's
// largest magnitude).

// Binary exponent of |v| from its fp32 exponent field (-127 for zero and fp32 subnormals).
__device__ __forceinline__ int f32_exp(float v) {
  return (int)((__float_as_uint(v) >> 23) & 0xFFu) - 127;
}

// Scale exponent of a block whose largest element exponent is emax (E8M0 byte = s + 127).
__device__ __forceinline__ int mx_shift(int emax) { return min(max(emax - 7, -127), 127); }

// E4M3 code of v (|v| <= 2^8), rounded to nearest even; *q receives the value it encodes.
__device__ __forceinline__ uint32_t e4m3_rne(float v, float* q) {
  const float a = fabsf(v);
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const int e = max(f32_exp(a), -6);  // below 2^-6 the subnormals share that binade's step
  const float m = __builtin_rintf(__builtin_amdgcn_ldexpf(a, 3 - e));  // a / step, in [0, 16]
  *q = __builtin_copysignf(__builtin_amdgcn_ldexpf(m, e - 3), v);
  const uint32_t mi = (uint32_t)m;
  uint32_t code;
  if (mi < 8)
    code = mi;  // subnormal (only in the binade of 2^-6)
  else if (mi < 16)
    code = ((uint32_t)(e + 7) << 3) | (mi - 8);
  else
    code = (uint32_t)(e + 8) << 3;  // rounded up into the next binade
  return sign | code;
}

// hi and lo codes of one element of a block with scale exponent s.
__device__ __forceinline__ void mx_pair(float h, int s, uint32_t* hi, uint32_t* lo) {
  const float hp = __builtin_amdgcn_ldexpf(h, -s);
  float qh, ql;
  *hi = e4m3_rne(hp, &qh);
  *lo = e4m3_rne(hp - qh, &ql);  // hp - qh is exact in fp32
}

// Maximum over the 16 lanes of a DPP row; every lane of the row gets it.
__device__ __forceinline__ int row_max_i(int v) {
  v = max(v, dpp_i<0xB1>(v));
  v = max(v, dpp_i<0x4E>(v));
  v = max(v, dpp_i<0x141>(v));
  v = max(v, dpp_i<0x140>(v));
  return v;
}
// ... and over the 32 lanes of a half wave.
__device__ __forceinline__ int half_max_i(int v) {
  v = row_max_i(v);
  return max(v, swz_xor16_i(v));
}

// D += A * B on the matrix cores: A = 16 rows x 128 K of E2M1 codes (lane l: row l%16, K
// 32*(l/16) .. +32, 16 bytes, low nibble first) with E8M0 scale byte OPA of sa for the lane's
// 32 elements; B = 128 K x 16 columns of E4M3 (lane l: column l%16, K 16*(l/16) .. +16 in
// b0 and K 64 + 16*(l/16) .. +16 in b1) with E8M0 scale byte 0 of sb for the 32-element block
// l/16 of column l%16.  D: lane l, register i = row 4*(l/16) + i, column l%16.
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
template <int OPA>
__device__ __forceinline__ f32x4_t mfma_mx(const uint4& a, const uint4& b0, const uint4& b1,
                                           f32x4_t c, uint32_t sa, uint32_t sb) {
  const i32x8_t A = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const i32x8_t B = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                     (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 0, OPA, (int)sa, 0, (int)sb);
}

}  // namespace moe
