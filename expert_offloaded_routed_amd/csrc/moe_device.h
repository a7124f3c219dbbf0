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

// Sum over the 64 lanes; every lane gets the same (deterministically ordered) total.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
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

}  // namespace moe
