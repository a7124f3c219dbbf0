// Expert image packing: canonical matrices <-> the image layouts described in moe_internal.h
// (the MXFP4 kernel layout; the six row-major sections of the other formats).  Pure host code.
#include <string.h>

#include "moe.h"
#include "moe_internal.h"

namespace moe {
moe_status fail(moe_status st, const char* fmt, ...);
moe_status ok();
moe_status check_shape(const moe_shape* s);

// Copy direction: pack (canonical -> image) or unpack (image -> canonical).
// Gate/up tiles: lane l < 32 is gate row 32t+l, lane l >= 32 up row 32t+l-32; block b of the
// lane's row at (b*64 + l)*16, scale words after the codes (see moe_internal.h).
template <bool PACK>
static void tiles(uint8_t* img, int n_tiles, int rows_per_lane_group, int nb, int ng,
                  size_t tile_bytes, uint8_t* const* codes, uint8_t* const* scales, int K) {
  const size_t row_code_bytes = (size_t)K / 2;
  const size_t row_scale_bytes = (size_t)K / 32;
  for (int t = 0; t < n_tiles; ++t) {
    uint8_t* tb = img + (size_t)t * tile_bytes;
    for (int lane = 0; lane < 64; ++lane) {
      const int mat = rows_per_lane_group == 32 ? (lane >> 5) : 0;
      const int row = t * rows_per_lane_group + (rows_per_lane_group == 32 ? (lane & 31) : lane);
      uint8_t* c = codes[mat] + (size_t)row * row_code_bytes;
      uint8_t* s = scales[mat] + (size_t)row * row_scale_bytes;
      for (int b = 0; b < nb; ++b) {
        uint8_t* dst = tb + ((size_t)b * 64 + lane) * 16;
        if (PACK)
          memcpy(dst, c + (size_t)b * 16, 16);
        else
          memcpy(c + (size_t)b * 16, dst, 16);
      }
      for (int q = 0; q < ng; ++q) {
        uint8_t* dst = tb + (size_t)nb * 1024 + ((size_t)q * 64 + lane) * 4;
        for (int i = 0; i < 4; ++i) {
          const int b = 4 * q + i;
          if (PACK)
            dst[i] = b < nb ? s[b] : 127;
          else if (b < nb)
            s[b] = dst[i];
        }
      }
    }
  }
}

// Down tiles: 16 rows; at K step s lane l holds row l%16, block 4s + l/16 (see moe_internal.h).
template <bool PACK>
static void down_tiles(uint8_t* img, const ImageLayout& L, uint8_t* codes, uint8_t* scales) {
  const int nb = L.nb_i;
  const size_t row_code_bytes = (size_t)L.I / 2;
  const size_t row_scale_bytes = (size_t)L.I / 32;
  for (int t = 0; t < L.dn_tiles; ++t) {
    uint8_t* tb = img + (size_t)t * L.dn_tile_bytes;
    for (int lane = 0; lane < 64; ++lane) {
      const int row = t * kDnRows + lane % 16;
      uint8_t* c = codes + (size_t)row * row_code_bytes;
      uint8_t* sc = scales + (size_t)row * row_scale_bytes;
      for (int st = 0; st < L.dn_ks; ++st) {
        const int b = 4 * st + lane / 16;
        if (b >= nb) continue;  // only in the partial step, whose stored lanes come first
        uint8_t* dst = tb + ((size_t)st * 64 + lane) * 16;
        if (PACK)
          memcpy(dst, c + (size_t)b * 16, 16);
        else
          memcpy(c + (size_t)b * 16, dst, 16);
      }
      for (int q = 0; q < L.dn_scale_words; ++q) {
        uint8_t* dst = tb + L.dn_code_bytes + ((size_t)q * 64 + lane) * 4;
        for (int i = 0; i < 4; ++i) {
          const int b = 4 * (4 * q + i) + lane / 16;
          if (PACK)
            dst[i] = b < nb ? sc[b] : 127;
          else if (b < nb)
            sc[b] = dst[i];
        }
      }
    }
  }
}

// The other formats: the six canonical arrays copied into (or out of) their image sections.
template <bool PACK>
static void fmt_sections(int fmt, int H, int I, uint8_t* img, uint8_t* const* arr) {
  const FmtLayout F = fmt_layout(fmt, H, I);
  const size_t off[6] = {F.gate, F.gate_s, F.up, F.up_s, F.down, F.down_s};
  const int N[6] = {I, I, I, I, H, H}, K[6] = {H, H, H, H, I, I};
  for (int a = 0; a < 6; ++a) {
    const size_t n = (a & 1) ? fmt_scale_bytes(fmt, N[a], K[a]) : fmt_elem_bytes(fmt, N[a], K[a]);
    if (n == 0) continue;
    if (PACK)
      memcpy(img + off[a], arr[a], n);
    else
      memcpy(arr[a], img + off[a], n);
  }
}

}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_pack_expert(const moe_shape* shape, const uint8_t* gate_codes,
                           const uint8_t* gate_scales, const uint8_t* up_codes,
                           const uint8_t* up_scales, const uint8_t* down_codes,
                           const uint8_t* down_scales, uint8_t* image) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (shape->format != MOE_FORMAT_MXFP4) {
    const bool scaled = shape->format != MOE_FORMAT_BF16;
    if (!gate_codes || !up_codes || !down_codes || !image ||
        (scaled && (!gate_scales || !up_scales || !down_scales)))
      return fail(MOE_ERR_INVALID_ARG, "moe_pack_expert: NULL pointer");
    memset(image, 0, expert_image_bytes(shape));
    uint8_t* arr[6] = {const_cast<uint8_t*>(gate_codes), const_cast<uint8_t*>(gate_scales),
                       const_cast<uint8_t*>(up_codes),   const_cast<uint8_t*>(up_scales),
                       const_cast<uint8_t*>(down_codes), const_cast<uint8_t*>(down_scales)};
    fmt_sections<true>(shape->format, shape->hidden, shape->inter, image, arr);
    return ok();
  }
  if (!gate_codes || !gate_scales || !up_codes || !up_scales || !down_codes || !down_scales || !image)
    return fail(MOE_ERR_INVALID_ARG, "moe_pack_expert: NULL pointer");
  const ImageLayout L = image_layout(shape->hidden, shape->inter);
  memset(image, 0, L.image_bytes);
  uint8_t* gc[2] = {const_cast<uint8_t*>(gate_codes), const_cast<uint8_t*>(up_codes)};
  uint8_t* gs[2] = {const_cast<uint8_t*>(gate_scales), const_cast<uint8_t*>(up_scales)};
  tiles<true>(image, L.gu_tiles, 32, L.nb_h, L.ng_h, L.gu_tile_bytes, gc, gs, L.H);
  down_tiles<true>(image + L.gu_bytes, L, const_cast<uint8_t*>(down_codes),
                   const_cast<uint8_t*>(down_scales));
  return ok();
}

moe_status moe_unpack_expert(const moe_shape* shape, const uint8_t* image, uint8_t* gate_codes,
                             uint8_t* gate_scales, uint8_t* up_codes, uint8_t* up_scales,
                             uint8_t* down_codes, uint8_t* down_scales) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (shape->format != MOE_FORMAT_MXFP4) {
    const bool scaled = shape->format != MOE_FORMAT_BF16;
    if (!gate_codes || !up_codes || !down_codes || !image ||
        (scaled && (!gate_scales || !up_scales || !down_scales)))
      return fail(MOE_ERR_INVALID_ARG, "moe_unpack_expert: NULL pointer");
    uint8_t* arr[6] = {gate_codes, gate_scales, up_codes, up_scales, down_codes, down_scales};
    fmt_sections<false>(shape->format, shape->hidden, shape->inter, const_cast<uint8_t*>(image), arr);
    return ok();
  }
  if (!gate_codes || !gate_scales || !up_codes || !up_scales || !down_codes || !down_scales || !image)
    return fail(MOE_ERR_INVALID_ARG, "moe_unpack_expert: NULL pointer");
  const ImageLayout L = image_layout(shape->hidden, shape->inter);
  uint8_t* img = const_cast<uint8_t*>(image);
  uint8_t* gc[2] = {gate_codes, up_codes};
  uint8_t* gs[2] = {gate_scales, up_scales};
  tiles<false>(img, L.gu_tiles, 32, L.nb_h, L.ng_h, L.gu_tile_bytes, gc, gs, L.H);
  down_tiles<false>(img + L.gu_bytes, L, down_codes, down_scales);
  return ok();
}

}  // extern "C"
