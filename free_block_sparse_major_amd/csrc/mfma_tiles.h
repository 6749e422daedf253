// MFMA tile helpers shared by the attention and probe kernels (gfx950).
//
// Operand layouts of v_mfma_f32_32x32x16_{bf16,f16} (wave64):
//   A (32 x 16): lane l holds row l%32, k = 8*(l/32) .. +8
//   B (16 x 32): lane l holds column l%32, k = 8*(l/32) .. +8
//   C (32 x 32): lane l holds column l%32, rows 8*(r/4) + 4*(l/32) + r%4, r = 0..15
// Scores are formed transposed (S^T = K Q^T): a lane owns one query and 32
// keys of a 64-key tile; O^T = V^T P^T keeps one query per lane as well.
//
// LDS tiles are 64 rows x D, row-major in 16-byte chunks with an XOR swizzle:
//   K (bf16): physical chunk = logical ^ (row % chunks-per-row)
//   V (fp16): physical chunk = logical ^ swz_v(row), a 64-byte-window rotation
// V^T fragments are read with ds_read_b64_tr_b16: inside each 16-lane group,
// source lane r points at V[k0 + r/4][d0 + 4(r%4) .. +3] and lane i receives
// V[k0 + j][d0 + i] for j = 0..3.
#pragma once

#include "common.h"

namespace spr {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

template <int D>
SPR_DEV int swz_v(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

template <int D>
SPR_DEV int k_slot(int row, int chunk) {
  return row * (D / 8) + (chunk ^ (row & (D / 8 - 1)));
}

template <int D>
SPR_DEV int v_slot(int row, int chunk) {
  return row * (D / 8) + (chunk ^ swz_v<D>(row));
}

// A operand of QK^T: keys 32*kb + n, dims 16 s + 8 g .. +8
template <int D>
SPR_DEV bf16x8_t k_frag(const uint4* kt, int row, int s, int g) {
  return __builtin_bit_cast(bf16x8_t, kt[k_slot<D>(row, 2 * s + g)]);
}

// A operand of PV for d block db and 16-key step u, keys in the slot order
// of the P fragment built from the C layout: slots 0..3 = keys 16u + 4g' +
// 0..3, slots 4..7 = keys 16u + 8 + 4g' + 0..3 (g' = lane / 32).
template <int D>
SPR_DEV f16x8_t v_frag(const uint4* vt, int lane, int u, int db) {
  const int G = lane >> 4, gi = lane & 15, gg = G >> 1;
  const int row1 = 16 * u + 4 * gg + (gi >> 2);
  const int row2 = row1 + 8;
  const int ch = 4 * db + 2 * (G & 1) + ((gi & 3) >> 1);
  const int hb = (gi & 1) * 8;
  const char* b1 = reinterpret_cast<const char*>(vt + v_slot<D>(row1, ch)) + hb;
  const char* b2 = reinterpret_cast<const char*>(vt + v_slot<D>(row2, ch)) + hb;
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)b1);
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)b2);
  return __builtin_bit_cast(f16x8_t, (short __attribute__((ext_vector_type(8)))){
                                         lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

// key index (0..63 in the tile) of C-layout register r of 32-key block kb
SPR_DEV int c_key(int kb, int r, int g) { return 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3); }

}  // namespace spr
