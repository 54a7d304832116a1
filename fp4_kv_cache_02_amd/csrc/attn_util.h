// Device helpers of the attention kernels: exact FP4 (E2M1 x E4M3) to fp16
// dequantisation, bf16 / fp16 packing for the matrix-core operands, and the
// per-head power-of-two scaling that brings a bf16 query into fp16's range.
#pragma once
#include "kernels.h"

namespace csa2 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// byte `sel` of `word` (two E2M1 codes, low nibble first) as fp16 at unit scale;
// sel is a compile-time constant after unrolling
CSA2_DEV half2_t fp4x2(uint32_t word, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3);
  }
}
CSA2_DEV uint32_t h2u(half2_t h) { return __builtin_bit_cast(uint32_t, h); }
CSA2_DEV half2_t u2h(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
// low halves of x and y as (x, y); high halves as (x, y): one byte permute
// each (the FP4 values of a main step), or a mask and a shift each (the
// window's bf16 words: with the permute there, a launch of whole window
// steps -- eight rows x six layers -- measured ~2.5 us slower)
CSA2_DEV uint32_t pack_lo(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x05040100u); }
CSA2_DEV uint32_t pack_hi(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x07060302u); }
CSA2_DEV uint32_t pack_lo_w(uint32_t x, uint32_t y) { return (x & 0xFFFFu) | (y << 16); }
CSA2_DEV uint32_t pack_hi_w(uint32_t x, uint32_t y) { return (x >> 16) | (y & 0xFFFF0000u); }

// Four E4M3 scales (the bytes of `w`) as fp16 pairs {s_i, s_i}: the hardware
// OCP E4M3 -> fp16 conversion at unit scale (exact: every E4M3 value,
// subnormals included, is an fp16 normal number), then each half doubled.
CSA2_DEV void scale_pairs4(uint32_t w, uint32_t (&o)[4]) {
  const uint32_t a = h2u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  const uint32_t b = h2u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
  o[0] = pack_lo(a, a);
  o[1] = pack_hi(a, a);
  o[2] = pack_lo(b, b);
  o[3] = pack_hi(b, b);
}

// 8 consecutive FP4 codes (one dword) times one E4M3 scale held as the fp16
// pair {s, s}, as fp16 (exact: an E2M1 value times an E4M3 value has at most
// six significant bits and lies within fp16's normal range).
CSA2_DEV half8_t dequant8(uint32_t word, half2_t sv) {
  const half2_t h0 = fp4x2(word, 0) * sv, h1 = fp4x2(word, 1) * sv;
  const half2_t h2 = fp4x2(word, 2) * sv, h3 = fp4x2(word, 3) * sv;
  half8_t r;
  r[0] = h0[0]; r[1] = h0[1]; r[2] = h1[0]; r[3] = h1[1];
  r[4] = h2[0]; r[5] = h2[1]; r[6] = h3[0]; r[7] = h3[1];
  return r;
}

CSA2_DEV bf8_t as_bf8(uint4 v) { return __builtin_bit_cast(bf8_t, v); }
CSA2_DEV half8_t as_h8(uint4 v) { return __builtin_bit_cast(half8_t, v); }
CSA2_DEV uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
CSA2_DEV uint4 mask4(uint4 v, uint32_t m) { return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m); }
CSA2_DEV float pick4(const float (&v)[4], int i) {
  return (i == 0) ? v[0] : (i == 1) ? v[1] : (i == 2) ? v[2] : v[3];
}

CSA2_DEV uint32_t bf16_abs_max8(uint4 v) {
  const uint32_t a = max(max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu), max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu));
  const uint32_t b = max(max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu), max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu));
  return max(a, b);
}
CSA2_DEV uint4 bf16x8_to_f16x8_scaled(uint4 v, float mul) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2_t h = {(_Float16)(bf16_lo(w[i]) * mul), (_Float16)(bf16_hi(w[i]) * mul)};
    o[i] = h2u(h);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}
}  // namespace csa2
