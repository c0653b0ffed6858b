// The NVFP4 block quantiser shared by the KV append, the QDQ emulation and
// the activation quantiser [P39129 NvFp4LinearLayerConfig docstring: two
// FP4 values per byte, one FP8-E4M3 scale per 16 values, a global fp32
// scale; P40177 "Key source snippets": the same format in the KV cache].
#pragma once

#include "device_common.hpp"

namespace nvfp4kv {

// The 16 bf16 values of one block (two 16-byte words) -> fp32.
__device__ __forceinline__ void bf16_block16(u32x4 a, u32x4 b, float (&x)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(a[i]);
    x[2 * i + 1] = bf16_hi(a[i]);
    x[8 + 2 * i] = bf16_lo(b[i]);
    x[8 + 2 * i + 1] = bf16_hi(b[i]);
  }
}

// Four E2M1 pairs -> one code word: byte j holds elements 2j (low nibble) and
// 2j + 1. The hardware convert with a unit scale rounds fp32 to nearest,
// ties to the even code, saturates at +-6 and keeps the sign of zeros and of
// values that round to zero; it differs from that rule only on NaN, which
// the quantiser below never produces from non-NaN inputs while 1 / d is
// finite.
__device__ __forceinline__ uint32_t e2m1_pack8(float a0, float a1, float a2, float a3, float a4, float a5, float a6,
                                               float a7) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a0, a1, 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a2, a3, 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a4, a5, 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a6, a7, 1.0f, 3);
  return w;
}

// Quantise one block under the per-tensor scale g: returns the E4M3 scale
// byte and sets the two code words (element 2k in the low nibble of byte k).
// Each line is a single fp32 operation with round-to-nearest-even: block
// scale s = E4M3(amax / (6 g)), step d = s * g, r = 1 / d (0 when d = 0),
// code = E2M1(x * r). For g >= 2^-119 the reciprocal of the smallest
// non-zero step is finite.
__device__ __forceinline__ uint32_t quantize_block16(const float (&x)[16], float g, uint32_t& w0, uint32_t& w1) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
  const float t6 = 6.0f * g;
  const float s32 = __fdiv_rn(amax, t6);
  const uint32_t s8 = e4m3_from_f32_sat(s32);
  const float d = e4m3_to_f32(s8) * g;
  const float r = (d == 0.0f) ? 0.0f : __fdiv_rn(1.0f, d);
  w0 = e2m1_pack8(x[0] * r, x[1] * r, x[2] * r, x[3] * r, x[4] * r, x[5] * r, x[6] * r, x[7] * r);
  w1 = e2m1_pack8(x[8] * r, x[9] * r, x[10] * r, x[11] * r, x[12] * r, x[13] * r, x[14] * r, x[15] * r);
  return s8;
}

// ---- FP8 KV rows [P40177 "Key source snippets": fp8_e4m3 / fp8_e5m2 cache
// dtypes]: code = FP8(RN32(x / g)), value = RN32(fp8 * g) ----------------

// fp32 -> FP8 byte, round to nearest even, magnitudes from the largest
// finite value up (infinity included) saturating to it, sign copied. E5M2:
// in binade [2^e, 2^(e+1)), e clamped to >= -14 (the subnormal step 2^-16
// continues below), n = rint(|q| * 2^(2-e)) and the byte is (e + 14) * 4 + n.
template <int FMT>
__device__ __forceinline__ uint32_t fp8_from_f32_sat(float q) {
  const float a = __builtin_fabsf(q);
  const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
  if constexpr (FMT == kFp8E4M3) {
    return e4m3_from_f32_sat(a) | sign;
  } else {
    if (!(a < 57344.0f)) return 0x7Bu | sign;
    int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;
    e = e < -14 ? -14 : e;
    const float n = __builtin_rintf(__builtin_ldexpf(a, 2 - e));
    return (uint32_t)((e + 14) * 4 + (int)n) | sign;
  }
}

// Four elements -> one word of FP8 codes (element k in byte k); g divides
// each element (one correctly rounded fp32 division).
template <int FMT>
__device__ __forceinline__ uint32_t fp8_pack4(float a0, float a1, float a2, float a3, float g) {
  return fp8_from_f32_sat<FMT>(__fdiv_rn(a0, g)) | (fp8_from_f32_sat<FMT>(__fdiv_rn(a1, g)) << 8) |
         (fp8_from_f32_sat<FMT>(__fdiv_rn(a2, g)) << 16) | (fp8_from_f32_sat<FMT>(__fdiv_rn(a3, g)) << 24);
}

// Eight FP8 codes (element k in byte k) -> 4 words of bf16 pairs:
// bf16_RNE(RN32(fp8 * g)); the codes convert to f16 exactly.
template <int FMT>
__device__ __forceinline__ void dequant_fp8x8(u32x2 c, float g, uint32_t (&o)[4]) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint32_t w = c[q];
    h2 a, b;
    if constexpr (FMT == kFp8E4M3) {
      a = fp8x2_to_h2<false>(w);
      b = fp8x2_to_h2<true>(w);
    } else {
      a = e5m2x2_to_h2<0, 1>(w, w);
      b = e5m2x2_to_h2<2, 3>(w, w);
    }
    o[2 * q] = pack_bf16x2((float)a[0] * g, (float)a[1] * g);
    o[2 * q + 1] = pack_bf16x2((float)b[0] * g, (float)b[1] * g);
  }
}

}  // namespace nvfp4kv
