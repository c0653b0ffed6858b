// Device helpers for the NVFP4 paged KV cache kernels (gfx950).
//
// Format [P39129 NvFp4LinearLayerConfig docstring; P40177 get_kv_cache_shape,
// get_dtype_for_flashinfer]: a (token, kv head) row is D/2 bytes of E2M1 codes
// (element 2k in the low nibble of byte k) followed by D/16 E4M3FN scales.
// FP8 caches (kFp8E4M3, kFp8E5M2) hold one code per element instead.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4kv {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Pool rows are only guaranteed 4-byte aligned (36-byte rows at D=64); these
// wrappers state that alignment so the compiler may still emit wide loads.
struct __attribute__((packed, aligned(4))) A4x2 { u32x2 v; };
struct __attribute__((packed, aligned(4))) A4x4 { u32x4 v; };

__device__ __forceinline__ uint32_t ld_u8(const uint8_t* p) { return *p; }
__device__ __forceinline__ uint32_t ld_u16(const uint8_t* p) { return *reinterpret_cast<const uint16_t*>(p); }
__device__ __forceinline__ uint32_t ld_u32(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ u32x2 ld_u32x2(const uint8_t* p) { return reinterpret_cast<const A4x2*>(p)->v; }
__device__ __forceinline__ u32x4 ld_u32x4(const uint8_t* p) { return reinterpret_cast<const A4x4*>(p)->v; }
__device__ __forceinline__ void st_u32x2(uint8_t* p, u32x2 v) { reinterpret_cast<A4x2*>(p)->v = v; }
__device__ __forceinline__ void st_u32x4(uint8_t* p, u32x4 v) { reinterpret_cast<A4x4*>(p)->v = v; }

// Cache formats [P40177 "Key source snippets": nvfp4 beside fp8_e4m3 and
// fp8_e5m2 in the backend's KV cache dtypes]. An NVFP4 row is D/2 code bytes
// then D/16 E4M3 block scales; an FP8 row is D codes under the per-tensor
// scale alone.
constexpr int kNvfp4 = 0;
constexpr int kFp8E4M3 = 1;
constexpr int kFp8E5M2 = 2;

// Pool geometry, strides in bytes (see nvfp4kv_cache).
struct Pool {
  uint8_t* data;
  int64_t num_blocks;
  int64_t sb, skv, st, sh;
  int32_t bs;
  int32_t bs_log2;  // block_size is a power of two
  int32_t hkv;
};

__device__ __forceinline__ int64_t clamp_block(int32_t id, int64_t num_blocks) {
  // Out-of-range ids are a caller error; clamping keeps every access inside
  // the pool so that bad metadata cannot fault the device. num_blocks is
  // below 2^31 (checked on the host), so 32-bit arithmetic suffices and stays
  // on the scalar unit for wave-uniform ids.
  const int32_t nb = (int32_t)num_blocks;
  int32_t v = id < 0 ? 0 : id;
  v = v >= nb ? nb - 1 : v;
  return (int64_t)v;
}

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 pair -> packed bf16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f2 v = {a, b};
  bf2 r = __builtin_convertvector(v, bf2);
  return __builtin_bit_cast(uint32_t, r);
}

// ---- E4M3FN --------------------------------------------------------------

// Non-negative finite fp32 -> E4M3FN byte, round to nearest even, values at
// or above 448 saturate to 0x7E. In binade [2^e, 2^(e+1)) (e clamped to >= -6,
// where the subnormal step 2^-9 takes over) the significand count is
// n = rint(s * 2^(3-e)) in [8, 16] (or [0, 8] below 2^-6) and the byte is
// (e + 6) * 8 + n; a round-up to 16 lands on the next binade's first code.
__device__ __forceinline__ uint32_t e4m3_from_f32_sat(float s) {
  if (!(s < 448.0f)) return 0x7Eu;
  int e = (int)((__float_as_uint(s) >> 23) & 0xFFu) - 127;
  e = e < -6 ? -6 : e;
  float n = __builtin_rintf(__builtin_ldexpf(s, 3 - e));
  return (uint32_t)((e + 6) * 8 + (int)n);
}

// E4M3FN byte (never NaN here) -> fp32, exact.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  int e = (int)((b >> 3) & 15u);
  int m = (int)(b & 7u);
  float v = e ? __builtin_ldexpf((float)(8 + m), e - 10) : __builtin_ldexpf((float)m, -9);
  return (b & 0x80u) ? -v : v;
}

// ---- E2M1 ----------------------------------------------------------------

// Two E2M1 codes in byte `sel` of w -> f16 pair (low nibble first), exact.
template <int SEL>
__device__ __forceinline__ h2 fp4x2_to_h2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

// Two E4M3 bytes (bytes 0,1 or 2,3 of w) -> f16 pair, exact.
template <bool HI>
__device__ __forceinline__ h2 fp8x2_to_h2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// f16 pair {byte A of a, byte B of b} of E5M2 codes: E5M2 is the upper byte
// of a binary16, so one byte permute (zeros below) converts exactly.
template <int A, int B>
__device__ __forceinline__ h2 e5m2x2_to_h2(uint32_t a, uint32_t b) {
  constexpr uint32_t sel = ((uint32_t)(4 + B) << 24) | (0x0Cu << 16) | ((uint32_t)A << 8) | 0x0Cu;
  return __builtin_bit_cast(h2, __builtin_amdgcn_perm(b, a, sel));
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ---- one 16-element block -------------------------------------------------

// Dequantise one block into 8 words of bf16 pairs: codes -> f16 with the
// hardware FP4 convert, times the E4M3 scale (exact in f16: at most 6
// significant bits), widened to fp32, times g (one fp32 RNE multiply), then
// bf16 RNE.
__device__ __forceinline__ void dequant_block16(u32x2 codes, uint32_t sbyte, float g, uint32_t (&o)[8]) {
  const h2 s = fp8x2_to_h2<false>(sbyte);
  const h2 ss = {s[0], s[0]};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint32_t c = codes[q];
    const h2 v0 = fp4x2_to_h2<0>(c) * ss;
    const h2 v1 = fp4x2_to_h2<1>(c) * ss;
    const h2 v2 = fp4x2_to_h2<2>(c) * ss;
    const h2 v3 = fp4x2_to_h2<3>(c) * ss;
    o[4 * q + 0] = pack_bf16x2((float)v0[0] * g, (float)v0[1] * g);
    o[4 * q + 1] = pack_bf16x2((float)v1[0] * g, (float)v1[1] * g);
    o[4 * q + 2] = pack_bf16x2((float)v2[0] * g, (float)v2[1] * g);
    o[4 * q + 3] = pack_bf16x2((float)v3[0] * g, (float)v3[1] * g);
  }
}

// Half a block (8 elements: one code word) into 4 words of bf16 pairs, with
// the same arithmetic as dequant_block16.
__device__ __forceinline__ void dequant_half8(uint32_t c, uint32_t sbyte, float g, uint32_t (&o)[4]) {
  const h2 s = fp8x2_to_h2<false>(sbyte);
  const h2 ss = {s[0], s[0]};
  const h2 v0 = fp4x2_to_h2<0>(c) * ss;
  const h2 v1 = fp4x2_to_h2<1>(c) * ss;
  const h2 v2 = fp4x2_to_h2<2>(c) * ss;
  const h2 v3 = fp4x2_to_h2<3>(c) * ss;
  o[0] = pack_bf16x2((float)v0[0] * g, (float)v0[1] * g);
  o[1] = pack_bf16x2((float)v1[0] * g, (float)v1[1] * g);
  o[2] = pack_bf16x2((float)v2[0] * g, (float)v2[1] * g);
  o[3] = pack_bf16x2((float)v3[0] * g, (float)v3[1] * g);
}

}  // namespace nvfp4kv
