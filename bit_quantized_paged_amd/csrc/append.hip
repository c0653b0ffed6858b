// Quantize-append with a slot mapping [P40177 "Key source snippets",
// _create_nvfp4_hnd_kv_cache; RFC47684 "Fix steps"].
//
// One lane owns one 16-element block of one (token, kv head, K|V) row, so the
// block amax needs no cross-lane traffic: it reads 32 bytes of bf16 and
// writes 8 bytes of codes plus its scale byte. Rows are dealt out in tiles
// of 16 tokens with the token fastest: consecutive lanes write consecutive
// rows of one kv head, which a sequence's tokens keep adjacent in a page, so
// a wave's stores fill whole cache lines (with the head fastest they spread
// over the head slabs and each line was completed by other workgroups). FP8 caches [P40177 "Key
// source snippets": fp8_e4m3 / fp8_e5m2] take the same lanes and write 16
// code bytes of x / g.
#include "quantize.hpp"
#include "launch.hpp"

namespace nvfp4kv {

template <int D, int FMT>
__global__ __launch_bounds__(256) void append_kernel(Pool pool, const uint16_t* __restrict__ key,
                                                     int64_t k_st, int64_t k_sh,
                                                     const uint16_t* __restrict__ value, int64_t v_st,
                                                     int64_t v_sh, const int64_t* __restrict__ slots,
                                                     int64_t num_tokens, const float* __restrict__ k_scale,
                                                     const float* __restrict__ v_scale) {
  constexpr int LPR = D / 16;  // lanes per row
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  constexpr int TT = kAppendTile;
  const int64_t row = gid / LPR;
  const int blk16 = (int)(gid % LPR);
  const int hkv = pool.hkv;
  // row = ((tile * 2 + kv) * hkv + h) * TT + ti, token t = tile * TT + ti
  const int64_t tiles = (num_tokens + TT - 1) / TT;
  if (row >= tiles * TT * 2 * hkv) return;
  const int ti = (int)(row % TT);
  const int64_t rest = row / TT;
  const int h = (int)(rest % hkv);
  const int kv = (int)((rest / hkv) & 1);
  const int64_t t = (rest / (2 * (int64_t)hkv)) * TT + ti;
  if (t >= num_tokens) return;

  const int64_t slot = slots[t];
  const int64_t cap = pool.num_blocks * pool.bs;
  if (slot < 0 || slot >= cap) return;

  const uint16_t* src = kv ? value + t * v_st + h * v_sh : key + t * k_st + h * k_sh;
  const u32x4* s4 = reinterpret_cast<const u32x4*>(src + blk16 * 16);
  float x[16];
  bf16_block16(s4[0], s4[1], x);
  const float g = kv ? *v_scale : *k_scale;
  const int64_t blk = slot / pool.bs;
  const int64_t off = slot % pool.bs;
  uint8_t* dst = pool.data + blk * pool.sb + kv * pool.skv + off * pool.st + h * pool.sh;
  if constexpr (FMT == kNvfp4) {
    uint32_t w0, w1;
    const uint32_t s8 = quantize_block16(x, g, w0, w1);
    st_u32x2(dst + blk16 * 8, u32x2{w0, w1});
    dst[D / 2 + blk16] = (uint8_t)s8;
  } else {
    u32x4 c;
#pragma unroll
    for (int q = 0; q < 4; ++q) c[q] = fp8_pack4<FMT>(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3], g);
    st_u32x4(dst + blk16 * 16, c);
  }
}

template <int FMT>
static hipError_t launch_append_f(const Pool& pool, int head_size, const void* key, int64_t k_st, int64_t k_sh,
                                  const void* value, int64_t v_st, int64_t v_sh, const int64_t* slots,
                                  int64_t num_tokens, const float* k_scale, const float* v_scale,
                                  hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int64_t lanes = append_lanes(num_tokens, pool.hkv, head_size);
  const int64_t blocks = (lanes + 255) / 256;
  const dim3 grid((unsigned)blocks);
  const uint16_t* k = static_cast<const uint16_t*>(key);
  const uint16_t* v = static_cast<const uint16_t*>(value);
  switch (head_size) {
    case 64:
      append_kernel<64, FMT><<<grid, 256, 0, stream>>>(pool, k, k_st, k_sh, v, v_st, v_sh, slots, num_tokens,
                                                  k_scale, v_scale);
      break;
    case 128:
      append_kernel<128, FMT><<<grid, 256, 0, stream>>>(pool, k, k_st, k_sh, v, v_st, v_sh, slots, num_tokens,
                                                   k_scale, v_scale);
      break;
    case 256:
      append_kernel<256, FMT><<<grid, 256, 0, stream>>>(pool, k, k_st, k_sh, v, v_st, v_sh, slots, num_tokens,
                                                   k_scale, v_scale);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_append(const Pool& pool, int head_size, const void* key, int64_t k_st, int64_t k_sh,
                         const void* value, int64_t v_st, int64_t v_sh, const int64_t* slots,
                         int64_t num_tokens, const float* k_scale, const float* v_scale, int fmt,
                         hipStream_t stream) {
  switch (fmt) {
    case kNvfp4:
      return launch_append_f<kNvfp4>(pool, head_size, key, k_st, k_sh, value, v_st, v_sh, slots, num_tokens,
                                     k_scale, v_scale, stream);
    case kFp8E4M3:
      return launch_append_f<kFp8E4M3>(pool, head_size, key, k_st, k_sh, value, v_st, v_sh, slots, num_tokens,
                                       k_scale, v_scale, stream);
    case kFp8E5M2:
      return launch_append_f<kFp8E5M2>(pool, head_size, key, k_st, k_sh, value, v_st, v_sh, slots, num_tokens,
                                       k_scale, v_scale, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace nvfp4kv
