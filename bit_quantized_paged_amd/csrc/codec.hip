// The codec on its own, for paths without native FP4 attention [P40177
// "Related context": the NVFP4 dequantization and quantize-dequantize (QDQ)
// emulation kernels for Hopper / AMD Instinct; RFC47684 "Fix steps":
// nvfp4_kv_dequantize_paged].
//
// Page-form dequantize: page p of the quantised pool becomes page p of a
// bf16 pool of the same geometry, so the same block table addresses both.
// QDQ: bf16 K/V rows are quantised exactly as the append writes them and
// replaced, in place, by the values the dequantize returns for them.
//
// FP8 caches take the page-form dequantize with the same lanes (8 codes each).
// Both are HBM-bound streams with one lane per 16-element block (8 code bytes
// + 1 scale byte <-> 32 bytes of bf16); consecutive lanes take consecutive
// blocks of one row, so the 32-byte bf16 accesses are coalesced.
#include "quantize.hpp"
#include "launch.hpp"

namespace nvfp4kv {

template <int D, int FMT>
__global__ __launch_bounds__(256) void dequant_pages_kernel(Pool pool, const int32_t* __restrict__ page_ids,
                                                            int32_t num_pages, const float* __restrict__ k_scale,
                                                            const float* __restrict__ v_scale,
                                                            uint16_t* __restrict__ out, int64_t ob, int64_t okv,
                                                            int64_t ot, int64_t oh) {
  constexpr int NB = D / 16;  // blocks per row
  const int i = blockIdx.x;
  if (i >= num_pages) return;
  const int64_t p = page_ids ? (int64_t)page_ids[i] : (int64_t)i;
  if (p < 0 || p >= pool.num_blocks) return;  // documented: ids outside the pool are skipped
  const int hkv = pool.hkv;
  const float gk = *k_scale;
  const float gv = *v_scale;
  // A lane owns half a block (8 elements: one code word and the block's
  // scale byte) and writes its 16 output bytes with one store, so a wave's
  // store covers 1 KB of consecutive output.
  constexpr int NH = 2 * NB;  // half blocks per row
  const int per_kv = pool.bs * hkv * NH;
  for (int w = threadIdx.x; w < 2 * per_kv; w += blockDim.x) {
    const int kv = w / per_kv;
    const int rem = w - kv * per_kv;
    const int hb = rem % NH;
    const int h = (rem / NH) % hkv;
    const int r = rem / (NH * hkv);
    const uint8_t* src = pool.data + p * pool.sb + kv * pool.skv + r * pool.st + h * pool.sh;
    uint32_t o[4];
    if constexpr (FMT == kNvfp4)
      dequant_half8(ld_u32(src + hb * 4), ld_u8(src + D / 2 + hb / 2), kv ? gv : gk, o);
    else
      dequant_fp8x8<FMT>(ld_u32x2(src + hb * 8), kv ? gv : gk, o);
    *reinterpret_cast<u32x4*>(out + p * ob + kv * okv + r * ot + h * oh + hb * 8) = u32x4{o[0], o[1], o[2], o[3]};
  }
}

template <int D>
__global__ __launch_bounds__(256) void qdq_kernel(uint16_t* __restrict__ key, int64_t k_st, int64_t k_sh,
                                                  uint16_t* __restrict__ value, int64_t v_st, int64_t v_sh,
                                                  int64_t num_tokens, int hkv, const float* __restrict__ k_scale,
                                                  const float* __restrict__ v_scale) {
  constexpr int LPR = D / 16;  // lanes per row
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / LPR;  // row = (t * 2 + kv) * hkv + h
  const int blk16 = (int)(gid % LPR);
  if (row >= num_tokens * 2 * hkv) return;
  const int h = (int)(row % hkv);
  const int kv = (int)((row / hkv) & 1);
  const int64_t t = row / (2 * (int64_t)hkv);
  uint16_t* p = (kv ? value + t * v_st + h * v_sh : key + t * k_st + h * k_sh) + blk16 * 16;
  u32x4* p4 = reinterpret_cast<u32x4*>(p);
  float x[16];
  bf16_block16(p4[0], p4[1], x);
  const float g = kv ? *v_scale : *k_scale;
  uint32_t w0, w1;
  const uint32_t s8 = quantize_block16(x, g, w0, w1);
  uint32_t o[8];
  dequant_block16(u32x2{w0, w1}, s8, g, o);
  p4[0] = u32x4{o[0], o[1], o[2], o[3]};
  p4[1] = u32x4{o[4], o[5], o[6], o[7]};
}

// FP8-E4M3 attention output -> bf16 [P40177 "Implementation breakdown" item
// 2: the forward pass dequantises the kernel's FP8 output back to the model
// dtype]. A lane converts 8 bytes: bf16 RNE of fp32(e4m3 * o_scale); the
// E4M3FN codes 0x7F and 0xFF are NaN.
__global__ __launch_bounds__(256) void fp8_to_bf16_kernel(const uint8_t* __restrict__ in, int64_t n8,
                                                          const float* __restrict__ o_scale,
                                                          uint16_t* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n8) return;
  const u32x2 w = ld_u32x2(in + gid * 8);
  const float os = *o_scale;
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t b0 = (w[k / 2] >> (16 * (k & 1))) & 0xFFu;
    const uint32_t b1 = (w[k / 2] >> (16 * (k & 1) + 8)) & 0xFFu;
    const float v0 = ((b0 & 0x7Fu) == 0x7Fu) ? __builtin_nanf("") : e4m3_to_f32(b0);
    const float v1 = ((b1 & 0x7Fu) == 0x7Fu) ? __builtin_nanf("") : e4m3_to_f32(b1);
    o[k] = pack_bf16x2(v0 * os, v1 * os);
  }
  *reinterpret_cast<u32x4*>(out + gid * 8) = u32x4{o[0], o[1], o[2], o[3]};
}

hipError_t launch_fp8_to_bf16(const void* in, int64_t n, const float* o_scale, void* out, hipStream_t stream) {
  const int64_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  fp8_to_bf16_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, stream>>>(static_cast<const uint8_t*>(in), n8, o_scale,
                                                                      static_cast<uint16_t*>(out));
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_dequant_pages_f(const Pool& pool, int head_size, const int32_t* page_ids, int32_t num_pages,
                                         const float* k_scale, const float* v_scale, void* out, int64_t ob,
                                         int64_t okv, int64_t ot, int64_t oh, hipStream_t stream) {
  if (num_pages == 0) return hipSuccess;
  uint16_t* o = static_cast<uint16_t*>(out);
  const dim3 grid((unsigned)num_pages);
  switch (head_size) {
    case 64:
      dequant_pages_kernel<64, FMT><<<grid, 256, 0, stream>>>(pool, page_ids, num_pages, k_scale, v_scale, o, ob, okv, ot, oh);
      break;
    case 128:
      dequant_pages_kernel<128, FMT><<<grid, 256, 0, stream>>>(pool, page_ids, num_pages, k_scale, v_scale, o, ob, okv, ot,
                                                          oh);
      break;
    case 256:
      dequant_pages_kernel<256, FMT><<<grid, 256, 0, stream>>>(pool, page_ids, num_pages, k_scale, v_scale, o, ob, okv, ot,
                                                          oh);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dequant_pages(const Pool& pool, int head_size, const int32_t* page_ids, int32_t num_pages,
                                const float* k_scale, const float* v_scale, void* out, int64_t ob, int64_t okv,
                                int64_t ot, int64_t oh, int fmt, hipStream_t stream) {
  switch (fmt) {
    case kNvfp4:
      return launch_dequant_pages_f<kNvfp4>(pool, head_size, page_ids, num_pages, k_scale, v_scale, out, ob, okv,
                                            ot, oh, stream);
    case kFp8E4M3:
      return launch_dequant_pages_f<kFp8E4M3>(pool, head_size, page_ids, num_pages, k_scale, v_scale, out, ob, okv,
                                              ot, oh, stream);
    case kFp8E5M2:
      return launch_dequant_pages_f<kFp8E5M2>(pool, head_size, page_ids, num_pages, k_scale, v_scale, out, ob, okv,
                                              ot, oh, stream);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_qdq(int head_size, void* key, int64_t k_st, int64_t k_sh, void* value, int64_t v_st, int64_t v_sh,
                      int64_t num_tokens, int num_kv_heads, const float* k_scale, const float* v_scale,
                      hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int64_t lanes = num_tokens * 2 * num_kv_heads * (head_size / 16);
  const dim3 grid((unsigned)((lanes + 255) / 256));
  uint16_t* k = static_cast<uint16_t*>(key);
  uint16_t* v = static_cast<uint16_t*>(value);
  switch (head_size) {
    case 64:
      qdq_kernel<64><<<grid, 256, 0, stream>>>(k, k_st, k_sh, v, v_st, v_sh, num_tokens, num_kv_heads, k_scale, v_scale);
      break;
    case 128:
      qdq_kernel<128><<<grid, 256, 0, stream>>>(k, k_st, k_sh, v, v_st, v_sh, num_tokens, num_kv_heads, k_scale,
                                                v_scale);
      break;
    case 256:
      qdq_kernel<256><<<grid, 256, 0, stream>>>(k, k_st, k_sh, v, v_st, v_sh, num_tokens, num_kv_heads, k_scale,
                                                v_scale);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nvfp4kv
