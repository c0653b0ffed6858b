// Paged dequantize [RFC47684 "Fix steps": nvfp4_kv_dequantize_paged].
//
// One workgroup per (page, sequence). A lane turns half a 16-element block
// (4 code bytes + the block's scale byte) into 8 bf16 values: codes -> f16
// with the hardware FP4 convert, times the E4M3 scale (exact in f16: at most
// 6 significant bits), widened to fp32, times g (one fp32 RNE multiply), then
// bf16 RNE. Consecutive lanes take consecutive halves of one output row, so
// the 16-byte stores and the 4-byte loads are coalesced. FP8 caches take the
// same lanes: 8 code bytes -> bf16_RNE(fp32(fp8) * g).
#include "quantize.hpp"
#include "launch.hpp"

namespace nvfp4kv {

template <int D, int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(Pool pool, const int32_t* __restrict__ block_table,
                                                      int32_t max_blocks, const int32_t* __restrict__ seq_lens,
                                                      const int32_t* __restrict__ cu_out, int32_t cap_len,
                                                      const float* __restrict__ k_scale,
                                                      const float* __restrict__ v_scale,
                                                      uint16_t* __restrict__ out_k, uint16_t* __restrict__ out_v,
                                                      int64_t out_rows) {
  constexpr int NB = D / 16;  // blocks per row
  const int b = blockIdx.y;
  const int p = blockIdx.x;
  const int bs = pool.bs;
  int L = seq_lens[b];
  L = L < 0 ? 0 : (L > cap_len ? cap_len : L);
  const int tok0 = p * bs;
  if (tok0 >= L) return;
  const int rows = (L - tok0) < bs ? (L - tok0) : bs;
  const int64_t blk = clamp_block(block_table[(int64_t)b * max_blocks + p], pool.num_blocks);
  const int hkv = pool.hkv;
  const int64_t out0 = (int64_t)cu_out[b] + tok0;
  const float gk = *k_scale;
  const float gv = *v_scale;
  // A lane owns half a block (8 elements: one code word and the block's
  // scale byte) and writes its 16 output bytes with one store, so a wave's
  // store covers 1 KB of consecutive output.
  constexpr int NH = 2 * NB;  // half blocks per row
  const int per_kv = rows * hkv * NH;
  for (int w = threadIdx.x; w < 2 * per_kv; w += blockDim.x) {
    const int kv = w / per_kv;
    const int rem = w - kv * per_kv;
    const int hb = rem % NH;
    const int h = (rem / NH) % hkv;
    const int r = rem / (NH * hkv);
    const int64_t orow = out0 + r;
    if (orow < 0 || orow >= out_rows) continue;
    const uint8_t* src = pool.data + blk * pool.sb + kv * pool.skv + r * pool.st + h * pool.sh;
    uint32_t o[4];
    if constexpr (FMT == kNvfp4)
      dequant_half8(ld_u32(src + hb * 4), ld_u8(src + D / 2 + hb / 2), kv ? gv : gk, o);
    else
      dequant_fp8x8<FMT>(ld_u32x2(src + hb * 8), kv ? gv : gk, o);
    uint16_t* dst = (kv ? out_v : out_k) + (orow * hkv + h) * D + hb * 8;
    *reinterpret_cast<u32x4*>(dst) = u32x4{o[0], o[1], o[2], o[3]};
  }
}

template <int FMT>
static hipError_t launch_dequant_f(const Pool& pool, int head_size, const int32_t* block_table, int32_t max_blocks,
                                   const int32_t* seq_lens, const int32_t* cu_out, int32_t num_seqs,
                                   int32_t max_seq_len, const float* k_scale, const float* v_scale, void* out_k,
                                   void* out_v, int64_t out_rows, hipStream_t stream) {
  if (num_seqs == 0 || max_seq_len <= 0) return hipSuccess;
  int64_t cap = (int64_t)max_blocks * pool.bs;
  if (cap > max_seq_len) cap = max_seq_len;
  const int pages = (int)((cap + pool.bs - 1) / pool.bs);
  if (pages == 0) return hipSuccess;
  const dim3 grid((unsigned)pages, (unsigned)num_seqs);
  uint16_t* ok = static_cast<uint16_t*>(out_k);
  uint16_t* ov = static_cast<uint16_t*>(out_v);
  switch (head_size) {
    case 64:
      dequant_kernel<64, FMT><<<grid, 256, 0, stream>>>(pool, block_table, max_blocks, seq_lens, cu_out, (int32_t)cap,
                                                   k_scale, v_scale, ok, ov, out_rows);
      break;
    case 128:
      dequant_kernel<128, FMT><<<grid, 256, 0, stream>>>(pool, block_table, max_blocks, seq_lens, cu_out, (int32_t)cap,
                                                    k_scale, v_scale, ok, ov, out_rows);
      break;
    case 256:
      dequant_kernel<256, FMT><<<grid, 256, 0, stream>>>(pool, block_table, max_blocks, seq_lens, cu_out, (int32_t)cap,
                                                    k_scale, v_scale, ok, ov, out_rows);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dequant(const Pool& pool, int head_size, const int32_t* block_table, int32_t max_blocks,
                          const int32_t* seq_lens, const int32_t* cu_out, int32_t num_seqs, int32_t max_seq_len,
                          const float* k_scale, const float* v_scale, void* out_k, void* out_v,
                          int64_t out_rows, int fmt, hipStream_t stream) {
  switch (fmt) {
    case kNvfp4:
      return launch_dequant_f<kNvfp4>(pool, head_size, block_table, max_blocks, seq_lens, cu_out, num_seqs,
                                      max_seq_len, k_scale, v_scale, out_k, out_v, out_rows, stream);
    case kFp8E4M3:
      return launch_dequant_f<kFp8E4M3>(pool, head_size, block_table, max_blocks, seq_lens, cu_out, num_seqs,
                                        max_seq_len, k_scale, v_scale, out_k, out_v, out_rows, stream);
    case kFp8E5M2:
      return launch_dequant_f<kFp8E5M2>(pool, head_size, block_table, max_blocks, seq_lens, cu_out, num_seqs,
                                        max_seq_len, k_scale, v_scale, out_k, out_v, out_rows, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace nvfp4kv
