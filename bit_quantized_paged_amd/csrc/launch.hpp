// Host-side launchers of the HIP kernels (one per operation); the C ABI in
// api.hip validates arguments and calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "device_common.hpp"

namespace nvfp4kv {

// `fmt` below is the cache format: kNvfp4, kFp8E4M3 or kFp8E5M2.

// Lanes of an append launch: tiles of kAppendTile tokens, K and V of every
// kv head, one lane per 16 elements.
constexpr int kAppendTile = 16;
inline int64_t append_lanes(int64_t num_tokens, int hkv, int head_size) {
  return (num_tokens + kAppendTile - 1) / kAppendTile * kAppendTile * 2 * hkv * (head_size / 16);
}
hipError_t launch_append(const Pool& pool, int head_size, const void* key, int64_t k_st, int64_t k_sh,
                         const void* value, int64_t v_st, int64_t v_sh, const int64_t* slots,
                         int64_t num_tokens, const float* k_scale, const float* v_scale, int fmt,
                         hipStream_t stream);

hipError_t launch_dequant(const Pool& pool, int head_size, const int32_t* block_table, int32_t max_blocks,
                          const int32_t* seq_lens, const int32_t* cu_out, int32_t num_seqs, int32_t max_seq_len,
                          const float* k_scale, const float* v_scale, void* out_k, void* out_v,
                          int64_t out_rows, int fmt, hipStream_t stream);

hipError_t launch_dequant_pages(const Pool& pool, int head_size, const int32_t* page_ids, int32_t num_pages,
                                const float* k_scale, const float* v_scale, void* out, int64_t ob, int64_t okv,
                                int64_t ot, int64_t oh, int fmt, hipStream_t stream);

hipError_t launch_qdq(int head_size, void* key, int64_t k_st, int64_t k_sh, void* value, int64_t v_st, int64_t v_sh,
                      int64_t num_tokens, int num_kv_heads, const float* k_scale, const float* v_scale,
                      hipStream_t stream);

// Largest batch of one decode call.
constexpr int kDecodeMaxSeqs = 4096;

// Decode workspace: [arrival counters][partial outputs][partial (max, sum)].
// The counter region takes counter_region_bytes (by default 4096 sequences'
// worth for num_kv_heads, a place that depends only on num_kv_heads); the
// partials need decode_partial_bytes after it.
size_t decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_size);
size_t decode_partial_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_size);

hipError_t launch_decode(const Pool& pool, int head_size, const void* q, int64_t q_st, int64_t q_sh,
                         int num_q_heads, const int32_t* block_table, int32_t max_blocks,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len, const float* k_scale,
                         const float* v_scale, float sm_scale, const float* o_scale, void* out, void* workspace,
                         int fmt, hipStream_t stream, int64_t counter_region_bytes = -1);

// The library-owned decode scratch of nvfp4_paged_attention_decode_noalloc:
// kScratchCounterBytes of arrival counters (one per (sequence, kv head),
// index b * num_kv_heads + h < kScratchCounters), then the partials, in all
// at most kScratchBytes. scratch_for_current_device returns its address on
// the current device, set up on the first call there (counters cleared by a
// kernel on `stream`).
constexpr int64_t kScratchBytes = 32ll << 20;
constexpr int64_t kScratchCounters = 65536;
constexpr int64_t kScratchCounterBytes = kScratchCounters * 4;
hipError_t scratch_for_current_device(hipStream_t stream, void** ptr);

// FP8-E4M3 bytes -> bf16: bf16 RNE of fp32(e4m3 * o_scale); n a multiple of 8.
hipError_t launch_fp8_to_bf16(const void* in, int64_t n, const float* o_scale, void* out, hipStream_t stream);
hipError_t launch_act_quant(const void* x, int64_t x_row_stride, int32_t m, int32_t k, const float* global_scale,
                            void* codes, void* scales, bool swizzled, hipStream_t stream);

// Decode kernel a call with these sizes launches on the current device:
// 1 = one workgroup per (sequence, kv head), 0 = split-K, -1 = bad head size.
int decode_plan(int num_seqs, int num_kv_heads, int head_size, int block_size, int max_blocks, int max_seq_len,
                int fmt);

// Dynamic LDS bytes of the decode split kernel (must stay within 160 KiB).
size_t decode_lds_bytes(int num_seqs, int grp, int head_size, int fmt);

hipError_t launch_prefill(const Pool& pool, int head_size, const void* q, int64_t q_st, int64_t q_sh,
                          int num_q_heads, const int32_t* cu_q, int32_t max_q_len, int32_t total_q,
                          const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                          int32_t num_seqs, int32_t max_seq_len, const float* k_scale, const float* v_scale,
                          float sm_scale, int causal, const float* o_scale, void* out, int fmt, void* workspace,
                          hipStream_t stream);

// Workspace bytes of the key-split prefill on the current device (0 for a
// head size the library does not build).
size_t prefill_workspace_bytes(int head_size);

// Sequences a key-split prefill launch takes at most.
constexpr int kPrefillSplitSeqsMax = 4096;

}  // namespace nvfp4kv
