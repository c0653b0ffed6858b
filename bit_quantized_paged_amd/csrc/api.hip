// extern "C" entry points of libnvfp4kv.so: argument validation, then one
// launcher call. Nothing here allocates or synchronises.
#include <stdarg.h>
#include <stdio.h>

#include "../../include/nvfp4kv.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

nvfp4kv_status fail(nvfp4kv_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

nvfp4kv_status ok() {
  g_err[0] = '\0';
  return NVFP4KV_OK;
}

nvfp4kv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(NVFP4KV_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

nvfp4kv_status check_cache(const nvfp4kv_cache* c, nvfp4kv::Pool& p, int* fmt = nullptr) {
  if (c == nullptr) return fail(NVFP4KV_INVALID_ARGUMENT, "cache descriptor is NULL");
  if (c->data == nullptr) return fail(NVFP4KV_INVALID_ARGUMENT, "cache data is NULL");
  if (c->kv_dtype != NVFP4KV_KV_NVFP4 && c->kv_dtype != NVFP4KV_KV_FP8_E4M3 && c->kv_dtype != NVFP4KV_KV_FP8_E5M2)
    return fail(NVFP4KV_INVALID_ARGUMENT, "cache.kv_dtype %d is not a cache format", c->kv_dtype);
  if (c->head_size != 64 && c->head_size != 128 && c->head_size != 256)
    return fail(NVFP4KV_UNSUPPORTED, "head_size %d not supported (64, 128, 256)", c->head_size);
  if (c->block_size != 16 && c->block_size != 32 && c->block_size != 64)
    return fail(NVFP4KV_UNSUPPORTED, "block_size %d not supported (16, 32, 64)", c->block_size);
  if (c->num_kv_heads < 1) return fail(NVFP4KV_INVALID_ARGUMENT, "num_kv_heads must be >= 1");
  if (c->num_blocks < 1) return fail(NVFP4KV_INVALID_ARGUMENT, "num_blocks must be >= 1");
  if ((int64_t)c->num_blocks * c->block_size > INT32_MAX)
    return fail(NVFP4KV_UNSUPPORTED, "num_blocks * block_size exceeds 2^31");
  if (!aligned(c->data, 16)) return fail(NVFP4KV_INVALID_ARGUMENT, "cache data must be 16-byte aligned");
  const int64_t s[4] = {c->stride_block, c->stride_kv, c->stride_token, c->stride_head};
  for (int k = 0; k < 4; ++k)
    if (s[k] < 0 || s[k] % 4 != 0)
      return fail(NVFP4KV_INVALID_ARGUMENT, "cache strides must be non-negative multiples of 4 bytes");
  if (c->kv_dtype != NVFP4KV_KV_NVFP4)
    for (int k = 0; k < 4; ++k)
      if (s[k] % 16 != 0)
        return fail(NVFP4KV_INVALID_ARGUMENT, "FP8 cache strides must be multiples of 16 bytes");
  // rows of a page are addressed with 32-bit offsets
  if (c->stride_token > (1 << 26)) return fail(NVFP4KV_UNSUPPORTED, "stride_token above 2^26 bytes");
  // the decode copies address a page's K and V rows from one 32-bit window
  if (c->stride_kv > (1 << 30)) return fail(NVFP4KV_UNSUPPORTED, "stride_kv above 2^30 bytes");
  p.data = c->data;
  p.num_blocks = c->num_blocks;
  p.sb = c->stride_block;
  p.skv = c->stride_kv;
  p.st = c->stride_token;
  p.sh = c->stride_head;
  p.bs = c->block_size;
  p.bs_log2 = c->block_size == 16 ? 4 : (c->block_size == 32 ? 5 : 6);
  p.hkv = c->num_kv_heads;
  if (fmt) *fmt = c->kv_dtype == NVFP4KV_KV_NVFP4 ? nvfp4kv::kNvfp4
                  : c->kv_dtype == NVFP4KV_KV_FP8_E4M3 ? nvfp4kv::kFp8E4M3 : nvfp4kv::kFp8E5M2;
  return ok();
}

nvfp4kv_status check_bf16_rows(const void* ptr, int64_t st, int64_t sh, const char* name) {
  if (ptr == nullptr) return fail(NVFP4KV_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned(ptr, 16)) return fail(NVFP4KV_INVALID_ARGUMENT, "%s must be 16-byte aligned", name);
  if (st < 0 || sh < 0 || st % 8 != 0 || sh % 8 != 0)
    return fail(NVFP4KV_INVALID_ARGUMENT, "%s strides must be non-negative multiples of 8 elements", name);
  return ok();
}

}  // namespace

extern "C" {

int32_t nvfp4_kv_full_dim(int32_t head_size) {
  if (head_size <= 0 || head_size % 16 != 0) return -1;
  return head_size / 2 + head_size / 16;
}

const char* nvfp4kv_status_string(nvfp4kv_status s) {
  switch (s) {
    case NVFP4KV_OK: return "ok";
    case NVFP4KV_INVALID_ARGUMENT: return "invalid argument";
    case NVFP4KV_UNSUPPORTED: return "unsupported";
    case NVFP4KV_WORKSPACE_TOO_SMALL: return "workspace too small";
    case NVFP4KV_HIP_ERROR: return "hip error";
    default: return "unknown status";
  }
}

const char* nvfp4kv_last_error(void) { return g_err; }

nvfp4kv_status nvfp4_kv_append(const nvfp4kv_cache* cache, const void* key, int64_t key_stride_token,
                               int64_t key_stride_head, const void* value, int64_t value_stride_token,
                               int64_t value_stride_head, const int64_t* slot_mapping, int64_t num_tokens,
                               const float* k_scale, const float* v_scale, void* stream) {
  nvfp4kv::Pool p;
  int fmt = 0;
  nvfp4kv_status s = check_cache(cache, p, &fmt);
  if (s) return s;
  if (num_tokens < 0) return fail(NVFP4KV_INVALID_ARGUMENT, "num_tokens must be >= 0");
  if (num_tokens == 0) return ok();
  if ((s = check_bf16_rows(key, key_stride_token, key_stride_head, "key"))) return s;
  if ((s = check_bf16_rows(value, value_stride_token, value_stride_head, "value"))) return s;
  if (slot_mapping == nullptr) return fail(NVFP4KV_INVALID_ARGUMENT, "slot_mapping is NULL");
  if (k_scale == nullptr || v_scale == nullptr) return fail(NVFP4KV_INVALID_ARGUMENT, "k_scale/v_scale is NULL");
  const int64_t lanes = nvfp4kv::append_lanes(num_tokens, p.hkv, cache->head_size);
  if (lanes / 256 >= (int64_t)INT32_MAX) return fail(NVFP4KV_UNSUPPORTED, "too many tokens for one call");
  return hip_status(nvfp4kv::launch_append(p, cache->head_size, key, key_stride_token, key_stride_head, value,
                                           value_stride_token, value_stride_head, slot_mapping, num_tokens,
                                           k_scale, v_scale, fmt, static_cast<hipStream_t>(stream)),
                    "nvfp4_kv_append launch");
}

nvfp4kv_status nvfp4_kv_dequant_paged(const nvfp4kv_cache* cache, const int32_t* block_table,
                                      int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                      const int32_t* cu_seqlens_out, int32_t num_seqs, int32_t max_seq_len,
                                      const float* k_scale, const float* v_scale, void* out_key,
                                      void* out_value, int64_t out_rows, void* stream) {
  nvfp4kv::Pool p;
  int fmt = 0;
  nvfp4kv_status s = check_cache(cache, p, &fmt);
  if (s) return s;
  if (num_seqs < 0 || num_seqs > 65535) return fail(NVFP4KV_INVALID_ARGUMENT, "num_seqs must be in [0, 65535]");
  if (num_seqs == 0 || max_seq_len <= 0 || out_rows <= 0) return ok();
  if (max_blocks_per_seq < 1) return fail(NVFP4KV_INVALID_ARGUMENT, "max_blocks_per_seq must be >= 1");
  if (!block_table || !seq_lens || !cu_seqlens_out) return fail(NVFP4KV_INVALID_ARGUMENT, "metadata pointer is NULL");
  if (!k_scale || !v_scale) return fail(NVFP4KV_INVALID_ARGUMENT, "k_scale/v_scale is NULL");
  if (!out_key || !out_value) return fail(NVFP4KV_INVALID_ARGUMENT, "output pointer is NULL");
  if (!aligned(out_key, 16) || !aligned(out_value, 16))
    return fail(NVFP4KV_INVALID_ARGUMENT, "outputs must be 16-byte aligned");
  return hip_status(nvfp4kv::launch_dequant(p, cache->head_size, block_table, max_blocks_per_seq, seq_lens,
                                            cu_seqlens_out, num_seqs, max_seq_len, k_scale, v_scale, out_key,
                                            out_value, out_rows, fmt, static_cast<hipStream_t>(stream)),
                    "nvfp4_kv_dequant_paged launch");
}

nvfp4kv_status nvfp4_kv_dequant_pages(const nvfp4kv_cache* cache, const int32_t* page_ids, int32_t num_pages,
                                      const float* k_scale, const float* v_scale, void* out,
                                      int64_t out_stride_block, int64_t out_stride_kv, int64_t out_stride_token,
                                      int64_t out_stride_head, void* stream) {
  nvfp4kv::Pool p;
  int fmt = 0;
  nvfp4kv_status s = check_cache(cache, p, &fmt);
  if (s) return s;
  if (num_pages < 0) return fail(NVFP4KV_INVALID_ARGUMENT, "num_pages must be >= 0");
  if (num_pages == 0) return ok();
  if (!k_scale || !v_scale) return fail(NVFP4KV_INVALID_ARGUMENT, "k_scale/v_scale is NULL");
  if (out == nullptr || !aligned(out, 16)) return fail(NVFP4KV_INVALID_ARGUMENT, "out must be a 16-byte aligned pointer");
  const int64_t st[4] = {out_stride_block, out_stride_kv, out_stride_token, out_stride_head};
  for (int64_t v : st)
    if (v < 0 || v % 8 != 0)
      return fail(NVFP4KV_INVALID_ARGUMENT, "out strides must be non-negative multiples of 8 elements");
  return hip_status(nvfp4kv::launch_dequant_pages(p, cache->head_size, page_ids, num_pages, k_scale, v_scale, out,
                                                  out_stride_block, out_stride_kv, out_stride_token, out_stride_head,
                                                  fmt, static_cast<hipStream_t>(stream)),
                    "nvfp4_kv_dequant_pages launch");
}

nvfp4kv_status nvfp4_kv_qdq(void* key, int64_t key_stride_token, int64_t key_stride_head, void* value,
                            int64_t value_stride_token, int64_t value_stride_head, int64_t num_tokens,
                            int32_t num_kv_heads, int32_t head_size, const float* k_scale, const float* v_scale,
                            void* stream) {
  if (head_size != 64 && head_size != 128 && head_size != 256)
    return fail(NVFP4KV_UNSUPPORTED, "head_size must be 64, 128 or 256");
  if (num_kv_heads < 1) return fail(NVFP4KV_INVALID_ARGUMENT, "num_kv_heads must be >= 1");
  if (num_tokens < 0) return fail(NVFP4KV_INVALID_ARGUMENT, "num_tokens must be >= 0");
  if (num_tokens == 0) return ok();
  nvfp4kv_status s;
  if ((s = check_bf16_rows(key, key_stride_token, key_stride_head, "key"))) return s;
  if ((s = check_bf16_rows(value, value_stride_token, value_stride_head, "value"))) return s;
  if (k_scale == nullptr || v_scale == nullptr) return fail(NVFP4KV_INVALID_ARGUMENT, "k_scale/v_scale is NULL");
  const int64_t lanes = num_tokens * 2 * num_kv_heads * (head_size / 16);
  if (lanes / 256 >= (int64_t)INT32_MAX) return fail(NVFP4KV_UNSUPPORTED, "too many tokens for one call");
  return hip_status(nvfp4kv::launch_qdq(head_size, key, key_stride_token, key_stride_head, value, value_stride_token,
                                        value_stride_head, num_tokens, num_kv_heads, k_scale, v_scale,
                                        static_cast<hipStream_t>(stream)),
                    "nvfp4_kv_qdq launch");
}

size_t nvfp4_paged_attention_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                   int32_t head_size) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
      head_size <= 0)
    return 0;
  return nvfp4kv::decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_size);
}

int32_t nvfp4_paged_attention_decode_plan(int32_t num_seqs, int32_t num_kv_heads, int32_t head_size,
                                          int32_t block_size, int32_t max_blocks_per_seq, int32_t max_seq_len,
                                          int32_t kv_dtype) {
  if (num_seqs < 0 || num_kv_heads < 1 || block_size < 1 || max_blocks_per_seq < 1) return -1;
  const int fmt = kv_dtype == NVFP4KV_KV_NVFP4      ? nvfp4kv::kNvfp4
                  : kv_dtype == NVFP4KV_KV_FP8_E4M3 ? nvfp4kv::kFp8E4M3
                  : kv_dtype == NVFP4KV_KV_FP8_E5M2 ? nvfp4kv::kFp8E5M2
                                                    : -1;
  if (fmt < 0) return -1;
  return nvfp4kv::decode_plan(num_seqs, num_kv_heads, head_size, block_size, max_blocks_per_seq, max_seq_len, fmt);
}

// Checks shared by the decode entry points (everything but the workspace).
static nvfp4kv_status decode_check(const nvfp4kv_cache* cache, const void* q, int64_t q_stride_token,
                                   int64_t q_stride_head, int32_t num_q_heads, const int32_t* block_table,
                                   int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                                   const float* k_scale, const float* v_scale, const void* out, nvfp4kv::Pool& p,
                                   int& fmt) {
  nvfp4kv_status s = check_cache(cache, p, &fmt);
  if (s) return s;
  if (num_seqs < 0 || num_seqs > nvfp4kv::kDecodeMaxSeqs)
    return fail(NVFP4KV_UNSUPPORTED, "num_seqs must be in [0, %d]", nvfp4kv::kDecodeMaxSeqs);
  if (num_q_heads < 1 || num_q_heads % p.hkv != 0)
    return fail(NVFP4KV_INVALID_ARGUMENT, "num_q_heads must be a positive multiple of num_kv_heads");
  const int grp = num_q_heads / p.hkv;
  if (grp > 16) return fail(NVFP4KV_UNSUPPORTED, "num_q_heads / num_kv_heads must be <= 16");
  if (num_seqs == 0) return ok();
  if ((s = check_bf16_rows(q, q_stride_token, q_stride_head, "q"))) return s;
  if (max_blocks_per_seq < 1) return fail(NVFP4KV_INVALID_ARGUMENT, "max_blocks_per_seq must be >= 1");
  if ((int64_t)max_blocks_per_seq * p.bs > INT32_MAX / 2)
    return fail(NVFP4KV_UNSUPPORTED, "max_blocks_per_seq * block_size too large");
  // the device schedule sums 32-key steps over the batch in 32-bit integers
  if ((int64_t)num_seqs * (((int64_t)max_blocks_per_seq * p.bs + 31) / 32) * p.hkv >= INT32_MAX)
    return fail(NVFP4KV_UNSUPPORTED, "num_seqs * max_blocks_per_seq * block_size too large for one call");
  if (!block_table || !seq_lens) return fail(NVFP4KV_INVALID_ARGUMENT, "metadata pointer is NULL");
  if (!k_scale || !v_scale) return fail(NVFP4KV_INVALID_ARGUMENT, "k_scale/v_scale is NULL");
  if (out == nullptr || !aligned(out, 16)) return fail(NVFP4KV_INVALID_ARGUMENT, "out must be a 16-byte aligned pointer");
  if (nvfp4kv::decode_lds_bytes(num_seqs, grp, cache->head_size, fmt) > 163840)
    return fail(NVFP4KV_UNSUPPORTED, "num_seqs / group size / head_size combination exceeds the LDS budget");
  return ok();
}

static nvfp4kv_status decode_impl(const nvfp4kv_cache* cache, const void* q, int64_t q_stride_token,
                                  int64_t q_stride_head, int32_t num_q_heads, const int32_t* block_table,
                                  int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                                  int32_t max_seq_len, const float* k_scale, const float* v_scale, float sm_scale,
                                  const float* o_scale, void* out, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  nvfp4kv::Pool p;
  int fmt = 0;
  nvfp4kv_status s = decode_check(cache, q, q_stride_token, q_stride_head, num_q_heads, block_table,
                                  max_blocks_per_seq, seq_lens, num_seqs, k_scale, v_scale, out, p, fmt);
  if (s || num_seqs == 0) return s;
  const size_t need = nvfp4kv::decode_workspace_bytes(num_seqs, num_q_heads, p.hkv, cache->head_size);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(NVFP4KV_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  if (!aligned(workspace, 16)) return fail(NVFP4KV_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  return hip_status(nvfp4kv::launch_decode(p, cache->head_size, q, q_stride_token, q_stride_head, num_q_heads,
                                           block_table, max_blocks_per_seq, seq_lens, num_seqs, max_seq_len,
                                           k_scale, v_scale, sm_scale, o_scale, out, workspace, fmt,
                                           static_cast<hipStream_t>(stream)),
                    "nvfp4_paged_attention_decode launch");
}

nvfp4kv_status nvfp4_paged_attention_decode(const nvfp4kv_cache* cache, const void* q, int64_t q_stride_token,
                                            int64_t q_stride_head, int32_t num_q_heads,
                                            const int32_t* block_table, int32_t max_blocks_per_seq,
                                            const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                                            const float* k_scale, const float* v_scale, float sm_scale,
                                            void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(cache, q, q_stride_token, q_stride_head, num_q_heads, block_table, max_blocks_per_seq, seq_lens,
                     num_seqs, max_seq_len, k_scale, v_scale, sm_scale, nullptr, out, workspace, workspace_bytes,
                     stream);
}

nvfp4kv_status nvfp4_paged_attention_decode_noalloc(const nvfp4kv_cache* cache, const void* q,
                                                    int64_t q_stride_token, int64_t q_stride_head,
                                                    int32_t num_q_heads, const int32_t* block_table,
                                                    int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                                    int32_t num_seqs, int32_t max_seq_len, const float* k_scale,
                                                    const float* v_scale, float sm_scale, void* out, void* stream) {
  nvfp4kv::Pool p;
  int fmt = 0;
  nvfp4kv_status s = decode_check(cache, q, q_stride_token, q_stride_head, num_q_heads, block_table,
                                  max_blocks_per_seq, seq_lens, num_seqs, k_scale, v_scale, out, p, fmt);
  if (s || num_seqs == 0) return s;
  if ((int64_t)num_seqs * p.hkv > nvfp4kv::kScratchCounters)
    return fail(NVFP4KV_WORKSPACE_TOO_SMALL, "num_seqs * num_kv_heads = %lld exceeds the %lld split counters of the "
                "library's decode scratch", (long long)num_seqs * p.hkv, (long long)nvfp4kv::kScratchCounters);
  const int64_t need = nvfp4kv::kScratchCounterBytes +
                       (int64_t)nvfp4kv::decode_partial_bytes(num_seqs, num_q_heads, p.hkv, cache->head_size);
  if (need > nvfp4kv::kScratchBytes)
    return fail(NVFP4KV_WORKSPACE_TOO_SMALL, "this batch needs %lld bytes of decode scratch; the library's array "
                "holds %lld (use nvfp4_paged_attention_decode with a workspace)", (long long)need,
                (long long)nvfp4kv::kScratchBytes);
  void* scratch = nullptr;
  hipError_t e = nvfp4kv::scratch_for_current_device(static_cast<hipStream_t>(stream), &scratch);
  if (e != hipSuccess) return hip_status(e, "nvfp4_paged_attention_decode_noalloc scratch set-up");
  return hip_status(nvfp4kv::launch_decode(p, cache->head_size, q, q_stride_token, q_stride_head, num_q_heads,
                                           block_table, max_blocks_per_seq, seq_lens, num_seqs, max_seq_len,
                                           k_scale, v_scale, sm_scale, nullptr, out, scratch, fmt,
                                           static_cast<hipStream_t>(stream), nvfp4kv::kScratchCounterBytes),
                    "nvfp4_paged_attention_decode_noalloc launch");
}

nvfp4kv_status nvfp4_paged_attention_decode_fp8(const nvfp4kv_cache* cache, const void* q, int64_t q_stride_token,
                                                int64_t q_stride_head, int32_t num_q_heads,
                                                const int32_t* block_table, int32_t max_blocks_per_seq,
                                                const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                                                const float* k_scale, const float* v_scale, float sm_scale,
                                                const float* o_scale, void* out_fp8, void* workspace,
                                                size_t workspace_bytes, void* stream) {
  if (o_scale == nullptr) return fail(NVFP4KV_INVALID_ARGUMENT, "o_scale is NULL");
  return decode_impl(cache, q, q_stride_token, q_stride_head, num_q_heads, block_table, max_blocks_per_seq, seq_lens,
                     num_seqs, max_seq_len, k_scale, v_scale, sm_scale, o_scale, out_fp8, workspace,
                     workspace_bytes, stream);
}

nvfp4kv_status nvfp4_fp8_to_bf16(const void* in, int64_t n, const float* o_scale, void* out, void* stream) {
  if (n < 0 || n % 8 != 0) return fail(NVFP4KV_INVALID_ARGUMENT, "n must be a non-negative multiple of 8");
  if (n == 0) return ok();
  if (in == nullptr || !aligned(in, 8)) return fail(NVFP4KV_INVALID_ARGUMENT, "in must be an 8-byte aligned pointer");
  if (out == nullptr || !aligned(out, 16))
    return fail(NVFP4KV_INVALID_ARGUMENT, "out must be a 16-byte aligned pointer");
  if (o_scale == nullptr) return fail(NVFP4KV_INVALID_ARGUMENT, "o_scale is NULL");
  return hip_status(nvfp4kv::launch_fp8_to_bf16(in, n, o_scale, out, static_cast<hipStream_t>(stream)),
                    "nvfp4_fp8_to_bf16 launch");
}

int64_t nvfp4_quant_activations_scale_bytes(int64_t m, int32_t k, int32_t swizzled) {
  if (m < 0 || k <= 0 || k % 16 != 0) return -1;
  const int64_t nc = k / 16;
  if (!swizzled) return m * nc;
  return ((m + 127) / 128) * 128 * ((nc + 3) / 4) * 4;
}

nvfp4kv_status nvfp4_quant_activations(const void* x, int64_t x_row_stride, int64_t m, int32_t k,
                                       const float* global_scale, int32_t swizzled, void* codes, void* scales,
                                       void* stream) {
  if (k <= 0 || k % 16 != 0) return fail(NVFP4KV_INVALID_ARGUMENT, "k must be a positive multiple of 16");
  if (m < 0) return fail(NVFP4KV_INVALID_ARGUMENT, "m must be >= 0");
  if (m == 0) return ok();
  if (m > INT32_MAX - 128) return fail(NVFP4KV_UNSUPPORTED, "m too large");
  if (x == nullptr || !aligned(x, 16)) return fail(NVFP4KV_INVALID_ARGUMENT, "x must be a 16-byte aligned pointer");
  if (x_row_stride < k || x_row_stride % 8 != 0)
    return fail(NVFP4KV_INVALID_ARGUMENT, "x_row_stride must be a multiple of 8 and >= k");
  if (global_scale == nullptr) return fail(NVFP4KV_INVALID_ARGUMENT, "global_scale is NULL");
  if (codes == nullptr || !aligned(codes, 4) || scales == nullptr || !aligned(scales, 4))
    return fail(NVFP4KV_INVALID_ARGUMENT, "codes and scales must be 4-byte aligned pointers");
  // one workgroup per 128 rows and 128 columns
  if (((m + 127) / 128) * ((k + 127) / 128) >= (int64_t)INT32_MAX)
    return fail(NVFP4KV_UNSUPPORTED, "m * k too large for one call");
  return hip_status(nvfp4kv::launch_act_quant(x, x_row_stride, (int32_t)m, k, global_scale, codes, scales,
                                              swizzled != 0, static_cast<hipStream_t>(stream)),
                    "nvfp4_quant_activations launch");
}

static nvfp4kv_status prefill_impl(const nvfp4kv_cache* cache, const void* q, int64_t q_stride_token,
                                             int64_t q_stride_head, int32_t num_q_heads,
                                             const int32_t* cu_seqlens_q, int32_t max_q_len, int32_t total_q,
                                             const int32_t* block_table, int32_t max_blocks_per_seq,
                                             const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                                             const float* k_scale, const float* v_scale, float sm_scale,
                                             int32_t causal, const float* o_scale, void* out, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  nvfp4kv::Pool p;
  int fmt = 0;
  nvfp4kv_status s = check_cache(cache, p, &fmt);
  if (s) return s;
  if (num_seqs < 0 || num_seqs > 65535) return fail(NVFP4KV_INVALID_ARGUMENT, "num_seqs must be in [0, 65535]");
  if (num_q_heads < 1 || num_q_heads % p.hkv != 0)
    return fail(NVFP4KV_INVALID_ARGUMENT, "num_q_heads must be a positive multiple of num_kv_heads");
  if (p.hkv > 65535) return fail(NVFP4KV_UNSUPPORTED, "num_kv_heads too large");
  if (max_q_len < 0 || total_q < 0) return fail(NVFP4KV_INVALID_ARGUMENT, "max_q_len and total_q must be >= 0");
  if (num_seqs == 0 || total_q == 0) return ok();
  if ((s = check_bf16_rows(q, q_stride_token, q_stride_head, "q"))) return s;
  if (max_blocks_per_seq < 1) return fail(NVFP4KV_INVALID_ARGUMENT, "max_blocks_per_seq must be >= 1");
  if ((int64_t)max_blocks_per_seq * p.bs > INT32_MAX / 2)
    return fail(NVFP4KV_UNSUPPORTED, "max_blocks_per_seq * block_size too large");
  if ((int64_t)max_q_len * (num_q_heads / p.hkv) > INT32_MAX / 2)
    return fail(NVFP4KV_UNSUPPORTED, "max_q_len too large");
  if (!cu_seqlens_q || !block_table || !seq_lens) return fail(NVFP4KV_INVALID_ARGUMENT, "metadata pointer is NULL");
  if (!k_scale || !v_scale) return fail(NVFP4KV_INVALID_ARGUMENT, "k_scale/v_scale is NULL");
  if (out == nullptr || !aligned(out, 16)) return fail(NVFP4KV_INVALID_ARGUMENT, "out must be a 16-byte aligned pointer");
  if (workspace == nullptr && workspace_bytes != 0)
    return fail(NVFP4KV_INVALID_ARGUMENT, "workspace is NULL but workspace_bytes is not 0");
  if (workspace != nullptr) {
    if (!aligned(workspace, 256)) return fail(NVFP4KV_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    if (workspace_bytes < nvfp4kv::prefill_workspace_bytes(cache->head_size))
      return fail(NVFP4KV_INVALID_ARGUMENT,
                  "workspace smaller than nvfp4_paged_attention_prefill_workspace_size(head_size)");
    if (num_seqs > nvfp4kv::kPrefillSplitSeqsMax)
      return fail(NVFP4KV_INVALID_ARGUMENT, "num_seqs must be <= 4096 with a workspace");
  }
  return hip_status(nvfp4kv::launch_prefill(p, cache->head_size, q, q_stride_token, q_stride_head, num_q_heads,
                                            cu_seqlens_q, max_q_len, total_q, block_table, max_blocks_per_seq,
                                            seq_lens, num_seqs, max_seq_len, k_scale, v_scale, sm_scale,
                                            causal ? 1 : 0, o_scale, out, fmt, workspace,
                                            static_cast<hipStream_t>(stream)),
                    "nvfp4_paged_attention_prefill launch");
}

size_t nvfp4_paged_attention_prefill_workspace_size(int32_t head_size) {
  if (head_size != 64 && head_size != 128 && head_size != 256) return 0;
  return nvfp4kv::prefill_workspace_bytes(head_size);
}

nvfp4kv_status nvfp4_paged_attention_prefill(const nvfp4kv_cache* cache, const void* q, int64_t q_stride_token,
                                             int64_t q_stride_head, int32_t num_q_heads,
                                             const int32_t* cu_seqlens_q, int32_t max_q_len, int32_t total_q,
                                             const int32_t* block_table, int32_t max_blocks_per_seq,
                                             const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                                             const float* k_scale, const float* v_scale, float sm_scale,
                                             int32_t causal, void* out, void* workspace, size_t workspace_bytes,
                                             void* stream) {
  return prefill_impl(cache, q, q_stride_token, q_stride_head, num_q_heads, cu_seqlens_q, max_q_len, total_q,
                      block_table, max_blocks_per_seq, seq_lens, num_seqs, max_seq_len, k_scale, v_scale, sm_scale,
                      causal, nullptr, out, workspace, workspace_bytes, stream);
}

nvfp4kv_status nvfp4_paged_attention_prefill_fp8(const nvfp4kv_cache* cache, const void* q, int64_t q_stride_token,
                                                 int64_t q_stride_head, int32_t num_q_heads,
                                                 const int32_t* cu_seqlens_q, int32_t max_q_len, int32_t total_q,
                                                 const int32_t* block_table, int32_t max_blocks_per_seq,
                                                 const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                                                 const float* k_scale, const float* v_scale, float sm_scale,
                                                 int32_t causal, const float* o_scale, void* out_fp8, void* workspace,
                                                 size_t workspace_bytes, void* stream) {
  if (o_scale == nullptr) return fail(NVFP4KV_INVALID_ARGUMENT, "o_scale is NULL");
  return prefill_impl(cache, q, q_stride_token, q_stride_head, num_q_heads, cu_seqlens_q, max_q_len, total_q,
                      block_table, max_blocks_per_seq, seq_lens, num_seqs, max_seq_len, k_scale, v_scale, sm_scale,
                      causal, o_scale, out_fp8, workspace, workspace_bytes, stream);
}

}  // extern "C"
