/*
 * nvfp4kv — NVFP4-quantised paged KV cache for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libnvfp4kv.so. Every buffer argument is a DEVICE pointer owned by
 * the caller; the library allocates nothing and keeps no state. Every call is
 * asynchronous and ordered on the given HIP stream (pass a hipStream_t as
 * `stream`; NULL means the default stream). Calls return a status; on a
 * non-zero status nothing was launched (argument errors) or a launch failed
 * (NVFP4KV_HIP_ERROR), and nvfp4kv_last_error() describes why.
 *
 * Sources of the operations (pages the method is described on):
 *   [P40177] "FlashInfer backend adds end-to-end NVFP4 KV cache support"
 *            (vLLM PR 40177 summary): "Key source snippets" —
 *            get_kv_cache_shape (pool shape, packed width D/2 + D/16),
 *            get_dtype_for_flashinfer (uint8 holding FP4 data and the FP8
 *            block scale), _create_nvfp4_hnd_kv_cache (slot-mapping writer
 *            with per-tensor kv scales, HND physical order);
 *            "Implementation breakdown" 1 and 3 (prefill/decode attention
 *            reading the packed cache and its block-scale view).
 *   [P39129] "Move NVFP4 GEMM management into NvFp4LinearKernel" (vLLM PR
 *            39129 report): NvFp4LinearLayerConfig docstring — two FP4
 *            values per byte, FP8-E4M3 scale per 16 elements, fp32 global
 *            scale.
 *   [RFC47684] "[RFC]: FlashInfer NVFP4 KV serving on pre-SM100 GPUs":
 *            "Cause analysis" / "Fix steps" — quantize-append with slot
 *            mapping and the paged dequantize of the fallback read path.
 *
 * Cache row format (readings of the pages, which print no bit layout): a
 * (token, kv head) row of head_size D elements is D/2 bytes of E2M1 codes
 * (element 2k in the low nibble of byte k, code = sign | e1 e0 | m) followed
 * by D/16 E4M3FN block scales (block j covers elements 16j..16j+15). An
 * element decodes as e2m1(code) * e4m3(scale) * g, with g the per-tensor
 * fp32 kv scale (k_scale for keys, v_scale for values).
 */
#ifndef NVFP4KV_H
#define NVFP4KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t nvfp4kv_status;
#define NVFP4KV_OK 0
#define NVFP4KV_INVALID_ARGUMENT 1   /* null pointer, bad size, bad stride */
#define NVFP4KV_UNSUPPORTED 2        /* shape the kernels are not built for */
#define NVFP4KV_WORKSPACE_TOO_SMALL 3
#define NVFP4KV_HIP_ERROR 4          /* a kernel launch failed */

/*
 * KV pool descriptor. Logical shape (num_blocks, 2, block_size,
 * num_kv_heads, full_dim) uint8 [P40177 get_kv_cache_shape]; index 0 of the
 * second axis holds keys, 1 values. Strides are in BYTES for the first four
 * axes; the last axis is contiguous. The HND physical order of [P40177
 * _create_nvfp4_hnd_kv_cache] (num_blocks, 2, num_kv_heads, block_size,
 * full_dim) is this descriptor with stride_token = full_dim and
 * stride_head = block_size * full_dim; NHD is stride_head = full_dim.
 * Requirements: data 16-byte aligned, every stride a multiple of 4,
 * stride_token <= 2^26 and stride_kv <= 2^30 bytes (NVFP4KV_UNSUPPORTED
 * otherwise).
 *
 * kv_dtype selects the row format [P40177 "Key source snippets": the
 * backend's KV cache dtypes list fp8_e4m3 and fp8_e5m2 beside nvfp4, and
 * get_dtype_for_flashinfer maps them to float8_e4m3fn, float8_e5m2 and
 * uint8]:
 *   NVFP4KV_KV_NVFP4: the packed row above, full_dim = D/2 + D/16;
 *   NVFP4KV_KV_FP8_E4M3 / _FP8_E5M2: D bytes, one OCP FP8 code per element
 *     (E4M3FN: bias 7, largest 448, 0x7F/0xFF NaN; E5M2: bias 15, largest
 *     57344), value fp8 * g. Every stride must then be a multiple of 16.
 *     Every entry point that takes a cache takes FP8 caches too.
 */
#define NVFP4KV_KV_NVFP4 0
#define NVFP4KV_KV_FP8_E4M3 1
#define NVFP4KV_KV_FP8_E5M2 2

typedef struct nvfp4kv_cache {
  uint8_t* data;
  int64_t num_blocks;
  int32_t block_size;     /* 16, 32 or 64 */
  int32_t num_kv_heads;
  int32_t head_size;      /* 64, 128 or 256 */
  int32_t kv_dtype;       /* NVFP4KV_KV_NVFP4 (0), _FP8_E4M3 (1) or _FP8_E5M2 (2) */
  int64_t stride_block;
  int64_t stride_kv;
  int64_t stride_token;
  int64_t stride_head;
} nvfp4kv_cache;

/* Packed row width in bytes: head_size/2 + head_size/16 [P40177
 * get_kv_cache_shape]; -1 if head_size is not a positive multiple of 16. */
int32_t nvfp4_kv_full_dim(int32_t head_size);

/*
 * Quantize-append with a slot mapping [P40177 _create_nvfp4_hnd_kv_cache;
 * RFC47684 "Fix steps": nvfp4_quantize_append_paged_kv_cache_with_slot_mapping].
 *
 * key, value: bf16 [num_tokens, num_kv_heads, head_size]; strides in
 *   ELEMENTS for the token and head axes (multiples of 8), last axis
 *   contiguous, 16-byte aligned base.
 * slot_mapping: int64 [num_tokens]; token t is written to block
 *   slot / block_size, row slot % block_size. Slots < 0 or >= num_blocks *
 *   block_size are skipped. Slots must be unique within a call.
 * k_scale, v_scale: device fp32 scalars g (finite, >= 2^-119 so that the
 *   reciprocal of every non-zero block step is finite), the dequantisation
 *   multipliers. Per 16-element block: s = E4M3_RNE_sat(amax / (6 g)),
 *   codes = E2M1_RNE_sat(x * (1 / (s g))), each step one fp32 RNE operation.
 *   FP8 caches: code = FP8_RNE(x / g) (one fp32 division), magnitudes from
 *   the format's largest finite value up saturating to it, sign kept.
 *   Key and value values must be finite or infinite, never NaN.
 * num_tokens == 0 is a no-op.
 */
nvfp4kv_status nvfp4_kv_append(const nvfp4kv_cache* cache,
                               const void* key, int64_t key_stride_token, int64_t key_stride_head,
                               const void* value, int64_t value_stride_token, int64_t value_stride_head,
                               const int64_t* slot_mapping, int64_t num_tokens,
                               const float* k_scale, const float* v_scale, void* stream);

/*
 * Paged dequantize [RFC47684 "Fix steps": nvfp4_kv_dequantize_paged]: every
 * sequence's keys and values, gathered through the block table, written as
 * bf16 rows. Sequence b's token j (j < seq_lens[b]) lives in block
 * block_table[b * max_blocks_per_seq + j / block_size], row j % block_size,
 * and is written to row cu_seqlens_out[b] + j of out_key / out_value
 * (bf16 [out_rows, num_kv_heads, head_size], contiguous). Values are
 * bf16_RNE(fp32(e2m1 * e4m3) * g).
 *
 * block_table: int32 [num_seqs, max_blocks_per_seq]; seq_lens: int32
 * [num_seqs]; cu_seqlens_out: int32 [num_seqs] (first output row per
 * sequence). max_seq_len: host upper bound of seq_lens (sizes the grid).
 * Device-side, lengths are clamped to min(max_seq_len, max_blocks_per_seq *
 * block_size), block ids to [0, num_blocks) and rows past out_rows are
 * dropped, so bad metadata yields wrong values, never an out-of-range access.
 */
nvfp4kv_status nvfp4_kv_dequant_paged(const nvfp4kv_cache* cache,
                                      const int32_t* block_table, int32_t max_blocks_per_seq,
                                      const int32_t* seq_lens, const int32_t* cu_seqlens_out,
                                      int32_t num_seqs, int32_t max_seq_len,
                                      const float* k_scale, const float* v_scale,
                                      void* out_key, void* out_value, int64_t out_rows, void* stream);

/*
 * Page-form dequantize [P40177 "Related context": the NVFP4 dequantization
 * kernels for Hopper / AMD Instinct; RFC47684 "Fix steps":
 * nvfp4_kv_dequantize_paged]: page p of the quantised cache becomes page p
 * of a bf16 cache of the same geometry, so one block table addresses both
 * (an attention kernel without FP4 support can then read the bf16 pages).
 * out[p][kv][t][h][d] = bf16_RNE(fp32(e2m1 * e4m3) * g), g = k_scale for
 * kv = 0 and v_scale for kv = 1: the values nvfp4_kv_dequant_paged returns.
 *
 * page_ids: device int32 [num_pages], the pages to convert (NULL converts
 *   pages 0 .. num_pages - 1); ids outside [0, num_blocks) are skipped.
 * out: caller-owned bf16 pages addressed as out + p * out_stride_block +
 *   kv * out_stride_kv + t * out_stride_token + h * out_stride_head + d
 *   (strides in ELEMENTS, non-negative multiples of 8; d contiguous;
 *   16-byte aligned). Pages not listed are left untouched.
 */
nvfp4kv_status nvfp4_kv_dequant_pages(const nvfp4kv_cache* cache, const int32_t* page_ids, int32_t num_pages,
                                      const float* k_scale, const float* v_scale, void* out,
                                      int64_t out_stride_block, int64_t out_stride_kv, int64_t out_stride_token,
                                      int64_t out_stride_head, void* stream);

/*
 * Quantize-dequantize emulation in place [P40177 "Related context": the QDQ
 * emulation kernels for Hopper / AMD Instinct]: every 16-element block of
 * every K and V row is quantised exactly as nvfp4_kv_append writes it and
 * replaced by the bf16 values nvfp4_kv_dequant_paged would return for it,
 * so a bf16 cache sees the same values an NVFP4 cache would hold.
 *
 * key, value: bf16 [num_tokens, num_kv_heads, head_size], strides in
 * ELEMENTS (non-negative multiples of 8), last axis contiguous, 16-byte
 * aligned; modified in place. Rows must not overlap (key and value must be
 * distinct memory). head_size: 64, 128 or 256.
 */
nvfp4kv_status nvfp4_kv_qdq(void* key, int64_t key_stride_token, int64_t key_stride_head,
                            void* value, int64_t value_stride_token, int64_t value_stride_head,
                            int64_t num_tokens, int32_t num_kv_heads, int32_t head_size,
                            const float* k_scale, const float* v_scale, void* stream);

/*
 * Workspace (bytes) that nvfp4_paged_attention_decode needs for a batch of
 * num_seqs sequences; it does not depend on the sequence lengths.
 */
size_t nvfp4_paged_attention_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                                   int32_t num_kv_heads, int32_t head_size);

/*
 * Which decode kernel nvfp4_paged_attention_decode launches for a batch of
 * these sizes on the current device (arguments as in that call):
 *   NVFP4KV_DECODE_PER_PAIR (1): one workgroup per (sequence, kv head) whose
 *     waves share the sequence's keys; no split-K, the workspace is not
 *     touched. Chosen when num_seqs * num_kv_heads is at least the device's
 *     compute-unit count and the longest sequence (max_seq_len, or
 *     max_blocks_per_seq * block_size when max_seq_len <= 0) needs at most 8
 *     steps of 32 keys per wave (waves per workgroup: NVFP4 12, 8 at
 *     head_size 256; FP8 12 at head_size 64, 8 at 128, 4 at 256).
 *   NVFP4KV_DECODE_SPLIT_K (0): every other batch; sequences are cut into
 *     units of about equal size, one per resident workgroup, and the last
 *     unit of a (sequence, kv head) to finish merges the others' partials.
 * kv_dtype: the cache's NVFP4KV_KV_* format. Returns -1 for a head_size
 * the library does not build or an unknown kv_dtype. Both kernels give
 * results within the same tolerance of the exact attention; bits may differ
 * between them.
 */
#define NVFP4KV_DECODE_SPLIT_K 0
#define NVFP4KV_DECODE_PER_PAIR 1
int32_t nvfp4_paged_attention_decode_plan(int32_t num_seqs, int32_t num_kv_heads, int32_t head_size,
                                          int32_t block_size, int32_t max_blocks_per_seq, int32_t max_seq_len,
                                          int32_t kv_dtype);

/*
 * Decode attention over the quantised pages [P40177 "Implementation
 * breakdown" 1 and 3; RFC47684 "Cause analysis": the paged read path].
 *
 * One query token per sequence, attending to all seq_lens[b] cached keys of
 * its sequence (the token's own key must already be appended). q head h
 * reads kv head h / (num_q_heads / num_kv_heads). Scores are
 * (q . k^) * sm_scale with k^ = e2m1 * e4m3 * k_scale; the output is
 * softmax(scores) . v^ with v^ = e2m1 * e4m3 * v_scale, rounded to bf16.
 *
 * q: bf16 [num_seqs, num_q_heads, head_size], strides in ELEMENTS (multiples
 *   of 8), last axis contiguous, 16-byte aligned. out: bf16 [num_seqs,
 *   num_q_heads, head_size] contiguous. A sequence with no key yields zeros.
 * num_q_heads / num_kv_heads must be an integer in [1, 16]; num_seqs <= 4096.
 * max_seq_len: host upper bound of seq_lens, used only to pick the kernel
 * and size the grid (a wrong value costs speed, not correctness); lengths
 * are clamped to max_blocks_per_seq * block_size on the device.
 * The result is deterministic: the same inputs give the same bits.
 * workspace: device scratch of at least
 *   nvfp4_paged_attention_decode_workspace_size(...) bytes, 16-byte aligned,
 *   ZERO-FILLED before its first use. It holds per-(sequence, kv head)
 *   arrival counters, at places that depend only on num_kv_heads, which
 *   every completed call leaves at zero again: one zero fill at allocation
 *   suffices for any later call with the same num_kv_heads and a batch the
 *   workspace is large enough for. Calls that share a workspace must be
 *   ordered on one stream. A workspace that breaks this contract gives wrong
 *   outputs, never an out-of-range access.
 */
nvfp4kv_status nvfp4_paged_attention_decode(const nvfp4kv_cache* cache,
                                            const void* q, int64_t q_stride_token, int64_t q_stride_head,
                                            int32_t num_q_heads,
                                            const int32_t* block_table, int32_t max_blocks_per_seq,
                                            const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                                            const float* k_scale, const float* v_scale, float sm_scale,
                                            void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode attention that allocates nothing and takes no workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same inputs,
 * kernels, output and contract as nvfp4_paged_attention_decode (bit-identical
 * results), except that the split-K counters and partials live in a
 * device-resident array the library owns: 32 MiB on each GPU it runs on,
 * set up by the first call on that GPU (which also clears its counters with
 * a kernel on `stream`) and held until the process ends. Counters occupy
 * the first 256 KiB (one per (sequence, kv head): num_seqs * num_kv_heads
 * must be <= 65536), partials the rest; a batch whose partials do not fit
 * (about 2048 + num_seqs * num_kv_heads slots of num_q_heads / num_kv_heads
 * * (head_size + 2) floats) returns NVFP4KV_WORKSPACE_TOO_SMALL and launches
 * nothing. Every call on one GPU shares that GPU's array and leaves its
 * counters at zero; calls that overlap on one GPU (other streams, other
 * host threads) race on it and give wrong results.
 */
nvfp4kv_status nvfp4_paged_attention_decode_noalloc(const nvfp4kv_cache* cache,
                                                    const void* q, int64_t q_stride_token, int64_t q_stride_head,
                                                    int32_t num_q_heads,
                                                    const int32_t* block_table, int32_t max_blocks_per_seq,
                                                    const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                                                    const float* k_scale, const float* v_scale, float sm_scale,
                                                    void* out, void* stream);

/*
 * Decode attention with FP8-E4M3 output [P40177 "Implementation breakdown"
 * item 2: the NVFP4 attention kernel emits FP8 into a preallocated buffer
 * and the forward pass dequantises it to the model dtype; "Risks and
 * impact": that adds a rounding step]. Same inputs, kernels and contract as
 * nvfp4_paged_attention_decode; instead of bf16 it writes, for each output
 * value y, the E4M3FN byte of RN32(y / o_scale) rounded to nearest even and
 * saturating at 448 (sign in bit 7). o_scale: device fp32 scalar (> 0).
 * out_fp8: uint8 [num_seqs, num_q_heads, head_size] contiguous, 16-byte
 * aligned. nvfp4_fp8_to_bf16 turns it back into bf16.
 */
nvfp4kv_status nvfp4_paged_attention_decode_fp8(const nvfp4kv_cache* cache,
                                                const void* q, int64_t q_stride_token, int64_t q_stride_head,
                                                int32_t num_q_heads,
                                                const int32_t* block_table, int32_t max_blocks_per_seq,
                                                const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                                                const float* k_scale, const float* v_scale, float sm_scale,
                                                const float* o_scale, void* out_fp8, void* workspace,
                                                size_t workspace_bytes, void* stream);

/*
 * The FP8 output's epilogue [P40177 "Implementation breakdown" item 2]:
 * out[i] = bf16_RNE(fp32(e4m3(in[i]) * o_scale)); the E4M3FN NaN codes 0x7F
 * and 0xFF give NaN. in: n bytes, 8-byte aligned; out: bf16 [n], 16-byte
 * aligned; n a multiple of 8.
 */
nvfp4kv_status nvfp4_fp8_to_bf16(const void* in, int64_t n, const float* o_scale, void* out, void* stream);

/*
 * Workspace (bytes) that nvfp4_paged_attention_prefill (and _fp8) needs for
 * the key split on the current device: arrival counters and two part
 * records for each workgroup the device holds at once. It depends only on
 * the device and head_size (0 for a head size the library does not build).
 */
size_t nvfp4_paged_attention_prefill_workspace_size(int32_t head_size);

/*
 * Chunked-prefill attention over the quantised pages [P40177
 * "Implementation breakdown" 1 and 3]. Sequence b has q_b = cu_seqlens_q[b+1]
 * - cu_seqlens_q[b] new query tokens, the last q_b of its seq_lens[b]
 * tokens; its keys and values (including the new chunk) must already be
 * appended. With causal != 0 query i of the chunk sees keys
 * j <= seq_lens[b] - q_b + i (bottom-right alignment), otherwise all keys.
 * Same scores, softmax and GQA mapping as decode.
 *
 * q: bf16 [total_q, num_q_heads, head_size] (element strides, multiples of
 *   8, last axis contiguous); cu_seqlens_q: int32 [num_seqs + 1];
 *   max_q_len: host hint of the largest q_b, used only to size the grid
 *   (workgroups loop over the column tiles of the actual q_b, so a wrong
 *   value, even 0, costs speed, not correctness); rows past total_q are
 *   neither read nor written. out: bf16 [total_q, num_q_heads,
 *   head_size] contiguous.
 * workspace: NULL (workspace_bytes 0) runs one workgroup per (sequence,
 *   column block of the chunk, kv head), each over all the keys its
 *   columns see. Otherwise device scratch of at least
 *   nvfp4_paged_attention_prefill_workspace_size(head_size) bytes, 256-byte
 *   aligned, ZERO-FILLED before its first use, with num_seqs <= 4096: the
 *   launch then has one workgroup per resident slot, each taking an equal
 *   share of all the jobs' 32-key steps, and a job cut between workgroups
 *   is merged by its last part to finish (its arrival counter, in the
 *   workspace, is left at zero again, so one zero fill suffices). Calls that
 *   share a workspace must be ordered on one stream. Both forms are
 *   deterministic and agree within the attention tolerance; their bits may
 *   differ. A bad workspace argument returns NVFP4KV_INVALID_ARGUMENT.
 */
nvfp4kv_status nvfp4_paged_attention_prefill(const nvfp4kv_cache* cache,
                                             const void* q, int64_t q_stride_token, int64_t q_stride_head,
                                             int32_t num_q_heads, const int32_t* cu_seqlens_q,
                                             int32_t max_q_len, int32_t total_q,
                                             const int32_t* block_table, int32_t max_blocks_per_seq,
                                             const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                                             const float* k_scale, const float* v_scale, float sm_scale,
                                             int32_t causal, void* out,
                                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Chunked-prefill attention with FP8-E4M3 output [P40177 "Implementation
 * breakdown" item 2]: same inputs, kernel and contract as
 * nvfp4_paged_attention_prefill, writing the E4M3FN byte of RN32(y /
 * o_scale) (round to nearest even, saturating at 448, sign in bit 7) for
 * each output value y, like nvfp4_paged_attention_decode_fp8. out_fp8:
 * uint8 [total_q, num_q_heads, head_size] contiguous, 16-byte aligned.
 */
nvfp4kv_status nvfp4_paged_attention_prefill_fp8(const nvfp4kv_cache* cache,
                                                 const void* q, int64_t q_stride_token, int64_t q_stride_head,
                                                 int32_t num_q_heads,
                                                 const int32_t* cu_seqlens_q, int32_t max_q_len, int32_t total_q,
                                                 const int32_t* block_table, int32_t max_blocks_per_seq,
                                                 const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                                                 const float* k_scale, const float* v_scale, float sm_scale,
                                                 int32_t causal, const float* o_scale, void* out_fp8,
                                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * NVFP4 quantisation of an activation matrix [P39129 "Implementation
 * breakdown": the FP4 linear kernels call scaled_fp4_quant(x,
 * input_global_scale_inv, is_sf_swizzled_layout=True) on their input, and
 * swizzle_blockscale rearranges block scales into the GEMM's layout]. The
 * block codec is nvfp4_kv_append's: per 16 consecutive elements of a row,
 * s = E4M3(amax / (6 g)) and code_i = E2M1(x_i / (s g)), with g the
 * global_scale (the dequantisation multiplier, x ~ e2m1 * s * g).
 *
 * x: bf16 [m, k], row stride x_row_stride ELEMENTS (a multiple of 8, >= k),
 *   16-byte aligned; k a positive multiple of 16.
 * global_scale: device fp32 scalar (finite, >= 2^-119); x holds no NaN.
 * codes: uint8 [m, k/2] contiguous, 4-byte aligned; element 2i of a row in
 *   the low nibble of byte i.
 * scales: uint8, 4-byte aligned, nvfp4_quant_activations_scale_bytes(m, k,
 *   swizzled) bytes. swizzled = 0: row-major [m, k/16]. swizzled = 1: the
 *   128 x 4 tile layout of block-scaled FP4 GEMM operands: the [m, k/16]
 *   scale matrix padded with zeros to R = 128 * ceil(m / 128) rows and
 *   C = 4 * ceil(k / 64) columns; the scale of row r, column c sits at byte
 *   512 * ((r / 128) * (C / 4) + c / 4) + 16 * (r % 32) + 4 * ((r % 128) / 32)
 *   + c % 4. Every byte of the buffer, padding included, is written.
 * m = 0 is a no-op.
 */
nvfp4kv_status nvfp4_quant_activations(const void* x, int64_t x_row_stride, int64_t m, int32_t k,
                                       const float* global_scale, int32_t swizzled, void* codes, void* scales,
                                       void* stream);

/* Bytes of the scale buffer nvfp4_quant_activations writes (-1 for bad m, k). */
int64_t nvfp4_quant_activations_scale_bytes(int64_t m, int32_t k, int32_t swizzled);

/* Human-readable name of a status code (static string). */
const char* nvfp4kv_status_string(nvfp4kv_status status);

/* Message of the last failing call on this host thread ("" if none). */
const char* nvfp4kv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4KV_H */
