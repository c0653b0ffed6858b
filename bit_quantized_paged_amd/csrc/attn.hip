// Paged attention over the NVFP4 cache: split-K decode (the split merge is
// done by the last-arriving workgroup of each sequence) and chunked prefill [P40177 "Implementation breakdown" 1 and 3; RFC47684
// "Cause analysis": the paged read path].
#include <atomic>
#include <map>
#include <mutex>

#include "attn_core.hpp"
#include "launch.hpp"

namespace nvfp4kv {

// ---------------------------------------------------------------------------
// Decode schedule. A unit is (sequence, split, kv head); a sequence of s
// 32-key steps has ceil(s / tps) splits that share its steps evenly. tps is
// chosen on the device from the actual lengths so
// that the batch yields about `target` units of equal size (target = the
// number of decode workgroups the GPU holds at once, so that all units run in
// a single round), which keeps
// ragged batches balanced without a host round trip. Every workgroup derives
// the same schedule: per-sequence unit counts and their exclusive prefix sum
// in LDS.
// ---------------------------------------------------------------------------
constexpr int kDecodeTargetMax = 2048;  // upper bound of `target` (sizes the workspace)
constexpr int kDecodeMinTps = 4;
constexpr int kStep = 32;
constexpr int kMergeCols = 8;  // columns merged per LDS round

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

// Agent-scope (all XCDs) coherent store / load of a split-K partial.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's stores have completed (s_waitcnt vmcnt(0)); the
// signal fences keep the compiler from moving memory operations across it.
__device__ __forceinline__ void wait_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d);
    if (lane >= d) v += t;
  }
  return v;
}

// Block-wide exclusive scan (NW waves); also returns the total.
template <int NW>
__device__ __forceinline__ int block_excl_scan(int v, int* s_red, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) s_red[w] = incl;
  __syncthreads();
  int off = 0;
  total = 0;
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    const int t = s_red[k];
    off += (k < w) ? t : 0;
    total += t;
  }
  __syncthreads();
  return incl - v + off;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// The schedule of a batch of at most 64 sequences, built by wave 0 alone
// (lane b holds sequence b) with wave-level scans; the other waves wait at
// one barrier. Same result as the block-wide version below.
__device__ void decode_schedule_small(const int32_t* __restrict__ seq_lens, int B, int cap, int hkv, int target,
                                      int* s_pref, int* s_len, int& total_units) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int L = lane < B ? clamp_len(seq_lens[lane], cap) : 0;
    const int st = ceil_div(L, kStep);
    const int total_steps = wave_sum_i(st);
    const int64_t work = (int64_t)total_steps * hkv;
    int t = (int)((work + target - 1) / target);
    int tps = t < kDecodeMinTps ? kDecodeMinTps : t;
    auto units = [&](int tt) { return lane < B ? max(1, ceil_div(st, tt)) : 0; };
    int total = wave_sum_i(units(tps));
    if ((int64_t)total * hkv > target && (int64_t)B * hkv <= target && total_steps > tps) {
      int lo = tps, hi = total_steps;  // lo does not fit, hi fits
      while (hi - lo > 1) {
        const int mid = lo + (hi - lo) / 2;
        if ((int64_t)wave_sum_i(units(mid)) * hkv <= target) hi = mid;
        else lo = mid;
      }
      tps = hi;
      total = wave_sum_i(units(tps));
    }
    const int n = units(tps);
    const int incl = wave_incl_scan(n);
    if (lane < B) {
      s_len[lane] = L;
      s_pref[lane] = incl - n;
    }
    if (lane == 0) s_pref[B] = total;
  }
  __syncthreads();
  total_units = s_pref[B];
}

// s_pref[b] = first unit (per head) of sequence b, s_pref[B] = units per head.
template <int NW>
__device__ void decode_schedule(const int32_t* __restrict__ seq_lens, int B, int cap, int hkv, int target,
                                int* s_pref, int* s_len, int* s_red, int& tps, int& total_units) {
  const int per = ceil_div(B, 64 * NW);
  const int b0 = threadIdx.x * per;
  const int b1 = (b0 + per < B) ? b0 + per : B;
  int steps_local = 0;
  for (int b = b0; b < b1; ++b) {
    const int L = clamp_len(seq_lens[b], cap);
    const int s = ceil_div(L, kStep);
    s_len[b] = L;
    s_pref[b] = s;
    steps_local += s;
  }
  int total_steps;
  (void)block_excl_scan<NW>(steps_local, s_red, total_steps);
  const int64_t work = (int64_t)total_steps * hkv;
  int t = (int)((work + target - 1) / target);
  tps = t < kDecodeMinTps ? kDecodeMinTps : t;
  // units (per kv head) at t steps per unit; a sequence without keys still
  // gets one (empty) unit, which writes zeros
  auto units_at = [&](int tt, int& run_out) {
    int loc = 0;
    for (int b = b0; b < b1; ++b) loc += max(1, ceil_div(s_pref[b], tt));
    int tot;
    run_out = block_excl_scan<NW>(loc, s_red, tot);
    return tot;
  };
  int run;
  int total = units_at(tps, run);
  // Short sequences round their unit counts up, so the even share can yield
  // more units than workgroups, and a second round then doubles some
  // workgroups' work. Take instead the smallest unit size whose units fit one
  // round (binary search; at total_steps every sequence is one unit, which
  // fits whenever the batch alone does).
  if ((int64_t)total * hkv > target && (int64_t)B * hkv <= target && total_steps > tps) {
    int lo = tps, hi = total_steps;  // lo does not fit, hi fits
    while (hi - lo > 1) {
      const int mid = lo + (hi - lo) / 2;
      int r;
      if ((int64_t)units_at(mid, r) * hkv <= target) hi = mid;
      else lo = mid;
    }
    tps = hi;
    total = units_at(tps, run);
  }
  for (int b = b0; b < b1; ++b) {
    const int n = max(1, ceil_div(s_pref[b], tps));
    s_pref[b] = run;
    run += n;
  }
  if (threadIdx.x == 0) s_pref[B] = total;
  total_units = total;
  __syncthreads();
}

__device__ __forceinline__ float uniform_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

struct DecodeArgs {
  Pool pool;
  const uint16_t* q;
  int64_t q_st, q_sh;
  int hq, grp;
  const int32_t* bt;
  int32_t max_blocks;
  const int32_t* seq_lens;
  int B;
  const float* k_scale;
  const float* v_scale;
  float sm_scale;
  uint16_t* out;           // bf16 output [B, hq, D] (when o_scale is null)
  uint8_t* out8;           // FP8-E4M3 output [B, hq, D] (when o_scale is set)
  const float* o_scale;    // per-tensor FP8 output scale, or null for bf16 output
  uint32_t* ws_cnt;  // [B * hkv] arrival counters; zero between calls
  float* ws_o;       // [slot][grp][D]   normalised partial outputs
  float* ws_ml;      // [slot][grp][2]   (max, sum) of each partial, base-2 scores
  int target;        // units the schedule aims for (<= kDecodeTargetMax)
};

// Attention output element idx (of [B, hq, D]) with value y: bf16 RNE, or
// with an output scale os the FP8-E4M3 byte of RN32(y / os), round to
// nearest even, saturating at 448, sign in bit 7 [P40177 "Implementation
// breakdown" item 2: the FP8 output of the NVFP4 attention kernel].
__device__ __forceinline__ uint32_t fp8_e4m3_out(float y, float os) {
  const float q = __fdiv_rn(y, os);
  return e4m3_from_f32_sat(__builtin_fabsf(q)) | ((__float_as_uint(q) >> 24) & 0x80u);
}
// Output elements idx .. idx + 3 (idx a multiple of 4) with values y * g.
__device__ __forceinline__ void store_out4(const DecodeArgs& a, float os, int64_t idx, f4 y, float g) {
  if (a.o_scale)
    *reinterpret_cast<uint32_t*>(a.out8 + idx) = fp8_e4m3_out(y[0] * g, os) | (fp8_e4m3_out(y[1] * g, os) << 8) |
                                                 (fp8_e4m3_out(y[2] * g, os) << 16) |
                                                 (fp8_e4m3_out(y[3] * g, os) << 24);
  else
    *reinterpret_cast<u32x2*>(a.out + idx) = u32x2{pack_bf16x2(y[0] * g, y[1] * g), pack_bf16x2(y[2] * g, y[3] * g)};
}

// LDS ints of the schedule: unit prefix [B + 1] and clamped lengths [B],
// each padded to 16 bytes.
__host__ __device__ inline int decode_lds_pref_ints(int B) { return ((B + 1 + 3) / 4) * 4 + ((B + 3) / 4) * 4; }

__device__ __forceinline__ float wave_max64(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// 16 agent-coherent bytes at byte offset `off` from the wave-uniform base.
__device__ __forceinline__ f4 ld_agent4(const float* base, uint32_t off) {
  const rsrc_t r = make_rsrc(reinterpret_cast<const uint8_t*>(base), 0x7FFFFFFF);
  return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16 /* sc1 */));
}
// The agent-coherent (sc1, written through to the device's coherence point)
// store of 16 bytes at byte offset `off` from the wave-uniform base.
__device__ __forceinline__ void st_agent4(float* base, uint32_t off, f4 v) {
  const rsrc_t r = make_rsrc(reinterpret_cast<const uint8_t*>(base), 0x7FFFFFFF);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 16 /* sc1 */);
}

// Merge the n partial results of (b, h) (slots slot0, slot0 + hkv, ...) into
// the output with log-sum-exp weights. Every thread owns 4 consecutive
// outputs of one column and merges the splits itself, kSplitBatch at a time
// with an online maximum: the (max, sum) pairs and the partial outputs of a
// batch are all requested before any is used, so a batch costs one round trip
// to the agent-coherent level, not one per load.
constexpr int kSplitBatch = 16;

template <int D, int NW>
__device__ void combine_splits(const DecodeArgs& a, int b, int h, int64_t slot0, int n) {
  const int hkv = a.pool.hkv;
  const int grp = a.grp;
  const float gv = *a.v_scale;
  const float os = a.o_scale ? *a.o_scale : 1.0f;
  const int64_t out0 = ((int64_t)b * a.hq + h * grp) * D;
  constexpr int D4 = D / 4;
  for (int e = threadIdx.x; e < grp * D4; e += 64 * NW) {
    const int col = e / D4;
    const int d4 = e - col * D4;
    const uint32_t off = (uint32_t)((col * D + 4 * d4) * 4);
    float M = -__builtin_inff(), lt = 0.0f;
    f4 o = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n; s0 += kSplitBatch) {
      float m[kSplitBatch], l[kSplitBatch];
      f4 v[kSplitBatch];
#pragma unroll
      for (int u = 0; u < kSplitBatch; ++u) {
        const int s = s0 + u < n ? s0 + u : n - 1;  // clamped: past-the-end entries are dropped below
        const int64_t slot = slot0 + (int64_t)s * hkv;
        const float* ml = a.ws_ml + (slot * grp + col) * 2;
        m[u] = ld_agent(ml);
        l[u] = ld_agent(ml + 1);
        v[u] = ld_agent4(a.ws_o + slot * grp * D, off);
      }
      float bm = M;
#pragma unroll
      for (int u = 0; u < kSplitBatch; ++u) bm = (s0 + u < n) ? __builtin_fmaxf(bm, m[u]) : bm;
      // rescale what is merged so far to the batch's maximum, then add the batch
      const float r = (M == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(M - bm);
      lt *= r;
      o *= r;
#pragma unroll
      for (int u = 0; u < kSplitBatch; ++u) {
        const float f = (s0 + u < n && m[u] != -__builtin_inff()) ? __builtin_amdgcn_exp2f(m[u] - bm) * l[u] : 0.0f;
        lt += f;
        o += f * v[u];
      }
      M = bm;
    }
    const float sc = (lt > 0.0f ? 1.0f / lt : 0.0f) * gv;
    const int64_t idx = out0 + col * D + 4 * d4;
    if (a.o_scale) {
      *reinterpret_cast<uint32_t*>(a.out8 + idx) =
          fp8_e4m3_out(o[0] * sc, os) | (fp8_e4m3_out(o[1] * sc, os) << 8) | (fp8_e4m3_out(o[2] * sc, os) << 16) |
          (fp8_e4m3_out(o[3] * sc, os) << 24);
    } else {
      uint32_t* dst = reinterpret_cast<uint32_t*>(a.out + idx);
      dst[0] = pack_bf16x2(o[0] * sc, o[1] * sc);
      dst[1] = pack_bf16x2(o[2] * sc, o[3] * sc);
    }
  }
}

// How a decode kernel streams pages into its per-wave ring of NS LDS stages
// (see attn_core.hpp):
//  kModeDmaCompact: NVFP4, contiguous 16-byte aligned rows: 16-byte
//    global->LDS copies;
//  kModeDmaGeneral: NVFP4, any row stride: 4-byte global->LDS copies;
//  kModeFp8E4M3, kModeFp8E5M2: FP8 rows (16-byte strides): 16-byte copies.
constexpr int kModeDmaGeneral = 0;
constexpr int kModeDmaCompact = 1;
constexpr int kModeFp8E4M3 = 2;
constexpr int kModeFp8E5M2 = 3;

constexpr int mode_fmt(int mode) {
  return mode == kModeFp8E4M3 ? kFp8E4M3 : mode == kModeFp8E5M2 ? kFp8E5M2 : kNvfp4;
}

// Stages of the per-wave LDS ring (DMA modes): enough bytes in flight per CU
// while several workgroups fit in the 160 KB of LDS.
template <int D>
struct DecodeStages {
  static constexpr int NS = (D == 64) ? 3 : 2;
};

// Stages of the split kernel's rings. An FP8 step at D = 256 is 16 KB, so two
// stages per wave would leave room for one workgroup per CU; with one stage,
// refilled as soon as the step is in registers, two fit.
template <int D, int MODE>
struct SplitStages {
  static constexpr int NS = (D == 256 && mode_fmt(MODE) != kNvfp4) ? 1 : DecodeStages<D>::NS;
};

// Waves per split-kernel workgroup. At head sizes up to 128 one 8-wave
// workgroup per CU (two waves per SIMD, the CU's units four times longer)
// streams faster than three 4-wave workgroups (three waves per SIMD): at the
// long-context batch 62 us against 66, with 4 splits per (sequence, kv head)
// to combine instead of 12. At 256 two 4-wave workgroups per CU.
template <int D>
struct SplitWaves {
  static constexpr int NW = (D == 256) ? 4 : 8;
};

template <int D, int MODE>
struct DecodeLds {
  static constexpr int NW = SplitWaves<D>::NW;
  static constexpr int dma_stage = StageGeo<D, MODE == kModeDmaCompact, mode_fmt(MODE)>::STAGE;
  static constexpr int stream = NW * SplitStages<D, MODE>::NS * dma_stage;
  static constexpr int merge = NW * kMergeCols * D * 4;
  static constexpr int area = stream > merge ? stream : merge;  // streams, then merge and combine scratch
};

// Waves per SIMD the register budget is sized for (the loads in flight live
// in LDS, so registers hold one step's working set; D = 256 needs more).
template <int D, int MODE>
struct DecodeOcc {
  static constexpr int waves = (D == 256) ? 2 : 3;
};

// One wave's share of a (sequence, kv head) unit: steps k0, k0 + NWS, ...
// below st1, streamed through the wave's ring of NS stages (step k + (NS - 1)
// * NWS is copied while step k, already in LDS, is computed). The query load
// is issued first so that it is in flight with the block-table reads the
// first copies wait for. Leaves the wave's softmax state in W; every copy has
// landed when it returns.
template <int D, bool COMPACT, int FMT, int NS, int NWS>
__device__ __forceinline__ void decode_stream(WaveAttn<D, 1, FMT>& W, uint8_t* ring, const Pool& pool,
                                              const int32_t* bt_row, int max_blocks, int L, int h, int k0, int st1,
                                              const uint16_t* qrow, float qk_factor,
                                              const DmaOffsets<D, COMPACT, FMT>& dof, const LdsLane& ll, int j) {
  using SG = StageGeo<D, COMPACT, FMT>;
  const auto qraw = WaveAttn<D, 1, FMT>::load_q_raw(qrow, j);
  StepIds nxt = lds_prologue<D, COMPACT, NS, FMT>(ring, k0, NWS, st1, bt_row, L, max_blocks, pool, h, dof);
  if constexpr (NS == 1) {
    // One stage: step k0's copy goes out before the query conversion, and
    // each later step's copy as soon as the previous step's bytes are in
    // registers (the reader waits for its LDS reads), so the copy streams in
    // while that step computes.
    dma_step<D, COMPACT, FMT>(ring, pool, nxt, h, k0 * kStep, dof);
    nxt = ids_for_step(bt_row, k0 + NWS, st1, L, max_blocks, pool);
    W.set_q(0, qraw, qk_factor);
    for (int k = k0; k < st1; k += NWS) {
      wait_vmcnt<0>();
      SubRaw<D, FMT> R[2];
      lds_read_step<D, FMT>(R, ring, ll);
      dma_step<D, COMPACT, FMT>(ring, pool, nxt, h, (k + NWS) * kStep, dof);
      nxt = ids_for_step(bt_row, k + 2 * NWS, st1, L, max_blocks, pool);
      const int kb = k * kStep;
      const bool partial = kb + kStep > L;
      if (partial) mask_step(R, kb, L, j);
      W.step(R, kb, j, partial);
    }
    wait_vmcnt<0>();
    return;
  }
  W.set_q(0, qraw, qk_factor);
  int slot = 0;
  for (int k = k0; k < st1; k += NWS) {
    const int fill = (slot + NS - 1) % NS;
    dma_step<D, COMPACT, FMT>(ring + fill * SG::STAGE, pool, nxt, h, (k + (NS - 1) * NWS) * kStep, dof);
    nxt = ids_for_step(bt_row, k + NS * NWS, st1, L, max_blocks, pool);
    wait_vmcnt<(NS - 1) * SG::NC>();
    SubRaw<D, FMT> R[2];
    lds_read_step<D, FMT>(R, ring + slot * SG::STAGE, ll);
    const int kb = k * kStep;
    const bool partial = kb + kStep > L;
    if (partial) mask_step(R, kb, L, j);
    W.step(R, kb, j, partial);
    slot = (slot + 1 == NS) ? 0 : slot + 1;
  }
  wait_vmcnt<0>();
}

// Merge the NWS waves' softmax states of a unit through LDS (s_ml: [NWS + 1]
// [16] (max, sum), the last row the merged (max, sum) of each column; s_o:
// [NWS][kMergeCols][D], which may overlap the drained rings), kMergeCols
// columns at a time: one thread per column turns the waves' maxima into
// normalised weights (written over the maxima), then every thread merges 4
// consecutive outputs of a column. emit(col, d, on, M, lt) gets outputs d ..
// d + 3 of column col: on = o / lt (0 when lt == 0), with the column's merged
// max M and sum lt.
template <int D, int NWS, int FMT, typename Emit>
__device__ __forceinline__ void merge_waves(const WaveAttn<D, 1, FMT>& W, float* s_ml, float* s_o, int grp, int w,
                                            int i, int j, Emit&& emit) {
  using G = Geo<D>;
  constexpr int D4 = D / 4;
  float* s_st = s_ml + NWS * 16 * 2;
  const float lsum = W.lsum(0);
  if (j == 0) {
    s_ml[(w * 16 + i) * 2] = W.m[0];
    s_ml[(w * 16 + i) * 2 + 1] = lsum;
  }
  for (int c0 = 0; c0 < grp; c0 += kMergeCols) {
    const int nc = (grp - c0 < kMergeCols) ? grp - c0 : kMergeCols;
    if (i >= c0 && i < c0 + nc) {
      float* dst = s_o + (w * kMergeCols + (i - c0)) * D;
#pragma unroll
      for (int t = 0; t < G::DPL; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(4 * j + r) * G::DPL + t] = W.acc[0][t][r];
    }
    __syncthreads();
    if ((int)threadIdx.x < nc) {
      const int col = c0 + threadIdx.x;
      float M = -__builtin_inff();
#pragma unroll
      for (int ww = 0; ww < NWS; ++ww) M = __builtin_fmaxf(M, s_ml[(ww * 16 + col) * 2]);
      float f[NWS];
      float lt = 0.0f;
#pragma unroll
      for (int ww = 0; ww < NWS; ++ww) {
        const float mw = s_ml[(ww * 16 + col) * 2];
        f[ww] = (mw == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
        lt += f[ww] * s_ml[(ww * 16 + col) * 2 + 1];
      }
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
#pragma unroll
      for (int ww = 0; ww < NWS; ++ww) s_ml[(ww * 16 + col) * 2] = f[ww] * inv;
      s_st[col * 2] = M;
      s_st[col * 2 + 1] = lt;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < nc * D4; e += 64 * NWS) {
      const int cc = e / D4;
      const int col = c0 + cc;
      const int d = 4 * (e - cc * D4);
      f4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ww = 0; ww < NWS; ++ww)
        o += s_ml[(ww * 16 + col) * 2] * *reinterpret_cast<const f4*>(s_o + (ww * kMergeCols + cc) * D + d);
      emit(col, d, o, s_st[col * 2], s_st[col * 2 + 1]);
    }
    __syncthreads();
  }
}

template <int D, int MODE>
__global__ __launch_bounds__(64 * SplitWaves<D>::NW) __attribute__((amdgpu_waves_per_eu(DecodeOcc<D, MODE>::waves))) void
decode_split_kernel(DecodeArgs a) {
  constexpr int NW = SplitWaves<D>::NW;
  constexpr int FMT = mode_fmt(MODE);
  constexpr bool COMPACT = MODE == kModeDmaCompact;
  using SG = StageGeo<D, COMPACT, FMT>;
  constexpr int NS = SplitStages<D, MODE>::NS;
  extern __shared__ __align__(16) char smem[];
  int* s_pref = reinterpret_cast<int*>(smem);
  int* s_len = s_pref + ((a.B + 1 + 3) / 4) * 4;
  int* s_red = s_pref + decode_lds_pref_ints(a.B);
  float* s_ml = reinterpret_cast<float*>(s_red + 16);  // [NW waves + merged][16 cols][2]
  uint8_t* rings = reinterpret_cast<uint8_t*>(s_ml + (NW + 1) * 16 * 2);  // per-wave stream area
  float* s_o = reinterpret_cast<float*>(rings);         // [NW waves][kMergeCols][D], after the streams

  // The scales are read with vector loads issued first: their latency then
  // overlaps the schedule's own loads (a scalar load here would be waited
  // for together with the kernel arguments the schedule needs).
  const float ksc = __builtin_bit_cast(
      float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(reinterpret_cast<const uint8_t*>(a.k_scale), 4), 0, 0, 0));
  const float vsc = __builtin_bit_cast(
      float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(reinterpret_cast<const uint8_t*>(a.v_scale), 4), 0, 0, 0));
  const int hkv = a.pool.hkv;
  const int cap = a.max_blocks * a.pool.bs;
  int tps, total;
  if (a.B <= 64)
    decode_schedule_small(a.seq_lens, a.B, cap, hkv, a.target, s_pref, s_len, total);
  else
    decode_schedule<NW>(a.seq_lens, a.B, cap, hkv, a.target, s_pref, s_len, s_red, tps, total);
  total = __builtin_amdgcn_readfirstlane(total);
  const float qk_factor = a.sm_scale * uniform_f32(ksc) * kLog2e;
  const float gv = uniform_f32(vsc);
  const float os = a.o_scale ? *a.o_scale : 1.0f;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int i = lane & 15, j = lane >> 4;
  const int grp = a.grp;
  const DmaOffsets<D, COMPACT, FMT> dof = dma_offsets<D, COMPACT, FMT>(a.pool.st, a.pool.skv, lane);
  uint8_t* ring = rings + w * NS * SG::STAGE;
  const LdsLane ll = lds_lane<D, FMT>(i, j);

  for (int u = blockIdx.x; u < total * hkv; u += gridDim.x) {
    const int ubs = u / hkv;
    const int h = u - ubs * hkv;
    // sequence of this unit: the last b with s_pref[b] <= ubs (the prefix
    // rises strictly and starts at 0), found by a 64-way search of two LDS
    // rounds: the lanes test every stride-th entry, then the entries of the
    // chosen stride (B <= kDecodeMaxSeqs = 4096, so the stride is at most 64)
    const int stride = (a.B + 63) >> 6;
    int idx = lane * stride;
    uint64_t hits = __builtin_amdgcn_ballot_w64(idx < a.B && s_pref[idx] <= ubs);
    const int c0 = (__builtin_popcountll(hits) - 1) * stride;
    idx = c0 + lane;
    hits = __builtin_amdgcn_ballot_w64(lane < stride && idx < a.B && s_pref[idx] <= ubs);
    const int b = c0 + __builtin_popcountll(hits) - 1;
    const int pb = __builtin_amdgcn_readfirstlane(s_pref[b]);
    const int split = ubs - pb;
    const int nsplit = __builtin_amdgcn_readfirstlane(s_pref[b + 1]) - pb;
    const int L = __builtin_amdgcn_readfirstlane(s_len[b]);
    const int steps = ceil_div(L, kStep);
    // the sequence's steps are dealt evenly over its nsplit units: the first
    // steps % nsplit units take one step more (nsplit <= steps when steps > 0)
    const int sq = steps / nsplit, sr = steps - sq * nsplit;
    const int st0 = split * sq + (split < sr ? split : sr);
    const int st1 = st0 + sq + (split < sr ? 1 : 0);

    const int32_t* bt_row = a.bt + (int64_t)b * a.max_blocks;
    const int k0 = st0 + w;  // the wave's steps: k0, k0 + NW, ... below st1
    WaveAttn<D, 1, FMT> W;
    W.init();
    const bool valid = i < grp;
    const uint16_t* qrow = valid ? a.q + (int64_t)b * a.q_st + (int64_t)(h * grp + i) * a.q_sh : nullptr;
    W.lim[0] = valid ? L - 1 : -1;

    decode_stream<D, COMPACT, FMT, NS, NW>(W, ring, a.pool, bt_row, a.max_blocks, L, h, k0, st1, qrow, qk_factor, dof,
                                           ll, j);
    __syncthreads();  // every wave's ring is drained before the rings become the merge buffer
    merge_waves<D, NW>(W, s_ml, s_o, grp, w, i, j, [&](int col, int d, f4 on, float M, float lt) {
      if (nsplit == 1) {
        store_out4(a, os, ((int64_t)b * a.hq + h * grp + col) * D + d, on, gv);
      } else {
        const int64_t slot = (int64_t)ubs * hkv + h;
        st_agent4(a.ws_o + slot * grp * D, (uint32_t)((col * D + d) * 4), on);
        if (d == 0) {
          st_agent(a.ws_ml + (slot * grp + col) * 2, M);
          st_agent(a.ws_ml + (slot * grp + col) * 2 + 1, lt);
        }
      }
    });
    if (nsplit > 1) {
      // The last of the sequence's splits to arrive merges all of them
      // (log-sum-exp weights) and resets the counter for the next call.
      // Partials travel through agent-coherent stores and loads (they
      // bypass the per-XCD L2), so the hand-off needs only every store to
      // have completed before the counter moves, not an L2 flush.
      wait_stores();
      __syncthreads();
      if (threadIdx.x == 0)
        s_red[15] = (__hip_atomic_fetch_add(&a.ws_cnt[(int64_t)b * hkv + h], 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(nsplit - 1));
      __syncthreads();
      if (s_red[15]) {
        combine_splits<D, NW>(a, b, h, (int64_t)s_pref[b] * hkv + h, nsplit);
        if (threadIdx.x == 0)
          __hip_atomic_store(&a.ws_cnt[(int64_t)b * hkv + h], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
    }
    // Retire this unit's stores here: the compiler's wait tracking does not
    // order stores against loads, so a store still counted as pending when
    // the next unit's pipelined loop starts makes it wait for every load in
    // flight at the top of each iteration.
    wait_stores();
  }
}

// ---------------------------------------------------------------------------
// Decode without split-K: one workgroup of NW waves per (sequence, kv head).
// The waves take interleaved steps and merge in LDS, and the workgroup writes
// the bf16 output itself: no schedule, no partials, no combine. Chosen when
// the batch alone gives every CU a (sequence, kv head) pair and no sequence
// needs more than a few steps per wave; longer or fewer sequences go to the
// split kernel.
// ---------------------------------------------------------------------------
template <int D, int FMT>
struct PairGeo {
  // waves per workgroup: as many rings as the LDS of one CU holds (one
  // workgroup per CU); FP8 stages are larger
  static constexpr int NW = (FMT == kNvfp4) ? ((D == 256) ? 8 : 12) : ((D == 64) ? 12 : (D == 128) ? 8 : 4);
  static constexpr int kMaxStepsPerWave = 8;
};

template <int D, int MODE>
struct PairLds {
  static constexpr int NW = PairGeo<D, mode_fmt(MODE)>::NW;
  static constexpr int stream =
      NW * DecodeStages<D>::NS * StageGeo<D, MODE == kModeDmaCompact, mode_fmt(MODE)>::STAGE;
  static constexpr int merge = NW * kMergeCols * D * 4;
  static constexpr int bytes = (NW + 1) * 16 * 2 * 4 + (stream > merge ? stream : merge);
  static_assert(bytes <= 160 * 1024, "one workgroup per CU");
};

template <int D, int MODE>
__global__ __launch_bounds__((64 * PairGeo<D, mode_fmt(MODE)>::NW)) void decode_pair_kernel(DecodeArgs a) {
  constexpr int FMT = mode_fmt(MODE);
  constexpr int NW = PairGeo<D, FMT>::NW;
  constexpr bool COMPACT = MODE == kModeDmaCompact;
  using SG = StageGeo<D, COMPACT, FMT>;
  constexpr int NS = DecodeStages<D>::NS;
  extern __shared__ __align__(16) char smem[];
  float* s_ml = reinterpret_cast<float*>(smem);                     // [NW waves + merged][16 cols][2]
  uint8_t* rings = reinterpret_cast<uint8_t*>(s_ml + (NW + 1) * 16 * 2);  // per-wave stream area
  float* s_o = reinterpret_cast<float*>(rings);                     // [NW][kMergeCols][D], after the streams

  const float ksc = __builtin_bit_cast(
      float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(reinterpret_cast<const uint8_t*>(a.k_scale), 4), 0, 0, 0));
  const float vsc = __builtin_bit_cast(
      float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(reinterpret_cast<const uint8_t*>(a.v_scale), 4), 0, 0, 0));
  const int hkv = a.pool.hkv;
  const int b = blockIdx.x / hkv;
  const int h = blockIdx.x - b * hkv;
  const int L = clamp_len(ld_uniform(a.seq_lens, b), a.max_blocks * a.pool.bs);
  const float qk_factor = a.sm_scale * uniform_f32(ksc) * kLog2e;
  const float gv = uniform_f32(vsc);
  const float os = a.o_scale ? *a.o_scale : 1.0f;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, j = lane >> 4;
  const int grp = a.grp;
  const DmaOffsets<D, COMPACT, FMT> dof = dma_offsets<D, COMPACT, FMT>(a.pool.st, a.pool.skv, lane);
  uint8_t* ring = rings + w * NS * SG::STAGE;
  const LdsLane ll = lds_lane<D, FMT>(i, j);
  WaveAttn<D, 1, FMT> W;
  W.init();
  const bool valid = i < grp;
  const uint16_t* qrow = valid ? a.q + (int64_t)b * a.q_st + (int64_t)(h * grp + i) * a.q_sh : nullptr;
  W.lim[0] = valid ? L - 1 : -1;
  decode_stream<D, COMPACT, FMT, NS, NW>(W, ring, a.pool, a.bt + (int64_t)b * a.max_blocks, a.max_blocks, L, h, w, ceil_div(L, kStep),
                                    qrow, qk_factor, dof, ll, j);
  __syncthreads();  // every wave's ring is drained before the rings become the merge buffer
  merge_waves<D, NW>(W, s_ml, s_o, grp, w, i, j, [&](int col, int d, f4 on, float, float) {
    store_out4(a, os, ((int64_t)b * a.hq + h * grp + col) * D + d, on, gv);
  });
}

// Workspace: [arrival counters][partial outputs][partial (max, sum)]. The
// counters are sized for the largest batch a call may have, so their place
// depends only on num_kv_heads: calls with different batch sizes can share a
// workspace without one call's partials landing on another's counters.
static int64_t counter_bytes(int num_kv_heads) {
  return (((int64_t)kDecodeMaxSeqs * num_kv_heads * 4 + 255) / 256) * 256;
}

size_t decode_partial_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_size) {
  const int64_t grp = num_q_heads / num_kv_heads;
  const int64_t slots = kDecodeTargetMax + (int64_t)num_seqs * num_kv_heads;
  return (size_t)(slots * grp * head_size * 4 + slots * grp * 2 * 4);
}

size_t decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_size) {
  return (size_t)counter_bytes(num_kv_heads) + decode_partial_bytes(num_seqs, num_q_heads, num_kv_heads, head_size);
}

template <int D, int MODE>
static size_t decode_lds_bytes_m(int num_seqs) {
  return (size_t)(decode_lds_pref_ints(num_seqs) + 16) * 4 + (SplitWaves<D>::NW + 1) * 16 * 2 * 4 +
         DecodeLds<D, MODE>::area;
}

template <int D>
static size_t decode_lds_bytes_t(int num_seqs, int fmt) {
  // both NVFP4 modes use the same stage geometry, both FP8 formats another
  static_assert(DecodeLds<D, kModeDmaGeneral>::area == DecodeLds<D, kModeDmaCompact>::area, "mode LDS sizes");
  static_assert(DecodeLds<D, kModeFp8E4M3>::area == DecodeLds<D, kModeFp8E5M2>::area, "mode LDS sizes");
  return fmt == kNvfp4 ? decode_lds_bytes_m<D, kModeDmaCompact>(num_seqs)
                       : decode_lds_bytes_m<D, kModeFp8E4M3>(num_seqs);
}

size_t decode_lds_bytes(int num_seqs, int grp, int head_size, int fmt) {
  (void)grp;
  switch (head_size) {
    case 64: return decode_lds_bytes_t<64>(num_seqs, fmt);
    case 128: return decode_lds_bytes_t<128>(num_seqs, fmt);
    default: return decode_lds_bytes_t<256>(num_seqs, fmt);
  }
}

// Workgroups of a decode kernel variant that the device holds at once (an
// occupancy query, not a device sync), cached per device, variant and LDS
// size: the split kernel's LDS grows with the batch, so a few sizes recur.
// Host threads may call concurrently; the cache is guarded by a mutex.
constexpr int kMaxDevices = 64;

struct OccupancyCache {
  std::mutex mu;
  std::map<size_t, int> by_lds[kMaxDevices];
};

static int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  return dev;
}

static int device_cus() {
  static std::atomic<int> cached[kMaxDevices];
  const int dev = current_device();
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

template <int D, int MODE>
static int resident_workgroups(size_t lds) {
  static OccupancyCache cache;
  const int dev = current_device();
  {
    std::lock_guard<std::mutex> lock(cache.mu);
    const auto it = cache.by_lds[dev].find(lds);
    if (it != cache.by_lds[dev].end()) return it->second;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_split_kernel<D, MODE>, 64 * SplitWaves<D>::NW,
                                                   lds) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  int n = per_cu * device_cus();
  n = n > kDecodeTargetMax ? kDecodeTargetMax : n;
  std::lock_guard<std::mutex> lock(cache.mu);
  cache.by_lds[dev][lds] = n;
  return n;
}

// 32-key steps of the longest sequence, as far as the host knows it.
static int64_t host_max_steps(int max_blocks, int bs, int max_seq_len) {
  const int64_t cap = (int64_t)max_blocks * bs;
  const int64_t lens = max_seq_len > 0 ? (max_seq_len < cap ? max_seq_len : cap) : cap;
  return (lens + kStep - 1) / kStep;
}

// The per-pair kernel when the batch alone gives every CU a (sequence, kv
// head) pair and no sequence needs more than kMaxStepsPerWave steps per wave.
template <int D, int FMT>
static bool use_pair_kernel(int num_seqs, int hkv, int64_t max_steps) {
  return (int64_t)num_seqs * hkv >= device_cus() &&
         max_steps <= (int64_t)PairGeo<D, FMT>::NW * PairGeo<D, FMT>::kMaxStepsPerWave;
}

template <int FMT>
static int decode_plan_f(int num_seqs, int num_kv_heads, int head_size, int64_t steps) {
  switch (head_size) {
    case 64: return use_pair_kernel<64, FMT>(num_seqs, num_kv_heads, steps) ? 1 : 0;
    case 128: return use_pair_kernel<128, FMT>(num_seqs, num_kv_heads, steps) ? 1 : 0;
    case 256: return use_pair_kernel<256, FMT>(num_seqs, num_kv_heads, steps) ? 1 : 0;
    default: return -1;
  }
}

int decode_plan(int num_seqs, int num_kv_heads, int head_size, int block_size, int max_blocks, int max_seq_len,
                int fmt) {
  const int64_t steps = host_max_steps(max_blocks, block_size, max_seq_len);
  switch (fmt) {
    case kNvfp4: return decode_plan_f<kNvfp4>(num_seqs, num_kv_heads, head_size, steps);
    case kFp8E4M3: return decode_plan_f<kFp8E4M3>(num_seqs, num_kv_heads, head_size, steps);
    case kFp8E5M2: return decode_plan_f<kFp8E5M2>(num_seqs, num_kv_heads, head_size, steps);
    default: return -1;
  }
}

template <int D, int MODE>
static hipError_t launch_decode_v(DecodeArgs a, int max_seq_len, hipStream_t stream) {
  const int hkv = a.pool.hkv;
  const int64_t steps = host_max_steps(a.max_blocks, a.pool.bs, max_seq_len);
  constexpr int FMT = mode_fmt(MODE);
  if (use_pair_kernel<D, FMT>(a.B, hkv, steps)) {
    decode_pair_kernel<D, MODE><<<a.B * hkv, 64 * PairGeo<D, FMT>::NW, PairLds<D, MODE>::bytes, stream>>>(a);
    return hipGetLastError();
  }
  const size_t lds = decode_lds_bytes_m<D, MODE>(a.B);
  a.target = resident_workgroups<D, MODE>(lds);
  // an upper bound of the units the schedule can produce for this batch
  int64_t want = (int64_t)a.B * hkv * ((steps + kDecodeMinTps - 1) / kDecodeMinTps);
  want = want < (int64_t)a.B * hkv ? (int64_t)a.B * hkv : want;
  const int grid = (int)(want < a.target ? want : a.target);
  decode_split_kernel<D, MODE><<<grid, 64 * SplitWaves<D>::NW, lds, stream>>>(a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_decode_t(DecodeArgs a, int max_seq_len, int fmt, hipStream_t stream) {
  // FP8 rows are copied in 16-byte chunks whatever their stride (the API
  // requires 16-byte aligned strides for them)
  if (fmt == kFp8E4M3) return launch_decode_v<D, kModeFp8E4M3>(a, max_seq_len, stream);
  if (fmt == kFp8E5M2) return launch_decode_v<D, kModeFp8E5M2>(a, max_seq_len, stream);
  // 16-byte chunks need contiguous, 16-byte aligned page rows (HND layout)
  const bool compact = a.pool.st == D / 2 + D / 16 && a.pool.sb % 16 == 0 && a.pool.skv % 16 == 0 &&
                       a.pool.sh % 16 == 0 && (reinterpret_cast<uintptr_t>(a.pool.data) % 16) == 0;
  return compact ? launch_decode_v<D, kModeDmaCompact>(a, max_seq_len, stream)
                 : launch_decode_v<D, kModeDmaGeneral>(a, max_seq_len, stream);
}

hipError_t launch_decode(const Pool& pool, int head_size, const void* q, int64_t q_st, int64_t q_sh,
                         int num_q_heads, const int32_t* block_table, int32_t max_blocks,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len, const float* k_scale,
                         const float* v_scale, float sm_scale, const float* o_scale, void* out, void* workspace,
                         int fmt, hipStream_t stream, int64_t counter_region_bytes) {
  if (num_seqs == 0) return hipSuccess;
  DecodeArgs a;
  a.pool = pool;
  a.q = static_cast<const uint16_t*>(q);
  a.q_st = q_st;
  a.q_sh = q_sh;
  a.hq = num_q_heads;
  a.grp = num_q_heads / pool.hkv;
  a.bt = block_table;
  a.max_blocks = max_blocks;
  a.seq_lens = seq_lens;
  a.B = num_seqs;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.sm_scale = sm_scale;
  a.out = static_cast<uint16_t*>(out);
  a.out8 = static_cast<uint8_t*>(out);
  a.o_scale = o_scale;
  const int64_t slots = kDecodeTargetMax + (int64_t)num_seqs * pool.hkv;
  a.ws_cnt = static_cast<uint32_t*>(workspace);
  const int64_t cbytes = counter_region_bytes >= 0 ? counter_region_bytes : counter_bytes(pool.hkv);
  a.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + cbytes);
  a.ws_ml = a.ws_o + slots * a.grp * head_size;
  switch (head_size) {
    case 64: return launch_decode_t<64>(a, max_seq_len, fmt, stream);
    case 128: return launch_decode_t<128>(a, max_seq_len, fmt, stream);
    case 256: return launch_decode_t<256>(a, max_seq_len, fmt, stream);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// Chunked prefill. Columns of (sequence b, kv head h) are (token, group head)
// pairs, token-major; a workgroup owns NW*16*NT consecutive columns (16*NT
// per wave) and walks keys 0 .. the last key its columns see, its waves
// sharing the dequantisation of each step. No split along the keys: long
// chunks already give many workgroups.
// ---------------------------------------------------------------------------
struct PrefillPlanRow;

struct PrefillArgs {
  Pool pool;
  const uint16_t* q;
  int64_t q_st, q_sh;
  int hq, grp;
  const int32_t* cu_q;
  int total_q;
  const int32_t* bt;
  int32_t max_blocks;
  const int32_t* seq_lens;
  const float* k_scale;
  const float* v_scale;
  float sm_scale;
  int causal;
  uint16_t* out;         // bf16 output (when o_scale is null)
  uint8_t* out8;         // FP8-E4M3 output (when o_scale is set)
  const float* o_scale;  // per-tensor FP8 output scale, or null
  int num_seqs;
  int longest_first;     // blockIdx.z is a rank in order of decreasing length (num_seqs <= kPrefillRankMax)
  const PrefillPlanRow* plan;  // key split: the plan of every rank (null: no split)
  uint32_t* ws_cnt;            // key split: arrival counters of cut jobs, zero between calls
  float* ws_part;              // key split: part records (PrefillPartGeo<D>::BYTES each)
};

// Query rows [q0, q0 + qlen) of the batch that are sequence b's chunk, and
// its key count L (cu_seqlens_q clamped to [0, total_q], lengths to the
// block table's capacity).
__device__ __forceinline__ void prefill_seq_geom(const PrefillArgs& a, int b, int& q0, int& qlen, int& L) {
  int x0 = a.cu_q[b], x1 = a.cu_q[b + 1];
  x0 = x0 < 0 ? 0 : (x0 > a.total_q ? a.total_q : x0);
  x1 = x1 < x0 ? x0 : (x1 > a.total_q ? a.total_q : x1);
  q0 = x0;
  qlen = x1 - x0;
  L = clamp_len(a.seq_lens[b], a.max_blocks * a.pool.bs);
}

// The same, as wave-uniform values (scalar registers).
__device__ __forceinline__ void prefill_seq_geom_u(const PrefillArgs& a, int b, int& q0, int& qlen, int& L) {
  prefill_seq_geom(a, b, q0, qlen, L);
  q0 = __builtin_amdgcn_readfirstlane(q0);
  qlen = __builtin_amdgcn_readfirstlane(qlen);
  L = __builtin_amdgcn_readfirstlane(L);
}

// 32-key steps a workgroup of kCols columns starting at column wg_col walks:
// up to the last key its last column sees (all L keys without the causal
// mask).
template <int kCols>
__device__ __forceinline__ int prefill_job_steps(int causal, int grp, int L, int qlen, int wg_col) {
  const int ncols = qlen * grp;
  const int wg_last = ((wg_col + kCols < ncols) ? wg_col + kCols : ncols) - 1;
  int kmax = causal ? L - qlen + wg_last / grp + 1 : L;
  kmax = kmax > L ? L : (kmax < 0 ? 0 : kmax);
  return ceil_div(kmax, kStep);
}

// Batches of up to this many sequences are walked longest first: the grid's
// sequence axis is a rank, so the longest sequences' workgroups are
// dispatched first and the short ones fill in behind them (longest-
// processing-time order), instead of a long sequence late in the batch
// setting the end.
constexpr int kPrefillRankMax = 256;

// The sequence of rank r in order of decreasing key length (ties: lower
// index first), ranked by the workgroup through s (kPrefillRankMax + 1 ints
// of LDS that are free until the function returns).
__device__ int prefill_seq_of_rank(const PrefillArgs& a, int r, int* s) {
  const int B = a.num_seqs;
  const int cap = a.max_blocks * a.pool.bs;
  for (int t = threadIdx.x; t < B; t += blockDim.x) s[t] = clamp_len(a.seq_lens[t], cap);
  __syncthreads();
  for (int t = threadIdx.x; t < B; t += blockDim.x) {
    const int kt = s[t];
    int rank = 0;
    for (int u = 0; u < B; ++u) {
      const int ku = s[u];
      rank += (ku > kt || (ku == kt && u < t)) ? 1 : 0;
    }
    if (rank == r) s[B] = t;
  }
  __syncthreads();
  const int b = s[B];
  __syncthreads();  // s is reused (the copies' ring) from here on
  return b;
}

template <int D>
__device__ __forceinline__ void store_column(uint16_t* orow, const f4 (&acc)[Geo<D>::DPL], float scale, int j) {
  constexpr int DPL = Geo<D>::DPL;
  // lane (i, j) holds d = (4j + r) * DPL + t, a contiguous run of 4*DPL values
  uint32_t pk[2 * DPL];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int t = 0; t < DPL; t += 2)
      pk[(r * DPL + t) / 2] = pack_bf16x2(acc[t][r] * scale, acc[t + 1][r] * scale);
  u32x4* dst = reinterpret_cast<u32x4*>(orow + 4 * j * DPL);
#pragma unroll
  for (int c = 0; c < DPL / 2; ++c) dst[c] = u32x4{pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]};
}

// The same column as FP8-E4M3 bytes (fp8_e4m3_out of each value), stored
// r by r: the DPL bytes (4j + r) * DPL + t, t < DPL, are consecutive.
template <int D>
__device__ __forceinline__ void store_column_fp8(uint8_t* orow, const f4 (&acc)[Geo<D>::DPL], float scale, float os,
                                                 int j) {
  constexpr int DPL = Geo<D>::DPL;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    uint32_t pk[DPL / 4];
#pragma unroll
    for (int k = 0; k < DPL / 4; ++k) {
      pk[k] = fp8_e4m3_out(acc[4 * k][r] * scale, os) | (fp8_e4m3_out(acc[4 * k + 1][r] * scale, os) << 8) |
              (fp8_e4m3_out(acc[4 * k + 2][r] * scale, os) << 16) | (fp8_e4m3_out(acc[4 * k + 3][r] * scale, os) << 24);
    }
    uint8_t* dst = orow + (4 * j + r) * DPL;
    if constexpr (DPL == 4) {
      *reinterpret_cast<uint32_t*>(dst) = pk[0];
    } else if constexpr (DPL == 8) {
      *reinterpret_cast<u32x2*>(dst) = u32x2{pk[0], pk[1]};
    } else {
#pragma unroll
      for (int c = 0; c < DPL / 16; ++c)
        reinterpret_cast<u32x4*>(dst)[c] = u32x4{pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]};
    }
  }
}

// Prefill ring stages: the step being dequantised and the ones in flight.
// NVFP4: as many stages (up to 4) as the 6-bit vmcnt counter can cover; FP8
// stages are 1.8x larger: 2 at D >= 128.
template <int D, bool COMPACT, int FMT = kNvfp4>
struct PrefillStages {
  static constexpr int NC = StageGeo<D, COMPACT, FMT>::NC;
  static constexpr int NS_MAX = (FMT == kNvfp4 || D == 64) ? 4 : 2;
  static constexpr int NS = (63 / NC + 1) < NS_MAX ? (63 / NC + 1) : NS_MAX;
  static_assert(NS >= 2, "the prefill pipeline reads one stage while the next lands");
};

template <bool B>
struct SteadyTag {
  static constexpr bool value = B;
};

// Waves per prefill workgroup (NW) and 16-column tiles per wave (NT): a
// workgroup shares the dequantisation of each step among its NW waves and
// owns NW * 16 * NT query columns. At head size 256 the accumulators of two
// tiles would leave one wave per SIMD; eight waves of one tile each keep the
// 128 columns per workgroup at two waves per SIMD.
template <int D>
struct PrefillGeo {
  static constexpr int NW = (D == 256) ? 8 : 4;
  static constexpr int NT = (D == 64) ? 4 : (D == 128) ? 2 : 1;
  static constexpr int kCols = NW * 16 * NT;
  // One workgroup fills a CU at head size 256, so a third operand buffer
  // (for the deferred PV product) costs no occupancy there; at the smaller
  // head sizes it would cost a workgroup per CU.
  static constexpr bool kDeferPV = (D == 256);
  static constexpr int kOpBufs = kDeferPV ? 3 : 2;
};

// Waves per SIMD the prefill register budget is sized for: without the hint
// the compiler spends the whole register file of one wave. Head size 128
// fits three workgroups per CU in LDS and is held to three waves (168
// registers); the rest to two.
template <int D, bool COMPACT, bool FP8OUT, int FMT>
struct PrefillOcc {
  static constexpr int waves = (D == 128) ? 3 : 2;
};

// NVFP4 at head sizes 128 and 256, where a workgroup has as many waves (NW)
// as a lane has K chunks (KW) and twice as many V^T tiles: wave w's share of
// a step is K chunk w of both subtiles and V^T tiles 2w and 2w + 1. Both
// tiles take, from each of the lane's four V rows, the two nibbles of one
// byte: byte B = w % 4 of the row's code word W = w / 4 (the lane's D/32
// code bytes of a row are D/128 words). Lane (i, j) reads, per subtile, the
// code word of K chunk w of row i with that chunk's block-scale byte, and
// word W of its four V rows with their scale bytes.
template <int D>
struct ShareRaw {
  uint32_t k[2];
  uint32_t ks[2];
  uint32_t v[2][4];
  uint32_t vs[2][4];
};

template <int D>
__device__ __forceinline__ void lds_read_share(ShareRaw<D>& R, const uint8_t* stage, const LdsLane& o, int w) {
  static_assert(D == 128 || D == 256, "share reader: head sizes 128 and 256");
  constexpr int FD = D / 2 + D / 16;
  constexpr int SUB = StageGeo<D, true>::SUB;
  static_assert(StageGeo<D, true>::SUB == StageGeo<D, false>::SUB, "subtile size is the copy's");
  static_assert((D == 256 && FD == 144 && SUB == 4608) || (D == 128 && FD == 72 && SUB == 2304), "reader offsets");
  const uint32_t s0 = lds_addr(stage);
  // chunk w of quarter j: code word w of the lane's run, block (j D/4 + 8 w) / 16
  const uint32_t ak = s0 + o.k + 4u * (uint32_t)w, aks = s0 + o.ks + ((uint32_t)w >> 1);
  const uint32_t av = s0 + o.v + 4u * (uint32_t)(w >> 2), avs = s0 + o.vs;
#define NVFP4KV_SHARE_READ(R1, R2, R3, SB0, SB1)                                                              \
  asm volatile("ds_read_b32 %0, %20\n\t"                                                                   \
               "ds_read_u8 %1, %21\n\t"                                                                    \
               "ds_read_b32 %2, %22\n\t"                                                                   \
               "ds_read_b32 %3, %22 offset:" #R1 "\n\t"                                                    \
               "ds_read_b32 %4, %22 offset:" #R2 "\n\t"                                                    \
               "ds_read_b32 %5, %22 offset:" #R3 "\n\t"                                                    \
               "ds_read_u8 %6, %23\n\t"                                                                    \
               "ds_read_u8 %7, %23 offset:" #R1 "\n\t"                                                     \
               "ds_read_u8 %8, %23 offset:" #R2 "\n\t"                                                     \
               "ds_read_u8 %9, %23 offset:" #R3 "\n\t"                                                     \
               "ds_read_b32 %10, %20 offset:" #SB0 "\n\t"                                                  \
               "ds_read_u8 %11, %21 offset:" #SB0 "\n\t"                                                   \
               "ds_read_b32 %12, %22 offset:" #SB0 "\n\t"                                                  \
               "ds_read_b32 %13, %22 offset:" #SB1 "+" #R1 "\n\t"                                          \
               "ds_read_b32 %14, %22 offset:" #SB1 "+" #R2 "\n\t"                                          \
               "ds_read_b32 %15, %22 offset:" #SB1 "+" #R3 "\n\t"                                          \
               "ds_read_u8 %16, %23 offset:" #SB0 "\n\t"                                                   \
               "ds_read_u8 %17, %23 offset:" #SB1 "+" #R1 "\n\t"                                           \
               "ds_read_u8 %18, %23 offset:" #SB1 "+" #R2 "\n\t"                                           \
               "ds_read_u8 %19, %23 offset:" #SB1 "+" #R3 "\n\t"                                           \
               "s_waitcnt lgkmcnt(0)"                                                                      \
               : "=&v"(R.k[0]), "=&v"(R.ks[0]), "=&v"(R.v[0][0]), "=&v"(R.v[0][1]), "=&v"(R.v[0][2]),     \
                 "=&v"(R.v[0][3]), "=&v"(R.vs[0][0]), "=&v"(R.vs[0][1]), "=&v"(R.vs[0][2]), "=&v"(R.vs[0][3]), \
                 "=&v"(R.k[1]), "=&v"(R.ks[1]), "=&v"(R.v[1][0]), "=&v"(R.v[1][1]), "=&v"(R.v[1][2]),      \
                 "=&v"(R.v[1][3]), "=&v"(R.vs[1][0]), "=&v"(R.vs[1][1]), "=&v"(R.vs[1][2]), "=&v"(R.vs[1][3]) \
               : "v"(ak), "v"(aks), "v"(av), "v"(avs)                                                      \
               : "memory")
  if constexpr (D == 256)
    NVFP4KV_SHARE_READ(144, 288, 432, 4608, 4608);
  else
    NVFP4KV_SHARE_READ(72, 144, 216, 2304, 2304);
#undef NVFP4KV_SHARE_READ
}

// This wave's share of the step's MFMA operands (NVFP4, head size 128 or
// 256) from its own raw bytes: the same values make_ops stores.
template <int D, int NW, bool FULL = false>
__device__ __forceinline__ void prefill_dequant_share(const uint8_t* stage, const LdsLane& ll, int kb, int L, int j,
                                                      int w, uint32_t slot) {
  static_assert(Geo<D>::KW == NW && Geo<D>::DPL == 2 * NW, "share layout");
  ShareRaw<D> R;
  lds_read_share<D>(R, stage, ll, w);
  if (!FULL && kb + kStep > L) {
    // value rows (codes and scales) of keys >= L read as zeros
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = kb + 16 * sb + 4 * j + r < L;
        R.v[sb][r] = ok ? R.v[sb][r] : 0u;
        R.vs[sb][r] = ok ? R.vs[sb][r] : 0u;
      }
  }
  // K chunk w of each subtile: 8 codes times their block scale
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const h2 sp = fp8x2_to_h2<false>(R.ks[sb]);
    const h2 ss = {sp[0], sp[0]};
    const uint32_t c = R.k[sb];
    const h2 a0 = fp4x2_to_h2<0>(c) * ss;
    const h2 a1 = fp4x2_to_h2<1>(c) * ss;
    const h2 a2 = fp4x2_to_h2<2>(c) * ss;
    const h2 a3 = fp4x2_to_h2<3>(c) * ss;
    lds_store_op(slot + (uint32_t)(sb * Geo<D>::KW + w) * 1024u,
                 h8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]});
  }
  // V^T tiles 2w (low nibbles, d even) and 2w + 1 (high nibbles): for the key
  // pair (a, b) = (4j + 2p, 4j + 2p + 1) of a subtile, one byte permute puts
  // byte B of the two rows side by side, each byte converts to its two
  // values times its row's block scale, and two half-word permutes pair the
  // keys' d-even and d-odd values.
  const uint32_t B = (uint32_t)w & 3u;
  const uint32_t sel = 0x0C0C0000u | ((4u + B) << 8) | B;
  h4 t0[2], t1[2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    h2 ca[2], cb[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const uint32_t x = __builtin_amdgcn_perm(R.v[sb][2 * p + 1], R.v[sb][2 * p], sel);
      const h2 sc = fp8x2_to_h2<false>(__builtin_amdgcn_perm(R.vs[sb][2 * p + 1], R.vs[sb][2 * p], 0x0C0C0400u));
      const h2 sa = {sc[0], sc[0]}, sbb = {sc[1], sc[1]};
      ca[p] = fp4x2_to_h2<0>(x) * sa;   // (a d-even, a d-odd)
      cb[p] = fp4x2_to_h2<1>(x) * sbb;  // (b d-even, b d-odd)
    }
    t0[sb] = h4{ca[0][0], cb[0][0], ca[1][0], cb[1][0]};
    t1[sb] = h4{ca[0][1], cb[0][1], ca[1][1], cb[1][1]};
  }
  const uint32_t vslot = slot + (uint32_t)(2 * Geo<D>::KW + 2 * w) * 1024u;
  lds_store_op(vslot, h8{t0[0][0], t0[0][1], t0[0][2], t0[0][3], t0[1][0], t0[1][1], t0[1][2], t0[1][3]});
  lds_store_op(vslot + 1024u, h8{t1[0][0], t1[0][1], t1[0][2], t1[0][3], t1[1][0], t1[1][1], t1[1][2], t1[1][3]});
}

// This wave's share of the MFMA operands of the raw step at `stage` (first
// key kb), dequantised into the operand buffer whose lane slot is `slot`.
// FULL: the caller knows every key of the step is below L.
template <int D, int FMT, int NW, bool FULL = false>
__device__ __forceinline__ void prefill_dequant(const uint8_t* stage, const LdsLane& ll, int kb, int L, int j, int w,
                                                uint32_t slot) {
  if constexpr (FMT == kNvfp4 && (D == 128 || D == 256)) {
    prefill_dequant_share<D, NW, FULL>(stage, ll, kb, L, j, w, slot);
  } else {
    SubRaw<D, FMT> R[2];
    lds_read_step<D, FMT>(R, stage, ll);
    if (!FULL && kb + kStep > L) mask_step(R, kb, L, j);
    VPairs<D, FMT> vp[2];
    make_pairs(R[0], vp[0]);
    make_pairs(R[1], vp[1]);
    make_ops<D, 0, NW>(R, vp, w, slot);
  }
}

// S^T of a step for this wave's column tiles from the K operands of its
// operand buffer (E = subtile * KW + chunk), eight (head size 64: four) at a
// time.
template <int D, int NT, int FMT>
__device__ __forceinline__ void prefill_scores(WaveAttn<D, NT, FMT>& W, uint32_t slot, f4 (&s)[2][NT]) {
  using G = Geo<D>;
  constexpr int NK = 2 * G::KW;
  // four at a time at head size 128, whose step loop is at its register budget
  constexpr int GS = (NK < 8 || D == 128) ? 4 : 8;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int n = 0; n < NT; ++n) s[sb][n] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < NK / GS; ++g) {
    h8 t[GS];
    if constexpr (GS == 8)
      lds_load_ops8(t, slot + g * GS * 1024);
    else
      lds_load_ops4(t, slot + g * GS * 1024);
#pragma unroll
    for (int e = 0; e < GS; ++e) {
      const int E = g * GS + e;
#pragma unroll
      for (int n = 0; n < NT; ++n)
        s[E / G::KW][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(t[e], W.q[n][E % G::KW], s[E / G::KW][n], 0, 0, 0);
    }
  }
}

// O^T += V^T . P^T of a step from the V^T operands of its operand buffer
// (E = 2 KW + tile), with the running sums when they come from the matrix
// unit.
template <int D, int NT, int FMT>
__device__ __forceinline__ void prefill_pv(WaveAttn<D, NT, FMT>& W, uint32_t slot, const h8 (&p)[NT]) {
  using G = Geo<D>;
  constexpr int GS = G::DPL < 8 ? G::DPL : 8;
  const uint32_t v0 = slot + 2 * G::KW * 1024;
#pragma unroll
  for (int g = 0; g < G::DPL / GS; ++g) {
    h8 t[GS];
    if constexpr (GS == 8)
      lds_load_ops8(t, v0 + g * GS * 1024);
    else
      lds_load_ops4(t, v0 + g * GS * 1024);
#pragma unroll
    for (int e = 0; e < GS; ++e)
#pragma unroll
      for (int n = 0; n < NT; ++n)
        W.acc[n][g * GS + e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(t[e], p[n], W.acc[n][g * GS + e], 0, 0, 0);
  }
  if constexpr (WaveAttn<D, NT>::kMfmaSum) W.sum_ops(p);
}

// One workgroup's part of a job (sequence, column block, kv head) under the
// key split: the job's steps are cut into n consecutive ranges, each its own
// workgroup; this one is part self. Part p leaves its state in record rec0 +
// p of the workspace, and arrival counter cnt counts the parts done. With
// n = 1 the workgroup writes the output itself.
struct PrefillPart {
  int n;
  int self;
  int rec0;
  int cnt;
};

template <int D, int NT>
__device__ __forceinline__ void prefill_put_part(const PrefillArgs& a, const WaveAttn<D, NT>& W, const PrefillPart& pt, int w, int lane);
template <int D, int NT>
__device__ __forceinline__ void prefill_merge_parts(const PrefillArgs& a, WaveAttn<D, NT>& W, const PrefillPart& pt, int w, int lane);

// Columns [wg_col, wg_col + NW 16 NT) of the chunk of sequence b (first
// query row q0, qlen rows, L keys) for kv head h, over the job's steps
// [k_lo, k_hi) (clamped to the steps the columns see): the workgroup's NW
// waves share the dequantisation of each 32-key step and each runs its own
// 16 NT columns' products. A part of a split job (pt.n > 1) leaves its state
// in the workspace; the last part to arrive merges them all and writes the
// output. s_flag: one int of LDS for the arrival result (the ring's first
// word: the ring is idle once the step loop is done).
template <int D, int NT, bool COMPACT, bool FP8OUT, int FMT>
__device__ __forceinline__ void prefill_columns(const PrefillArgs& a, uint8_t* ring, uint8_t* opbuf, int b, int h,
                                                int q0, int qlen, int L, int wg_col, int k_lo, int k_hi,
                                                const PrefillPart& pt, int* s_flag) {
  using G = Geo<D>;
  using SG = StageGeo<D, COMPACT, FMT>;
  using OG = OpGeo<D>;
  constexpr int NS = PrefillStages<D, COMPACT, FMT>::NS;
  // Opaque per call: the lane offsets below are then derived again in each
  // inlined call instead of being kept live from one call to the next.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int i = lane & 15, j = lane >> 4;
  const int grp = a.grp;
  const int ncols = qlen * grp;
  const int col_base = wg_col + w * 16 * NT;

  WaveAttn<D, NT> W;
  W.init();
  const float qk_factor = a.sm_scale * (*a.k_scale) * kLog2e;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int c = col_base + 16 * n + i;
    const bool valid = c < ncols;
    const int tok = c / grp, g = c - (c / grp) * grp;
    const uint16_t* qrow =
        valid ? a.q + (int64_t)(q0 + tok) * a.q_st + (int64_t)(h * grp + g) * a.q_sh : nullptr;
    W.load_q(n, qrow, j, qk_factor);
    int lim = a.causal ? L - qlen + tok : L - 1;
    lim = lim > L - 1 ? L - 1 : lim;
    W.lim[n] = valid ? lim : -1;
  }
  // the steps of this range: the job's steps (up to the last visible key of
  // its last column) within [k_lo, k_hi)
  constexpr int kWgCols = PrefillGeo<D>::NW * 16 * NT;
  const int job_steps = prefill_job_steps<kWgCols>(a.causal, grp, L, qlen, wg_col);
  const int kend = k_hi < job_steps ? k_hi : job_steps;
  const int kbeg = k_lo < kend ? k_lo : kend;
  // keys this wave's columns see (none if it has no column), and below
  // min_full every valid column of the wave sees every key
  const bool has_cols = col_base < ncols;
  const int c_last = ((col_base + 16 * NT < ncols) ? col_base + 16 * NT : ncols) - 1;
  int kw = has_cols ? (a.causal ? L - qlen + c_last / grp + 1 : L) : 0;
  kw = kw > L ? L : (kw < 0 ? 0 : kw);
  const int min_full = a.causal ? L - qlen + col_base / grp + 1 : L;
  const int32_t* bt_row = a.bt + (int64_t)b * a.max_blocks;
  const LdsLane ll = lds_lane<D, FMT>(i, j);
  const uint32_t op_lane = lds_addr(opbuf) + lane * 16;

  // ---- the waves share each 32-key step, in a pipeline with one barrier
  // per step. Wave 0 copies raw steps into the NS-stage ring (NS - 1 ahead);
  // each wave dequantises its share of a step's MFMA operands into that
  // step's operand buffer one iteration before the step's products, so the
  // dequantisation of step k + 1 overlaps the products of step k on the
  // matrix unit. Iteration k runs, per wave: the scores of step k; with a
  // deferred PV product (three operand buffers, step s in buffer s % 3) the
  // PV product of step k - 1, whose probabilities the previous iteration
  // left; the dequantisation of step k + 1; the softmax of step k, and
  // without deferral (two buffers, s % 2) the PV product of step k; then the
  // barrier. At the barrier that opens iteration k every operand of step k is
  // in place and raw step k + 1 has landed; ring stage k % NS (raw step k,
  // dequantised in iteration k - 1) is free, and so is the buffer that step
  // k + 1 takes (it held step k - 2, or step k - 1 without deferral, both
  // last read in iteration k - 1).
  // Ring stage and operand buffer indices count from kbeg.
  const bool copier = w == 0;
  if (copier) {
    const DmaOffsets<D, COMPACT, FMT> dof = dma_offsets<D, COMPACT, FMT>(a.pool.st, a.pool.skv, lane);
#pragma unroll
    for (int s = 0; s < NS; ++s)
      dma_step<D, COMPACT, FMT>(ring + s * SG::STAGE, a.pool,
                                ids_for_step(bt_row, kbeg + s, kend, L, a.max_blocks, a.pool), h, (kbeg + s) * kStep,
                                dof);
  }
  StepIds nxt = ids_for_step(bt_row, kbeg + NS, kend, L, a.max_blocks, a.pool);
  wait_vmcnt<(NS - 1) * SG::NC>();  // the copier: step kbeg has landed (others: no-op)
  lds_barrier();
  if (kbeg < kend) prefill_dequant<D, FMT, PrefillGeo<D>::NW>(ring, ll, kbeg * kStep, L, j, w, op_lane);
  constexpr bool kDefer = PrefillGeo<D>::kDeferPV;
  // With the deferred PV product (head size 256, one workgroup per CU) the
  // waves dequantise after their products, which then queue on the matrix
  // unit while the vector ALU works; at the smaller head sizes several
  // workgroups share a CU and every wave dequantises first, which keeps the
  // scores out of registers during the dequantisation (measured on
  // mixed_serving 890 us against 904 us with the dequantisation first and
  // 912 us with half the waves each way; chunked_prefill 1616 us against
  // 1707 us with it last).
  const bool deq_first = !kDefer;
  h8 p[NT];
  bool pv_pending = false;  // wave-uniform: the previous step's PV product is due (deferral only)
  // operand buffers of steps k, k + 1 and (deferral) k - 1
  uint32_t buf_cur = 0, buf_next = OG::BYTES, buf_prev = 2 * OG::BYTES;
  if constexpr (D != 256) {
    // Iterations in the middle of the range, where every wave has columns,
    // step k needs no mask for any of them and a next step is dequantised
    // (needing none either), run without the branches on these conditions:
    // every wave of the CU runs those on the one scalar unit they share. The
    // bound is workgroup-uniform (wave 0's columns are the earliest, so its
    // first masked key is the lowest).
    const int wg_min_full = a.causal ? L - qlen + wg_col / grp + 1 : L;
    const bool all_cols = wg_col + (PrefillGeo<D>::NW - 1) * 16 * NT < ncols;
    int ks = wg_min_full / kStep;
    ks = ks < L / kStep - 1 ? ks : L / kStep - 1;
    ks = ks < kend - 1 ? ks : kend - 1;
    if (!all_cols) ks = kbeg;
    auto iteration = [&](const int k, auto steady_tag) {
      constexpr bool S = decltype(steady_tag)::value;
      wait_vmcnt<(NS - 2) * SG::NC>();  // the copier: step k + 1 has landed
      lds_barrier();
      const int kk = k - kbeg;
      if (copier) {
        // per-lane copy offsets: held for NVFP4 rows in 16-byte copies; in the
        // other copy forms at head size 128 derived again each step (held, they
        // would spill: the step loop there is at its register budget)
        int t = threadIdx.x;
        if constexpr (D == 128 && !(COMPACT && FMT == kNvfp4)) asm volatile("" : "+v"(t));
        const DmaOffsets<D, COMPACT, FMT> dof = dma_offsets<D, COMPACT, FMT>(a.pool.st, a.pool.skv, t & 63);
        dma_step<D, COMPACT, FMT>(ring + (kk % NS) * SG::STAGE, a.pool, nxt, h, (k + NS) * kStep, dof);
        // the ids of the copier's next step, read one iteration ahead (the
        // other waves never use them; the scalar unit is shared by the CU)
        nxt = ids_for_step(bt_row, k + NS + 1, kend, L, a.max_blocks, a.pool);
      }
      const int kb = k * kStep;
      const bool mine = S || kb < kw;
      f4 sc[2][NT];
      const bool deq = S || k + 1 < kend;
      if (deq_first && deq)
        prefill_dequant<D, FMT, PrefillGeo<D>::NW, S>(ring + ((kk + 1) % NS) * SG::STAGE, ll, kb + kStep, L, j, w,
                                                       op_lane + buf_next);
      if (mine) prefill_scores(W, op_lane + buf_cur, sc);
      if (kDefer && (S || pv_pending)) prefill_pv(W, op_lane + buf_prev, p);
      if (!deq_first && deq)
        prefill_dequant<D, FMT, PrefillGeo<D>::NW, S>(ring + ((kk + 1) % NS) * SG::STAGE, ll, kb + kStep, L, j, w,
                                                       op_lane + buf_next);
      if (mine) {
        W.softmax(sc, kb, j, !S && kb + kStep > min_full, p);
        if (!kDefer) prefill_pv(W, op_lane + buf_cur, p);
      }
      pv_pending = kDefer && mine;
      if constexpr (kDefer) {
        const uint32_t t = buf_prev;
        buf_prev = buf_cur;
        buf_cur = buf_next;
        buf_next = t;
      } else {
        const uint32_t t = buf_cur;
        buf_cur = buf_next;
        buf_next = t;
      }
    };
    int k = kbeg;
    for (; k < ks; ++k) iteration(k, SteadyTag<true>{});
    for (; k < kend; ++k) iteration(k, SteadyTag<false>{});
  } else {
    // head size 256: the plain loop (the two-form version above takes this
    // kernel to the whole register file, with spills, and even in its
    // general form alone compiles to a slower schedule)
    for (int k = kbeg; k < kend; ++k) {
      wait_vmcnt<(NS - 2) * SG::NC>();  // the copier: step k + 1 has landed
      lds_barrier();
      const int kk = k - kbeg;
      if (copier) {
        // per-lane copy offsets: held for NVFP4 rows in 16-byte copies; in the
        // other copy forms at head size 128 derived again each step (held, they
        // would spill: the step loop there is at its register budget)
        int t = threadIdx.x;
        if constexpr (D == 128 && !(COMPACT && FMT == kNvfp4)) asm volatile("" : "+v"(t));
        const DmaOffsets<D, COMPACT, FMT> dof = dma_offsets<D, COMPACT, FMT>(a.pool.st, a.pool.skv, t & 63);
        dma_step<D, COMPACT, FMT>(ring + (kk % NS) * SG::STAGE, a.pool, nxt, h, (k + NS) * kStep, dof);
        // the ids of the copier's next step, read one iteration ahead (the
        // other waves never use them; the scalar unit is shared by the CU)
        nxt = ids_for_step(bt_row, k + NS + 1, kend, L, a.max_blocks, a.pool);
      }
      const int kb = k * kStep;
      const bool mine = kb < kw;
      f4 sc[2][NT];
      const bool deq = k + 1 < kend;
      if (deq_first && deq)
        prefill_dequant<D, FMT, PrefillGeo<D>::NW>(ring + ((kk + 1) % NS) * SG::STAGE, ll, kb + kStep, L, j, w,
                                                    op_lane + buf_next);
      if (mine) prefill_scores(W, op_lane + buf_cur, sc);
      if (kDefer && pv_pending) prefill_pv(W, op_lane + buf_prev, p);
      if (!deq_first && deq)
        prefill_dequant<D, FMT, PrefillGeo<D>::NW>(ring + ((kk + 1) % NS) * SG::STAGE, ll, kb + kStep, L, j, w,
                                                    op_lane + buf_next);
      if (mine) {
        W.softmax(sc, kb, j, kb + kStep > min_full, p);
        if (!kDefer) prefill_pv(W, op_lane + buf_cur, p);
      }
      pv_pending = kDefer && mine;
      if constexpr (kDefer) {
        const uint32_t t = buf_prev;
        buf_prev = buf_cur;
        buf_cur = buf_next;
        buf_next = t;
      } else {
        const uint32_t t = buf_cur;
        buf_cur = buf_next;
        buf_next = t;
      }
    }
  }
  if (kDefer && pv_pending) prefill_pv(W, op_lane + buf_prev, p);
  wait_vmcnt<0>();

  // (split jobs run the main column tiling only)
  if (NT == PrefillGeo<D>::NT && pt.n > 1) {
    // Every part leaves its state; the last to arrive (the count before its
    // increment is n - 1) merges the n states in part order, so the result
    // does not depend on the order of arrival, and resets the counter. The
    // states travel through agent-coherent stores and loads (they bypass the
    // per-XCD L2), so the hand-off needs every store complete before the
    // counter moves, not an L2 flush.
    if constexpr (NT == PrefillGeo<D>::NT) prefill_put_part<D, NT>(a, W, pt, w, lane);
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0)
      *s_flag = (__hip_atomic_fetch_add(&a.ws_cnt[pt.cnt], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 (uint32_t)(pt.n - 1))
                    ? 1
                    : 0;
    __syncthreads();
    const bool last = *s_flag != 0;
    __syncthreads();  // every wave has read the flag before the ring is written again
    if (!last) return;
    if constexpr (NT == PrefillGeo<D>::NT) prefill_merge_parts<D, NT>(a, W, pt, w, lane);
    if (threadIdx.x == 0)
      __hip_atomic_store(&a.ws_cnt[pt.cnt], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  const float gv = *a.v_scale;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const float lt = W.lsum(n);
    const int c = col_base + 16 * n + i;
    if (c < ncols) {
      const int tok = c / grp, g = c - (c / grp) * grp;
      const int64_t row = ((int64_t)(q0 + tok) * a.hq + h * grp + g) * D;
      if constexpr (FP8OUT)
        store_column_fp8<D>(a.out8 + row, W.acc[n], lt > 0.0f ? gv / lt : 0.0f, *a.o_scale, j);
      else
        store_column<D>(a.out + row, W.acc[n], lt > 0.0f ? gv / lt : 0.0f, j);
    }
  }
}

// ---------------------------------------------------------------------------
// Key split of the prefill grid. The grid's dispatch order stays: kv heads,
// then column blocks from the last one back, then sequences longest first,
// so the workgroups of one sequence run side by side and read the same keys
// from the same L2 (measured at chunked_prefill: 94% L2 hits in this order
// against 13-20% when every workgroup took an equal share of one line of all
// the jobs' steps). A job of the sequence of rank r is cut into P_r
// consecutive key ranges, each its own workgroup: grid z runs over slices,
// the P_r parts of rank 0, then those of rank 1, ..., so a rank's parts run
// side by side too, and the slices past the last part (the grid holds as
// many as the records could need) are empty and come last. P_r is guided by
// the work left: the parts are about max(kPrefillMinPart, 2 R / (3 slots))
// steps, R the steps of ranks r .. last and slots the workgroups the device
// holds at once, so the long early ranks stay whole and the last rounds are
// cut fine enough to end together. Cut jobs need part records; when the
// tail's records would exceed the workspace's, the earlier of those ranks
// stay whole, and so do they when the cut ranks' extra slices would exceed
// the grid's. One workgroup (prefill_plan_kernel) derives the slices, with
// each rank's sequence, P_r and record and counter bases, into a table the
// prefill workgroups read.
// ---------------------------------------------------------------------------
constexpr int kPrefillParts = 3;     // parts per job at most
constexpr int kPrefillMinPart = 32;  // steps

struct PrefillPlanRow {  // one grid z slice
  int32_t seq;       // sequence of the slice's rank
  int32_t parts;     // P_r (0: an empty slice)
  int32_t part;      // which part of the rank's jobs
  int32_t rec_base;  // first part record of the rank's cut jobs
  int32_t cnt_base;  // first arrival counter of the rank's cut jobs
  int32_t pad[3];
};

// A part's state in the workspace, lane-major so that every store and load
// is a whole 64-lane row: per (wave, column tile, accumulator quad) the
// lanes' 16-byte O^T quads, then per (wave, column tile) the lanes' (running
// max, running sum) pairs.
template <int D>
struct PrefillPartGeo {
  static constexpr int NW = PrefillGeo<D>::NW, NT = PrefillGeo<D>::NT, DPL = Geo<D>::DPL;
  static constexpr int ACC_BYTES = NW * NT * DPL * 64 * 16;
  static constexpr int BYTES = ACC_BYTES + NW * NT * 64 * 8;
  static_assert(BYTES % 256 == 0, "records stay 256-byte aligned");
};


template <int D>
__device__ __forceinline__ rsrc_t prefill_part_rsrc(const PrefillArgs& a, const PrefillPart& pt, int p) {
  using PG = PrefillPartGeo<D>;
  return make_rsrc(reinterpret_cast<const uint8_t*>(a.ws_part) + (int64_t)(pt.rec0 + p) * PG::BYTES, PG::BYTES);
}

template <int D, int NT>
__device__ __forceinline__ void prefill_put_part(const PrefillArgs& a, const WaveAttn<D, NT>& W, const PrefillPart& pt, int w, int lane) {
  using PG = PrefillPartGeo<D>;
  static_assert(NT == PG::NT, "split jobs use the main column tiling");
  constexpr int DPL = Geo<D>::DPL;
  const rsrc_t r = prefill_part_rsrc<D>(a, pt, pt.self);
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int t = 0; t < DPL; ++t)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, W.acc[n][t]), r,
                                             (uint32_t)((((w * NT + n) * DPL + t) * 64 + lane) * 16), 0, 16 /* sc1 */);
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    float lv;
    if constexpr (WaveAttn<D, NT>::kMfmaSum) lv = W.lacc[n][0];
    else lv = W.l[n];
    // two 4-byte stores: a pair built from W.m[n] would be read as one
    // 8-byte load across the array, which keeps W.m out of registers
    const uint32_t off = (uint32_t)(PG::ACC_BYTES + ((w * NT + n) * 64 + lane) * 8);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, W.m[n]), r, off, 0, 16 /* sc1 */);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lv), r, off + 4, 0, 16 /* sc1 */);
  }
}

// The job's state from its n parts, in part order: the maximum over the
// parts' running maxima, then the sum of each part's accumulators and
// running sum weighted by 2^(its max - that maximum). Each lane merges its
// own entries (every part ran the same columns on the same lanes).
template <int D, int NT>
__device__ __forceinline__ void prefill_merge_parts(const PrefillArgs& a, WaveAttn<D, NT>& W, const PrefillPart& pt, int w, int lane) {
  using PG = PrefillPartGeo<D>;
  constexpr int DPL = Geo<D>::DPL;
  float M[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) M[n] = -__builtin_inff();
  for (int p = 0; p < pt.n; ++p) {
    const rsrc_t r = prefill_part_rsrc<D>(a, pt, p);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const u32x2 ml = __builtin_amdgcn_raw_buffer_load_b64(r, (uint32_t)(PG::ACC_BYTES + ((w * NT + n) * 64 + lane) * 8),
                                                            0, 16 /* sc1 */);
      M[n] = __builtin_fmaxf(M[n], __uint_as_float(ml[0]));
    }
  }
  float lt[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    lt[n] = 0.0f;
#pragma unroll
    for (int t = 0; t < DPL; ++t) W.acc[n][t] = f4{0.f, 0.f, 0.f, 0.f};
  }
  for (int p = 0; p < pt.n; ++p) {
    const rsrc_t r = prefill_part_rsrc<D>(a, pt, p);
    u32x2 ml[NT];
    f4 v[NT][DPL];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      ml[n] = __builtin_amdgcn_raw_buffer_load_b64(r, (uint32_t)(PG::ACC_BYTES + ((w * NT + n) * 64 + lane) * 8), 0,
                                                   16 /* sc1 */);
#pragma unroll
      for (int t = 0; t < DPL; ++t)
        v[n][t] = __builtin_bit_cast(
            f4, __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)((((w * NT + n) * DPL + t) * 64 + lane) * 16), 0,
                                                      16 /* sc1 */));
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const float mp = __uint_as_float(ml[n][0]);
      const float f = (mp == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mp - M[n]);
      lt[n] += f * __uint_as_float(ml[n][1]);
#pragma unroll
      for (int t = 0; t < DPL; ++t) W.acc[n][t] += f * v[n][t];
    }
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    W.m[n] = M[n];
    if constexpr (WaveAttn<D, NT>::kMfmaSum) W.lacc[n] = f4{lt[n], lt[n], lt[n], lt[n]};
    else W.l[n] = lt[n];
  }
}

__device__ __forceinline__ int64_t wave_incl_scan64(int64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t t = __shfl_up(v, d);
    if (lane >= d) v += t;
  }
  return v;
}


// Block-wide exclusive scans of K int64 values at once (one pair of
// barriers for all K); also returns the totals. s_red: K * NW int64.
template <int NW, int K>
__device__ __forceinline__ void block_excl_scan64x(int64_t (&v)[K], int64_t* s_red, int64_t (&total)[K]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int64_t incl[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    incl[k] = wave_incl_scan64(v[k]);
    if (lane == 63) s_red[k * NW + w] = incl[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < K; ++k) {
    int64_t off = 0;
    total[k] = 0;
#pragma unroll
    for (int u = 0; u < NW; ++u) {
      const int64_t t = s_red[k * NW + u];
      off += (u < w) ? t : 0;
      total[k] += t;
    }
    v[k] = incl[k] - v[k] + off;
  }
  __syncthreads();
}

// The plan (one workgroup of kPlanThreads). LDS: per rank its work (int64),
// sequence, longest job and column blocks; per sequence its clamped length
// and chunk length (all loaded in one pass).
constexpr int kPlanThreads = 256;

__host__ __device__ inline size_t prefill_plan_lds_bytes(int B) {
  return (size_t)B * 8 + (size_t)B * 4 * 5 + 3 * (kPlanThreads / 64) * 8 + 16;
}

template <int D>
__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(PrefillArgs a, PrefillPlanRow* plan, int slots,
                                                                    int rec_cap, int extra_cap) {
  constexpr int kCols = PrefillGeo<D>::kCols;
  constexpr int NWP = kPlanThreads / 64;
  extern __shared__ __align__(16) char smem[];
  const int B = a.num_seqs;
  const int hkv = a.pool.hkv;
  int64_t* s_w = reinterpret_cast<int64_t*>(smem);  // [B] work of rank r
  int* s_len = reinterpret_cast<int*>(s_w + B);     // [B] clamped length of sequence b
  int* s_qlen = s_len + B;                          // [B] chunk length of sequence b
  int* s_seq = s_qlen + B;                          // [B] sequence of rank r
  int* s_nmax = s_seq + B;                          // [B] steps of rank r's longest job
  int* s_nblk = s_nmax + B;                         // [B] column blocks of rank r
  int64_t* s_red = reinterpret_cast<int64_t*>(s_nblk + B + (B & 1));  // [3 NWP], 8-byte aligned

  for (int t = threadIdx.x; t < B; t += kPlanThreads) {
    int q0, qlen, L;
    prefill_seq_geom(a, t, q0, qlen, L);
    s_len[t] = L;
    s_qlen[t] = qlen;
  }
  __syncthreads();
  // ranks: longest first, ties in index order (the order prefill_seq_of_rank
  // gives); index order for batches the grid does not rank
  for (int t = threadIdx.x; t < B; t += kPlanThreads) {
    int rank = t;
    if (a.longest_first) {
      const int kt = s_len[t];
      rank = 0;
      for (int u = 0; u < B; ++u) {
        const int ku = s_len[u];
        rank += (ku > kt || (ku == kt && u < t)) ? 1 : 0;
      }
    }
    s_seq[rank] = t;
  }
  __syncthreads();
  // each thread a contiguous run of ranks
  const int per = (B + kPlanThreads - 1) / kPlanThreads;
  const int r0 = threadIdx.x * per;
  const int r1 = (r0 + per < B) ? r0 + per : B;
  const int grp = a.grp;
  const int dq = kCols / grp, dr = kCols - (kCols / grp) * grp;  // kCols = dq grp + dr
  int64_t sc1[1] = {0};
  for (int r = r0; r < r1; ++r) {
    const int b = s_seq[r];
    const int L = s_len[b], qlen = s_qlen[b];
    const int nblk = ceil_div(qlen * grp, kCols);
    int64_t work = 0;
    int nmax = 0;
    if (!a.causal || nblk == 0) {
      nmax = nblk > 0 ? max(1, ceil_div(L, kStep)) : 0;  // every block sees all L keys
      work = (int64_t)nblk * nmax;
    } else {
      // prefill_job_steps of each block without a division per block: the
      // token of block cb's last column is tq = ((cb + 1) kCols - 1) / grp,
      // stepped by dq (plus one when the remainder tr carries); the last
      // block ends at the chunk's last token
      int tq = (kCols - 1) / grp, tr = (kCols - 1) - ((kCols - 1) / grp) * grp;
      for (int cb = 0; cb < nblk; ++cb) {
        const int tok = cb == nblk - 1 ? qlen - 1 : tq;
        int kmax = L - qlen + tok + 1;
        kmax = kmax > L ? L : (kmax < 0 ? 0 : kmax);
        const int n = max(1, (kmax + kStep - 1) / kStep);
        work += n;
        nmax = n > nmax ? n : nmax;
        tq += dq;
        tr += dr;
        if (tr >= grp) {
          tr -= grp;
          ++tq;
        }
      }
    }
    s_w[r] = work * hkv;
    s_nmax[r] = nmax;
    s_nblk[r] = nblk;
    sc1[0] += work * hkv;
  }
  int64_t total[1];
  block_excl_scan64x<NWP, 1>(sc1, s_red, total);
  int64_t run = sc1[0];
  // P_r from the work of ranks r .. last
  constexpr int kPer = kPrefillSplitSeqsMax / kPlanThreads;
  static_assert(kPer * kPlanThreads == kPrefillSplitSeqsMax, "ranks per thread");
  int P[kPer];
  int64_t sc2[2] = {0, 0};  // records, extra slices
  for (int r = r0; r < r1; ++r) {
    const int64_t rest = total[0] - run;  // ranks r .. last
    run += s_w[r];
    int64_t part = (2 * rest + 3 * (int64_t)slots - 1) / (3 * (int64_t)slots);
    part = part < kPrefillMinPart ? kPrefillMinPart : part;
    int pr = (int)((s_nmax[r] + part - 1) / part);
    pr = pr < 1 ? 1 : (pr > kPrefillParts ? kPrefillParts : pr);
    P[r - r0] = pr;
    sc2[0] += pr > 1 ? (int64_t)s_nblk[r] * hkv * pr : 0;
    sc2[1] += pr - 1;
  }
  // tail first: a rank is cut only if its records and extra slices and those
  // of every later cut rank fit in rec_cap and extra_cap
  int64_t tot2[2];
  block_excl_scan64x<NWP, 2>(sc2, s_red, tot2);
  int64_t rec_run = sc2[0], ext_run = sc2[1];
  int64_t sc3[3] = {0, 0, 0};  // kept records, counters, extra slices
  for (int r = r0; r < r1; ++r) {
    const int64_t rec = P[r - r0] > 1 ? (int64_t)s_nblk[r] * hkv * P[r - r0] : 0;
    const int64_t ext = P[r - r0] - 1;
    if (tot2[0] - rec_run > rec_cap || tot2[1] - ext_run > extra_cap) P[r - r0] = 1;  // ranks r .. last
    rec_run += rec;
    ext_run += ext;
    sc3[0] += P[r - r0] > 1 ? (int64_t)s_nblk[r] * hkv * P[r - r0] : 0;
    sc3[1] += P[r - r0] > 1 ? (int64_t)s_nblk[r] * hkv : 0;
    sc3[2] += P[r - r0] - 1;
  }
  int64_t tot3[3];
  block_excl_scan64x<NWP, 3>(sc3, s_red, tot3);
  int64_t rec_base = sc3[0], cnt_base = sc3[1];
  int64_t z = sc3[2] + r0;  // first slice of rank r0
  for (int r = r0; r < r1; ++r) {
    PrefillPlanRow row = {};
    row.seq = s_seq[r];
    row.parts = P[r - r0];
    row.rec_base = (int32_t)rec_base;
    row.cnt_base = (int32_t)cnt_base;
    for (int p = 0; p < row.parts; ++p) {
      row.part = p;
      plan[z + p] = row;
    }
    z += row.parts;
    if (row.parts > 1) {
      rec_base += (int64_t)s_nblk[r] * hkv * row.parts;
      cnt_base += (int64_t)s_nblk[r] * hkv;
    }
  }
  // the slices past the last part: empty
  const PrefillPlanRow none = {};
  for (int64_t e = B + tot3[2] + threadIdx.x; e < (int64_t)B + extra_cap; e += kPlanThreads) plan[e] = none;
}

template <int D, int NT, bool COMPACT, bool FP8OUT, int FMT>
__global__ __launch_bounds__(64 * PrefillGeo<D>::NW) __attribute__((amdgpu_waves_per_eu(PrefillOcc<D, COMPACT, FP8OUT, FMT>::waves))) void prefill_kernel(
    PrefillArgs a) {
  using SG = StageGeo<D, COMPACT, FMT>;
  constexpr int NS = PrefillStages<D, COMPACT, FMT>::NS;
  extern __shared__ __align__(16) char smem[];
  uint8_t* ring = reinterpret_cast<uint8_t*>(smem);  // [NS] raw steps
  uint8_t* opbuf = ring + NS * SG::STAGE;             // [kOpBufs] operand buffers

  // Dispatch order (x fastest): kv heads, then column blocks from the last
  // one back (under a causal mask the later columns see the most keys), then
  // sequences longest first, so the longest jobs start first. With the key
  // split, grid z runs over the plan's slices (a rank's parts in turn; an
  // empty slice has nothing to do).
  const int h = blockIdx.x;
  const int cb = (int)(gridDim.y - 1 - blockIdx.y);
  int b, parts = 1, part = 0, rec_base = 0, cnt_base = 0;
  if (a.plan != nullptr) {
    const PrefillPlanRow row = a.plan[blockIdx.z];
    parts = __builtin_amdgcn_readfirstlane(row.parts);
    if (parts == 0) return;
    part = __builtin_amdgcn_readfirstlane(row.part);
    b = __builtin_amdgcn_readfirstlane(row.seq);
    rec_base = __builtin_amdgcn_readfirstlane(row.rec_base);
    cnt_base = __builtin_amdgcn_readfirstlane(row.cnt_base);
  } else {
    b = a.longest_first ? prefill_seq_of_rank(a, blockIdx.z, reinterpret_cast<int*>(ring)) : (int)blockIdx.z;
  }
  int q0, qlen, L;
  prefill_seq_geom(a, b, q0, qlen, L);
  const int ncols = qlen * a.grp;
  constexpr int kCols = PrefillGeo<D>::NW * 16 * NT;  // columns per workgroup
  const PrefillPart whole = {1, 0, 0, 0};
  if (cb * kCols < ncols) {
    int k_lo = 0, k_hi = INT32_MAX;
    PrefillPart pt = whole;
    if (parts > 1) {
      // part p of the job's steps; record (cb hkv + h) P + p and counter
      // cb hkv + h of the rank's block
      const int n = prefill_job_steps<kCols>(a.causal, a.grp, L, qlen, cb * kCols);
      k_lo = (int)((int64_t)n * part / parts);
      k_hi = (int)((int64_t)n * (part + 1) / parts);
      pt.n = parts;
      pt.self = part;
      pt.rec0 = rec_base + (cb * a.pool.hkv + h) * parts;
      pt.cnt = cnt_base + cb * a.pool.hkv + h;
    }
    prefill_columns<D, NT, COMPACT, FP8OUT, FMT>(a, ring, opbuf, b, h, q0, qlen, L, cb * kCols, k_lo, k_hi, pt,
                                                 reinterpret_cast<int*>(ring));
  }
  // The grid is sized from the host's max_q_len hint. If a chunk is longer,
  // the grid's last column block takes the columns past the grid, one
  // 16-column tile per wave at a time (this rarely taken path then needs no
  // more registers than the main one), so a wrong hint costs speed, never
  // rows. The workgroup's waves take the branch and the loop together.
  if (cb == (int)gridDim.y - 1 && part == 0)
    for (int c0 = (int)gridDim.y * kCols; c0 < ncols; c0 += PrefillGeo<D>::NW * 16)
      prefill_columns<D, 1, COMPACT, FP8OUT, FMT>(a, ring, opbuf, b, h, q0, qlen, L, c0, 0, INT32_MAX, whole, nullptr);
}

template <int D, bool COMPACT, int FMT>
size_t prefill_lds_bytes() {
  return (size_t)PrefillStages<D, COMPACT, FMT>::NS * StageGeo<D, COMPACT, FMT>::STAGE + PrefillGeo<D>::kOpBufs * OpGeo<D>::BYTES;
}

template <int D, int NT, int FMT>
static void launch_prefill_fp8(const PrefillArgs& a, const dim3& grid, hipStream_t stream) {
  const size_t lds = prefill_lds_bytes<D, false, FMT>();
  if (a.o_scale == nullptr)
    prefill_kernel<D, NT, false, false, FMT><<<grid, 64 * PrefillGeo<D>::NW, lds, stream>>>(a);
  else
    prefill_kernel<D, NT, false, true, FMT><<<grid, 64 * PrefillGeo<D>::NW, lds, stream>>>(a);
}

// Column blocks on the grid's y axis: from the host's max_q_len hint (at
// most 65535; a longer chunk's remaining columns go to the last block's loop)
template <int D, int NT>
static int64_t prefill_grid_y(int grp, int max_q_len) {
  const int64_t cols = (int64_t)(max_q_len > 0 ? max_q_len : 1) * grp;
  const int64_t per_wg = PrefillGeo<D>::NW * 16 * NT;
  const int64_t gy = (cols + per_wg - 1) / per_wg;
  return gy > 65535 ? 65535 : gy;
}

template <int D, int NT>
static hipError_t launch_prefill_t(const PrefillArgs& a, int num_seqs, int max_q_len, int fmt, int extra_slices,
                                   hipStream_t stream) {
  // max_q_len only sizes the grid: workgroups loop over the column tiles of
  // the actual chunk lengths, so any hint (even 0) gives every row
  const int64_t gy = prefill_grid_y<D, NT>(a.grp, max_q_len);
  const unsigned gz = (unsigned)num_seqs + (a.plan != nullptr ? (unsigned)extra_slices : 0u);
  const dim3 grid((unsigned)a.pool.hkv, (unsigned)gy, gz);
  if (fmt == kFp8E4M3 || fmt == kFp8E5M2) {
    // FP8 rows are copied in 16-byte chunks whatever their stride
    if (fmt == kFp8E4M3)
      launch_prefill_fp8<D, NT, kFp8E4M3>(a, grid, stream);
    else
      launch_prefill_fp8<D, NT, kFp8E5M2>(a, grid, stream);
    return hipGetLastError();
  }
  // 16-byte copies need contiguous, 16-byte aligned page rows (HND layout)
  const bool compact = a.pool.st == D / 2 + D / 16 && a.pool.sb % 16 == 0 && a.pool.skv % 16 == 0 &&
                       a.pool.sh % 16 == 0 && (reinterpret_cast<uintptr_t>(a.pool.data) % 16) == 0;
  const bool fp8 = a.o_scale != nullptr;
  if (compact && !fp8)
    prefill_kernel<D, NT, true, false, kNvfp4><<<grid, 64 * PrefillGeo<D>::NW, prefill_lds_bytes<D, true, kNvfp4>(), stream>>>(a);
  else if (compact)
    prefill_kernel<D, NT, true, true, kNvfp4><<<grid, 64 * PrefillGeo<D>::NW, prefill_lds_bytes<D, true, kNvfp4>(), stream>>>(a);
  else if (!fp8)
    prefill_kernel<D, NT, false, false, kNvfp4><<<grid, 64 * PrefillGeo<D>::NW, prefill_lds_bytes<D, false, kNvfp4>(), stream>>>(a);
  else
    prefill_kernel<D, NT, false, true, kNvfp4><<<grid, 64 * PrefillGeo<D>::NW, prefill_lds_bytes<D, false, kNvfp4>(), stream>>>(a);
  return hipGetLastError();
}

// Workgroups per CU the prefill kernel holds (LDS and register budget):
// head size 256 one 8-wave workgroup, 128 three 4-wave ones, 64 two. The key
// split's plan sizes its parts for that many slots, and its workspace holds
// two part records per slot.
static int prefill_wg_per_cu(int head_size) { return head_size == 256 ? 1 : head_size == 128 ? 3 : 2; }

static int64_t prefill_slots(int head_size) { return (int64_t)prefill_wg_per_cu(head_size) * device_cus(); }

// slices: B ranks plus at most 2 B extra parts
constexpr int64_t kPrefillPlanBytes = 3 * (int64_t)kPrefillSplitSeqsMax * sizeof(PrefillPlanRow);

static int64_t prefill_counter_bytes(int head_size) { return ((prefill_slots(head_size) * 4 + 255) / 256) * 256; }

static int64_t prefill_part_bytes(int head_size) {
  switch (head_size) {
    case 64: return PrefillPartGeo<64>::BYTES;
    case 128: return PrefillPartGeo<128>::BYTES;
    case 256: return PrefillPartGeo<256>::BYTES;
    default: return 0;
  }
}

// Workspace: [plan slices of 3 kPrefillSplitSeqsMax][arrival counters, one
// per slot][part records, two per slot]. Cut jobs have at least two parts,
// so the counters cover every cut job the records allow.
size_t prefill_workspace_bytes(int head_size) {
  const int64_t part = prefill_part_bytes(head_size);
  if (part == 0) return 0;
  return (size_t)(kPrefillPlanBytes + prefill_counter_bytes(head_size) + 2 * prefill_slots(head_size) * part);
}

hipError_t launch_prefill(const Pool& pool, int head_size, const void* q, int64_t q_st, int64_t q_sh,
                          int num_q_heads, const int32_t* cu_q, int32_t max_q_len, int32_t total_q,
                          const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                          int32_t num_seqs, int32_t max_seq_len, const float* k_scale, const float* v_scale,
                          float sm_scale, int causal, const float* o_scale, void* out, int fmt, void* workspace,
                          hipStream_t stream) {
  (void)max_seq_len;
  if (num_seqs == 0 || total_q <= 0) return hipSuccess;
  PrefillArgs a;
  a.pool = pool;
  a.q = static_cast<const uint16_t*>(q);
  a.q_st = q_st;
  a.q_sh = q_sh;
  a.hq = num_q_heads;
  a.grp = num_q_heads / pool.hkv;
  a.cu_q = cu_q;
  a.total_q = total_q;
  a.bt = block_table;
  a.max_blocks = max_blocks;
  a.seq_lens = seq_lens;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.sm_scale = sm_scale;
  a.causal = causal;
  a.out = static_cast<uint16_t*>(out);
  a.out8 = static_cast<uint8_t*>(out);
  a.o_scale = o_scale;
  a.num_seqs = num_seqs;
  a.longest_first = (num_seqs > 1 && num_seqs <= kPrefillRankMax) ? 1 : 0;
  a.plan = nullptr;
  a.ws_cnt = nullptr;
  a.ws_part = nullptr;
  int extra = 0;
  if (workspace != nullptr) {
    // the key split: the plan first (one workgroup), then the grid with
    // kPrefillParts part slots per sequence
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    PrefillPlanRow* plan = reinterpret_cast<PrefillPlanRow*>(ws);
    a.ws_cnt = reinterpret_cast<uint32_t*>(ws + kPrefillPlanBytes);
    a.ws_part = reinterpret_cast<float*>(ws + kPrefillPlanBytes + prefill_counter_bytes(head_size));
    const int slots = (int)prefill_slots(head_size);
    const int rec_cap = 2 * slots;
    // extra slices: a cut rank of gy column blocks takes at least 2 gy hkv
    // records per extra part, so rec_cap / (gy hkv) extra slices cover the
    // records' worth (the plan keeps within it; at most 2 per sequence)
    int64_t gy = head_size == 64    ? prefill_grid_y<64, PrefillGeo<64>::NT>(a.grp, max_q_len)
                 : head_size == 128 ? prefill_grid_y<128, PrefillGeo<128>::NT>(a.grp, max_q_len)
                                    : prefill_grid_y<256, PrefillGeo<256>::NT>(a.grp, max_q_len);
    int64_t x = rec_cap / (gy * pool.hkv);
    x = x < 1 ? 1 : (x > 2 * (int64_t)num_seqs ? 2 * (int64_t)num_seqs : x);
    extra = (int)x;
    const size_t plds = prefill_plan_lds_bytes(num_seqs);
    switch (head_size) {
      case 64: prefill_plan_kernel<64><<<1, kPlanThreads, plds, stream>>>(a, plan, slots, rec_cap, extra); break;
      case 128: prefill_plan_kernel<128><<<1, kPlanThreads, plds, stream>>>(a, plan, slots, rec_cap, extra); break;
      case 256: prefill_plan_kernel<256><<<1, kPlanThreads, plds, stream>>>(a, plan, slots, rec_cap, extra); break;
      default: return hipErrorInvalidValue;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.plan = plan;
  }
  switch (head_size) {
    case 64: return launch_prefill_t<64, PrefillGeo<64>::NT>(a, num_seqs, max_q_len, fmt, extra, stream);
    case 128: return launch_prefill_t<128, PrefillGeo<128>::NT>(a, num_seqs, max_q_len, fmt, extra, stream);
    case 256: return launch_prefill_t<256, PrefillGeo<256>::NT>(a, num_seqs, max_q_len, fmt, extra, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nvfp4kv
