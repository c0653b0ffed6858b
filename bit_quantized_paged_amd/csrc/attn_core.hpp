// Wave-level paged attention engine over the NVFP4 cache (gfx950).
//
// Attention reads the packed pages and their block-scale bytes directly
// [P40177 "Implementation breakdown" 1 and 3: prefill/decode wrappers run on
// the packed cache plus its block-scale view].
//
// A wave owns 16*NT "query columns" (q rows; in decode the GQA heads of one
// token) and walks the keys of one sequence/kv head in steps of 32 keys
// (two 16-key subtiles). With lane = 16*j + i:
//
//  * S^T = K^ . Q^T on v_mfma_f32_16x16x32_f16. Lane (i, j) loads key i's
//    code bytes [j*D/8, (j+1)*D/8) with one wide load; chunk c of the
//    reduction uses its word c. Q is laid out with the same (j, c) -> element
//    map, so the contraction is over a fixed permutation of d and needs no
//    shuffles. Codes become f16 with the hardware FP4 convert and are scaled
//    by their E4M3 block scale (both exact in f16), g_K is folded into the
//    per-column score factor.
//  * The MFMA result gives lane (i, j) the scores of column i for keys
//    4j..4j+3 of the subtile: the row max needs two cross-lane steps and the
//    probabilities are already in the B-operand layout of the PV product.
//  * O^T = V^ T . P^T on the same MFMA. Lane (i, j) needs, for one d, keys
//    4j..4j+3 of each subtile: it loads D/32 bytes of each of those four rows
//    (d in [i*D/16, (i+1)*D/16)), and a nibble transpose (two masks and a
//    shift per key pair) puts the two keys of a pair into one byte, which the
//    FP4 convert turns into the f16 pair the MFMA wants. PV product t covers
//    d = i*D/16 + t.
//  * Online softmax in base 2 with a lazy maximum: the running max of a
//    column only moves (and the accumulators are only rescaled) when a score
//    exceeds it by more than 8, so probabilities stay <= 256 in f16.
#pragma once

#include "device_common.hpp"

namespace nvfp4kv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyMax = 8.0f;

template <int D>
struct Geo {
  static constexpr int DPL = D / 16;                // V: d per lane = PV products
  static constexpr int KW = D / 32;                 // K: code words per lane = QK chunks
  static constexpr int VB = DPL / 2;                // V: code bytes per key per lane
  static constexpr int VW = VB >= 4 ? VB / 4 : 1;   // V: words per key per lane
};

template <int D>
struct SubRaw {  // raw bytes of one 16-key subtile for one lane
  uint32_t k[Geo<D>::KW];
  uint32_t ks;
  uint32_t v[4][Geo<D>::VW];
  uint32_t vs[4];
};

template <int D>
__device__ __forceinline__ void zero_sub(SubRaw<D>& R) {
#pragma unroll
  for (int c = 0; c < Geo<D>::KW; ++c) R.k[c] = 0;
  R.ks = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int w = 0; w < Geo<D>::VW; ++w) R.v[r][w] = 0;
    R.vs[r] = 0;
  }
}

// Byte offsets of this lane's loads inside a 16-row subtile; they depend only
// on the lane and the row stride, so a wave computes them once.
template <int D>
struct LaneOffsets {
  uint32_t k, ks, v, vs;  // v / vs: row 4j of the lane's four value rows
  int32_t st;             // row stride; value row 4j + r adds r * st (scalar)
};

template <int D>
__device__ __forceinline__ LaneOffsets<D> lane_offsets(int64_t st, int i, int j) {
  LaneOffsets<D> o;
  const uint32_t s = (uint32_t)st;
  o.k = i * s + j * (D / 8);
  o.ks = i * s + D / 2 + j * (D / 64);
  o.v = 4 * j * s + i * Geo<D>::VB;
  o.vs = 4 * j * s + D / 2 + (i * Geo<D>::DPL) / 16;
  o.st = (int32_t)st;
  return o;
}

// Pages are read with raw buffer loads: a wave-uniform descriptor per
// subtile (base = first row of the subtile, size = the bytes its 16 rows
// span) plus the lane offsets above. A subtile with nothing to read gets size
// 0, which makes the hardware return zeros without touching memory, so the
// loads of a step are issued unconditionally and every access is
// range-checked against its own page.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw (unformatted) buffer, gfx9 family

__device__ __forceinline__ rsrc_t make_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, bytes, kRsrcWord3);
}

template <int D>
__device__ __forceinline__ void load_sub(SubRaw<D>& R, rsrc_t kr, rsrc_t vr, const LaneOffsets<D>& o) {
  if constexpr (D == 64) {
    const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(kr, o.k, 0, 0);
    R.k[0] = w[0];
    R.k[1] = w[1];
    R.ks = __builtin_amdgcn_raw_buffer_load_b8(kr, o.ks, 0, 0);
  } else if constexpr (D == 128) {
    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(kr, o.k, 0, 0);
    R.k[0] = w[0];
    R.k[1] = w[1];
    R.k[2] = w[2];
    R.k[3] = w[3];
    R.ks = __builtin_amdgcn_raw_buffer_load_b16(kr, o.ks, 0, 0);
  } else {
    const u32x4 w0 = __builtin_amdgcn_raw_buffer_load_b128(kr, o.k, 0, 0);
    const u32x4 w1 = __builtin_amdgcn_raw_buffer_load_b128(kr, o.k + 16, 0, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      R.k[c] = w0[c];
      R.k[4 + c] = w1[c];
    }
    R.ks = __builtin_amdgcn_raw_buffer_load_b32(kr, o.ks, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int so = r * o.st;
    if constexpr (D == 64) {
      R.v[r][0] = __builtin_amdgcn_raw_buffer_load_b16(vr, o.v, so, 0);
    } else if constexpr (D == 128) {
      R.v[r][0] = __builtin_amdgcn_raw_buffer_load_b32(vr, o.v, so, 0);
    } else {
      const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(vr, o.v, so, 0);
      R.v[r][0] = w[0];
      R.v[r][1] = w[1];
    }
    R.vs[r] = __builtin_amdgcn_raw_buffer_load_b8(vr, o.vs, so, 0);
  }
}

// Zero the value rows of keys >= L (unwritten rows may hold NaN scale bytes;
// their probability is 0 but 0 * NaN would poison the accumulator).
template <int D>
__device__ __forceinline__ void mask_sub_values(SubRaw<D>& R, int key0, int L, int j) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const bool ok = key0 + 4 * j + r < L;
#pragma unroll
    for (int w = 0; w < Geo<D>::VW; ++w) R.v[r][w] = ok ? R.v[r][w] : 0u;
    R.vs[r] = ok ? R.vs[r] : 0u;
  }
}

// Dequantised K chunk c of this lane: 8 f16 = codes * block scale.
template <int D, int C>
__device__ __forceinline__ h8 k_chunk(const SubRaw<D>& R) {
  constexpr int SI = C / 2;  // scale byte index within the lane's scales
  const h2 sp = (SI < 2) ? fp8x2_to_h2<false>(R.ks) : fp8x2_to_h2<true>(R.ks);
  const _Float16 s = sp[SI & 1];
  const h2 ss = {s, s};
  const uint32_t w = R.k[C];
  const h2 a0 = fp4x2_to_h2<0>(w) * ss;
  const h2 a1 = fp4x2_to_h2<1>(w) * ss;
  const h2 a2 = fp4x2_to_h2<2>(w) * ss;
  const h2 a3 = fp4x2_to_h2<3>(w) * ss;
  return h8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
}

// Value rows of one subtile rearranged so that each byte holds the codes of
// two keys (4j+2p, 4j+2p+1) at one d.
template <int D>
struct VPairs {
  uint32_t ev[2][Geo<D>::VW];  // [pair][word]: byte b <-> d offset 8w + 2b
  uint32_t od[2][Geo<D>::VW];  //                byte b <-> d offset 8w + 2b + 1
  h2 s[2];                     // block scales of the pair's two keys
};

template <int D>
__device__ __forceinline__ void make_pairs(const SubRaw<D>& R, VPairs<D>& P) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int w = 0; w < Geo<D>::VW; ++w) {
      const uint32_t a = R.v[2 * p][w];
      const uint32_t b = R.v[2 * p + 1][w];
      P.ev[p][w] = (a & 0x0F0F0F0Fu) | ((b & 0x0F0F0F0Fu) << 4);
      P.od[p][w] = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
    }
  }
  const uint32_t sw = R.vs[0] | (R.vs[1] << 8) | (R.vs[2] << 16) | (R.vs[3] << 24);
  P.s[0] = fp8x2_to_h2<false>(sw);
  P.s[1] = fp8x2_to_h2<true>(sw);
}

template <int D, int T>
__device__ __forceinline__ h4 v_operand(const VPairs<D>& P) {
  constexpr int W = T / 8;
  constexpr int BYTE = (T % 8) / 2;
  const uint32_t w0 = (T & 1) ? P.od[0][W] : P.ev[0][W];
  const uint32_t w1 = (T & 1) ? P.od[1][W] : P.ev[1][W];
  const h2 a = fp4x2_to_h2<BYTE>(w0) * P.s[0];
  const h2 b = fp4x2_to_h2<BYTE>(w1) * P.s[1];
  return h4{a[0], a[1], b[0], b[1]};
}

__device__ __forceinline__ float wave_max_j(float v) {
  v = __builtin_fmaxf(v, __shfl_xor(v, 16));
  return __builtin_fmaxf(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float wave_sum_j(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

template <int D, int NT>
struct WaveAttn {
  using G = Geo<D>;
  h8 q[NT][G::KW];       // B operand of S^T, per column tile and chunk
  float sf[NT];          // per-column factor: sm_scale * g_K * log2(e) / qscale
  int lim[NT];           // last visible key of the column (-1: none)
  f4 acc[NT][G::DPL];    // O^T accumulators
  float m[NT];           // running max (base-2 scores)
  float l[NT];           // this lane's share of the running sum

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      m[n] = -__builtin_inff();
      l[n] = 0.0f;
#pragma unroll
      for (int t = 0; t < G::DPL; ++t) acc[n][t] = f4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // Load column tile n: qrow points at the column's D bf16 values (nullptr:
  // padding column). The row is scaled by a power of two so that its largest
  // magnitude lies in [1, 2) before the exact-range f16 conversion; the
  // inverse goes into sf.
  __device__ __forceinline__ void load_q(int n, const uint16_t* qrow, int j, float base_factor) {
    constexpr int E = D / 4;  // bf16 elements per lane
    uint32_t w[E / 2];
    if (qrow != nullptr) {
      const u32x4* p = reinterpret_cast<const u32x4*>(qrow + j * E);
#pragma unroll
      for (int c = 0; c < E / 8; ++c) {
        const u32x4 x = p[c];
        w[4 * c] = x[0];
        w[4 * c + 1] = x[1];
        w[4 * c + 2] = x[2];
        w[4 * c + 3] = x[3];
      }
    } else {
#pragma unroll
      for (int c = 0; c < E / 2; ++c) w[c] = 0;
    }
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < E / 2; ++c)
      amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fabsf(bf16_lo(w[c])), __builtin_fabsf(bf16_hi(w[c]))));
    amax = wave_max_j(amax);
    int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 127;
    e = (amax == 0.0f) ? 0 : (e < -120 ? -120 : e);
    sf[n] = __builtin_ldexpf(base_factor, e);
#pragma unroll
    for (int c = 0; c < G::KW; ++c) {
      h8 v;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v[2 * t] = (_Float16)__builtin_ldexpf(bf16_lo(w[4 * c + t]), -e);
        v[2 * t + 1] = (_Float16)__builtin_ldexpf(bf16_hi(w[4 * c + t]), -e);
      }
      q[n][c] = v;
    }
  }

  // One 32-key step starting at absolute key kb; R[0], R[1] hold the two
  // subtiles' raw bytes (keys >= L already zeroed in the value rows). With
  // masked false (wave-uniform) every key of the step is visible to every
  // valid column and the per-key limit test is skipped.
  __device__ __forceinline__ void step(const SubRaw<D> (&R)[2], int kb, int j, bool masked) {
    // ---- S^T = K^ . Q^T for both subtiles
    f4 s[2][NT];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int n = 0; n < NT; ++n) s[sb][n] = f4{0.f, 0.f, 0.f, 0.f};
      chunks<0>(R[sb], s[sb]);
    }
    // ---- online softmax
    h8 p[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float x[8];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) x[4 * sb + r] = s[sb][n][r] * sf[n];
      }
      if (masked) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int key = kb + 16 * (k >> 2) + 4 * j + (k & 3);
          x[k] = (key <= lim[n]) ? x[k] : -__builtin_inff();
        }
      }
      float mx = x[0];
#pragma unroll
      for (int k = 1; k < 8; ++k) mx = __builtin_fmaxf(mx, x[k]);
      mx = wave_max_j(mx);
      const bool grow = mx > m[n] + kLazyMax;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float mnew = grow ? mx : m[n];
        const float alpha = grow ? __builtin_amdgcn_exp2f(m[n] - mnew) : 1.0f;  // exp2(-inf) = 0
        l[n] *= alpha;
#pragma unroll
        for (int t = 0; t < G::DPL; ++t) acc[n][t] *= alpha;
        m[n] = mnew;
      }
      const float mu = (m[n] == -__builtin_inff()) ? 0.0f : m[n];
      // probabilities go to f16 in pairs; the running sum adds exactly the
      // f16 values the PV product uses (dot with (1, 1)), so constant values
      // come back unchanged
      const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
      float ps = l[n];
#pragma unroll
      for (int k = 0; k < 8; k += 2) {
        const h2 e = __builtin_bit_cast(
            h2, __builtin_amdgcn_cvt_pkrtz(__builtin_amdgcn_exp2f(x[k] - mu), __builtin_amdgcn_exp2f(x[k + 1] - mu)));
        ps = __builtin_amdgcn_fdot2(e, one, ps, false);
        p[n][k] = e[0];
        p[n][k + 1] = e[1];
      }
      l[n] = ps;
    }
    // ---- O^T += V^ T . P^T
    VPairs<D> vp[2];
    make_pairs(R[0], vp[0]);
    make_pairs(R[1], vp[1]);
    pv<0>(vp, p);
  }

  template <int C>
  __device__ __forceinline__ void chunks(const SubRaw<D>& R, f4 (&s)[NT]) {
    if constexpr (C < G::KW) {
      const h8 a = k_chunk<D, C>(R);
#pragma unroll
      for (int n = 0; n < NT; ++n) s[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, q[n][C], s[n], 0, 0, 0);
      chunks<C + 1>(R, s);
    }
  }

  template <int T>
  __device__ __forceinline__ void pv(const VPairs<D> (&vp)[2], const h8 (&p)[NT]) {
    if constexpr (T < G::DPL) {
      const h4 a0 = v_operand<D, T>(vp[0]);
      const h4 a1 = v_operand<D, T>(vp[1]);
      const h8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n][T] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, p[n], acc[n][T], 0, 0, 0);
      pv<T + 1>(vp, p);
    }
  }
};

// Block ids of the two 16-key subtiles of the step at kb and whether they
// hold keys below `lim` (L for a step of this wave, 0 for a prefetch past the
// wave's range). kb, lim and bt_row are wave-uniform.
struct StepIds {
  int32_t id[2];
  bool ok[2];
};

// The block table is read-only for the whole kernel; reading it through the
// constant address space lets these wave-uniform loads use the scalar cache,
// so waiting for them never waits on the vector loads of the data pipeline.
typedef __attribute__((address_space(4))) const int32_t const_i32;

__device__ __forceinline__ int32_t ld_uniform(const int32_t* p, int idx) {
  return ((const const_i32*)(uintptr_t)p)[idx];
}

__device__ __forceinline__ StepIds step_ids(const int32_t* bt_row, int kb, int lim, const Pool& pool) {
  StepIds s;
  s.ok[0] = kb < lim;
  s.ok[1] = kb + 16 < lim;
  const int page = kb >> pool.bs_log2;
  s.id[0] = ld_uniform(bt_row, s.ok[0] ? page : 0);
  s.id[1] = (pool.bs == 16) ? ld_uniform(bt_row, s.ok[1] ? page + 1 : 0) : s.id[0];
  return s;
}

// Issue the loads of the 32-key step at kb.
template <int D>
__device__ __forceinline__ void load_step(SubRaw<D> (&R)[2], const Pool& pool, const StepIds& ids, int h, int kb,
                                          const LaneOffsets<D>& o) {
  const int extent = 15 * (int)pool.st + D / 2 + D / 16;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const int row0 = (kb + 16 * sb) & (pool.bs - 1);
    const int64_t blk = clamp_block(ids.id[sb], pool.num_blocks);
    const uint8_t* kbase = pool.data + blk * pool.sb + (int64_t)h * pool.sh + (int64_t)row0 * pool.st;
    const int n = ids.ok[sb] ? extent : 0;
    load_sub<D>(R[sb], make_rsrc(kbase, n), make_rsrc(kbase + pool.skv, n), o);
  }
  // keep the scheduler from hoisting work on the previous step's data above
  // these loads (that would make their issue wait for that data)
  __builtin_amdgcn_sched_barrier(0);
}

// Stream the steps k0, k0 + ks, ... (< kend) through two register buffers:
// the data of the next step is in flight while a step is computed, and block
// ids are read one step further ahead. ids_at(k) must return not-ok ids for
// k >= kend; run(R, k) consumes step k.
template <int D, typename IdsAt, typename Run>
__device__ __forceinline__ void stream_steps(int k0, int ks, int kend, const Pool& pool, int h,
                                             const LaneOffsets<D>& off, IdsAt ids_at, Run run) {
  if (k0 >= kend) return;
  SubRaw<D> A[2], B[2];
  load_step<D>(A, pool, ids_at(k0), h, k0 * 32, off);
  StepIds ib = ids_at(k0 + ks);
  int k = k0;
  while (true) {
    load_step<D>(B, pool, ib, h, (k + ks) * 32, off);
    const StepIds ia = ids_at(k + 2 * ks);
    run(A, k);
    if (k + ks >= kend) break;
    load_step<D>(A, pool, ia, h, (k + 2 * ks) * 32, off);
    ib = ids_at(k + 3 * ks);
    run(B, k + ks);
    k += 2 * ks;
    if (k >= kend) break;
  }
}

// ---------------------------------------------------------------------------
// LDS-staged stream (decode). Each wave owns a ring of NS stages in LDS; a
// stage holds one 32-key step: for each 16-key subtile its K rows then its V
// rows, each 16 x full_dim bytes, densely. The copy into a stage is a fixed
// number of direct global->LDS buffer loads (no registers held while in
// flight): 16-byte chunks when a page's rows are contiguous (HND layout),
// 4-byte chunks for any other row stride. Lane l of a load lands at the
// load's LDS base + l * chunk; a subtile's K and V chunks form one list (V
// lanes add the K->V stride to their offset), and the lanes past the end of
// the list read out of range, which writes zeros to the padding after the
// subtile. No load is ever predicated, so every step issues exactly the same
// number of loads (a step past the wave's range uses zero-size descriptors:
// zeros, no memory traffic) and the wait before reading stage i is the
// constant vmcnt <= (NS - 1) * loads_per_step. The compiler does not order
// these loads against LDS reads, so that wait is explicit and fenced.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

template <int D, bool COMPACT>
struct StageGeo {
  static constexpr int FD = D / 2 + D / 16;
  static constexpr int SLAB = 16 * FD;                       // bytes of 16 rows
  static constexpr int CHUNK = COMPACT ? 16 : 4;             // bytes per lane per load
  static constexpr int CH = SLAB / CHUNK;                    // chunks per slab
  static constexpr int NCS = (2 * CH + 63) / 64;             // loads per subtile (K + V)
  static constexpr int NC = 2 * NCS;                         // loads per step
  static constexpr int SUB = NCS * 64 * CHUNK;               // LDS bytes per subtile (padded)
  static constexpr int STAGE = 2 * SUB;                      // LDS bytes per stage
};

// Per-lane byte offsets (relative to the subtile's first K row) of this
// lane's chunk in each load of a subtile, and whether it is a V chunk (which
// adds the K->V stride); loop invariant.
template <int D, bool COMPACT>
struct DmaOffsets {
  uint32_t v[StageGeo<D, COMPACT>::NCS];
  uint32_t isv;  // bit t: load t's chunk of this lane is a V chunk
};

constexpr uint32_t kOutOfRange = 0x7FFFFFF0u;  // >= any descriptor size used here

template <int D, bool COMPACT>
__device__ __forceinline__ DmaOffsets<D, COMPACT> dma_offsets(int64_t st, int lane) {
  using SG = StageGeo<D, COMPACT>;
  DmaOffsets<D, COMPACT> o;
  o.isv = 0;
#pragma unroll
  for (int t = 0; t < SG::NCS; ++t) {
    const int c = 64 * t + lane;
    const int cc = c < SG::CH ? c : c - SG::CH;  // chunk within its slab
    uint32_t off;
    if constexpr (COMPACT) {
      off = (uint32_t)(cc * 16);
    } else {
      constexpr int WPR = SG::FD / 4;  // dwords per row
      off = (uint32_t)((cc / WPR) * (int)st + 4 * (cc % WPR));
    }
    o.v[t] = (c < 2 * SG::CH) ? off : kOutOfRange;
    o.isv |= (c >= SG::CH && c < 2 * SG::CH) ? (1u << t) : 0u;
  }
  return o;
}

__device__ __forceinline__ lds_void* to_lds(uint8_t* p) { return (lds_void*)p; }

// Copy the step at kb (ids from step_ids) into the stage at dst.
template <int D, bool COMPACT>
__device__ __forceinline__ void dma_step(uint8_t* dst, const Pool& pool, const StepIds& ids, int h, int kb,
                                         const DmaOffsets<D, COMPACT>& o) {
  using SG = StageGeo<D, COMPACT>;
  const int extent = (int)pool.skv + 15 * (int)pool.st + SG::FD;
  const uint32_t skv = (uint32_t)pool.skv;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const int row0 = (kb + 16 * sb) & (pool.bs - 1);
    const int64_t blk = clamp_block(ids.id[sb], pool.num_blocks);
    const uint8_t* base = pool.data + blk * pool.sb + (int64_t)h * pool.sh + (int64_t)row0 * pool.st;
    const rsrc_t r = make_rsrc(base, ids.ok[sb] ? extent : 0);
#pragma unroll
    for (int t = 0; t < SG::NCS; ++t) {
      const uint32_t voff = o.v[t] + (((o.isv >> t) & 1u) ? skv : 0u);
      if constexpr (COMPACT)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, to_lds(dst + sb * SG::SUB + t * 64 * 16), 16, voff, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, to_lds(dst + sb * SG::SUB + t * 64 * 4), 4, voff, 0, 0, 0);
    }
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
}

// This lane's raw bytes of one subtile, read from its two slabs in LDS (the
// same per-lane pattern the direct global loads use).
template <int D>
__device__ __forceinline__ void lds_read_sub(SubRaw<D>& R, const uint8_t* kslab, const uint8_t* vslab, int i,
                                             int j) {
  constexpr int FD = D / 2 + D / 16;
  const uint8_t* krow = kslab + i * FD;
  if constexpr (D == 64) {
    const u32x2 w = ld_u32x2(krow + j * 8);
    R.k[0] = w[0];
    R.k[1] = w[1];
    R.ks = ld_u8(krow + 32 + j);
  } else if constexpr (D == 128) {
    const u32x4 w = ld_u32x4(krow + j * 16);
    R.k[0] = w[0];
    R.k[1] = w[1];
    R.k[2] = w[2];
    R.k[3] = w[3];
    R.ks = ld_u16(krow + 64 + 2 * j);
  } else {
    const u32x4 w0 = ld_u32x4(krow + j * 32);
    const u32x4 w1 = ld_u32x4(krow + j * 32 + 16);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      R.k[c] = w0[c];
      R.k[4 + c] = w1[c];
    }
    R.ks = ld_u32(krow + 128 + 4 * j);
  }
  const uint8_t* vrow = vslab + 4 * j * FD;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if constexpr (D == 64) {
      R.v[r][0] = ld_u16(vrow + r * FD + 2 * i);
      R.vs[r] = ld_u8(vrow + r * FD + 32 + (i >> 2));
    } else if constexpr (D == 128) {
      R.v[r][0] = ld_u32(vrow + r * FD + 4 * i);
      R.vs[r] = ld_u8(vrow + r * FD + 64 + (i >> 1));
    } else {
      const u32x2 w = ld_u32x2(vrow + r * FD + 8 * i);
      R.v[r][0] = w[0];
      R.v[r][1] = w[1];
      R.vs[r] = ld_u8(vrow + r * FD + 128 + i);
    }
  }
}

// Stream steps k0, k0 + ks, ... (< kend) of a sequence with L keys (block
// table row bt_row) through the wave's LDS ring `ring` (NS stages).
// lds_prologue issues the first NS - 1 copies (so that other loads, e.g. the
// queries, overlap them) and returns the ids of the next step to copy; the
// caller's loop then copies step k + (NS - 1) * ks, waits for stage k and
// computes it, and drains with wait_vmcnt<0>() at the end.
__device__ __forceinline__ StepIds ids_for_step(const int32_t* bt_row, int k, int kend, int L, const Pool& pool) {
  return step_ids(bt_row, k * 32, k < kend ? L : 0, pool);
}

template <int D, bool COMPACT, int NS>
__device__ __forceinline__ StepIds lds_prologue(uint8_t* ring, int k0, int ks, int kend, const int32_t* bt_row, int L,
                                                const Pool& pool, int h, const DmaOffsets<D, COMPACT>& dof) {
  using SG = StageGeo<D, COMPACT>;
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    dma_step<D, COMPACT>(ring + s * SG::STAGE, pool, ids_for_step(bt_row, k0 + s * ks, kend, L, pool), h,
                         (k0 + s * ks) * 32, dof);
  return ids_for_step(bt_row, k0 + (NS - 1) * ks, kend, L, pool);
}

// Read this lane's raw bytes of both subtiles of the stage at `stage`.
template <int D, bool COMPACT>
__device__ __forceinline__ void lds_read_step(SubRaw<D> (&R)[2], const uint8_t* stage, int i, int j) {
  using SG = StageGeo<D, COMPACT>;
  lds_read_sub<D>(R[0], stage, stage + SG::SLAB, i, j);
  lds_read_sub<D>(R[1], stage + SG::SUB, stage + SG::SUB + SG::SLAB, i, j);
}

template <int D>
__device__ __forceinline__ void mask_step(SubRaw<D> (&R)[2], int kb, int L, int j) {
  if (kb + 32 > L) {
    mask_sub_values<D>(R[0], kb, L, j);
    mask_sub_values<D>(R[1], kb + 16, L, j);
  }
}

}  // namespace nvfp4kv
