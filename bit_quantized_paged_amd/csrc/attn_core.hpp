// Wave-level paged attention engine over the NVFP4 (and FP8) cache (gfx950).
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
//  * FP8 caches [P40177 "Key source snippets": fp8_e4m3 / fp8_e5m2 beside
//    nvfp4] take the same lanes and elements with one byte per element:
//    K chunks and V tiles convert to f16 exactly (E4M3 by the hardware pair
//    convert, E5M2 by a byte permute, being the upper byte of a binary16),
//    with no block scale. The format is a template parameter (FMT) of the
//    raw-step types, the stage geometry and WaveAttn.
//  * Online softmax in base 2 with a lazy maximum: the running max of a
//    column only moves (and the accumulators are only rescaled) when a score
//    exceeds it by more than 8, so probabilities stay <= 256 in f16.
#pragma once

#include "device_common.hpp"

namespace nvfp4kv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyMax = 8.0f;

template <int D, int FMT>
struct RowBytes {
  static constexpr int value = (FMT == kNvfp4) ? D / 2 + D / 16 : D;
};

template <int D>
struct Geo {
  static constexpr int DPL = D / 16;                // V: d per lane = PV products
  static constexpr int KW = D / 32;                 // K: code words per lane = QK chunks
  static constexpr int VB = DPL / 2;                // V: code bytes per key per lane
  static constexpr int VW = VB >= 4 ? VB / 4 : 1;   // V: words per key per lane
};

// Raw bytes of one 16-key subtile for lane (i, j) = (lane % 16, lane / 16):
// K row i, the quarter j of its elements (d in [D/4 j, D/4 (j+1)), the
// operands of k_chunk), and V rows 4j..4j+3, the D/16 elements
// d in [D/16 i, D/16 (i+1)) of each (the lane's rows of the V^T tiles).
// FP8 (this template): one byte per element.
template <int D, int FMT = kNvfp4>
struct SubRaw {
  uint32_t k[D / 16];
  uint32_t v[4][D / 64];
};

// NVFP4: the same elements as nibbles, plus the E4M3 scale bytes of their
// 16-element blocks.
template <int D>
struct SubRaw<D, kNvfp4> {
  uint32_t k[Geo<D>::KW];
  uint32_t ks;
  uint32_t v[4][Geo<D>::VW];
  uint32_t vs[4];
};

// Pages are read with raw buffer loads: a wave-uniform descriptor per
// subtile (base = first row of the subtile, size = the bytes its 16 rows
// span) plus per-lane offsets. A subtile with nothing to read gets size 0,
// which makes the hardware return zeros without touching memory, so the
// loads of a step are issued unconditionally and every access is
// range-checked against its own page.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw (unformatted) buffer, gfx9 family

__device__ __forceinline__ rsrc_t make_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, bytes, kRsrcWord3);
}

// Zero the value rows of keys >= L (unwritten rows may hold NaN codes or
// scale bytes; their probability is 0 but 0 * NaN would poison the
// accumulator).
template <int D, int FMT>
__device__ __forceinline__ void mask_sub_values(SubRaw<D, FMT>& R, int key0, int L, int j) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const bool ok = key0 + 4 * j + r < L;
    if constexpr (FMT == kNvfp4) {
#pragma unroll
      for (int w = 0; w < Geo<D>::VW; ++w) R.v[r][w] = ok ? R.v[r][w] : 0u;
      R.vs[r] = ok ? R.vs[r] : 0u;
    } else {
#pragma unroll
      for (int w = 0; w < D / 64; ++w) R.v[r][w] = ok ? R.v[r][w] : 0u;
    }
  }
}


// Dequantised NVFP4 K chunk c of this lane: 8 f16 = codes * block scale.
template <int D, int C>
__device__ __forceinline__ h8 k_chunk_nvfp4(const SubRaw<D, kNvfp4>& R) {
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

// K chunk c of this lane as 8 f16 (the A operand of S^T = K^ Q^T): NVFP4
// codes times their block scale, or FP8 codes converted exactly (the
// per-tensor scale is applied to the scores).
template <int D, int C, int FMT>
__device__ __forceinline__ h8 k_chunk(const SubRaw<D, FMT>& R) {
  if constexpr (FMT == kNvfp4) {
    return k_chunk_nvfp4<D, C>(R);
  } else {
    const uint32_t w0 = R.k[2 * C], w1 = R.k[2 * C + 1];
    h2 a0, a1, a2, a3;
    if constexpr (FMT == kFp8E4M3) {
      a0 = fp8x2_to_h2<false>(w0);
      a1 = fp8x2_to_h2<true>(w0);
      a2 = fp8x2_to_h2<false>(w1);
      a3 = fp8x2_to_h2<true>(w1);
    } else {
      a0 = e5m2x2_to_h2<0, 1>(w0, w0);
      a1 = e5m2x2_to_h2<2, 3>(w0, w0);
      a2 = e5m2x2_to_h2<0, 1>(w1, w1);
      a3 = e5m2x2_to_h2<2, 3>(w1, w1);
    }
    return h8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
  }
}

// Value rows of one subtile arranged for the V^T tiles.
// NVFP4: each byte holds the codes of two keys (4j+2p, 4j+2p+1) at one d.
// FP8: the rows as read; a tile takes its two keys' bytes with one permute.
template <int D, int FMT = kNvfp4>
struct VPairs {
  uint32_t raw[4][D / 64];
};

template <int D>
struct VPairs<D, kNvfp4> {
  uint32_t ev[2][Geo<D>::VW];  // [pair][word]: byte b <-> d offset 8w + 2b
  uint32_t od[2][Geo<D>::VW];  //                byte b <-> d offset 8w + 2b + 1
  h2 s[2];                     // block scales of the pair's two keys
};

template <int D, int FMT>
__device__ __forceinline__ void make_pairs(const SubRaw<D, FMT>& R, VPairs<D, FMT>& P) {
  if constexpr (FMT == kNvfp4) {
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
    // (vs0, vs1) and (vs2, vs3) side by side in the low bytes: one permute each
    P.s[0] = fp8x2_to_h2<false>(__builtin_amdgcn_perm(R.vs[1], R.vs[0], 0x0C0C0400u));
    P.s[1] = fp8x2_to_h2<false>(__builtin_amdgcn_perm(R.vs[3], R.vs[2], 0x0C0C0400u));
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int w = 0; w < D / 64; ++w) P.raw[r][w] = R.v[r][w];
  }
}

// V^T tile T: this lane's row d = D/16 i + T, keys 4j..4j+3 as f16.
template <int D, int T, int FMT>
__device__ __forceinline__ h4 v_operand(const VPairs<D, FMT>& P) {
  h2 a, b;
  if constexpr (FMT == kNvfp4) {
    constexpr int W = T / 8;
    constexpr int BYTE = (T % 8) / 2;
    const uint32_t w0 = (T & 1) ? P.od[0][W] : P.ev[0][W];
    const uint32_t w1 = (T & 1) ? P.od[1][W] : P.ev[1][W];
    a = fp4x2_to_h2<BYTE>(w0) * P.s[0];
    b = fp4x2_to_h2<BYTE>(w1) * P.s[1];
  } else if constexpr (FMT == kFp8E4M3) {
    // byte B of keys (0, 1) and (2, 3) side by side, then one pair convert
    constexpr int W = T / 4;
    constexpr uint32_t sel = 0x0C0C0000u | ((uint32_t)(4 + T % 4) << 8) | (uint32_t)(T % 4);
    a = fp8x2_to_h2<false>(__builtin_amdgcn_perm(P.raw[1][W], P.raw[0][W], sel));
    b = fp8x2_to_h2<false>(__builtin_amdgcn_perm(P.raw[3][W], P.raw[2][W], sel));
  } else {
    constexpr int W = T / 4;
    constexpr int B = T % 4;
    a = e5m2x2_to_h2<B, B>(P.raw[0][W], P.raw[1][W]);
    b = e5m2x2_to_h2<B, B>(P.raw[2][W], P.raw[3][W]);
  }
  return h4{a[0], a[1], b[0], b[1]};
}

// Reductions over j (lane bits 4 and 5): lanes l and l ^ 16, then l and
// l ^ 32. The row swap (16-lane rows 0 <-> 1, 2 <-> 3) and the half swap of
// gfx950 exchange a register's rows in the VALU without an LDS round trip;
// with both operands the same value, the two results of a swap hold, in every
// lane, x[l] and x[l ^ 16] (x[l ^ 32]) in the same order for both lanes of a
// pair, so every lane of a pair gets the same bits.
__device__ __forceinline__ float wave_max_j(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __builtin_fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// Maxima of scores. fmaxf first quiets signalling NaNs: on operands the
// compiler cannot prove canonical (matrix-unit results, lane swaps) that is
// two extra v_max per call. The median of a, b and +inf is their maximum
// (v_med3_f32, no quieting), and its result lets the compiler chain further
// maxima (v_max3_f32) without quieting either. pinf must hold +inf in a
// register the compiler cannot see into, or it folds the median back into
// fmaxf. Scores are never NaN here (every visible key has finite codes and
// scales; hidden keys are set to -inf before any maximum). Written in C, not
// as assembly, so that the compiler keeps the wait states a vector read of
// matrix-unit results needs.
__device__ __forceinline__ float opaque_pinf() {
  float pinf = __builtin_inff();
  asm volatile("" : "+s"(pinf));
  return pinf;
}
__device__ __forceinline__ float max_med3(float a, float b, float pinf) { return __builtin_amdgcn_fmed3f(a, b, pinf); }
__device__ __forceinline__ float wave_max_j_med3(float v, float pinf) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = max_med3(__uint_as_float(a[0]), __uint_as_float(a[1]), pinf);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max_med3(__uint_as_float(b[0]), __uint_as_float(b[1]), pinf);
}
__device__ __forceinline__ float wave_sum_j(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D, int NT, int FMT = kNvfp4>
struct WaveAttn {
  using G = Geo<D>;
  h8 q[NT][G::KW];       // B operand of S^T, per column tile and chunk
  float sf[NT];          // per-column factor |sm_scale * g_K| * log2(e) / qscale (> 0)
  int lim[NT];           // last visible key of the column (-1: none)
  f4 acc[NT][G::DPL];    // O^T accumulators
  float m[NT];           // running max (base-2 scores); -FLT_MAX until the column has a visible key
  // Running sums. With one column tile (decode) they come from the matrix
  // unit: a ones tile times P^T (every entry = the lane's column sum). With
  // several (prefill) the four extra accumulators per tile would cost
  // occupancy, so each lane sums its own probabilities on the vector unit.
  static constexpr bool kMfmaSum = (NT == 1);
  f4 lacc[NT];           // kMfmaSum
  float l[NT];           // otherwise: this lane's share of the running sum

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      // finite, so that -m is a usable exp2 offset from the first step on:
      // a hidden score (-inf) still gives exp2(-inf) = 0, and the first
      // visible one always moves the max (alpha then underflows to 0, as
      // exp2(-inf) would). Merges weight such an empty state by
      // exp2(-FLT_MAX - M) = 0, or by 1 when every state is empty, with zero
      // sums and accumulators either way.
      m[n] = -3.40282347e38f;
      if constexpr (kMfmaSum) lacc[n] = f4{0.f, 0.f, 0.f, 0.f};
      else l[n] = 0.0f;
#pragma unroll
      for (int t = 0; t < G::DPL; ++t) acc[n][t] = f4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // Query columns are loaded in two halves so that other loads can be
  // issued while these are in flight: load_q_raw issues this lane's share of
  // the column's D bf16 values (qrow nullptr: padding column), set_q turns
  // them into column tile n. The row is scaled by a power of two so that its
  // largest magnitude lies in [1, 2) before the exact-range f16 conversion;
  // the inverse goes into sf. The softmax folds sf into its max and exp2
  // argument, which needs sf > 0: a negative factor's sign moves into the
  // query (exact), and a zero one becomes the smallest normal float (every
  // logit is then 0 to within 2^-100, as it should be).
  struct QRaw {
    uint32_t w[D / 8];
  };

  __device__ __forceinline__ static QRaw load_q_raw(const uint16_t* qrow, int j) {
    constexpr int E = D / 4;  // bf16 elements per lane
    QRaw r;
    if (qrow != nullptr) {
      const u32x4* p = reinterpret_cast<const u32x4*>(qrow + j * E);
#pragma unroll
      for (int c = 0; c < E / 8; ++c) {
        const u32x4 x = p[c];
        r.w[4 * c] = x[0];
        r.w[4 * c + 1] = x[1];
        r.w[4 * c + 2] = x[2];
        r.w[4 * c + 3] = x[3];
      }
    } else {
#pragma unroll
      for (int c = 0; c < E / 2; ++c) r.w[c] = 0;
    }
    return r;
  }

  __device__ __forceinline__ void set_q(int n, const QRaw& r, float base_factor) {
    constexpr int E = D / 4;
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < E / 2; ++c)
      amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fabsf(bf16_lo(r.w[c])), __builtin_fabsf(bf16_hi(r.w[c]))));
    amax = wave_max_j(amax);
    int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 127;
    e = (amax == 0.0f) ? 0 : (e < -120 ? -120 : e);
    const float sgn = base_factor < 0.0f ? -1.0f : 1.0f;
    sf[n] = __builtin_fmaxf(__builtin_ldexpf(base_factor * sgn, e), 1.17549435e-38f);
#pragma unroll
    for (int c = 0; c < G::KW; ++c) {
      h8 v;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v[2 * t] = (_Float16)(__builtin_ldexpf(bf16_lo(r.w[4 * c + t]), -e) * sgn);
        v[2 * t + 1] = (_Float16)(__builtin_ldexpf(bf16_hi(r.w[4 * c + t]), -e) * sgn);
      }
      q[n][c] = v;
    }
  }

  __device__ __forceinline__ void load_q(int n, const uint16_t* qrow, int j, float base_factor) {
    set_q(n, load_q_raw(qrow, j), base_factor);
  }

  // One 32-key step starting at absolute key kb; R[0], R[1] hold the two
  // subtiles' raw bytes (keys >= L already zeroed in the value rows). With
  // masked false (wave-uniform) every key of the step is visible to every
  // valid column and the per-key limit test is skipped.
  __device__ __forceinline__ void step(const SubRaw<D, FMT> (&R)[2], int kb, int j, bool masked) {
    // ---- S^T = K^ . Q^T for both subtiles
    f4 s[2][NT];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int n = 0; n < NT; ++n) s[sb][n] = f4{0.f, 0.f, 0.f, 0.f};
      chunks<0>(R[sb], s[sb]);
    }
    h8 p[NT];
    softmax(s, kb, j, masked, p);
    // ---- O^T += V^ T . P^T
    VPairs<D, FMT> vp[2];
    make_pairs(R[0], vp[0]);
    make_pairs(R[1], vp[1]);
    pv<0>(vp, p);
  }

  // The step's halves from operands already dequantised into the MFMA lane
  // layout: ka[sb][c] = k_chunk<c>(subtile sb); va[t] = the V^T tile t that
  // pv builds (both subtiles' keys).
  __device__ __forceinline__ void scores_ops(const h8 (&ka)[2][G::KW], f4 (&s)[2][NT]) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int n = 0; n < NT; ++n) s[sb][n] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < G::KW; ++c)
#pragma unroll
        for (int n = 0; n < NT; ++n)
          s[sb][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[sb][c], q[n][c], s[sb][n], 0, 0, 0);
    }
  }
  __device__ __forceinline__ void pv_ops(const h8 (&va)[G::DPL], const h8 (&p)[NT]) {
#pragma unroll
    for (int t = 0; t < G::DPL; ++t)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[t], p[n], acc[n][t], 0, 0, 0);
    if constexpr (kMfmaSum) sum_ops(p);
  }
  // Column sums of P^T (the exact f16 values the PV product uses) on the
  // matrix unit: a ones tile times P^T, accumulated in fp32.
  __device__ __forceinline__ void sum_ops(const h8 (&p)[NT]) {
    const _Float16 o = (_Float16)1.0f;
    const h8 ones = {o, o, o, o, o, o, o, o};
#pragma unroll
    for (int n = 0; n < NT; ++n) lacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, p[n], lacc[n], 0, 0, 0);
  }
  // The running sum of column tile n for this lane's column (the same value
  // in the four lanes of the column).
  __device__ __forceinline__ float lsum(int n) const {
    if constexpr (kMfmaSum) return lacc[n][0];
    else return wave_sum_j(l[n]);
  }

  // Online softmax of a step's scores (base 2, lazy rescale) into the f16
  // probabilities p of each column tile. The scale sf (> 0) is applied once
  // to the raw max and inside each exp2 argument (one fma per score).
  __device__ __forceinline__ void softmax(const f4 (&s)[2][NT], int kb, int j, bool masked, h8 (&p)[NT]) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float x[8];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) x[4 * sb + r] = s[sb][n][r];
      }
      if (masked) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int key = kb + 16 * (k >> 2) + 4 * j + (k & 3);
          x[k] = (key <= lim[n]) ? x[k] : -__builtin_inff();
        }
      }
      const float pinf = opaque_pinf();
      float rmx = max_med3(x[0], x[1], pinf);
#pragma unroll
      for (int k = 2; k < 8; ++k) rmx = __builtin_fmaxf(rmx, x[k]);
      // A column's running max moves only when the step's maximum, scaled,
      // exceeds it by more than kLazyMax. Scaling by sf > 0 is monotone (also
      // after rounding), so that holds exactly when it holds for the maximum
      // of some lane's own scores: each lane tests its own, and the maxima
      // across the column's lanes are formed only on the rare steps where a
      // test holds somewhere in the wave (a wave-uniform branch).
      if (__builtin_amdgcn_ballot_w64(rmx * sf[n] > m[n] + kLazyMax) != 0) {
        const float mx = wave_max_j_med3(rmx, pinf) * sf[n];  // sf > 0: a column with no visible key has -inf
        const bool grow = mx > m[n] + kLazyMax;
        const float mnew = grow ? mx : m[n];
        const float alpha = grow ? __builtin_amdgcn_exp2f(m[n] - mnew) : 1.0f;  // 0 from the initial max
        if constexpr (kMfmaSum) lacc[n] *= alpha;
        else l[n] *= alpha;
#pragma unroll
        for (int t = 0; t < G::DPL; ++t) acc[n][t] *= alpha;
        m[n] = mnew;
      }
      const float nmu = -m[n];
      // the sum adds exactly the f16 values the PV product uses (dot with
      // (1, 1)), so constant values come back unchanged
      const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
      float ps = kMfmaSum ? 0.0f : l[n];
#pragma unroll
      for (int k = 0; k < 8; k += 2) {
        const h2 e = __builtin_bit_cast(
            h2, __builtin_amdgcn_cvt_pkrtz(__builtin_amdgcn_exp2f(__builtin_fmaf(x[k], sf[n], nmu)),
                                           __builtin_amdgcn_exp2f(__builtin_fmaf(x[k + 1], sf[n], nmu))));
        if constexpr (!kMfmaSum) ps = __builtin_amdgcn_fdot2(e, one, ps, false);
        p[n][k] = e[0];
        p[n][k + 1] = e[1];
      }
      if constexpr (!kMfmaSum) l[n] = ps;
    }
  }

  template <int C>
  __device__ __forceinline__ void chunks(const SubRaw<D, FMT>& R, f4 (&s)[NT]) {
    if constexpr (C < G::KW) {
      const h8 a = k_chunk<D, C>(R);
#pragma unroll
      for (int n = 0; n < NT; ++n) s[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, q[n][C], s[n], 0, 0, 0);
      chunks<C + 1>(R, s);
    }
  }

  template <int T>
  __device__ __forceinline__ void pv(const VPairs<D, FMT> (&vp)[2], const h8 (&p)[NT]) {
    if constexpr (T == 0 && kMfmaSum) sum_ops(p);
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

// The table index does not depend on lim (it is clamped to the row's last
// entry instead), so the loads of the first steps can be in flight while the
// sequence length is still on its way; an id read for a subtile that is not
// ok is never used (its copy has size 0).
__device__ __forceinline__ StepIds step_ids(const int32_t* bt_row, int kb, int lim, int max_blocks,
                                            const Pool& pool) {
  StepIds s;
  s.ok[0] = kb < lim;
  s.ok[1] = kb + 16 < lim;
  const int page = kb >> pool.bs_log2;
  const int last = max_blocks - 1;
  s.id[0] = ld_uniform(bt_row, page < last ? page : last);
  s.id[1] = (pool.bs == 16) ? ld_uniform(bt_row, page + 1 < last ? page + 1 : last) : s.id[0];
  return s;
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

// LDS stage of one 32-key step: two subtiles, each its K slab (16 rows x
// full_dim bytes) followed by its V slab, packed densely (a subtile is padded
// only to 256 bytes). A subtile is copied by direct-to-LDS loads in which
// lane l of load t writes LDS byte off(t) + l * size(t) of the subtile:
//  compact (contiguous 16-byte aligned rows): N16 loads of 16 bytes per lane
//    (1 KB each), then N4 loads of 4 bytes per lane (256 B each) for the rest;
//  general (any row stride): loads of 4 bytes per lane, 256 B each.
// Lanes past the subtile's bytes read out of range, which writes zeros.
//  FP8 rows (D bytes, a multiple of 16; row strides multiples of 16): 16-byte
//    loads only, whatever the row stride. In the K slab, 16-byte chunk c of
//    row r sits at chunk c ^ fp8_k_swizzle(r) of its LDS row, so that the 16
//    lanes reading one chunk column of 16 rows (D-byte rows: same banks) hit
//    eight different 16-byte bank groups.
template <int D>
__host__ __device__ constexpr int fp8_k_swizzle(int row) {
  return (D == 64) ? ((row >> 1) & 3) : (row & 7);
}

template <int D, bool COMPACT, int FMT = kNvfp4>
struct StageGeo {
  static constexpr int FD = RowBytes<D, FMT>::value;
  static constexpr int SLAB = 16 * FD;                       // bytes of 16 rows
  static constexpr int BYTES = 2 * SLAB;                     // K and V of a subtile
  static constexpr int SUB = (BYTES + 255) / 256 * 256;      // LDS bytes per subtile
  static constexpr int STAGE = 2 * SUB;                      // LDS bytes per stage
  static constexpr int N16 = (COMPACT || FMT != kNvfp4) ? BYTES / 1024 : 0;  // 16-byte loads per subtile
  static constexpr int N4 = (BYTES - 1024 * N16 + 255) / 256;  // 4-byte loads per subtile
  static constexpr int NCS = N16 + N4;                       // loads per subtile
  static constexpr int NC = 2 * NCS;                         // loads per step
  static constexpr int size(int t) { return t < N16 ? 16 : 4; }
  static constexpr int off(int t) { return t < N16 ? 1024 * t : 1024 * N16 + 256 * (t - N16); }
  static_assert(off(NCS - 1) + 256 <= SUB, "loads overrun the subtile");
};

// Per-lane byte offset, relative to the subtile's first K row in the pool, of
// the bytes lane `lane` copies in each load of a subtile (V bytes include the
// K->V stride); loop invariant.
template <int D, bool COMPACT, int FMT = kNvfp4>
struct DmaOffsets {
  uint32_t v[StageGeo<D, COMPACT, FMT>::NCS];
};

constexpr uint32_t kOutOfRange = 0x7FFFFFF0u;  // >= any descriptor size used here

template <int D, bool COMPACT, int FMT = kNvfp4>
__device__ __forceinline__ DmaOffsets<D, COMPACT, FMT> dma_offsets(int64_t st, int64_t skv, int lane) {
  using SG = StageGeo<D, COMPACT, FMT>;
  DmaOffsets<D, COMPACT, FMT> o;
#pragma unroll
  for (int t = 0; t < SG::NCS; ++t) {
    const int x = SG::off(t) + SG::size(t) * lane;  // byte of the subtile's [K slab | V slab]
    const bool isv = x >= SG::SLAB;
    int y = isv ? x - SG::SLAB : x;                 // byte within its slab
    if constexpr (FMT != kNvfp4) {
      // the K chunk this LDS chunk holds (the swizzle is its own inverse)
      if (!isv) y = (y / D) * D + 16 * (((y % D) / 16) ^ fp8_k_swizzle<D>(y / D));
    }
    uint32_t off;
    if constexpr (COMPACT) {
      off = (uint32_t)y;                             // rows are contiguous
    } else {
      off = (uint32_t)((y / SG::FD) * (int)st + y % SG::FD);
    }
    off += isv ? (uint32_t)skv : 0u;
    o.v[t] = (x < SG::BYTES) ? off : kOutOfRange;
  }
  return o;
}

__device__ __forceinline__ lds_void* to_lds(uint8_t* p) { return (lds_void*)p; }

// Loads T, T + 1, ... of one subtile (the load width must be a literal).
template <int D, bool COMPACT, int FMT, int T>
__device__ __forceinline__ void dma_sub(uint8_t* dst, rsrc_t r, const DmaOffsets<D, COMPACT, FMT>& o) {
  using SG = StageGeo<D, COMPACT, FMT>;
  if constexpr (T < SG::NCS) {
    if constexpr (SG::size(T) == 16)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, to_lds(dst + SG::off(T)), 16, o.v[T], 0, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, to_lds(dst + SG::off(T)), 4, o.v[T], 0, 0, 0);
    dma_sub<D, COMPACT, FMT, T + 1>(dst, r, o);
  }
}

// Address of the first K row of a subtile: row row0 of block id (clamped to
// the pool), kv head h. The clamped block index is below 2^31, so its product
// with the block stride needs no sign extension, and the row term fits 32
// bits (row0 < 64 and row strides are below 2^26 by the descriptor checks):
// fewer scalar instructions per copy than full 64-bit products.
__device__ __forceinline__ const uint8_t* subtile_base(const Pool& pool, int32_t id, int h, int row0) {
  const uint32_t blk = (uint32_t)clamp_block(id, pool.num_blocks);
  return pool.data + (uint64_t)blk * (uint64_t)pool.sb + (int64_t)h * pool.sh +
         (uint64_t)((uint32_t)row0 * (uint32_t)pool.st);
}

// Copy the step at kb (ids from step_ids) into the stage at dst.
template <int D, bool COMPACT, int FMT = kNvfp4>
__device__ __forceinline__ void dma_step(uint8_t* dst, const Pool& pool, const StepIds& ids, int h, int kb,
                                         const DmaOffsets<D, COMPACT, FMT>& o) {
  using SG = StageGeo<D, COMPACT, FMT>;
  const int extent = (int)pool.skv + 15 * (int)pool.st + SG::FD;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const uint8_t* base = subtile_base(pool, ids.id[sb], h, (kb + 16 * sb) & (pool.bs - 1));
    dma_sub<D, COMPACT, FMT, 0>(dst + sb * SG::SUB, make_rsrc(base, ids.ok[sb] ? extent : 0), o);
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

// Stream steps k0, k0 + ks, ... (< kend) of a sequence with L keys (block
// table row bt_row) through the wave's LDS ring `ring` (NS stages).
// lds_prologue issues the first NS - 1 copies (so that other loads, e.g. the
// queries, overlap them) and returns the ids of the next step to copy; the
// caller's loop then copies step k + (NS - 1) * ks, waits for stage k and
// computes it, and drains with wait_vmcnt<0>() at the end.
__device__ __forceinline__ StepIds ids_for_step(const int32_t* bt_row, int k, int kend, int L, int max_blocks,
                                                const Pool& pool) {
  return step_ids(bt_row, k * 32, k < kend ? L : 0, max_blocks, pool);
}

template <int D, bool COMPACT, int NS, int FMT = kNvfp4>
__device__ __forceinline__ StepIds lds_prologue(uint8_t* ring, int k0, int ks, int kend, const int32_t* bt_row, int L,
                                                int max_blocks, const Pool& pool, int h,
                                                const DmaOffsets<D, COMPACT, FMT>& dof) {
  using SG = StageGeo<D, COMPACT, FMT>;
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    dma_step<D, COMPACT, FMT>(ring + s * SG::STAGE, pool,
                              ids_for_step(bt_row, k0 + s * ks, kend, L, max_blocks, pool), h, (k0 + s * ks) * 32,
                              dof);
  return ids_for_step(bt_row, k0 + (NS - 1) * ks, kend, L, max_blocks, pool);
}

// ---- step reader for stages filled by direct-to-LDS loads ----------------
// The compiler cannot tell which LDS bytes an in-flight direct-to-LDS load
// will write, so before any LDS read it would wait for every load in flight,
// including the stages still streaming in. The step's reads are therefore
// issued from one asm block, which the compiler does not inspect for LDS
// accesses, and which itself waits for its reads (lgkmcnt(0)) before it
// returns; the caller orders it after the stage's wait_vmcnt.

// Per-lane byte offsets, within a stage, of what lane (i, j) reads of
// subtile 0 (subtile 1 is StageGeo::SUB further): K row i, quarter j of its
// codes (the k_chunk operands) and the scales of that quarter; V rows
// 4j..4j+3, the codes of the lane's D/16 dims (2 bytes for D = 64, 4 for
// 128, 8 for 256, one scale block) and that block's scale byte.
struct LdsLane {
  uint32_t k, ks, v, vs;
  uint32_t k2, k3;  // FP8 at D = 256: the third and fourth K chunks
};

template <int D, int FMT = kNvfp4>
__device__ __forceinline__ LdsLane lds_lane(int i, int j) {
  LdsLane o;
  if constexpr (FMT == kNvfp4) {
    constexpr int FD = D / 2 + D / 16;
    o.k = (uint32_t)(i * FD + (D / 8) * j);
    o.ks = (uint32_t)(i * FD + D / 2 + (D / 64) * j);
    o.v = (uint32_t)(16 * FD + 4 * j * FD + (D / 32) * i);
    o.vs = (uint32_t)(16 * FD + 4 * j * FD + D / 2 + ((i * D) >> 8));
    o.k2 = 0;
    o.k3 = 0;
  } else {
    // K chunks (D/64) * j + c of row i, through the swizzle; for D = 64 one
    // chunk, 128 two (k, ks), 256 four (k, ks, k2, k3)
    constexpr int NKC = D / 64;
    uint32_t a[4] = {0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < NKC; ++c) a[c] = (uint32_t)(i * D + 16 * ((NKC * j + c) ^ fp8_k_swizzle<D>(i)));
    o.k = a[0];
    o.ks = a[1];
    o.k2 = a[2];
    o.k3 = a[3];
    o.v = (uint32_t)(16 * D + 4 * j * D + (D / 16) * i);
    o.vs = 0;
  }
  return o;
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

template <int D>
__device__ __forceinline__ void lds_read_step_async_safe(SubRaw<D> (&R)[2], const uint8_t* stage, const LdsLane& o);

static_assert(StageGeo<64, true>::SUB == 1280 && StageGeo<64, false>::SUB == 1280, "D = 64 reader offsets");
static_assert(StageGeo<128, true>::SUB == 2304 && StageGeo<128, false>::SUB == 2304, "D = 128 reader offsets");
static_assert(StageGeo<256, true>::SUB == 4608 && StageGeo<256, false>::SUB == 4608, "D = 256 reader offsets");

// D = 64: row 36 bytes, subtile 1280 bytes.
template <>
__device__ __forceinline__ void lds_read_step_async_safe<64>(SubRaw<64> (&R)[2], const uint8_t* stage,
                                                             const LdsLane& o) {
  const uint32_t s = lds_addr(stage);
  const uint32_t ak = s + o.k, aks = s + o.ks, av = s + o.v, avs = s + o.vs;
  asm volatile(
      "ds_read_b32 %0, %22\n\t"
      "ds_read_b32 %1, %22 offset:4\n\t"
      "ds_read_u8 %2, %23\n\t"
      "ds_read_u16 %3, %24\n\t"
      "ds_read_u16 %4, %24 offset:36\n\t"
      "ds_read_u16 %5, %24 offset:72\n\t"
      "ds_read_u16 %6, %24 offset:108\n\t"
      "ds_read_u8 %7, %25\n\t"
      "ds_read_u8 %8, %25 offset:36\n\t"
      "ds_read_u8 %9, %25 offset:72\n\t"
      "ds_read_u8 %10, %25 offset:108\n\t"
      "ds_read_b32 %11, %22 offset:1280\n\t"
      "ds_read_b32 %12, %22 offset:1284\n\t"
      "ds_read_u8 %13, %23 offset:1280\n\t"
      "ds_read_u16 %14, %24 offset:1280\n\t"
      "ds_read_u16 %15, %24 offset:1316\n\t"
      "ds_read_u16 %16, %24 offset:1352\n\t"
      "ds_read_u16 %17, %24 offset:1388\n\t"
      "ds_read_u8 %18, %25 offset:1280\n\t"
      "ds_read_u8 %19, %25 offset:1316\n\t"
      "ds_read_u8 %20, %25 offset:1352\n\t"
      "ds_read_u8 %21, %25 offset:1388\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(R[0].k[0]), "=&v"(R[0].k[1]), "=&v"(R[0].ks), "=&v"(R[0].v[0][0]), "=&v"(R[0].v[1][0]),
        "=&v"(R[0].v[2][0]), "=&v"(R[0].v[3][0]), "=&v"(R[0].vs[0]), "=&v"(R[0].vs[1]), "=&v"(R[0].vs[2]),
        "=&v"(R[0].vs[3]), "=&v"(R[1].k[0]), "=&v"(R[1].k[1]), "=&v"(R[1].ks), "=&v"(R[1].v[0][0]),
        "=&v"(R[1].v[1][0]), "=&v"(R[1].v[2][0]), "=&v"(R[1].v[3][0]), "=&v"(R[1].vs[0]), "=&v"(R[1].vs[1]),
        "=&v"(R[1].vs[2]), "=&v"(R[1].vs[3])
      : "v"(ak), "v"(aks), "v"(av), "v"(avs)
      : "memory");
}

// D = 128: row 72 bytes, subtile 2304 bytes.
template <>
__device__ __forceinline__ void lds_read_step_async_safe<128>(SubRaw<128> (&R)[2], const uint8_t* stage,
                                                              const LdsLane& o) {
  const uint32_t s = lds_addr(stage);
  const uint32_t ak = s + o.k, aks = s + o.ks, av = s + o.v, avs = s + o.vs;
  u32x2 k0a, k0b, k1a, k1b;
  asm volatile(
      "ds_read_b64 %0, %22\n\t"
      "ds_read_b64 %1, %22 offset:8\n\t"
      "ds_read_u16 %2, %23\n\t"
      "ds_read_b32 %3, %24\n\t"
      "ds_read_b32 %4, %24 offset:72\n\t"
      "ds_read_b32 %5, %24 offset:144\n\t"
      "ds_read_b32 %6, %24 offset:216\n\t"
      "ds_read_u8 %7, %25\n\t"
      "ds_read_u8 %8, %25 offset:72\n\t"
      "ds_read_u8 %9, %25 offset:144\n\t"
      "ds_read_u8 %10, %25 offset:216\n\t"
      "ds_read_b64 %11, %22 offset:2304\n\t"
      "ds_read_b64 %12, %22 offset:2312\n\t"
      "ds_read_u16 %13, %23 offset:2304\n\t"
      "ds_read_b32 %14, %24 offset:2304\n\t"
      "ds_read_b32 %15, %24 offset:2376\n\t"
      "ds_read_b32 %16, %24 offset:2448\n\t"
      "ds_read_b32 %17, %24 offset:2520\n\t"
      "ds_read_u8 %18, %25 offset:2304\n\t"
      "ds_read_u8 %19, %25 offset:2376\n\t"
      "ds_read_u8 %20, %25 offset:2448\n\t"
      "ds_read_u8 %21, %25 offset:2520\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k0a), "=&v"(k0b), "=&v"(R[0].ks), "=&v"(R[0].v[0][0]), "=&v"(R[0].v[1][0]), "=&v"(R[0].v[2][0]),
        "=&v"(R[0].v[3][0]), "=&v"(R[0].vs[0]), "=&v"(R[0].vs[1]), "=&v"(R[0].vs[2]), "=&v"(R[0].vs[3]),
        "=&v"(k1a), "=&v"(k1b), "=&v"(R[1].ks), "=&v"(R[1].v[0][0]), "=&v"(R[1].v[1][0]), "=&v"(R[1].v[2][0]),
        "=&v"(R[1].v[3][0]), "=&v"(R[1].vs[0]), "=&v"(R[1].vs[1]), "=&v"(R[1].vs[2]), "=&v"(R[1].vs[3])
      : "v"(ak), "v"(aks), "v"(av), "v"(avs)
      : "memory");
  R[0].k[0] = k0a[0];
  R[0].k[1] = k0a[1];
  R[0].k[2] = k0b[0];
  R[0].k[3] = k0b[1];
  R[1].k[0] = k1a[0];
  R[1].k[1] = k1a[1];
  R[1].k[2] = k1b[0];
  R[1].k[3] = k1b[1];
}

// D = 256: row 144 bytes, subtile 4608 bytes.
template <>
__device__ __forceinline__ void lds_read_step_async_safe<256>(SubRaw<256> (&R)[2], const uint8_t* stage,
                                                              const LdsLane& o) {
  const uint32_t s = lds_addr(stage);
  const uint32_t ak = s + o.k, aks = s + o.ks, av = s + o.v, avs = s + o.vs;
  u32x4 k0a, k0b, k1a, k1b;
  u32x2 v0[4], v1[4];
  asm volatile(
      "ds_read_b128 %0, %22\n\t"
      "ds_read_b128 %1, %22 offset:16\n\t"
      "ds_read_b32 %2, %23\n\t"
      "ds_read_b64 %3, %24\n\t"
      "ds_read_b64 %4, %24 offset:144\n\t"
      "ds_read_b64 %5, %24 offset:288\n\t"
      "ds_read_b64 %6, %24 offset:432\n\t"
      "ds_read_u8 %7, %25\n\t"
      "ds_read_u8 %8, %25 offset:144\n\t"
      "ds_read_u8 %9, %25 offset:288\n\t"
      "ds_read_u8 %10, %25 offset:432\n\t"
      "ds_read_b128 %11, %22 offset:4608\n\t"
      "ds_read_b128 %12, %22 offset:4624\n\t"
      "ds_read_b32 %13, %23 offset:4608\n\t"
      "ds_read_b64 %14, %24 offset:4608\n\t"
      "ds_read_b64 %15, %24 offset:4752\n\t"
      "ds_read_b64 %16, %24 offset:4896\n\t"
      "ds_read_b64 %17, %24 offset:5040\n\t"
      "ds_read_u8 %18, %25 offset:4608\n\t"
      "ds_read_u8 %19, %25 offset:4752\n\t"
      "ds_read_u8 %20, %25 offset:4896\n\t"
      "ds_read_u8 %21, %25 offset:5040\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k0a), "=&v"(k0b), "=&v"(R[0].ks), "=&v"(v0[0]), "=&v"(v0[1]), "=&v"(v0[2]), "=&v"(v0[3]),
        "=&v"(R[0].vs[0]), "=&v"(R[0].vs[1]), "=&v"(R[0].vs[2]), "=&v"(R[0].vs[3]), "=&v"(k1a), "=&v"(k1b),
        "=&v"(R[1].ks), "=&v"(v1[0]), "=&v"(v1[1]), "=&v"(v1[2]), "=&v"(v1[3]), "=&v"(R[1].vs[0]),
        "=&v"(R[1].vs[1]), "=&v"(R[1].vs[2]), "=&v"(R[1].vs[3])
      : "v"(ak), "v"(aks), "v"(av), "v"(avs)
      : "memory");
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    R[0].k[c] = k0a[c];
    R[0].k[4 + c] = k0b[c];
    R[1].k[c] = k1a[c];
    R[1].k[4 + c] = k1b[c];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    R[0].v[r][0] = v0[r][0];
    R[0].v[r][1] = v0[r][1];
    R[1].v[r][0] = v1[r][0];
    R[1].v[r][1] = v1[r][1];
  }
}

// FP8 stage readers: lane (i, j) reads D/4 bytes of K row i (its D/64
// 16-byte chunks, each at its swizzled place, addresses from lds_lane) and
// D/16 bytes of V rows 4j..4j+3 at 16*D + 4j*D + D/16*i, in both subtiles
// (the second 32*D bytes further). All offsets are 16-byte aligned for the
// 16-byte reads (the ring is).
template <int D, int FMT>
__device__ __forceinline__ void lds_read_step_fp8(SubRaw<D, FMT> (&R)[2], const uint8_t* stage, const LdsLane& o) {
  const uint32_t s = lds_addr(stage);
  const uint32_t ak = s + o.k, av = s + o.v;
  if constexpr (D == 64) {
    static_assert(StageGeo<64, false, FMT>::SUB == 2048, "D = 64 FP8 reader offsets");
    u32x4 k0, k1;
    asm volatile(
        "ds_read_b128 %0, %10\n\t"
        "ds_read_b32 %1, %11\n\t"
        "ds_read_b32 %2, %11 offset:64\n\t"
        "ds_read_b32 %3, %11 offset:128\n\t"
        "ds_read_b32 %4, %11 offset:192\n\t"
        "ds_read_b128 %5, %10 offset:2048\n\t"
        "ds_read_b32 %6, %11 offset:2048\n\t"
        "ds_read_b32 %7, %11 offset:2112\n\t"
        "ds_read_b32 %8, %11 offset:2176\n\t"
        "ds_read_b32 %9, %11 offset:2240\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k0), "=&v"(R[0].v[0][0]), "=&v"(R[0].v[1][0]), "=&v"(R[0].v[2][0]), "=&v"(R[0].v[3][0]),
          "=&v"(k1), "=&v"(R[1].v[0][0]), "=&v"(R[1].v[1][0]), "=&v"(R[1].v[2][0]), "=&v"(R[1].v[3][0])
        : "v"(ak), "v"(av)
        : "memory");
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      R[0].k[c] = k0[c];
      R[1].k[c] = k1[c];
    }
  } else if constexpr (D == 128) {
    static_assert(StageGeo<128, false, FMT>::SUB == 4096, "D = 128 FP8 reader offsets");
    const uint32_t ak1 = s + o.ks;
    u32x4 k0a, k0b, k1a, k1b;
    u32x2 v0[4], v1[4];
    asm volatile(
        "ds_read_b128 %0, %12\n\t"
        "ds_read_b128 %1, %14\n\t"
        "ds_read_b64 %2, %13\n\t"
        "ds_read_b64 %3, %13 offset:128\n\t"
        "ds_read_b64 %4, %13 offset:256\n\t"
        "ds_read_b64 %5, %13 offset:384\n\t"
        "ds_read_b128 %6, %12 offset:4096\n\t"
        "ds_read_b128 %7, %14 offset:4096\n\t"
        "ds_read_b64 %8, %13 offset:4096\n\t"
        "ds_read_b64 %9, %13 offset:4224\n\t"
        "ds_read_b64 %10, %13 offset:4352\n\t"
        "ds_read_b64 %11, %13 offset:4480\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k0a), "=&v"(k0b), "=&v"(v0[0]), "=&v"(v0[1]), "=&v"(v0[2]), "=&v"(v0[3]), "=&v"(k1a),
          "=&v"(k1b), "=&v"(v1[0]), "=&v"(v1[1]), "=&v"(v1[2]), "=&v"(v1[3])
        : "v"(ak), "v"(av), "v"(ak1)
        : "memory");
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      R[0].k[c] = k0a[c];
      R[0].k[4 + c] = k0b[c];
      R[1].k[c] = k1a[c];
      R[1].k[4 + c] = k1b[c];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      R[0].v[r][0] = v0[r][0];
      R[0].v[r][1] = v0[r][1];
      R[1].v[r][0] = v1[r][0];
      R[1].v[r][1] = v1[r][1];
    }
  } else {
    static_assert(D == 256 && StageGeo<256, false, FMT>::SUB == 8192, "D = 256 FP8 reader offsets");
    const uint32_t ak1 = s + o.ks, ak2 = s + o.k2, ak3 = s + o.k3;
    u32x4 k0[4], k1[4], v0[4], v1[4];
    asm volatile(
        "ds_read_b128 %0, %16\n\t"
        "ds_read_b128 %1, %18\n\t"
        "ds_read_b128 %2, %19\n\t"
        "ds_read_b128 %3, %20\n\t"
        "ds_read_b128 %4, %17\n\t"
        "ds_read_b128 %5, %17 offset:256\n\t"
        "ds_read_b128 %6, %17 offset:512\n\t"
        "ds_read_b128 %7, %17 offset:768\n\t"
        "ds_read_b128 %8, %16 offset:8192\n\t"
        "ds_read_b128 %9, %18 offset:8192\n\t"
        "ds_read_b128 %10, %19 offset:8192\n\t"
        "ds_read_b128 %11, %20 offset:8192\n\t"
        "ds_read_b128 %12, %17 offset:8192\n\t"
        "ds_read_b128 %13, %17 offset:8448\n\t"
        "ds_read_b128 %14, %17 offset:8704\n\t"
        "ds_read_b128 %15, %17 offset:8960\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k0[0]), "=&v"(k0[1]), "=&v"(k0[2]), "=&v"(k0[3]), "=&v"(v0[0]), "=&v"(v0[1]), "=&v"(v0[2]),
          "=&v"(v0[3]), "=&v"(k1[0]), "=&v"(k1[1]), "=&v"(k1[2]), "=&v"(k1[3]), "=&v"(v1[0]), "=&v"(v1[1]),
          "=&v"(v1[2]), "=&v"(v1[3])
        : "v"(ak), "v"(av), "v"(ak1), "v"(ak2), "v"(ak3)
        : "memory");
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        R[0].k[4 * q + c] = k0[q][c];
        R[1].k[4 * q + c] = k1[q][c];
        R[0].v[q][c] = v0[q][c];
        R[1].v[q][c] = v1[q][c];
      }
  }
}

// The step's raw bytes for either format (see the readers above).
template <int D, int FMT>
__device__ __forceinline__ void lds_read_step(SubRaw<D, FMT> (&R)[2], const uint8_t* stage, const LdsLane& o) {
  if constexpr (FMT == kNvfp4)
    lds_read_step_async_safe<D>(R, stage, o);
  else
    lds_read_step_fp8<D, FMT>(R, stage, o);
}

template <int D, int FMT>
__device__ __forceinline__ void mask_step(SubRaw<D, FMT> (&R)[2], int kb, int L, int j) {
  if (kb + 32 > L) {
    mask_sub_values(R[0], kb, L, j);
    mask_sub_values(R[1], kb + 16, L, j);
  }
}

}  // namespace nvfp4kv

namespace nvfp4kv {

// ---------------------------------------------------------------------------
// Shared operand tiles (prefill). The waves of a workgroup dequantise a
// step together: operand e of the step (K chunks e < 2 * KW, in the order
// (subtile, chunk); then the V^T tiles) is 64 lanes x 16 bytes in the lane
// layout the MFMA takes, stored at e * 1024 + lane * 16 of an operand
// buffer, so that every write and read is one conflict-free 16-byte LDS
// access per lane. The accesses are asm for the reason the step reader is:
// direct-to-LDS copies are in flight around them.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void lds_store_op(uint32_t addr, const h8& v) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// Eight consecutive operands starting at the operand whose lane slot is addr.
__device__ __forceinline__ void lds_load_ops8(h8 (&o)[8], uint32_t addr) {
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:1024\n\t"
      "ds_read_b128 %2, %8 offset:2048\n\t"
      "ds_read_b128 %3, %8 offset:3072\n\t"
      "ds_read_b128 %4, %8 offset:4096\n\t"
      "ds_read_b128 %5, %8 offset:5120\n\t"
      "ds_read_b128 %6, %8 offset:6144\n\t"
      "ds_read_b128 %7, %8 offset:7168\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
      : "v"(addr)
      : "memory");
}

// Four consecutive operands (head size 64: a step's K or V operands).
__device__ __forceinline__ void lds_load_ops4(h8 (&o)[4], uint32_t addr) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:1024\n\t"
      "ds_read_b128 %2, %4 offset:2048\n\t"
      "ds_read_b128 %3, %4 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(addr)
      : "memory");
}

// Workgroup barrier after this wave's LDS accesses have completed.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory"); }

template <int D>
struct OpGeo {
  static constexpr int NK = 2 * Geo<D>::KW;           // K operands per step
  static constexpr int NE = NK + Geo<D>::DPL;         // all operands per step
  static constexpr int BYTES = NE * 1024;             // one operand buffer
  static_assert(NK % 8 == 0 || D == 64, "K operands come in groups of 8");
};

// Operand E of the step, from its raw bytes (vp: make_pairs of both subtiles).
template <int D, int E, int FMT>
__device__ __forceinline__ h8 make_op(const SubRaw<D, FMT> (&R)[2], const VPairs<D, FMT> (&vp)[2]) {
  using G = Geo<D>;
  if constexpr (E < 2 * G::KW) {
    return k_chunk<D, E % G::KW>(R[E / G::KW]);
  } else {
    constexpr int T = E - 2 * G::KW;
    const h4 a0 = v_operand<D, T>(vp[0]);
    const h4 a1 = v_operand<D, T>(vp[1]);
    return h8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  }
}

// Build and store this wave's share of the step's operands (E = w, w + NW,
// ... for NW waves) at slot + E * 1024 (slot: this lane's place in the
// operand buffer).
template <int D, int E, int NW, int FMT>
__device__ __forceinline__ void make_ops(const SubRaw<D, FMT> (&R)[2], const VPairs<D, FMT> (&vp)[2], int w,
                                         uint32_t slot) {
  if constexpr (E < OpGeo<D>::NE) {
    if (E % NW == w) lds_store_op(slot + E * 1024, make_op<D, E>(R, vp));
    make_ops<D, E + 1, NW>(R, vp, w, slot);
  }
}

template <int D, int E0>
__device__ __forceinline__ void load_ops8(h8 (&ka)[2][Geo<D>::KW], h8 (&va)[Geo<D>::DPL], uint32_t slot) {
  using G = Geo<D>;
  h8 t[8];
  lds_load_ops8(t, slot + E0 * 1024);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int E = E0 + e;
    if (E < 2 * G::KW)
      ka[E / G::KW][E % G::KW] = t[e];
    else if (E < OpGeo<D>::NE)
      va[E - 2 * G::KW] = t[e];
  }
}

// Operands [E0, E1) of the buffer (groups of 8; slot: this lane's place in
// the buffer) into ka (K operands) or va (V^T tiles).
template <int D, int E0, int E1>
__device__ __forceinline__ void load_ops(h8 (&ka)[2][Geo<D>::KW], h8 (&va)[Geo<D>::DPL], uint32_t slot) {
  if constexpr (E0 < E1) {
    load_ops8<D, E0>(ka, va, slot);
    load_ops<D, E0 + 8, E1>(ka, va, slot);
  }
}

}  // namespace nvfp4kv
