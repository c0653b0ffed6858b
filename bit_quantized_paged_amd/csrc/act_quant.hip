// NVFP4 quantisation of an activation matrix with swizzled block scales
// [P39129 "Implementation breakdown": the FP4 linear kernels quantise their
// input with scaled_fp4_quant(x, input_global_scale_inv,
// is_sf_swizzled_layout=True) before the block-scaled GEMM, and
// swizzle_blockscale puts scales in the GEMM's tile layout].
//
// The block codec is the KV cache's (quantize_block16). Scales go either
// row-major [m, k/16] or into the 128-row x 4-column tile layout: the scale
// matrix is padded with zeros to a multiple of 128 rows and 4 columns, tile
// (i, j) is 512 consecutive bytes at index i * (cols / 4) + j, and row
// 128i + 32a + b keeps its 4 scales at bytes 16b + 4a .. 16b + 4a + 3.
//
// A workgroup owns 128 rows (one tile row) by KC columns (KC = 128: two
// scale tiles), so each 512-byte scale tile is written by one workgroup,
// padding included. A lane owns one 16-element block (32 bytes in, 8 code
// bytes out) in each of 128 / (2048 / KC) rows, and issues all its loads
// before it quantises; lanes 4q..4q+3 hold the 4 scales of one tile row and
// lane 4q stores them as one word.
#include "quantize.hpp"
#include "launch.hpp"

namespace nvfp4kv {

template <int KC, bool SWZ>
__global__ __launch_bounds__(256) void act_quant_kernel(const uint16_t* __restrict__ x, int64_t xs, int32_t m,
                                                        int32_t k, const float* __restrict__ gscale,
                                                        uint8_t* __restrict__ codes, uint8_t* __restrict__ sf,
                                                        int32_t nchunks) {
  constexpr int LPR = KC / 16;    // lanes per row segment
  constexpr int RPI = 256 / LPR;  // rows per pass of the workgroup
  static_assert(LPR % 4 == 0 && 128 % RPI == 0, "tile shape");
  const int tm = blockIdx.x / nchunks;
  const int chunk = blockIdx.x - tm * nchunks;
  const int lr = threadIdx.x / LPR;
  const int c = chunk * LPR + (threadIdx.x % LPR);  // block (scale column) index in the row
  const int nc = k >> 4;
  const bool cin = c < nc;
  const int ncp4 = (nc + 3) >> 2;  // scale-column tiles
  const float g = *gscale;
  constexpr int NIT = 128 / RPI;
  // All of a lane's loads are issued before any block is quantised. Rows past
  // m and blocks past k/16 load a clamped in-bounds address (m >= 1) and
  // their values are dropped.
  const int cl = cin ? c : nc - 1;
  u32x4 lo[NIT], hi[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int r = tm * 128 + it * RPI + lr;
    const int rl = r < m ? r : m - 1;
    const u32x4* p = reinterpret_cast<const u32x4*>(x + (int64_t)rl * xs + cl * 16);
    lo[it] = p[0];
    hi[it] = p[1];
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int rr = it * RPI + lr;  // row inside the tile row
    const int r = tm * 128 + rr;
    uint32_t s8 = 0;
    if (r < m && cin) {
      float v[16];
      bf16_block16(lo[it], hi[it], v);
      uint32_t w0, w1;
      s8 = quantize_block16(v, g, w0, w1);
      st_u32x2(codes + (int64_t)r * (k >> 1) + c * 8, u32x2{w0, w1});
      if (!SWZ) sf[(int64_t)r * nc + c] = (uint8_t)s8;
    }
    if (SWZ) {
      // every lane reaches this point: the trip count is uniform
      const uint32_t s1 = __shfl_down(s8, 1);
      const uint32_t s2 = __shfl_down(s8, 2);
      const uint32_t s3 = __shfl_down(s8, 3);
      if ((c & 3) == 0 && cin) {
        const int64_t off = ((int64_t)tm * ncp4 + (c >> 2)) * 512 + (rr & 31) * 16 + (rr >> 5) * 4;
        *reinterpret_cast<uint32_t*>(sf + off) = s8 | (s1 << 8) | (s2 << 16) | (s3 << 24);
      }
    }
  }
}

template <int KC>
static hipError_t launch_act_quant_t(const uint16_t* x, int64_t xs, int32_t m, int32_t k, const float* g,
                                     uint8_t* codes, uint8_t* sf, bool swizzled, hipStream_t stream) {
  const int nchunks = (k / 16 + KC / 16 - 1) / (KC / 16);
  const int64_t tiles = ((int64_t)m + 127) / 128;
  const dim3 grid((unsigned)(tiles * nchunks));
  if (swizzled)
    act_quant_kernel<KC, true><<<grid, 256, 0, stream>>>(x, xs, m, k, g, codes, sf, nchunks);
  else
    act_quant_kernel<KC, false><<<grid, 256, 0, stream>>>(x, xs, m, k, g, codes, sf, nchunks);
  return hipGetLastError();
}

hipError_t launch_act_quant(const void* x, int64_t x_row_stride, int32_t m, int32_t k, const float* global_scale,
                            void* codes, void* scales, bool swizzled, hipStream_t stream) {
  if (m == 0) return hipSuccess;
  return launch_act_quant_t<128>(static_cast<const uint16_t*>(x), x_row_stride, m, k, global_scale,
                                 static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales), swizzled, stream);
}

}  // namespace nvfp4kv
