// Measurement aid, not an operation of the method: a read-only stream of a
// device buffer, to give the benchmark the HBM read rate a kernel reading
// the same number of bytes reaches on the same device (the ceiling against
// which the attention kernels' cache-read stream is judged).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nvfp4kv_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Every lane reads 16-byte chunks i, i + S, ... (S = all lanes of the grid),
// four loads in flight, and folds them with XOR; one word per wave goes to
// sink so that no load can be dropped.
__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int64_t s = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * s < n16; i += 4 * s) {
    const u32x4 a = p[i], b = p[i + s], c = p[i + 2 * s], d = p[i + 3 * s];
    const u32x4 x = a ^ b ^ c ^ d;
    acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
  }
  for (; i < n16; i += s) {
    const u32x4 x = p[i];
    acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}


// The pages a decode batch reads, as a plain gather: workgroup u owns unit
// (sequence b, kv head h, split) of `splits` equal page ranges per sequence;
// its four waves take pages p0 + w, p0 + w + 4, ... and each reads a page's
// K slab and V slab (slab_bytes contiguous bytes each: page rows are
// contiguous), 16 bytes per lane and load, kPagesInFlight pages at a time.
// CPL 16-byte chunks per lane and slab: 2 (slabs of up to 2 KB: head sizes
// up to 128 at 16-row pages) or 4 (up to 4 KB); the smaller form holds half
// the registers, so it keeps more waves in flight where it suffices.
constexpr int kPagesInFlight = 4;
constexpr int kMaxChunksPerLane = 4;

template <int CPL>
__global__ __launch_bounds__(256) void read_pages_kernel(const uint8_t* __restrict__ pool, int64_t stride_block,
                                                         int64_t stride_kv, int64_t stride_head,
                                                         const int32_t* __restrict__ block_table, int max_blocks,
                                                         const int32_t* __restrict__ seq_lens, int num_kv_heads,
                                                         int splits, int block_size, int slab_bytes,
                                                         int64_t num_blocks, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int u = blockIdx.x;
  const int split = u % splits;
  const int h = (u / splits) % num_kv_heads;
  const int b = u / (splits * num_kv_heads);
  const int L = seq_lens[b] < 0 ? 0 : seq_lens[b];
  int pages = (L + block_size - 1) / block_size;
  pages = pages > max_blocks ? max_blocks : pages;
  const int p0 = (int)((int64_t)pages * split / splits), p1 = (int)((int64_t)pages * (split + 1) / splits);
  const int nc = slab_bytes / 16;
  const int32_t* row = block_table + (int64_t)b * max_blocks;
  uint32_t acc = 0;
  for (int p = p0 + w; p < p1; p += 4 * kPagesInFlight) {
    u32x4 v[kPagesInFlight][2][CPL];
#pragma unroll
    for (int k = 0; k < kPagesInFlight; ++k) {
      const int pk = p + 4 * k;
#pragma unroll
      for (int kv = 0; kv < 2; ++kv)
#pragma unroll
        for (int c = 0; c < CPL; ++c) v[k][kv][c] = u32x4{0u, 0u, 0u, 0u};
      if (pk < p1) {
        int64_t id = row[pk];
        id = id < 0 ? 0 : (id >= num_blocks ? num_blocks - 1 : id);
#pragma unroll
        for (int kv = 0; kv < 2; ++kv) {
          const u32x4* src = reinterpret_cast<const u32x4*>(pool + id * stride_block + kv * stride_kv +
                                                            (int64_t)h * stride_head);
#pragma unroll
          for (int c = 0; c < CPL; ++c)
            if (lane + 64 * c < nc) v[k][kv][c] = src[lane + 64 * c];
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kPagesInFlight; ++k)
#pragma unroll
      for (int kv = 0; kv < 2; ++kv)
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const u32x4 x = v[k][kv][c];
          acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
        }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  if (lane == 0) sink[blockIdx.x * 4 + w] = acc;
}

}  // namespace

extern "C" int32_t nvfp4kv_probe_read_stream(const void* data, int64_t bytes, int32_t grid, void* sink,
                                             int64_t sink_bytes, void* stream) {
  if (data == nullptr || sink == nullptr || bytes < 16 || bytes % 16 != 0 || grid < 1 ||
      (reinterpret_cast<uintptr_t>(data) % 16) != 0 || (reinterpret_cast<uintptr_t>(sink) % 4) != 0 ||
      sink_bytes < (int64_t)grid * 16)
    return 1;
  read_stream_kernel<<<grid, 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const u32x4*>(data), bytes / 16,
                                                                      static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int32_t nvfp4kv_probe_read_pages(const void* pool, int64_t num_blocks, int64_t stride_block,
                                            int64_t stride_kv, int64_t stride_head, int32_t slab_bytes,
                                            int32_t block_size, int32_t num_kv_heads, const int32_t* block_table,
                                            int32_t max_blocks, const int32_t* seq_lens, int32_t num_seqs,
                                            int32_t splits, void* sink, int64_t sink_bytes, void* stream) {
  const int64_t grid = (int64_t)num_seqs * num_kv_heads * splits;
  if (pool == nullptr || block_table == nullptr || seq_lens == nullptr || sink == nullptr || splits < 1 ||
      num_blocks < 1 || max_blocks < 1 || num_seqs < 1 || block_size < 1 || num_kv_heads < 1 || slab_bytes < 16 ||
      slab_bytes % 16 != 0 || slab_bytes > 64 * 16 * kMaxChunksPerLane || (reinterpret_cast<uintptr_t>(pool) % 16) != 0 ||
      stride_block % 16 != 0 || stride_kv % 16 != 0 || stride_head % 16 != 0 || grid > INT32_MAX ||
      (reinterpret_cast<uintptr_t>(sink) % 4) != 0 || sink_bytes < grid * 16)
    return 1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (slab_bytes <= 64 * 16 * 2)
    read_pages_kernel<2><<<(unsigned)grid, 256, 0, st>>>(static_cast<const uint8_t*>(pool), stride_block, stride_kv,
                                                          stride_head, block_table, max_blocks, seq_lens, num_kv_heads,
                                                          splits, block_size, slab_bytes, num_blocks,
                                                          static_cast<uint32_t*>(sink));
  else
    read_pages_kernel<4><<<(unsigned)grid, 256, 0, st>>>(static_cast<const uint8_t*>(pool), stride_block, stride_kv,
                                                          stride_head, block_table, max_blocks, seq_lens, num_kv_heads,
                                                          splits, block_size, slab_bytes, num_blocks,
                                                          static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
