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
