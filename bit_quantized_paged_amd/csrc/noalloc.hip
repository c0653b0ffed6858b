// The decode scratch that nvfp4_paged_attention_decode_noalloc uses instead
// of a caller workspace: a device-resident array of fixed size, one copy per
// GPU, held until the process ends. For callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).
#include <mutex>

#include "launch.hpp"

namespace nvfp4kv {
namespace {

// [kScratchCounterBytes of split-K arrival counters][partials]. In host code
// `scratch` names a host-side stand-in, not device memory: only the address
// hipGetSymbolAddress returns for the current device may reach a kernel.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

}  // namespace

hipError_t scratch_for_current_device(hipStream_t stream, void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    // Every completed decode leaves the counters it used at zero; they start
    // at zero through this clear, a kernel (not a memset node) on the first
    // caller's stream, ahead of that caller's decode.
    zero_words_kernel<<<(unsigned)(kScratchCounters / 256), 256, 0, stream>>>(static_cast<uint32_t*>(p),
                                                                             kScratchCounters);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace nvfp4kv
