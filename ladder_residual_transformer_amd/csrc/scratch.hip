// Library-owned device scratch for callers that cannot allocate device memory.
//
// `scratch` is a file-scope device array: every GPU the library runs on holds its own
// copy, at its own address, from the code object's load until the process ends.  In host
// code the array's name is only a stand-in for the symbol, not a device address, so the
// address of each device's copy is looked up once per device (hipGetSymbolAddress, with
// that device current) and kept here; every kernel argument, fill and copy uses that
// address.  Calls that use the array on one GPU share it: overlapping calls race, and
// each call clears what it needs at zero itself.
#include <algorithm>
#include <mutex>

#include "kernels.h"

namespace ladder {

static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
hipError_t g_status[kMaxDevices] = {};
bool g_done[kMaxDevices] = {};

// Zero n 16-byte words with vector stores (a kernel rather than a memset, so a caller
// may capture the step into a HIP graph).
__global__ __launch_bounds__(256) void zero_words_kernel(uint4* p, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace

hipError_t static_scratch_setup(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_done[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipErrorInvalidDevice;   // the caller makes dev current
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = e == hipSuccess ? p : nullptr;
    g_status[dev] = e;
    g_done[dev] = true;
  }
  return g_status[dev];
}

hipError_t static_scratch(int dev, void** ptr) {
  if (dev < 0 || dev >= kMaxDevices || !ptr) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_done[dev]) return hipErrorNotInitialized;
  *ptr = g_ptr[dev];
  return g_status[dev];
}

hipError_t launch_zero_bytes(void* p, size_t bytes, hipStream_t s) {
  if (!p || ((uintptr_t)p & 15u) || (bytes & 15u)) return hipErrorInvalidValue;
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_words_kernel, dim3(blocks), dim3(256), 0, s, (uint4*)p, n);
  return hipGetLastError();
}

}  // namespace ladder
