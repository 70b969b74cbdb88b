// Device memory for plans made by cp_plan_create_static: callers that cannot
// allocate device memory (code that forbids hipMalloc, such as serving loops
// or harnesses that own the device's memory) get their plan's scratch from a
// fixed array the library holds on every device it runs on.
//
// In host code `scratch` names a host-side stand-in, not device memory: the
// device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address is ever handed to kernels or
// copies.
#include <hip/hip_runtime.h>

#include <mutex>

#include "cp_device.h"

namespace cpms {

namespace {

// Every scratch buffer of one static plan: activations, partial sums, the K/V
// cache, the task lists and the plan state.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices];

__global__ __launch_bounds__(256) void fill_kernel(uint4* p, uint64_t n, uint32_t pattern) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = uint4{pattern, pattern, pattern, pattern};
}

}  // namespace

// Device address of this device's scratch array (`device` must be current).
hipError_t static_scratch(int device, void** ptr, size_t* bytes) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_addr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_addr[device] = p;
  }
  *ptr = g_addr[device];
  *bytes = kStaticScratchBytes;
  return hipSuccess;
}

// Fills [p, p + bytes) (bytes a multiple of 16) with a repeated 32-bit
// pattern, with a kernel on the null stream: static plans initialise their
// scratch without hipMemset.
hipError_t launch_fill(void* p, size_t bytes, uint32_t pattern) {
  const uint64_t n = bytes / 16;
  const unsigned blocks = (unsigned)(n < 256 * 1024 ? (n + 255) / 256 : 1024);
  hipLaunchKernelGGL(fill_kernel, dim3(blocks ? blocks : 1), dim3(256), 0, 0, (uint4*)p, n, pattern);
  return hipGetLastError();
}

}  // namespace cpms
