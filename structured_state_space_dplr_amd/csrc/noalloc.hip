// Library-owned device scratch for s4dplr_forward_noalloc: a file-scope
// device array that stands in for the caller's workspace, for callers that
// cannot allocate device memory.  Each GPU the library runs on holds its own
// copy of the array at its own address until the process ends.
//
// In host code the array's name is only a host-side stand-in, never a device
// address: its device address is looked up once per device, with that device
// current, by hipGetSymbolAddress, and that address (not the name) is what
// kernels and copies receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"
#include "tables.h"

namespace s4 {

// Largest forward workspace prefix the array holds: the tables, the
// generating function, the convolution weights and, for L >= 32768, the
// kernel buffer and the four-step intermediate.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
unsigned char* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

size_t noalloc_scratch_bytes() { return kNoallocScratchBytes; }

namespace {

// The plan's table region (tables.h), one entry per thread of a grid-stride
// loop, so that the no-allocation path copies nothing from host memory.
__global__ void table_kernel(TableSpec a) {
  const long total = table_entries(a);
  for (long g = blockIdx.x * (long)blockDim.x + threadIdx.x; g < total;
       g += (long)gridDim.x * blockDim.x)
    table_entry(a, g);
}

}  // namespace

hipError_t launch_plan_tables(const s4dplr_plan* p, unsigned char* w, hipStream_t s) {
  table_kernel<<<256, 256, 0, s>>>(plan_table_spec(p, w));
  return hipGetLastError();
}

hipError_t noalloc_scratch(unsigned char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<unsigned char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace s4
