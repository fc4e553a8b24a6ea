// Host-only stand-ins for the HIP runtime calls and kernel launchers used by
// api.cpp, so that the C-ABI host logic can be built with g++ and run under
// AddressSanitizer / UndefinedBehaviorSanitizer without a GPU.
#include <hip/hip_runtime_api.h>

#include <cstring>
#include <vector>

#include "internal.h"
#include "tables.h"

static int g_launches = 0;
int stub_launch_count() { return g_launches; }

extern "C" hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind,
                                     hipStream_t) {
  // the workspace pointer in the driver is real host memory
  std::memcpy(dst, src, n);
  return hipSuccess;
}
extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }

namespace s4 {
// the library's static scratch, played by host memory of the same size
static std::vector<unsigned char>* g_scratch = nullptr;
size_t noalloc_scratch_bytes() { return size_t(64) << 20; }
hipError_t noalloc_scratch(unsigned char** out) {
  if (!g_scratch) g_scratch = new std::vector<unsigned char>(noalloc_scratch_bytes());
  *out = g_scratch->data();
  return hipSuccess;
}
bool lds_path(const s4dplr_plan* p) { return p->log2L <= S4DPLR_LDS_MAX_LOG2L; }
// the device table kernel, played by the same per-entry formulas on the host
hipError_t launch_plan_tables(const s4dplr_plan* p, unsigned char* w, hipStream_t) {
  ++g_launches;
  const TableSpec a = plan_table_spec(p, w);
  const long n = table_entries(a);
  for (long g = 0; g < n; ++g) table_entry(a, g);
  return hipSuccess;
}
hipError_t launch_kernel_gen(const s4dplr_plan*, const float*, const float*, const float*,
                             const float*, const float*, const float*, const float*, float*,
                             unsigned char*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_generating_function(const s4dplr_plan*, const float*, const float*,
                                      const float*, const float*, const float*, const float*,
                                      float*, unsigned char*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_spectrum_from_time(const s4dplr_plan*, const float*, const float*,
                                     unsigned char*, hipStream_t, int) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_conv(const s4dplr_plan*, const float*, float*, unsigned char*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_corr(const s4dplr_plan*, const float*, const float*, float*, float*,
                       unsigned char*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_kernel_gen_bwd(const s4dplr_plan*, const float*, const float*, const float*,
                                 const float*, const float*, const float*, const float*, float*,
                                 float*, float*, float*, float*, float*, unsigned char*,
                                 hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_vandermonde(const s4dplr_plan*, const float*, const float*, const float*,
                              const float*, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_vandermonde_bwd(const s4dplr_plan*, const float*, const float*, const float*,
                                  const float*, const float*, float*, float*, float*, float*,
                                  unsigned char*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_layer_norm(const s4dplr_plan*, const float*, const float*, const float*, float*,
                             hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_block_epilogue(const s4dplr_plan*, const float*, const float*, const float*,
                                 const float*, float*, unsigned char*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_big_corr(const s4dplr_plan*, const float*, const float*, float*, float*,
                           unsigned char*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_big_ghat(const s4dplr_plan*, const float*, unsigned char*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_recurrent_prepare(const s4dplr_plan*, const float*, const float*,
                                    const float*, const float*, const float*, const float*,
                                    unsigned char*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_recurrent_scan(const s4dplr_plan*, const float*, const float*, float*, float*,
                                 int, unsigned char*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
}  // namespace s4
