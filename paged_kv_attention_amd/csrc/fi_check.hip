// fi_check.hip -- debug check of the device page tables a run call reads.
//
// The run calls trust that every page id they read lies in the caller's pool
// (the pages are gathered unconditionally). This optional check counts the
// ids outside [0, num_pages) so that a caller can verify its tables while
// debugging; it is not part of any run call.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "fi_host.h"

namespace fi {
namespace {

__global__ __launch_bounds__(64) void zero_count_kernel(int32_t* count) {
  if (threadIdx.x == 0) *count = 0;
}

// Grid-stride count of the out-of-range ids of one table; one atomic add per
// thread that found any.
__global__ __launch_bounds__(256) void count_bad_ids_kernel(const int32_t* ids, int64_t n,
                                                           int32_t num_pages, int32_t* count) {
  int32_t bad = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int32_t v = ids[i];
    bad += (v < 0 || v >= num_pages) ? 1 : 0;
  }
  if (bad) atomicAdd(count, bad);
}

}  // namespace

hipError_t launch_check_page_ids(const int32_t* kv_ids, int64_t n_kv, const int32_t* prefix_ids,
                                 int64_t n_prefix, int32_t num_pages, int32_t* count,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(zero_count_kernel, dim3(1), dim3(64), 0, stream, count);
  hipError_t e = hipGetLastError();
  const int32_t* ids[2] = {kv_ids, prefix_ids};
  const int64_t n[2] = {n_kv, n_prefix};
  for (int t = 0; t < 2 && e == hipSuccess; ++t) {
    if (!ids[t] || n[t] == 0) continue;
    const unsigned blocks = (unsigned)std::min<int64_t>(1024, (n[t] + 255) / 256);
    hipLaunchKernelGGL(count_bad_ids_kernel, dim3(blocks), dim3(256), 0, stream, ids[t], n[t],
                       num_pages, count);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace fi
