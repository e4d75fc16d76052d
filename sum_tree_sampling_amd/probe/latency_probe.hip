// latency_probe.hip -- the two measurement aids of include/per_probe.h: an
// empty kernel (the floor of a launch) and a single-lane chain of dependent
// loads (the floor of a walk down the tree, one level per load).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/per_probe.h"

namespace {

__global__ void __launch_bounds__(64) empty_kernel() {}

__global__ void __launch_bounds__(64) chain_kernel(const uint32_t* __restrict__ next,
                                                   uint32_t mask, int64_t depth,
                                                   uint32_t* __restrict__ out) {
  if (threadIdx.x != 0) return;
  uint32_t i = 0;
  for (int64_t k = 0; k < depth; ++k) i = next[i & mask];
  out[0] = i;
}

}  // namespace

extern "C" {

int per_probe_empty(int64_t launches, hipStream_t stream) {
  if (launches < 1) return -1;
  for (int64_t k = 0; k < launches; ++k)
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int per_probe_chain(const uint32_t* d_next, int64_t length, int64_t depth, uint32_t* d_out,
                    hipStream_t stream) {
  if (!d_next || !d_out || depth < 1 || length < 1 || length > (int64_t(1) << 30) ||
      (length & (length - 1)) != 0)
    return -1;
  hipLaunchKernelGGL(chain_kernel, dim3(1), dim3(64), 0, stream, d_next,
                     (uint32_t)(length - 1), depth, d_out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
