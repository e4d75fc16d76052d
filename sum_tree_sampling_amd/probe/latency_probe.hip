// latency_probe.hip -- the measurement aids of include/per_probe.h: an
// empty kernel (the floor of a launch), a single-lane chain of dependent
// loads (the floor of a walk down the tree, one level per load), and the
// cost an argument block adds to a launch, eager or replayed from a graph.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/per_probe.h"

namespace {

__global__ void __launch_bounds__(64) empty_kernel() {}

template <int BYTES>
struct ArgBlock {
  uint64_t w[BYTES / 8];
};

// Empty in effect: the store needs a first word no caller passes.
template <int BYTES>
__global__ void __launch_bounds__(64) args_kernel(ArgBlock<BYTES> a, uint32_t* out) {
  if (threadIdx.x == 0 && a.w[0] == 0x5EEDull) out[0] = 1u;
}

template <int BYTES>
hipError_t launch_cost(int64_t launches, bool graph, double* us) {
  ArgBlock<BYTES> a{};
  hipStream_t s = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipGraph_t g = nullptr;
  hipGraphExec_t ge = nullptr;
  uint32_t* out = nullptr;  // never written (see args_kernel)
  hipError_t e = hipStreamCreate(&s);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  auto batch = [&](int64_t n) {
    for (int64_t k = 0; k < n; ++k) hipLaunchKernelGGL(args_kernel<BYTES>, dim3(1), dim3(64), 0, s, a, out);
    return hipGetLastError();
  };
  if (e == hipSuccess && graph) {
    e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
    if (e == hipSuccess) {
      const hipError_t eb = batch(100);
      e = hipStreamEndCapture(s, &g);
      if (e == hipSuccess) e = eb;
    }
    if (e == hipSuccess) e = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
  }
  auto run = [&](int64_t n) {
    if (!graph) return batch(n);
    for (int64_t r = 0; r < n / 100; ++r) {
      const hipError_t el = hipGraphLaunch(ge, s);
      if (el != hipSuccess) return el;
    }
    return hipSuccess;
  };
  if (e == hipSuccess) e = run(200);  // warm-up
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipEventRecord(e0, s);
  if (e == hipSuccess) e = run(launches);
  if (e == hipSuccess) e = hipEventRecord(e1, s);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e == hipSuccess) *us = (double)ms * 1e3 / (double)launches;
  if (ge) (void)hipGraphExecDestroy(ge);
  if (g) (void)hipGraphDestroy(g);
  if (e1) (void)hipEventDestroy(e1);
  if (e0) (void)hipEventDestroy(e0);
  if (s) (void)hipStreamDestroy(s);
  return e;
}

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

int per_probe_launch_cost(int64_t launches, int arg_bytes, int graph, double* us_per_launch) {
  if (!us_per_launch || launches < 100 || launches > 100000 || launches % 100 != 0) return -1;
  hipError_t e;
  switch (arg_bytes) {
    case 16:
      e = launch_cost<16>(launches, graph != 0, us_per_launch);
      break;
    case 256:
      e = launch_cost<256>(launches, graph != 0, us_per_launch);
      break;
    case 512:
      e = launch_cost<512>(launches, graph != 0, us_per_launch);
      break;
    default:
      return -1;
  }
  return e == hipSuccess ? 0 : -4;
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
