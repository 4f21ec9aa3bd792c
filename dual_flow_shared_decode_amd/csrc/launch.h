// Kernel launch with optional dispatch events (hipExtLaunchKernelGGL records
// them from the dispatch itself, without extra commands on the stream) and
// optional dynamic LDS bytes.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "dfa_internal.h"

namespace dfa {

template <typename Kernel, typename Params>
hipError_t launch_kernel(Kernel kernel, dim3 grid, dim3 block, hipStream_t stream, const KernelEvents& ev,
                         const Params& params, size_t lds_bytes = 0) {
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, ev.start, ev.stop, 0, params);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, params);
  return hipGetLastError();
}

}  // namespace dfa
