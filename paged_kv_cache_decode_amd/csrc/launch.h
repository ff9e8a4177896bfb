// Kernel launch with optional per-dispatch timing (device code only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace pa {

// Launches `kernel`; while the library profiler is on, the start/stop events
// are attached to this dispatch itself (hipExtLaunchKernelGGL), so the
// elapsed time is the kernel's own execution, as a kernel trace reports it.
template <class... Params, class... Args>
hipError_t timed_launch(const char* name, void (*kernel)(Params...), dim3 grid, dim3 block,
                        hipStream_t stream, Args... args) {
  KernelTimer t(name, stream);
  if (t.start_)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, t.start_, t.stop_, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) t.commit();
  return e;
}

}  // namespace pa
