// Launchers for the gfx950 kernels (implemented in the .hip files) and the
// event-based kernel timer they report to.
#pragma once

#include <hip/hip_runtime.h>

#include "plan.h"

namespace pa {

// Launches the partition kernel and the log-sum-exp merge.  `workspace`
// holds plan.ws_bytes bytes.
hipError_t launch_decode(const DecodePlan& plan, void* workspace, hipStream_t stream);

// Wavefronts of the decode kernel the current device keeps resident for
// this instance (falls back to an MI355X's 256 CUs x 12 without a device).
int decode_worker_count(int dtype, int D, int G);

hipError_t launch_prefill(const PrefillPlan& plan, hipStream_t stream);

hipError_t launch_write_kv(const WriteKvPlan& plan, hipStream_t stream);

// Kernel timer: while enabled, KernelTimer brackets a launch with events.
bool profiler_enabled();
struct KernelTimer {
  KernelTimer(const char* name, hipStream_t stream);
  ~KernelTimer();
  const char* name_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr;
};

}  // namespace pa
