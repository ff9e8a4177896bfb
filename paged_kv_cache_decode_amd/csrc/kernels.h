// Launchers for the gfx950 kernels (implemented in the .hip files) and the
// event-based kernel timer they report to.
#pragma once

#include <hip/hip_runtime.h>

#include "plan.h"

namespace pa {

// Launches the partition kernel and the log-sum-exp merge.  `workspace`
// holds plan.ws_bytes bytes.
hipError_t launch_decode(const DecodePlan& plan, void* workspace, hipStream_t stream);

// This GPU's copy of pa_decode_noalloc's fixed workspace (decode.hip): its
// device address, looked up once per device, whose counter region is zeroed
// on `stream` at that first call.
hipError_t noalloc_workspace(hipStream_t stream, void** ws);

// Decode workers for this instance on the current device: one workgroup of
// kDecodeWaves wavefronts per compute unit (an MI355X's 256 CUs without a
// device).
int decode_worker_count(int dtype, int D, int G);

hipError_t launch_prefill(const PrefillPlan& plan, hipStream_t stream);

// pa_decode_shared_prefix's prefix step (`pre`, prefill in key-chunk mode)
// and suffix step (`dec`, with workspace `workspace`) as one kernel.
hipError_t launch_shared_prefix(const DecodePlan& dec, void* workspace, const PrefillPlan& pre,
                                hipStream_t stream);

// Joins partial attention states (pa_merge_states).
hipError_t launch_merge(const MergePlan& plan, hipStream_t stream);

// Joins a shared prefix's key chunks with the suffix step's state.
hipError_t launch_prefix_join(const PrefixJoinPlan& plan, hipStream_t stream);

hipError_t launch_write_kv(const WriteKvPlan& plan, hipStream_t stream);

hipError_t launch_copy_blocks(const CopyBlocksPlan& plan, hipStream_t stream);

// Shader-clock probe (pa_clock_probe): out[0] = shader clock ticks, out[1] =
// 100 MHz reference ticks over one wave's wait of `ticks` reference ticks.
hipError_t launch_clock_probe(int64_t ticks, int64_t* out, hipStream_t stream);

// Kernel timer.  While the profiler is enabled, a KernelTimer holds a pair
// of events that timed_launch (launch.h) binds to one kernel dispatch; the
// pair is queued for reading by commit() and released otherwise.
bool profiler_enabled();
struct KernelTimer {
  KernelTimer(const char* name, hipStream_t stream);
  ~KernelTimer();
  KernelTimer(const KernelTimer&) = delete;
  KernelTimer& operator=(const KernelTimer&) = delete;
  void commit();
  const char* name_;
  hipEvent_t start_ = nullptr;
  hipEvent_t stop_ = nullptr;
};

}  // namespace pa
