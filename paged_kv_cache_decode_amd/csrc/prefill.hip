// Paged prefill: kernel instances and launch.  The kernel's device code and
// design notes are in prefill_kernel.h.
#include "prefill_kernel.h"
#include "launch.h"

namespace pa {
namespace {

// Sixteen-wave workgroups (packed prompts) ask for at most 128 registers,
// four waves per SIMD; four-wave ones (the shared-prefix step) for at most
// 256.
template <class T, int HG, int RW>
__global__ __launch_bounds__(64 * HG * RW)
__attribute__((amdgpu_waves_per_eu(HG * RW == 16 ? 4 : 2))) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[PrefillLds<HG, RW>::kBytes];
  prefill_body<T, HG, RW>(a, blockIdx.x, lds);
}

template <class T, int HG, int RW>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
  const int64_t blocks = a.wg_per_xcd * 8;
  return timed_launch("prefill", prefill_kernel<T, HG, RW>, dim3((unsigned)blocks),
                      dim3(64 * HG * RW), stream, a);
}

// Workgroups of 16 waves (packed prompts) or 4 waves (the shared-prefix
// step): HG = min(G, 4) heads x (waves / HG) row slices.
template <class T>
hipError_t dispatch_shape(const PrefillPlan& pl, const PrefillArgs& a, hipStream_t stream) {
  const int hg = pl.G > 4 ? 4 : pl.G;
  switch (hg * 100 + hg * pl.row_waves) {
    case 116: return launch_prefill_t<T, 1, 16>(a, stream);
    case 216: return launch_prefill_t<T, 2, 8>(a, stream);
    case 416: return launch_prefill_t<T, 4, 4>(a, stream);
    case 104: return launch_prefill_t<T, 1, 4>(a, stream);
    case 204: return launch_prefill_t<T, 2, 2>(a, stream);
    case 404: return launch_prefill_t<T, 4, 1>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillPlan& pl, hipStream_t stream) {
  const PrefillArgs a = prefill_args(pl);
  if (a.n_wg == 0) return hipSuccess;
  switch (pl.dtype) {
    case PA_F16: return dispatch_shape<TF16>(pl, a, stream);
    case PA_BF16: return dispatch_shape<TBF16>(pl, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
