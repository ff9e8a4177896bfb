// pa_decode_shared_prefix's main kernel: its prefix step and suffix step in
// one launch.
//
// The prefix step (every sequence's query heads against the shared prefix
// keys, as one dense block on the matrix cores: prefill workgroups of four
// waves, keys split into chunks) and the suffix step (the decode kernel on
// each sequence's own keys) share no data until the join, and each leaves
// most of a compute unit idle: the suffix step streams HBM with one wave per
// SIMD, the prefix step is a short burst of matrix work.  Both run as the
// two kinds of workgroup of one kernel: workgroups [0, dec_groups) are
// decode workgroups, the rest prefill workgroups, and the two kinds share
// compute units (LDS sized for the larger, registers for either at two
// waves per SIMD).  A second kernel on the same stream then joins the
// prefix's chunks with the suffix state (prefix_join_kernel, decode.hip).
// One stream, two dispatches: no cross-stream events.  Measured on 256
// sequences sharing a 2048-token prefix (bf16, 32 / 8 heads): 123 us per
// call, against 129 us with the two steps as kernels on two streams joined
// by events, and 144 us with the prefix step first and the decode kernel
// starting from its result.  Putting the prefill workgroups first in the
// grid, or reading K in the MFMA layout, measured slower.
#include "decode_kernel.h"
#include "launch.h"
#include "prefill_kernel.h"

namespace pa {
namespace {

template <class T, int G>
struct SharedPrefixShape {
  static constexpr int kHG = G > 4 ? 4 : G;              // heads per prefill workgroup
  static constexpr int kRW = kPrefixStepWaves / kHG;     // 16-row waves per head
  static constexpr bool kKRows = G <= 4;                 // decode reads K as whole rows
  static constexpr int kDecLds = DecodeLds<T, 128, G, kKRows>::kBytes;
  static constexpr int kPreLds = PrefillLds<kHG, kRW>::kBytes;
  static constexpr int kLds = kPreLds > kDecLds ? kPreLds : kDecLds;
  static_assert(kHG * kRW == kDecodeWaves, "both kinds of workgroup have four waves");
};

template <class T, int G>
__global__ __launch_bounds__(64 * kDecodeWaves)
__attribute__((amdgpu_waves_per_eu(2))) void shared_prefix_kernel(DecodeArgs da, PrefillArgs pa,
                                                                  int dec_groups) {
  using Shape = SharedPrefixShape<T, G>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[Shape::kLds];
  if ((int)blockIdx.x < dec_groups) {
    decode_body<T, 128, G, Shape::kKRows>(da, blockIdx.x, dec_groups, lds);
  }
  else
    prefill_body<T, Shape::kHG, Shape::kRW>(pa, (int64_t)blockIdx.x - dec_groups, lds);
}

template <class T, int G>
hipError_t launch_t(const DecodeArgs& da, const PrefillArgs& pa, int dec_groups,
                    int64_t blocks, hipStream_t stream) {
  return timed_launch("shared_prefix", shared_prefix_kernel<T, G>, dim3((unsigned)blocks),
                      dim3(64 * kDecodeWaves), stream, da, pa, dec_groups);
}

template <class T>
hipError_t dispatch_g(int G, const DecodeArgs& da, const PrefillArgs& pa, int dec_groups,
                      int64_t blocks, hipStream_t stream) {
  switch (G) {
    case 1: return launch_t<T, 1>(da, pa, dec_groups, blocks, stream);
    case 2: return launch_t<T, 2>(da, pa, dec_groups, blocks, stream);
    case 4: return launch_t<T, 4>(da, pa, dec_groups, blocks, stream);
    case 8: return launch_t<T, 8>(da, pa, dec_groups, blocks, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_shared_prefix(const DecodePlan& dp, void* workspace, const PrefillPlan& pp,
                                hipStream_t stream) {
  if (dp.D != 128 || dp.grid[0] % 8 != 0) return hipErrorInvalidValue;
  const DecodeArgs da = decode_args(dp, workspace);
  const PrefillArgs pa = prefill_args(pp);
  const int dec_groups = (int)dp.grid[0];
  // Prefill workgroups follow the decode ones; dec_groups is a multiple of
  // 8, so each keeps the XCD its own number gives it.
  const int64_t blocks = dec_groups + (pa.n_wg > 0 ? pa.wg_per_xcd * 8 : 0);
  switch (dp.dtype) {
    case PA_F16: return dispatch_g<TF16>(dp.G, da, pa, dec_groups, blocks, stream);
    case PA_BF16: return dispatch_g<TBF16>(dp.G, da, pa, dec_groups, blocks, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
