// Paged decode: kernel instances, launch and worker planning, the
// fixed-workspace variant, pa_merge_states and the shared-prefix join.  The
// partition kernel's device code and design notes are in decode_kernel.h.
#include "decode_kernel.h"
#include "launch.h"

#include <map>
#include <mutex>
#include <tuple>

namespace pa {
namespace {

template <class T, int D, int G, bool kKRows>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_partitions_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[DecodeLds<T, D, G, kKRows>::kBytes];
  decode_body<T, D, G, kKRows>(a, blockIdx.x, gridDim.x, lds);
}

template <class T, int D, int G>
hipError_t launch_decode_t(const DecodePlan& pl, const DecodeArgs& a, hipStream_t stream) {
  // The suffix step after a shared prefix (fp16 / bf16, d = 128) reads K as
  // whole rows; with groups of 8 that instance would spill registers, so
  // those keep the operand-layout loads.
  if constexpr (D == 128 && !__is_same(T, TF32) && G <= 4) {
    if (pl.key_begin > 0)
      return timed_launch("decode_partitions", decode_partitions_kernel<T, D, G, true>,
                          dim3((unsigned)pl.grid[0]), dim3(pl.block_threads), stream, a);
  }
  return timed_launch("decode_partitions", decode_partitions_kernel<T, D, G, false>,
                      dim3((unsigned)pl.grid[0]), dim3(pl.block_threads), stream, a);
}

// One workgroup (kDecodeWaves wavefronts) per compute unit.  Measured on
// MI355X, one wavefront per SIMD streams K/V faster than two: fewer, longer
// slices mean fewer pipeline restarts at unit boundaries and fewer
// partitions, with enough bytes still in flight.
template <class T, int D, int G>
int resident_waves_t() {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(decode_partitions_kernel<T, D, G, false>),
          64 * kDecodeWaves, 0) != hipSuccess)
    return 0;
  return per_cu >= 1 ? cus * kDecodeWaves : 0;
}

template <class T>
int resident_waves_shape(int D, int G) {
  switch (D * 10 + G) {
    case 641: return resident_waves_t<T, 64, 1>();
    case 642: return resident_waves_t<T, 64, 2>();
    case 644: return resident_waves_t<T, 64, 4>();
    case 648: return resident_waves_t<T, 64, 8>();
    case 1281: return resident_waves_t<T, 128, 1>();
    case 1282: return resident_waves_t<T, 128, 2>();
    case 1284: return resident_waves_t<T, 128, 4>();
    case 1288: return resident_waves_t<T, 128, 8>();
    default: return 0;
  }
}

template <class T>
hipError_t dispatch_shape(const DecodePlan& pl, const DecodeArgs& a, hipStream_t stream) {
  switch (pl.D * 10 + pl.G) {
    case 641: return launch_decode_t<T, 64, 1>(pl, a, stream);
    case 642: return launch_decode_t<T, 64, 2>(pl, a, stream);
    case 644: return launch_decode_t<T, 64, 4>(pl, a, stream);
    case 648: return launch_decode_t<T, 64, 8>(pl, a, stream);
    case 1281: return launch_decode_t<T, 128, 1>(pl, a, stream);
    case 1282: return launch_decode_t<T, 128, 2>(pl, a, stream);
    case 1284: return launch_decode_t<T, 128, 4>(pl, a, stream);
    case 1288: return launch_decode_t<T, 128, 8>(pl, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int decode_worker_count(int dtype, int D, int G) {
  // Resident capacity of the current device for this instance, cached.
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, int>, int> cache;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  const auto key = std::make_tuple(dev, dtype, D, G);
  {
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  int w = 0;
  if (dev >= 0) {
    switch (dtype) {
      case PA_F32: w = resident_waves_shape<TF32>(D, G); break;
      case PA_F16: w = resident_waves_shape<TF16>(D, G); break;
      case PA_BF16: w = resident_waves_shape<TBF16>(D, G); break;
      default: break;
    }
  }
  // Without a device (planning only) assume an MI355X: 256 CUs.
  if (w <= 0) w = 256 * kDecodeWaves;
  std::lock_guard<std::mutex> lk(mu);
  cache[key] = w;
  return w;
}

namespace {

// pa_decode_noalloc's workspace: a file-scope device array, one copy per GPU
// that the library runs on, held until the process ends.  In host code its
// name is only a stand-in; the device address of the current GPU's copy
// comes from hipGetSymbolAddress (noalloc_workspace) and is what kernels
// and copies get.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0u;
}

}  // namespace

hipError_t noalloc_workspace(hipStream_t stream, void** ws) {
  static std::mutex mu;
  static std::map<int, void*> per_device;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  auto it = per_device.find(dev);
  if (it != per_device.end()) {
    *ws = it->second;
    return hipSuccess;
  }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  // Set-up on this GPU: the counter region starts at zero (a kernel, not a
  // memset, so that a first call inside a graph capture records no memset
  // node).  Every later call leaves the counters it uses at zero again.
  hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, stream,
                     static_cast<uint32_t*>(ptr), kNoAllocCounterBytes / 4);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  per_device[dev] = ptr;
  *ws = ptr;
  return hipSuccess;
}

hipError_t launch_decode(const DecodePlan& pl, void* workspace, hipStream_t stream) {
  const DecodeArgs a = decode_args(pl, workspace);
  switch (pl.dtype) {
    case PA_F32: return dispatch_shape<TF32>(pl, a, stream);
    case PA_F16: return dispatch_shape<TF16>(pl, a, stream);
    case PA_BF16: return dispatch_shape<TBF16>(pl, a, stream);
    default: return hipErrorInvalidValue;
  }
}


namespace {

// Joins P partial attention states of each (s, h): the part p attended a
// disjoint key set and gives its normalised output o_p and natural-log
// log-sum-exp lse_p.  With M = max_p lse_p and w_p = e^(lse_p - M):
//   out = sum_p w_p o_p / sum_p w_p,   lse = M + ln sum_p w_p
// -- the rescaling of the online softmax's running maximum and sum
// ("FlashAttention and PagedAttention: two fixes for two different
// bottlenecks", "FlashAttention - How it works"), applied to whole parts.
// Parts with lse = -inf attended no key; if all are, out = 0 and lse = -inf.
// One wavefront per (s, h); lane l holds values l*kV .. l*kV+kV-1.
struct MergeArgs {
  const float* po;
  int64_t po_p, po_s, po_h;
  const float* pl;
  int64_t pl_p, pl_s, pl_h;
  void* out;
  int64_t o_s, o_h;
  int out_dtype;
  float* lse;
  int64_t l_s, l_h;
  int P, S, H;
};

template <int D>
__global__ __launch_bounds__(256) void merge_states_kernel(MergeArgs a) {
  constexpr int kV = D / 64;
  const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (unit >= (int64_t)a.S * a.H) return;
  const int s = (int)(unit / a.H), h = (int)(unit % a.H);
  const float* lp = a.pl + (int64_t)s * a.pl_s + (int64_t)h * a.pl_h;
  float M = -INFINITY;
  for (int p = 0; p < a.P; ++p) M = fmaxf(M, lp[(int64_t)p * a.pl_p]);
  float acc[kV], wsum = 0.f;
#pragma unroll
  for (int e = 0; e < kV; ++e) acc[e] = 0.f;
  if (M != -INFINITY) {
    // Four parts' loads in flight together; parts past P enter as empty.
    const float* op = a.po + (int64_t)s * a.po_s + (int64_t)h * a.po_h + lane * kV;
    for (int p0 = 0; p0 < a.P; p0 += 4) {
      float l[4], o[4][kV];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool in = p0 + u < a.P;
        l[u] = in ? lp[(int64_t)(p0 + u) * a.pl_p] : -INFINITY;
#pragma unroll
        for (int e = 0; e < kV; ++e) o[u][e] = in ? op[(int64_t)(p0 + u) * a.po_p + e] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (l[u] == -INFINITY) continue;
        const float w = fast_exp2((l[u] - M) * 1.4426950408889634f);
        wsum += w;
#pragma unroll
        for (int e = 0; e < kV; ++e) acc[e] = fmaf(w, o[u][e], acc[e]);
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int64_t ob = (int64_t)s * a.o_s + (int64_t)h * a.o_h + lane * kV;
#pragma unroll
  for (int e = 0; e < kV; ++e) {
    const float v = acc[e] * inv;
    if (a.out_dtype == PA_F32)
      static_cast<float*>(a.out)[ob + e] = v;
    else if (a.out_dtype == PA_F16)
      static_cast<uint16_t*>(a.out)[ob + e] = to_f16_bits(v);
    else
      static_cast<uint16_t*>(a.out)[ob + e] = to_bf16_bits(v);
  }
  if (a.lse && lane == 0)
    a.lse[(int64_t)s * a.l_s + (int64_t)h * a.l_h] =
        wsum > 0.f ? M + __log2f(wsum) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_merge(const MergePlan& pl, hipStream_t stream) {
  MergeArgs a;
  a.po = pl.part_out;
  a.po_p = pl.po_p;
  a.po_s = pl.po_s;
  a.po_h = pl.po_h;
  a.pl = pl.part_lse;
  a.pl_p = pl.pl_p;
  a.pl_s = pl.pl_s;
  a.pl_h = pl.pl_h;
  a.out = pl.out;
  a.o_s = pl.o_s;
  a.o_h = pl.o_h;
  a.out_dtype = pl.out_dtype;
  a.lse = pl.lse;
  a.l_s = pl.l_s;
  a.l_h = pl.l_h;
  a.P = pl.P;
  a.S = pl.S;
  a.H = pl.H;
  const int64_t units = (int64_t)pl.S * pl.H;
  if (units == 0) return hipSuccess;
  const dim3 grid((unsigned)((units + 3) / 4));
  return pl.D == 64 ? timed_launch("merge_states", merge_states_kernel<64>, grid, dim3(256),
                                   stream, a)
                    : timed_launch("merge_states", merge_states_kernel<128>, grid, dim3(256),
                                   stream, a);
}

namespace {

// The last step of a shared-prefix decode: for each (s, h) the parts are the
// prefix's key chunks and the state of the sequence's own keys; with
// lse in log2 units, M = max_p lse_p and w_p = 2^(lse_p - M),
//   out = sum_p w_p o_p / sum_p w_p
// (the same whole-part rescaling as merge_states_kernel).  One wavefront per
// (s, h), lane l holding values l*kV .. l*kV+kV-1; all parts' loads are
// issued before any is used.
struct PrefixJoinArgs {
  const float* pre_o;
  const float* pre_lse;
  const float* suf_o;
  const float* suf_lse;
  void* out;
  int64_t o_ss, o_sh;
  int out_dtype;
  int n_pre, S, H;
};

template <int D>
__global__ __launch_bounds__(256) void prefix_join_kernel(PrefixJoinArgs a) {
  constexpr int kV = D / 64;
  constexpr int kP = kMaxPrefixChunks + 1;
  const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (unit >= (int64_t)a.S * a.H) return;
  const int s = (int)(unit / a.H), h = (int)(unit % a.H);
  float l[kP], o[kP][kV];
#pragma unroll
  for (int c = 0; c < kMaxPrefixChunks; ++c) {
    const bool in = c < a.n_pre;
    const int64_t row = ((int64_t)c * a.H + h) * a.S + s;
    l[c] = in ? a.pre_lse[row] : -INFINITY;
#pragma unroll
    for (int e = 0; e < kV; ++e) o[c][e] = in ? a.pre_o[row * D + lane * kV + e] : 0.f;
  }
  l[kP - 1] = a.suf_lse[unit] * 1.4426950408889634f;  // natural log -> log2
#pragma unroll
  for (int e = 0; e < kV; ++e) o[kP - 1][e] = a.suf_o[unit * D + lane * kV + e];
  float M = -INFINITY;
#pragma unroll
  for (int p = 0; p < kP; ++p) M = fmaxf(M, l[p]);
  float acc[kV], wsum = 0.f;
#pragma unroll
  for (int e = 0; e < kV; ++e) acc[e] = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int p = 0; p < kP; ++p) {
      if (l[p] == -INFINITY) continue;  // a part with no keys
      const float w = fast_exp2(l[p] - M);
      wsum += w;
#pragma unroll
      for (int e = 0; e < kV; ++e) acc[e] = fmaf(w, o[p][e], acc[e]);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int64_t ob = (int64_t)s * a.o_ss + (int64_t)h * a.o_sh + lane * kV;
#pragma unroll
  for (int e = 0; e < kV; ++e) {
    const float v = acc[e] * inv;
    if (a.out_dtype == PA_F32)
      static_cast<float*>(a.out)[ob + e] = v;
    else if (a.out_dtype == PA_F16)
      static_cast<uint16_t*>(a.out)[ob + e] = to_f16_bits(v);
    else
      static_cast<uint16_t*>(a.out)[ob + e] = to_bf16_bits(v);
  }
}

}  // namespace

hipError_t launch_prefix_join(const PrefixJoinPlan& pl, hipStream_t stream) {
  PrefixJoinArgs a;
  a.pre_o = pl.pre_o;
  a.pre_lse = pl.pre_lse;
  a.suf_o = pl.suf_o;
  a.suf_lse = pl.suf_lse;
  a.out = pl.out;
  a.o_ss = pl.o_ss;
  a.o_sh = pl.o_sh;
  a.out_dtype = pl.out_dtype;
  a.n_pre = pl.n_pre;
  a.S = pl.S;
  a.H = pl.H;
  const int64_t units = (int64_t)pl.S * pl.H;
  if (units == 0) return hipSuccess;
  if (pl.D != 128 || pl.n_pre > kMaxPrefixChunks) return hipErrorInvalidValue;
  return timed_launch("prefix_join", prefix_join_kernel<128>, dim3((unsigned)((units + 3) / 4)),
                      dim3(256), stream, a);
}

}  // namespace pa
