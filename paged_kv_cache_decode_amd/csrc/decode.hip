// Paged decode attention for gfx950: balanced split-context partitions and
// a log-sum-exp merge.
//
// One query token per sequence attends to the n_s keys of its paged KV
// cache.  The keys of a sequence are found through its block table
// (logical block j -> physical block), the address translation of
// "FlashAttention and PagedAttention: two fixes for two different
// bottlenecks", section "PagedAttention - How it works", and of
// "How PagedAttention and RadixAttention optimise KV-cache handling",
// "How PagedAttention works"; the math is eq. (4) of "Flash Attention vs
// Paged Attention" (attention over KV blocks), evaluated with the online
// softmax of the first page's "FlashAttention - How it works" (running
// maximum and running sum, no score matrix in memory).
//
// Work decomposition (MI355X: 256 CUs, 64-lane wavefronts).  A unit is one
// (sequence s, KV head g) pair with the G query heads that share g; it has
// ceil(n_s / 16) tiles of 16 keys.  The tiles of all units, KV-head major
// ((g, s) order), form one list of `total` tiles.  The kernel launches W
// wavefronts ("workers", as many as the device keeps resident) and gives
// worker i the contiguous slice [i*q, (i+1)*q) of the list,
// q = ceil(total / W), so every worker streams the same number of bytes
// whatever the mix of context lengths -- no tail of long partitions, no idle
// XCD.  Worker numbers are dealt so that each of the 8 XCDs (which receive
// workgroups round-robin) owns one contiguous eighth of the list: with
// head-major order an XCD then serves one or two KV heads, and K/V blocks
// that several sequences share (a common prompt prefix) stay in its L2.
// The piece of a unit that one worker covers is a partition: a worker that
// covers a whole unit writes `out` directly; otherwise it writes a
// normalised partial output and its log2-sum-exp, and the merge kernel
// joins the partitions of that unit.
//
// Per 16-key tile a worker:
//   * loads the K rows with the lane layout of the 16x16 MFMA B operand
//     (lane = key r16 and 16-byte column group c): every load instruction
//     reads 64 contiguous bytes of each of 16 rows;
//   * computes S = Q K^T on one MFMA chain; Q (the A operand) repeats the G
//     heads down its 16 rows, so every lane ends with the scores of its key
//     for all G heads (no transposes, no cross-lane traffic);
//   * does the online-softmax update with 16-lane DPP max reductions;
//   * loads the V rows with full-row coalescing (16 lanes x 16 bytes per
//     256-byte row) and accumulates p * v in fp32 on the VALU, reading the
//     probabilities of its key from a 256-byte per-wave LDS slot.
// Three register sets rotate so that two tiles are in flight while the third
// is being used (about 5 us of loaded memory latency has to be covered).
#include "device_common.h"
#include "kernels.h"
#include "launch.h"

#include <map>
#include <mutex>
#include <tuple>

namespace pa {
namespace {

template <class T, int D>
struct DecodeGeom {
  static constexpr int kElem = T::kBytes;
  static constexpr int kRowBytes = D * kElem;       // one key row of one head
  static constexpr int kKLoads = kRowBytes / 64;    // 16-byte K loads per lane per tile
  static constexpr int kLPR = kRowBytes / 16;       // lanes per V row
  static constexpr int kRPI = 64 / kLPR;            // V rows per load instruction
  static constexpr int kVLoads = kTileKeys / kRPI;  // V loads per lane per tile
  static constexpr int kE = 16 / kElem;             // elements per 16 bytes
  static_assert(kKLoads >= 1 && kRPI >= 1 && kVLoads >= 1, "unsupported row size");
};

struct DecodeArgs {
  const uint8_t* q;
  int64_t q_ss, q_sh;  // bytes
  const uint8_t* k;
  const uint8_t* v;
  const int32_t* bt;
  int64_t bt_ss;
  const int32_t* cl;
  void* out;
  int64_t o_ss, o_sh;  // elements
  int out_f32;
  float* part_o;     // [slots, G, D]
  float* part_lse;   // [slots, G] (log2 units)
  int2* unit_range;  // [Hkv * S]: first and last worker of each unit (g-major)
  int S, H, Hkv, W, bs_shift;
  float scale_log2;  // scale * log2(e)
};

// S = Q K^T on matrix cores for one 16-key tile.  Returns, per lane, the
// scores of key r16 for heads h < G in elements 0..G-1.
template <class T, int D>
__device__ __forceinline__ f32x4_t qk_tile(const u32x4_t* qf, const u32x4_t* kf) {
  using Geo = DecodeGeom<T, D>;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < Geo::kKLoads; ++i) {
    if constexpr (__is_same(T, TBF16)) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qf[i]),
                                                     __builtin_bit_cast(bf16x8_t, kf[i]), acc,
                                                     0, 0, 0);
    } else if constexpr (__is_same(T, TF16)) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, qf[i]),
                                                    __builtin_bit_cast(f16x8_t, kf[i]), acc, 0,
                                                    0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(qf[i][j]),
                                                   __uint_as_float(kf[i][j]), acc, 0, 0, 0);
    }
  }
  return acc;
}

__device__ __forceinline__ int uniform_i(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t wave_sum_i64(int64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return uniform_i64(v);
}

__device__ __forceinline__ int64_t wave_incl_scan_i64(int64_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ int tiles_of(int n) { return (n + kTileKeys - 1) / kTileKeys; }

template <class T, int D, int G>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_partitions_kernel(DecodeArgs a) {
  using Geo = DecodeGeom<T, D>;
  constexpr int kNW = kDecodeWaves;
  constexpr int kE = Geo::kE;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  // Hardware workgroup b runs on XCD b % 8; logical workgroup numbers give
  // each XCD a contiguous run of workers (the grid is a multiple of 8).
  const int groups = gridDim.x;
  const int logical = (blockIdx.x & 7) * (groups >> 3) + (blockIdx.x >> 3);
  const int worker = logical * kNW + w;
  if (worker >= a.W) return;

  __shared__ float p_lds[kNW][kTileKeys][4];
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[kNW][G * Geo::kRowBytes];

  // ---- this worker's slice of the global tile list ----
  // Tiles per KV head over all sequences (the list is g-major).  With at
  // most 64 sequences one load of the lengths serves both passes.
  const int lane_tiles = lane < a.S ? tiles_of(as_const(a.cl)[lane]) : 0;
  int64_t t_all = wave_sum_i64(lane_tiles);
  for (int c0 = 64; c0 < a.S; c0 += 64) {
    const int s = c0 + lane;
    t_all += wave_sum_i64(s < a.S ? (int64_t)tiles_of(as_const(a.cl)[s]) : 0);
  }
  const int64_t total = t_all * a.Hkv;
  const int64_t per = (total + a.W - 1) / a.W;
  const int64_t begin = (int64_t)worker * per;
  const int64_t end = min(total, begin + per);
  if (begin >= end) return;

  // KV head and sequence holding `begin`, and the list index of the first
  // tile of that sequence's unit.
  int g = (int)(begin / t_all);
  int s = 0;
  int64_t unit_first = (int64_t)g * t_all;
  {
    const int64_t r = begin - unit_first;
    int64_t pre = 0;
    for (int c0 = 0; c0 < a.S; c0 += 64) {
      const int ss = c0 + lane;
      const int64_t tl =
          c0 == 0 ? lane_tiles : (ss < a.S ? (int64_t)tiles_of(as_const(a.cl)[ss]) : 0);
      const int64_t incl = wave_incl_scan_i64(tl, lane);
      const int64_t chunk = uniform_i64(__shfl(incl, 63));
      if (pre + chunk > r) {
        const uint64_t hit = __ballot(pre + incl > r);
        const int f = __ffsll((unsigned long long)hit) - 1;
        s = c0 + f;
        pre += uniform_i64(__shfl(incl - tl, f));
        break;
      }
      pre += chunk;
    }
    unit_first += pre;
  }

  const int c = lane >> 4;    // 16-byte column group of the MFMA operands
  const int r16 = lane & 15;  // key (B operand) / head row (A operand)
  const int bmask = (1 << a.bs_shift) - 1;
  const uint32_t tok_stride = (uint32_t)a.Hkv * Geo::kRowBytes;  // bytes between slots
  const int64_t blk_stride = (int64_t)tok_stride << a.bs_shift;
  const int v_row = lane / Geo::kLPR;
  const uint32_t k_off = (uint32_t)r16 * tok_stride + c * 16;
  const uint32_t v_off = (uint32_t)v_row * tok_stride + (lane % Geo::kLPR) * 16;
  uint8_t* my_q = q_lds[w];
  const uint8_t* q_frag = my_q + (r16 % G) * Geo::kRowBytes + c * 16;

  int64_t t = begin;
  while (t < end) {
    // Unit (g, s) starting at list index unit_first; t lies in or after it.
    // (readfirstlane marks the loop state wave-uniform for the compiler, so
    // table and length reads below become scalar loads.)
    s = uniform_i(s);
    g = uniform_i(g);
    const int n = as_const(a.cl)[s];
    const int ts = tiles_of(n);
    if (t >= unit_first + ts) {  // empty or finished unit: next sequence / head
      unit_first += ts;
      if (++s == a.S) {
        s = 0;
        ++g;
      }
      continue;
    }
    const int j0 = uniform_i((int)(t - unit_first));
    const int j1 = uniform_i((int)min((int64_t)ts, end - unit_first));
    const int ntile = j1 - j0;
    const int hq0 = g * G;

    // Q of the G heads, fetched now and written to this wave's LDS slot once
    // the first K/V loads are in flight (being older, its wait does not hold
    // them up).  The previous unit's LDS reads were issued earlier by this
    // same wave, and LDS executes them in order.
    constexpr int kQChunks = G * Geo::kRowBytes / 16;
    constexpr int kQPer = (kQChunks + 63) / 64;
    u32x4_t qreg[kQPer];
#pragma unroll
    for (int j = 0; j < kQPer; ++j) {
      const int i = lane + 64 * j;
      const int h = i / (Geo::kRowBytes / 16), col = i % (Geo::kRowBytes / 16);
      if (i < kQChunks)
        qreg[j] = load16(a.q + (int64_t)s * a.q_ss + (int64_t)(hq0 + h) * a.q_sh + col * 16);
    }

    const const_i32_ptr bt_row = as_const(a.bt) + (int64_t)s * a.bt_ss;
    const uint8_t* kbase = a.k + (int64_t)g * Geo::kRowBytes;
    const uint8_t* vbase = a.v + (int64_t)g * Geo::kRowBytes;

    float m[G], l_lane[G], acc[G][kE];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
      l_lane[h] = 0.f;
#pragma unroll
      for (int e = 0; e < kE; ++e) acc[h][e] = 0.f;
    }

    u32x4_t kA[Geo::kKLoads], vA[Geo::kVLoads];
    u32x4_t kB[Geo::kKLoads], vB[Geo::kVLoads];
    u32x4_t kC[Geo::kKLoads], vC[Geo::kVLoads];

    auto load_tile = [&](int k, u32x4_t* kd, u32x4_t* vd) {
      const int key0 = uniform_i((j0 + min(k, ntile - 1)) * kTileKeys);
      const int phys = bt_row[key0 >> a.bs_shift];
      const int64_t row0 = (int64_t)phys * blk_stride + (int64_t)(key0 & bmask) * tok_stride;
      const uint8_t* kb = kbase + row0;
      const uint8_t* vb = vbase + row0;
#pragma unroll
      for (int i = 0; i < Geo::kKLoads; ++i) kd[i] = load16(kb + k_off + i * 64);
#pragma unroll
      for (int i = 0; i < Geo::kVLoads; ++i)
        vd[i] = load16(vb + (int64_t)(i * Geo::kRPI) * tok_stride + v_off);
    };

    auto compute_tile = [&](int k, const u32x4_t* kf, const u32x4_t* vf) {
      const int valid = n - (j0 + k) * kTileKeys;  // keys of this tile below n (>= 1)
      u32x4_t qf[Geo::kKLoads];
#pragma unroll
      for (int i = 0; i < Geo::kKLoads; ++i)
        qf[i] = *reinterpret_cast<const u32x4_t*>(q_frag + i * 64);
      const f32x4_t sc = qk_tile<T, D>(qf, kf);
      const bool key_ok = r16 < valid;
      float x[G], pr[G], mnew[G];
      bool grow = false;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        // Slots at or past n are selected away (they may hold NaN).
        x[h] = key_ok ? sc[h] * a.scale_log2 : -INFINITY;
        const float tmax = uniform(row16_max(x[h]));
        mnew[h] = fmaxf(m[h], tmax);
        grow |= mnew[h] > m[h];
      }
      if (grow) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float alpha = fast_exp2(m[h] - mnew[h]);
          l_lane[h] *= alpha;
#pragma unroll
          for (int e = 0; e < kE; ++e) acc[h][e] *= alpha;
          m[h] = mnew[h];
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        pr[h] = fast_exp2(x[h] - m[h]);
        l_lane[h] += pr[h];
      }
      // Hand each lane the probabilities of the key whose V row it holds.
      if (lane < kTileKeys) {
#pragma unroll
        for (int h = 0; h < G; ++h) p_lds[w][r16][h] = pr[h];
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < Geo::kVLoads; ++i) {
        const int key = i * Geo::kRPI + v_row;
        float pk[G];
#pragma unroll
        for (int h = 0; h < G; ++h) pk[h] = p_lds[w][key][h];
        u32x4_t raw = vf[i];
        if (key >= valid) raw = u32x4_t{0u, 0u, 0u, 0u};
        float vv[kE];
        Unpack<T>::run(raw, vv);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < kE; ++e) acc[h][e] = fmaf(pk[h], vv[e], acc[h][e]);
      }
      __builtin_amdgcn_wave_barrier();
    };

    // Three-way rotation over this partition's tiles: the steady-state loop
    // issues one tile's loads per computed tile (fixed waits); an epilogue
    // finishes the last one to five tiles without loading past the end.
    load_tile(0, kA, vA);
    load_tile(1, kB, vB);  // the first loads are clamped to the last tile
    load_tile(2, kC, vC);  // of a partition shorter than three tiles
#pragma unroll
    for (int j = 0; j < kQPer; ++j)
      if (lane + 64 * j < kQChunks) *reinterpret_cast<u32x4_t*>(my_q + (lane + 64 * j) * 16) = qreg[j];
    __builtin_amdgcn_wave_barrier();
    int k = 0;
    for (; k + 5 < ntile; k += 3) {
      compute_tile(k, kA, vA);
      load_tile(k + 3, kA, vA);
      compute_tile(k + 1, kB, vB);
      load_tile(k + 4, kB, vB);
      compute_tile(k + 2, kC, vC);
      load_tile(k + 5, kC, vC);
    }
    const int rest = ntile - k;  // 1..5; A, B, C hold tiles k, k + 1, k + 2
    compute_tile(k, kA, vA);
    if (rest > 3) load_tile(k + 3, kA, vA);
    if (rest > 1) compute_tile(k + 1, kB, vB);
    if (rest > 4) load_tile(k + 4, kB, vB);
    if (rest > 2) compute_tile(k + 2, kC, vC);
    if (rest > 3) compute_tile(k + 3, kA, vA);
    if (rest > 4) compute_tile(k + 4, kB, vB);

    // Partition totals: l over the 16 keys of a row, acc over lanes sharing
    // a column.
#pragma unroll
    for (int h = 0; h < G; ++h) l_lane[h] = row16_sum(l_lane[h]);
#pragma unroll
    for (int off = Geo::kLPR; off < 64; off <<= 1)
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < kE; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);

    const int u = g * a.S + s;  // unit index in list order
    const bool whole = j0 == 0 && j1 == ts;
    if (lane < Geo::kLPR) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float inv = 1.f / l_lane[h];
#pragma unroll
        for (int e = 0; e < kE; ++e) {
          const int d = lane * kE + e;
          if (whole) {
            store_out<T>(a.out, (int64_t)s * a.o_ss + (int64_t)(hq0 + h) * a.o_sh + d,
                         acc[h][e] * inv, a.out_f32 != 0);
          } else {
            a.part_o[((int64_t)(worker + u) * G + h) * D + d] = acc[h][e] * inv;
          }
        }
      }
    }
    if (lane == 0) {
      if (!whole) {
#pragma unroll
        for (int h = 0; h < G; ++h)
          a.part_lse[(int64_t)(worker + u) * G + h] = m[h] + __log2f(l_lane[h]);
      }
      if (j0 == 0) {
        // First worker of the unit records which workers hold its pieces.
        const int last = (int)((unit_first + ts - 1) / per);
        a.unit_range[u] = make_int2(worker, last);
      }
    }
    t = unit_first + j1;
  }
}

// Joins the partitions of units split over several workers:
// out = sum_p 2^(lse_p - M) o_p / sum_p 2^(lse_p - M),  M = max_p lse_p.
// Also writes the zero output of empty contexts.  One 256-thread workgroup
// per (sequence, query head): every thread accumulates 4 output columns
// over a strided subset of the partitions with independent 16-byte loads.
constexpr int kMergeThreads = 256;

template <class T, int D, int G>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs a) {
  constexpr int kChunks = D / 4;                    // 16-byte column chunks of a row
  constexpr int kGroups = kMergeThreads / kChunks;  // partition subsets
  const int hq = blockIdx.x, s = blockIdx.y;
  const int tid = threadIdx.x;
  const int n = a.cl[s];
  const int g = hq / G, h = hq % G;
  const int64_t ob = (int64_t)s * a.o_ss + (int64_t)hq * a.o_sh;
  if (n == 0) {
    for (int d = tid; d < D; d += kMergeThreads) store_out<T>(a.out, ob + d, 0.f, a.out_f32 != 0);
    return;
  }
  const int u = g * a.S + s;
  const int2 range = a.unit_range[u];
  const int np = range.y - range.x + 1;
  if (np <= 1) return;  // the single worker wrote `out` itself
  const int64_t slot0 = (int64_t)range.x + u;

  __shared__ float red[kMergeThreads / 64];
  __shared__ float wts[kMergeThreads];
  __shared__ f32x4_t part[kGroups][kChunks];

  float M = -INFINITY;
  for (int p = tid; p < np; p += kMergeThreads) M = fmaxf(M, a.part_lse[(slot0 + p) * G + h]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if ((tid & 63) == 0) red[tid >> 6] = M;
  __syncthreads();
  M = red[0];
#pragma unroll
  for (int i = 1; i < kMergeThreads / 64; ++i) M = fmaxf(M, red[i]);

  const int cidx = tid % kChunks, pg = tid / kChunks;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  for (int p0 = 0; p0 < np; p0 += kMergeThreads) {
    const int cnt = min(kMergeThreads, np - p0);
    __syncthreads();
    if (tid < cnt) {
      const float wv = fast_exp2(a.part_lse[(slot0 + p0 + tid) * G + h] - M);
      wts[tid] = wv;
      wsum += wv;
    }
    __syncthreads();
#pragma unroll 8
    for (int j = pg; j < cnt; j += kGroups) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(
          a.part_o + ((slot0 + p0 + j) * G + h) * D + cidx * 4);
      acc += wts[j] * v;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) wsum += __shfl_xor(wsum, o);
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = wsum;
  part[pg][cidx] = acc;
  __syncthreads();
  float W = red[0];
#pragma unroll
  for (int i = 1; i < kMergeThreads / 64; ++i) W += red[i];
  if (tid < kChunks) {
    f32x4_t o = part[0][tid];
#pragma unroll
    for (int g2 = 1; g2 < kGroups; ++g2) o += part[g2][tid];
    const float inv = 1.f / W;
#pragma unroll
    for (int e = 0; e < 4; ++e) store_out<T>(a.out, ob + tid * 4 + e, o[e] * inv, a.out_f32 != 0);
  }
}

template <class T, int D, int G>
hipError_t launch_decode_t(const DecodePlan& pl, const DecodeArgs& a, hipStream_t stream) {
  const hipError_t e =
      timed_launch("decode_partitions", decode_partitions_kernel<T, D, G>,
                   dim3((unsigned)pl.grid[0]), dim3(pl.block_threads), stream, a);
  if (e != hipSuccess) return e;
  return timed_launch("decode_merge", decode_merge_kernel<T, D, G>, dim3(pl.H, pl.S),
                      dim3(kMergeThreads), stream, a);
}

template <class T, int D, int G>
int resident_waves_t() {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(decode_partitions_kernel<T, D, G>),
          64 * kDecodeWaves, 0) != hipSuccess)
    return 0;
  return cus * per_cu * kDecodeWaves;
}

template <class T>
int resident_waves_shape(int D, int G) {
  switch (D * 10 + G) {
    case 641: return resident_waves_t<T, 64, 1>();
    case 642: return resident_waves_t<T, 64, 2>();
    case 644: return resident_waves_t<T, 64, 4>();
    case 1281: return resident_waves_t<T, 128, 1>();
    case 1282: return resident_waves_t<T, 128, 2>();
    case 1284: return resident_waves_t<T, 128, 4>();
    default: return 0;
  }
}

template <class T>
hipError_t dispatch_shape(const DecodePlan& pl, const DecodeArgs& a, hipStream_t stream) {
  switch (pl.D * 10 + pl.G) {
    case 641: return launch_decode_t<T, 64, 1>(pl, a, stream);
    case 642: return launch_decode_t<T, 64, 2>(pl, a, stream);
    case 644: return launch_decode_t<T, 64, 4>(pl, a, stream);
    case 1281: return launch_decode_t<T, 128, 1>(pl, a, stream);
    case 1282: return launch_decode_t<T, 128, 2>(pl, a, stream);
    case 1284: return launch_decode_t<T, 128, 4>(pl, a, stream);
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
  // Without a device (planning only) assume an MI355X: 256 CUs x 12 waves.
  if (w <= 0) w = 256 * 12;
  std::lock_guard<std::mutex> lk(mu);
  cache[key] = w;
  return w;
}

hipError_t launch_decode(const DecodePlan& pl, void* workspace, hipStream_t stream) {
  DecodeArgs a;
  const int e = pl.dtype == PA_F32 ? 4 : 2;
  a.q = static_cast<const uint8_t*>(pl.q);
  a.q_ss = pl.q_ss * e;
  a.q_sh = pl.q_sh * e;
  a.k = static_cast<const uint8_t*>(pl.k);
  a.v = static_cast<const uint8_t*>(pl.v);
  a.bt = pl.bt;
  a.bt_ss = pl.bt_ss;
  a.cl = pl.cl;
  a.out = pl.out;
  a.o_ss = pl.o_ss;
  a.o_sh = pl.o_sh;
  a.out_f32 = pl.out_dtype == PA_F32;
  a.part_o = static_cast<float*>(workspace);
  a.part_lse = a.part_o + pl.slots * pl.G * pl.D;
  a.unit_range = reinterpret_cast<int2*>(a.part_lse + pl.slots * pl.G);
  a.S = pl.S;
  a.H = pl.H;
  a.Hkv = pl.Hkv;
  a.W = pl.workers;
  a.bs_shift = __builtin_ctz(pl.B);
  a.scale_log2 = pl.scale * 1.4426950408889634f;
  switch (pl.dtype) {
    case PA_F32: return dispatch_shape<TF32>(pl, a, stream);
    case PA_F16: return dispatch_shape<TF16>(pl, a, stream);
    case PA_BF16: return dispatch_shape<TBF16>(pl, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
