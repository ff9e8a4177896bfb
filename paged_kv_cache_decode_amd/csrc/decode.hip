// Paged decode attention for gfx950: split-context partitions + LSE merge.
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
// Work decomposition (MI355X: 256 CUs, 64-lane wavefronts):
//   workgroup = (partition p of P keys, KV head g, sequence s), 4 waves.
//   Every wave takes 16-key tiles of the partition round-robin and keeps
//   its own (running max m, running sum l, accumulator) for the G query
//   heads that share KV head g.  At the end the 4 waves are merged through
//   LDS; a sequence that fits one partition writes `out` directly, others
//   write a normalised partial output plus log2-sum-exp per partition and
//   the merge kernel joins them.
//
// Per 16-key tile a wave:
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
// The next tile's K/V loads are issued before the current tile is used.
#include "device_common.h"
#include "kernels.h"

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
  float* part_o;    // [S, H, MP, D]
  float* part_lse;  // [S, H, MP] (log2 units)
  int H, Hkv, P, MP, bs_shift;
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

template <class T, int D, int G>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_partitions_kernel(DecodeArgs a) {
  using Geo = DecodeGeom<T, D>;
  constexpr int kNW = kDecodeWaves;
  constexpr int kE = Geo::kE;

  const int p = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n = a.cl[s];
  const int t_begin = p * a.P;
  if (p > 0 && t_begin >= n) return;  // partition past the context (whole workgroup)
  const int t_end = min(n, t_begin + a.P);
  const int ntiles = t_end > t_begin ? (t_end - t_begin + kTileKeys - 1) / kTileKeys : 0;
  const int my_tiles = ntiles > w ? (ntiles - w + kNW - 1) / kNW : 0;

  __shared__ float p_lds[kNW][kTileKeys][4];
  __shared__ float red_acc[kNW][G][D];
  __shared__ float red_m[kNW][G];
  __shared__ float red_l[kNW][G];

  const int c = lane >> 4;    // 16-byte column group of the MFMA operands
  const int r16 = lane & 15;  // key (B operand) / head row (A operand)
  const int hq0 = g * G;

  // Q as the MFMA A operand: row r16 holds head hq0 + r16 % G.
  u32x4_t qf[Geo::kKLoads];
  {
    const uint8_t* qrow = a.q + (int64_t)s * a.q_ss + (int64_t)(hq0 + r16 % G) * a.q_sh;
#pragma unroll
    for (int i = 0; i < Geo::kKLoads; ++i) qf[i] = load16(qrow + i * 64 + c * 16);
  }

  // Physical block of each of this wave's tiles, one per lane.
  const int32_t* bt_row = a.bt + (int64_t)s * a.bt_ss;
  int my_blk = 0;
  if (lane < my_tiles) my_blk = bt_row[(t_begin + kTileKeys * (w + lane * kNW)) >> a.bs_shift];

  const int64_t tok_stride = (int64_t)a.Hkv * Geo::kRowBytes;  // bytes between slots
  const int64_t blk_stride = tok_stride << a.bs_shift;
  const uint8_t* kbase = a.k + (int64_t)g * Geo::kRowBytes;
  const uint8_t* vbase = a.v + (int64_t)g * Geo::kRowBytes;
  const int bmask = (1 << a.bs_shift) - 1;
  const int v_row = lane / Geo::kLPR;
  const int v_col = (lane % Geo::kLPR) * 16;

  float m[G], l_lane[G], acc[G][kE];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l_lane[h] = 0.f;
#pragma unroll
    for (int e = 0; e < kE; ++e) acc[h][e] = 0.f;
  }

  u32x4_t kf[Geo::kKLoads], vf[Geo::kVLoads];
  u32x4_t kn[Geo::kKLoads], vn[Geo::kVLoads];

  auto load_tile = [&](int k, u32x4_t* kd, u32x4_t* vd) {
    const int tile_start = t_begin + kTileKeys * (w + k * kNW);
    const int phys = __builtin_amdgcn_readlane(my_blk, k);
    const int slot0 = tile_start & bmask;
    const uint8_t* kb = kbase + (int64_t)phys * blk_stride + (int64_t)(slot0 + r16) * tok_stride +
                        c * 16;
#pragma unroll
    for (int i = 0; i < Geo::kKLoads; ++i) kd[i] = load16(kb + i * 64);
    const uint8_t* vb = vbase + (int64_t)phys * blk_stride + (int64_t)(slot0 + v_row) * tok_stride +
                        v_col;
#pragma unroll
    for (int i = 0; i < Geo::kVLoads; ++i) vd[i] = load16(vb + (int64_t)(i * Geo::kRPI) * tok_stride);
  };

  if (my_tiles > 0) load_tile(0, kn, vn);
  for (int k = 0; k < my_tiles; ++k) {
#pragma unroll
    for (int i = 0; i < Geo::kKLoads; ++i) kf[i] = kn[i];
#pragma unroll
    for (int i = 0; i < Geo::kVLoads; ++i) vf[i] = vn[i];
    if (k + 1 < my_tiles) load_tile(k + 1, kn, vn);

    const int tile_start = t_begin + kTileKeys * (w + k * kNW);
    const int valid = t_end - tile_start;  // keys of this tile inside the partition (>= 1)

    const f32x4_t sc = qk_tile<T, D>(qf, kf);
    const bool key_ok = r16 < valid;
    float x[G], pr[G];
    bool grow = false;
    float mnew[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      // Slots at or past the end are selected away (they may hold NaN).
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
  }

  // Wave totals: l over the 16 keys of a row, acc over lanes sharing a column.
#pragma unroll
  for (int h = 0; h < G; ++h) l_lane[h] = row16_sum(l_lane[h]);
#pragma unroll
  for (int off = Geo::kLPR; off < 64; off <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < kE; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);
  if (lane < Geo::kLPR) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < kE; ++e) red_acc[w][h][lane * kE + e] = acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      red_m[w][h] = m[h];
      red_l[w][h] = l_lane[h];
    }
  }
  __syncthreads();

  // Merge the waves and write the output (or this partition's partial).
  const int np = n > a.P ? (n + a.P - 1) / a.P : 1;
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * kNW) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kNW; ++ww) M = fmaxf(M, red_m[ww][h]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < kNW; ++ww) {
        const float f = fast_exp2(red_m[ww][h] - M);
        L = fmaf(red_l[ww][h], f, L);
        O = fmaf(red_acc[ww][h][d], f, O);
      }
    }
    const int hq = hq0 + h;
    const float o = L > 0.f ? O / L : 0.f;
    if (np == 1) {
      store_out<T>(a.out, (int64_t)s * a.o_ss + (int64_t)hq * a.o_sh + d, o, a.out_f32 != 0);
    } else {
      const int64_t row = ((int64_t)s * a.H + hq) * a.MP + p;
      a.part_o[row * D + d] = o;
      if (d == 0) a.part_lse[row] = M + __log2f(L);
    }
  }
}

// Joins the partitions of sequences longer than one partition:
// out = sum_p 2^(lse_p - M) o_p / sum_p 2^(lse_p - M).
template <class T, int D>
__global__ __launch_bounds__(128) void decode_merge_kernel(DecodeArgs a) {
  const int hq = blockIdx.x, s = blockIdx.y;
  const int n = a.cl[s];
  const int np = n > a.P ? (n + a.P - 1) / a.P : 1;
  if (np <= 1) return;
  const int64_t row0 = ((int64_t)s * a.H + hq) * a.MP;
  const float* lse = a.part_lse + row0;
  const float* po = a.part_o + row0 * D;
  float M = -INFINITY;
  for (int pp = 0; pp < np; ++pp) M = fmaxf(M, lse[pp]);
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float W = 0.f, O = 0.f;
    for (int pp = 0; pp < np; ++pp) {
      const float f = fast_exp2(lse[pp] - M);
      W += f;
      O = fmaf(f, po[(int64_t)pp * D + d], O);
    }
    store_out<T>(a.out, (int64_t)s * a.o_ss + (int64_t)hq * a.o_sh + d, O / W, a.out_f32 != 0);
  }
}

template <class T, int D, int G>
hipError_t launch_decode_t(const DecodePlan& pl, const DecodeArgs& a, hipStream_t stream) {
  {
    KernelTimer t("decode_partitions", stream);
    hipLaunchKernelGGL((decode_partitions_kernel<T, D, G>),
                       dim3((unsigned)pl.grid[0], (unsigned)pl.grid[1], (unsigned)pl.grid[2]),
                       dim3(pl.block_threads), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.MP <= 1) return e;
  {
    KernelTimer t("decode_merge", stream);
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(pl.H, pl.S), dim3(128), 0, stream, a);
  }
  return hipGetLastError();
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
  a.part_lse = workspace ? a.part_o + (int64_t)pl.S * pl.H * pl.MP * pl.D : nullptr;
  a.H = pl.H;
  a.Hkv = pl.Hkv;
  a.P = pl.P;
  a.MP = pl.MP;
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
