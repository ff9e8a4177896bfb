// Causal (or full) paged prefill attention on gfx950 matrix cores.
//
// Packed query rows of several sequences attend to their paged K/V, read
// through the block table ("FlashAttention and PagedAttention: two fixes
// for two different bottlenecks", "PagedAttention - How it works"), with
// the fused tiling / online softmax / causal-skip of "FlashAttention - How
// it works" and "Flash Attention vs Paged Attention" (kernel fusion: matmul
// and softmax in one kernel, causal mask applied in-kernel, masked work
// skipped).
//
// Work decomposition:
//   workgroup = 64 query positions x the G query heads of one KV head
//   (2G waves; a wave owns 32 positions of one head).  K/V tiles of 64 keys
//   are gathered once per workgroup into LDS and feed all G heads.
//   Key tiles wholly above the diagonal are never loaded.
//
// Per 64-key tile a wave computes, on 32x32x16 MFMAs:
//   S^T = K Q^T   (A = K from LDS, B = Q from registers; bf16/f16 inputs,
//                  fp32 accumulate).  The transposed product leaves every
//                  score of query row r in lane r (and r + 32), so the
//                  row max / row sum of the online softmax are lane-local.
//   O^T += V^T P^T (A = V^T from LDS, B = P from the lane's own scores,
//                  rounded to fp16; fp32 accumulate).  V is written to LDS
//                  transposed (d-major) and converted to fp16 while it is
//                  staged; fp16 keeps P's rounding error 8x below bf16's.
//   O^T's layout again keeps row r in lane r, so the softmax rescale is a
//   per-lane multiply.
//
// Workgroups are ordered so that each XCD (8 per MI355X, fed round-robin)
// works through a contiguous slice of (KV head, sequence, query tile), with
// a sequence's query tiles longest-first; the tiles running together on an
// XCD then share the same K/V in its L2.
#include "device_common.h"
#include "kernels.h"

namespace pa {
namespace {

constexpr int kBN = 64;                  // keys per tile
constexpr int kD = 128;                  // head size
constexpr int kKRow = kD * 2 + 16;       // K tile row in LDS (bytes, padded)
constexpr int kVRow = kBN * 2 + 8;       // V^T tile row in LDS (bytes, padded)
constexpr int kKChunks = kBN * kD * 2 / 16;  // 16-byte chunks in a K tile (1024)
constexpr int kVUnits = (kBN / 2) * (kD / 8);  // (key pair, 8-column) units (512)

struct PrefillArgs {
  const uint8_t* q;
  int64_t q_st, q_sh;  // bytes
  const uint8_t* k;
  const uint8_t* v;
  const int32_t* bt;
  int64_t bt_ss;
  const int32_t* cl;
  const int32_t* qsl;
  void* out;
  int64_t o_st, o_sh;  // elements
  int out_f32;
  int S, Hkv, q_tiles, bs_shift, causal;
  int64_t n_wg;      // real workgroups (q_tiles * Hkv * S)
  int64_t wg_per_xcd;  // ceil(n_wg / 8)
  float scale_log2;
};

template <class T>
__device__ __forceinline__ f32x16_t mfma_qk(u32x4_t a, u32x4_t b, f32x16_t c) {
  if constexpr (__is_same(T, TBF16))
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma_pv(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Two fp16 values packed in a dword from two floats (round to nearest even).
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  f16x2_t h;
  h[0] = static_cast<_Float16>(lo);
  h[1] = static_cast<_Float16>(hi);
  return __builtin_bit_cast(uint32_t, h);
}

// Low / high 16-bit element of a storage dword, as fp16 bits.
template <class T>
__device__ __forceinline__ uint32_t pair_to_f16(uint32_t w0, uint32_t w1, bool high) {
  if constexpr (__is_same(T, TF16)) {
    return high ? ((w0 >> 16) | (w1 & 0xffff0000u)) : ((w0 & 0xffffu) | (w1 << 16));
  } else {
    return high ? pack_f16(bf16_hi(w0), bf16_hi(w1)) : pack_f16(bf16_lo(w0), bf16_lo(w1));
  }
}

template <class T, int G>
__global__ __launch_bounds__(128 * G) void prefill_kernel(PrefillArgs a) {
  constexpr int kNT = 128 * G;  // threads
  constexpr int kKPer = kKChunks / kNT;
  constexpr int kVPer = kVUnits / kNT;
  static_assert(kKPer * kNT == kKChunks && kVPer * kNT == kVUnits, "tile split");

  __shared__ __attribute__((aligned(16))) uint8_t k_lds[kBN * kKRow];
  __shared__ __attribute__((aligned(16))) uint8_t vt_lds[kD * kVRow];

  // XCD-aware order: hardware workgroup b runs on XCD b % 8; give each XCD
  // a contiguous slice of the logical order (g, s, query tile descending).
  const int64_t bid = blockIdx.x;
  const int64_t logical = (bid & 7) * a.wg_per_xcd + (bid >> 3);
  if (logical >= a.n_wg) return;
  const int per_g = a.S * a.q_tiles;
  const int g = (int)(logical / per_g);
  const int rem = (int)(logical % per_g);
  const int s = rem / a.q_tiles;
  const int qt = a.q_tiles - 1 - rem % a.q_tiles;

  const int q0 = a.qsl[s];
  const int L = a.qsl[s + 1] - q0;
  const int n = a.cl[s];
  if (qt * kPrefillRows >= L) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hl = w % G;          // head within the group
  const int half = w / G;        // which 32 of the 64 positions
  const int hq = g * G + hl;
  const int r32 = lane & 31;
  const int hi = lane >> 5;

  // This wave's rows: i = row0 + r32 (query index within the sequence).
  const int row0 = qt * kPrefillRows + half * 32;
  const int my_i = row0 + r32;
  const bool row_ok = my_i < L;
  const int shift = n - L;  // absolute position of row i is shift + i

  // Keys the workgroup needs: [0, kend).
  int kend = n;
  if (a.causal) kend = min(n, shift + min(qt * kPrefillRows + kPrefillRows, L));
  const int ntk = (kend + kBN - 1) / kBN;
  // Keys visible to this wave's first / last valid row.
  const int wave_last_i = min(row0 + 31, L - 1);
  const bool wave_active = row0 < L;
  const int vis_lo = a.causal ? shift + row0 : n - 1;         // first row's last key
  const int vis_hi = a.causal ? shift + wave_last_i : n - 1;  // last row's last key
  const int my_vis = a.causal ? shift + my_i : n - 1;

  // Q^T as the MFMA B operand: lane holds row r32, columns ks*16 + 8*hi.
  u32x4_t qf[kD / 16];
  {
    const uint8_t* qrow = a.q + (int64_t)(q0 + my_i) * a.q_st + (int64_t)hq * a.q_sh + hi * 16;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks)
      qf[ks] = row_ok ? load16(qrow + ks * 32) : u32x4_t{0u, 0u, 0u, 0u};
  }

  const int32_t* bt_row = a.bt + (int64_t)s * a.bt_ss;
  const int64_t tok_stride = (int64_t)a.Hkv * kD * 2;
  const int bmask = (1 << a.bs_shift) - 1;
  const uint8_t* kbase = a.k + (int64_t)g * kD * 2;
  const uint8_t* vbase = a.v + (int64_t)g * kD * 2;

  auto key_addr = [&](const uint8_t* base, int key) -> const uint8_t* {
    const int phys = bt_row[key >> a.bs_shift];
    return base + ((int64_t)phys << a.bs_shift) * tok_stride + (int64_t)(key & bmask) * tok_stride;
  };

  u32x4_t kreg[kKPer];
  u32x4_t vreg[kVPer][2];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int j = 0; j < kKPer; ++j) {
      const int chunk = tid + j * kNT;
      const int key = kt * kBN + (chunk >> 4);
      kreg[j] = key < kend ? load16(key_addr(kbase, key) + (chunk & 15) * 16)
                           : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < kVPer; ++j) {
      const int u = tid + j * kNT;
      const int key = kt * kBN + 2 * (u >> 4);
      const int col = (u & 15) * 16;
#pragma unroll
      for (int t = 0; t < 2; ++t)
        vreg[j][t] = key + t < kend ? load16(key_addr(vbase, key + t) + col)
                                    : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int j = 0; j < kKPer; ++j) {
      const int chunk = tid + j * kNT;
      *reinterpret_cast<u32x4_t*>(k_lds + (chunk >> 4) * kKRow + (chunk & 15) * 16) = kreg[j];
    }
#pragma unroll
    for (int j = 0; j < kVPer; ++j) {
      const int u = tid + j * kNT;
      const int kp = u >> 4;         // key pair
      const int d0 = (u & 15) * 8;   // first of 8 columns
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = pair_to_f16<T>(vreg[j][0][i], vreg[j][1][i], false);
        const uint32_t hv = pair_to_f16<T>(vreg[j][0][i], vreg[j][1][i], true);
        *reinterpret_cast<uint32_t*>(vt_lds + (d0 + 2 * i) * kVRow + kp * 4) = lo;
        *reinterpret_cast<uint32_t*>(vt_lds + (d0 + 2 * i + 1) * kVRow + kp * 4) = hv;
      }
    }
  };

  f32x16_t acc_o[kD / 32];
#pragma unroll
  for (int md = 0; md < kD / 32; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[md][r] = 0.f;
  float m_run = -INFINITY;  // running max of row r32 (log2 units)
  float l_lane = 0.f;       // running sum over this lane's keys

  if (ntk > 0) load_tile(0);
  for (int kt = 0; kt < ntk; ++kt) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (kt + 1 < ntk) load_tile(kt + 1);

    const int kbase_t = kt * kBN;
    if (!wave_active || kbase_t > vis_hi) continue;  // nothing visible for this wave
    const bool need_mask = kbase_t + kBN - 1 > vis_lo || kbase_t + kBN > n;

    // S^T = K Q^T for the tile's two 32-key blocks.
    f32x16_t sc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[mb][r] = 0.f;
      const uint8_t* krow = k_lds + (mb * 32 + r32) * kKRow + hi * 16;
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks)
        sc[mb] = mfma_qk<T>(*reinterpret_cast<const u32x4_t*>(krow + ks * 32), qf[ks], sc[mb]);
    }

    // Online softmax for row r32; key of element (mb, r) is
    // kbase_t + mb*32 + 8*(r/4) + 4*hi + r%4.
    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = sc[mb][r] * a.scale_log2;
        if (need_mask) {
          const int key = kbase_t + mb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key > my_vis) x = -INFINITY;
        }
        sc[mb][r] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    l_lane *= alpha;
#pragma unroll
    for (int md = 0; md < kD / 32; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[md][r] *= alpha;

    u32x4_t pf[2][2];  // B operand of P^T per (mb, qq)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pv[j] = fast_exp2(sc[mb][8 * qq + j] - m_new);
          l_lane += pv[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) pf[mb][qq][j] = pack_f16(pv[2 * j], pv[2 * j + 1]);
      }

    // O^T += V^T P^T.
#pragma unroll
    for (int md = 0; md < kD / 32; ++md) {
      const uint8_t* vrow = vt_lds + (md * 32 + r32) * kVRow;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          const int k0 = mb * 32 + 16 * qq + 4 * hi;
          const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vrow + k0 * 2);
          const u32x2_t hv = *reinterpret_cast<const u32x2_t*>(vrow + (k0 + 8) * 2);
          const u32x4_t av = {lo[0], lo[1], hv[0], hv[1]};
          acc_o[md] = mfma_pv(av, pf[mb][qq], acc_o[md]);
        }
    }
  }

  if (!row_ok) return;
  const float l_tot = l_lane + __shfl_xor(l_lane, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t obase = (int64_t)(q0 + my_i) * a.o_st + (int64_t)hq * a.o_sh;
#pragma unroll
  for (int md = 0; md < kD / 32; ++md)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = md * 32 + 8 * rg + 4 * hi;
      const float o0 = acc_o[md][4 * rg + 0] * inv, o1 = acc_o[md][4 * rg + 1] * inv;
      const float o2 = acc_o[md][4 * rg + 2] * inv, o3 = acc_o[md][4 * rg + 3] * inv;
      if (a.out_f32) {
        *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.out) + obase + d0) =
            f32x4_t{o0, o1, o2, o3};
      } else {
        uint16_t* op = static_cast<uint16_t*>(a.out) + obase + d0;
        u32x2_t pk;
        if constexpr (__is_same(T, TBF16)) {
          pk[0] = (uint32_t)to_bf16_bits(o0) | ((uint32_t)to_bf16_bits(o1) << 16);
          pk[1] = (uint32_t)to_bf16_bits(o2) | ((uint32_t)to_bf16_bits(o3) << 16);
        } else {
          pk[0] = (uint32_t)to_f16_bits(o0) | ((uint32_t)to_f16_bits(o1) << 16);
          pk[1] = (uint32_t)to_f16_bits(o2) | ((uint32_t)to_f16_bits(o3) << 16);
        }
        *reinterpret_cast<u32x2_t*>(op) = pk;
      }
    }
}

template <class T, int G>
hipError_t launch_prefill_t(const PrefillPlan& pl, const PrefillArgs& a, hipStream_t stream) {
  const int64_t blocks = a.wg_per_xcd * 8;
  KernelTimer t("prefill", stream);
  hipLaunchKernelGGL((prefill_kernel<T, G>), dim3((unsigned)blocks), dim3(128 * G), 0, stream,
                     a);
  return hipGetLastError();
}

template <class T>
hipError_t dispatch_group(const PrefillPlan& pl, const PrefillArgs& a, hipStream_t stream) {
  switch (pl.G) {
    case 1: return launch_prefill_t<T, 1>(pl, a, stream);
    case 2: return launch_prefill_t<T, 2>(pl, a, stream);
    case 4: return launch_prefill_t<T, 4>(pl, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillPlan& pl, hipStream_t stream) {
  PrefillArgs a;
  a.q = static_cast<const uint8_t*>(pl.q);
  a.q_st = pl.q_st * 2;
  a.q_sh = pl.q_sh * 2;
  a.k = static_cast<const uint8_t*>(pl.k);
  a.v = static_cast<const uint8_t*>(pl.v);
  a.bt = pl.bt;
  a.bt_ss = pl.bt_ss;
  a.cl = pl.cl;
  a.qsl = pl.qsl;
  a.out = pl.out;
  a.o_st = pl.o_st;
  a.o_sh = pl.o_sh;
  a.out_f32 = pl.out_dtype == PA_F32;
  a.S = pl.S;
  a.Hkv = pl.Hkv;
  a.q_tiles = pl.q_tiles;
  a.bs_shift = __builtin_ctz(pl.B);
  a.causal = pl.causal;
  a.n_wg = (int64_t)pl.q_tiles * pl.Hkv * pl.S;
  a.wg_per_xcd = (a.n_wg + 7) / 8;
  a.scale_log2 = pl.scale * 1.4426950408889634f;
  if (a.n_wg == 0) return hipSuccess;
  switch (pl.dtype) {
    case PA_F16: return dispatch_group<TF16>(pl, a, stream);
    case PA_BF16: return dispatch_group<TBF16>(pl, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
