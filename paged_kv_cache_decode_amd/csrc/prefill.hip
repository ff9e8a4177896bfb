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
//   workgroup = 32 * RW query positions (64 for packed prompts, 32 for the
//   shared-prefix step) x the G query heads of one KV
//   head (a wave owns 32 positions of one head).  K/V tiles of 64 keys
//   are gathered once per workgroup into LDS and feed all G heads.  Key
//   tiles wholly above the diagonal are never loaded.  LDS is double
//   buffered: while the waves compute on one tile the next one is written
//   to the other buffer from registers, and the tile after that is already
//   being fetched, so there is one barrier per tile.
//
// Per 32-key half of a 64-key tile a wave computes, on 32x32x16 MFMAs:
//   S^T = K Q^T   (A = K from LDS, B = Q from registers; bf16/f16 inputs,
//                  fp32 accumulate).  The transposed product leaves every
//                  score of query row r in lane r (and r + 32), so the
//                  row max / row sum of the online softmax are lane-local.
//   O^T += V^T P^T (A = V^T from LDS, B = P from the lane's own scores,
//                  rounded to fp16; fp32 accumulate).  V is written to LDS
//                  transposed (d-major) and converted to fp16 while it is
//                  staged; fp16 keeps P's rounding error 8x below bf16's.
// Softmax: the scale is folded into the exponent's FMA (p = 2^(s*c - m)
// with c = scale*log2 e); the running maximum is only raised when a row's
// new maximum exceeds it by more than 2^8 (p then stays below 256, exact
// in fp16's range), so the O rescale is rare; row sums accumulate the
// fp16 P values with v_dot2, consistent with what the P.V product uses.
// Only tiles that cross the diagonal (or the end of the context) run the
// masking code.
//
// Workgroups are ordered so that each XCD (8 per MI355X, fed round-robin)
// works through a contiguous slice of (KV head, sequence, query tile), with
// a sequence's query tiles longest-first; the tiles running together on an
// XCD then share the same K/V in its L2.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "launch.h"

namespace pa {
namespace {

constexpr int kBN = 64;                        // keys per tile
constexpr int kD = 128;                        // head size
constexpr int kKRow = kD * 2 + 16;             // K tile row in LDS (bytes, padded)
constexpr int kVRow = kBN * 2 + 8;             // V^T tile row in LDS (bytes, padded)
constexpr int kKBytes = kBN * kKRow;           // one K tile in LDS
constexpr int kVBytes = kD * kVRow;            // one V^T tile in LDS
constexpr int kKChunks = kBN * kD * 2 / 16;    // 16-byte chunks in a K tile (1024)
constexpr int kVUnits = (kBN / 2) * (kD / 8);  // (key pair, 8-column) units (512)
constexpr float kRescaleSlack = 8.f;           // lazy-rescale threshold (log2 units)

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
  int S, Hkv, MB, q_tiles, bs_shift, causal;
  // Pool layout (bytes): between consecutive slots of a block, and between
  // KV heads; blocks are Hkv*B*d*2 bytes apart.
  int tok_bytes;
  int64_t head_bytes;
  uint32_t q_sign;     // XORed into Q's 16-bit lanes (0x80008000 when scale < 0)
  // Head groups of more than 4 heads run as kv_div workgroups of 4 heads per
  // KV head (each reads that KV head's K/V): workgroup group g covers query
  // heads 4g .. 4g+3 and KV head g / kv_div.  kv_div = 1 otherwise.
  int kv_div;
  int64_t n_wg;        // real workgroups (q_tiles * Hkv * kv_div * S * n_chunks)
  int64_t wg_per_xcd;  // ceil(n_wg / 8)
  float c;             // |scale| * log2(e)
  // One sequence given by value (fixed_L >= 0): L = fixed_L rows, n =
  // fixed_n keys; qsl / cl are not read.
  int fixed_L, fixed_n;
  // Keys split into n_chunks chunks of chunk_tiles 64-key tiles; with
  // part_o set, each workgroup writes its normalised partial output and
  // log2-sum-exp instead of `out`, for a later kernel to merge:
  //   part_o [n_chunks, H, part_rows, d] f32, part_lse [n_chunks, H, part_rows].
  int n_chunks, chunk_tiles, H;
  int64_t part_rows;
  float* part_o;
  float* part_lse;
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

// Low / high 16-bit element of two storage dwords, as one fp16 pair.
template <class T>
__device__ __forceinline__ uint32_t pair_to_f16(uint32_t w0, uint32_t w1, bool high) {
  if constexpr (__is_same(T, TF16)) {
    return high ? ((w0 >> 16) | (w1 & 0xffff0000u)) : ((w0 & 0xffffu) | (w1 << 16));
  } else {
    return high ? pack_f16(bf16_hi(w0), bf16_hi(w1)) : pack_f16(bf16_lo(w0), bf16_lo(w1));
  }
}

// The value of lane l ^ 32 (v_permlane32_swap exchanges the wave's halves
// without going through LDS).
__device__ __forceinline__ float swap_halves(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  // r[0] holds the low half in both halves, r[1] the high half.
  const bool upper = (threadIdx.x & 32) != 0;
  return __builtin_bit_cast(float, upper ? r[0] : r[1]);
}

// V^T rows are stored with their key-pair columns XOR-swizzled by the row's
// 32-row group (even values, so the two dwords of a 4-key read stay
// adjacent); it spreads the transposing writes over the LDS banks.
__device__ __forceinline__ int vt_col(int d, int kp) { return kp ^ ((d >> 5) << 1); }

// RW waves per head: a workgroup covers 32 * RW query positions.  The
// 32-row instances (the shared-prefix step) ask for at most half the
// register file, so that two of their workgroups can share a CU (measured:
// prefix step 28 -> 25.5 us on the shared-prefix workload).
template <class T, int G, int RW>
__global__ __launch_bounds__(64 * RW * G)
__attribute__((amdgpu_waves_per_eu(RW == 1 ? 2 : 1))) void prefill_kernel(PrefillArgs a) {
  constexpr int kNT = 64 * RW * G;  // threads
  constexpr int kRows = 32 * RW;    // query positions per workgroup
  constexpr int kKPer = kKChunks / kNT;
  constexpr int kVPer = kVUnits / kNT;
  static_assert(kKPer * kNT == kKChunks && kVPer * kNT == kVUnits, "tile split");

  __shared__ __attribute__((aligned(16))) uint8_t k_lds[2][kKBytes];
  __shared__ __attribute__((aligned(16))) uint8_t vt_lds[2][kVBytes];

  // XCD-aware order: hardware workgroup b runs on XCD b % 8; give each XCD
  // a contiguous slice of the logical order (g, s, query tile descending).
  const int64_t bid = blockIdx.x;
  const int64_t logical_c = (bid & 7) * a.wg_per_xcd + (bid >> 3);
  if (logical_c >= a.n_wg) return;
  const int chunk = (int)(logical_c % a.n_chunks);
  const int64_t logical = logical_c / a.n_chunks;
  const int per_g = a.S * a.q_tiles;
  const int g = (int)(logical / per_g);
  const int rem = (int)(logical % per_g);
  const int s = rem / a.q_tiles;
  const int qt = a.q_tiles - 1 - rem % a.q_tiles;

  const const_i32_ptr qsl = as_const(a.qsl);
  const int q0 = a.fixed_L >= 0 ? 0 : qsl[s];
  const int L = a.fixed_L >= 0 ? a.fixed_L : qsl[s + 1] - q0;
  const int n = a.fixed_L >= 0 ? a.fixed_n : as_const(a.cl)[s];
  if (qt * kRows >= L) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hl = w % G;    // head within the group
  const int half = w / G;  // which 32 of the 64 positions
  const int hq = g * G + hl;
  const int r32 = lane & 31;
  const int hi = lane >> 5;

  // This wave's rows: i = row0 + r32 (query index within the sequence).
  const int row0 = qt * kRows + half * 32;
  const int my_i = row0 + r32;
  const bool row_ok = my_i < L;
  const int shift = n - L;  // absolute position of row i is shift + i

  // Keys the workgroup needs: [0, kend).
  int kend = n;
  if (a.causal) kend = min(n, shift + min(qt * kRows + kRows, L));
  const int ntk = (kend + kBN - 1) / kBN;
  // Per wave: tiles below `full` need no mask; tiles from `full` up to
  // `last` need one; later tiles hold no visible key for this wave.
  const bool wave_active = row0 < L;
  const int wave_last_i = min(row0 + 31, L - 1);
  const int vis_lo = a.causal ? shift + row0 : n - 1;         // first row's last key
  const int vis_hi = a.causal ? shift + wave_last_i : n - 1;  // last row's last key
  const int full = min(vis_lo + 1, n) / kBN;                  // fully visible tiles
  const int last = wave_active ? vis_hi / kBN : -1;
  const int my_vis = a.causal ? shift + my_i : n - 1;

  // Q^T as the MFMA B operand: lane holds row r32, columns ks*16 + 8*hi.
  u32x4_t qf[kD / 16];
  {
    const uint8_t* qrow = a.q + (int64_t)(q0 + my_i) * a.q_st + (int64_t)hq * a.q_sh + hi * 16;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      qf[ks] = row_ok ? load16(qrow + ks * 32) : u32x4_t{0u, 0u, 0u, 0u};
      qf[ks] ^= a.q_sign;
    }
  }

  const const_i32_ptr bt_row = as_const(a.bt) + (int64_t)s * a.bt_ss;
  const int tok_stride = a.tok_bytes;  // bytes between consecutive slots
  const int bmask = (1 << a.bs_shift) - 1;
  const int64_t block_bytes = (int64_t)(a.Hkv * kD * 2) << a.bs_shift;
  const uint8_t* kbase = a.k + (int64_t)(g / a.kv_div) * a.head_bytes;
  const uint8_t* vbase = a.v + (int64_t)(g / a.kv_div) * a.head_bytes;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // wave index (uniform)
  // Gather addressing.  Every load instruction of a wave covers 4 (K) or 8
  // (V) consecutive keys starting at a multiple of 4 (8), so all its lanes
  // sit in one KV block (B >= 16): the block's address comes from one scalar
  // table read and scalar arithmetic, and each lane adds a fixed offset.
  // Key starts at or past the end are clamped to the last 4 keys before
  // `kend` (a block the table maps); the rows they fetch are either masked
  // (K) or zeroed before use (V).
  const int kend_c = max(kend - 1, 0) & ~3;
  const uint32_t k_lane = (uint32_t)((lane >> 4) * tok_stride + (lane & 15) * 16);
  const uint32_t v_lane = (uint32_t)(2 * (lane >> 4) * tok_stride + (lane & 15) * 16);
  auto row_addr = [&](const uint8_t* base, int key) -> const uint8_t* {
    const int blk = key >> a.bs_shift;
    const int64_t phys = bt_row[blk];
    return base + phys * block_bytes + (int64_t)((key & bmask) * tok_stride);
  };

  // Global -> registers for tile kt.
  u32x4_t kreg[kKPer];
  u32x4_t vreg[kVPer][2];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int j = 0; j < kKPer; ++j) {
      const int kb = min(kt * kBN + 4 * wu + j * (kNT / 16), kend_c);
      kreg[j] = load16(row_addr(kbase, kb) + k_lane);
    }
#pragma unroll
    for (int j = 0; j < kVPer; ++j) {
      const int kb = min(kt * kBN + 8 * wu + j * (kNT / 8), kend_c & ~7);
      const uint8_t* p = row_addr(vbase, kb) + v_lane;
      vreg[j][0] = load16(p);
      vreg[j][1] = load16(p + tok_stride);
    }
  };
  // Registers -> LDS buffer `buf` (K row-major, V transposed to fp16).  In
  // the tile that reaches `kend`, V rows at or past it are zeroed first (they
  // may be clamped duplicates or unwritten slots; P is zero there, and a
  // zero row keeps the product finite).
  auto store_tile = [&](int kt, int buf) {
    uint8_t* kl = k_lds[buf];
    uint8_t* vl = vt_lds[buf];
#pragma unroll
    for (int j = 0; j < kKPer; ++j) {
      const int chunk = tid + j * kNT;
      *reinterpret_cast<u32x4_t*>(kl + (chunk >> 4) * kKRow + (chunk & 15) * 16) = kreg[j];
    }
    if ((kt + 1) * kBN > kend) {
#pragma unroll
      for (int j = 0; j < kVPer; ++j) {
        const int key = kt * kBN + 2 * ((tid + j * kNT) >> 4);
#pragma unroll
        for (int t = 0; t < 2; ++t)
          if (key + t >= kend) vreg[j][t] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int j = 0; j < kVPer; ++j) {
      const int u = tid + j * kNT;
      const int kp = u >> 4;        // key pair
      const int d0 = (u & 15) * 8;  // first of 8 columns
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = d0 + 2 * i;
        *reinterpret_cast<uint32_t*>(vl + d * kVRow + vt_col(d, kp) * 4) =
            pair_to_f16<T>(vreg[j][0][i], vreg[j][1][i], false);
        *reinterpret_cast<uint32_t*>(vl + (d + 1) * kVRow + vt_col(d + 1, kp) * 4) =
            pair_to_f16<T>(vreg[j][0][i], vreg[j][1][i], true);
      }
    }
  };

  f32x16_t acc_o[kD / 32];
#pragma unroll
  for (int md = 0; md < kD / 32; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[md][r] = 0.f;
  float m_run = -INFINITY;  // running max of row r32, scaled (log2 units)
  float l_lane = 0.f;       // running sum of this lane's P values

  // One 64-key tile of this wave as two 32-key halves, software-pipelined so
  // that matrix-core and vector work overlap inside the wave: both halves'
  // S^T = K Q^T MFMAs are issued first; the softmax of half 0 (VALU) then
  // runs while half 1's QK^T executes, and the softmax of half 1 while half
  // 0's O^T += V^T P^T executes.
  f16x2_t ones;
  ones[0] = ones[1] = static_cast<_Float16>(1.f);
  // S^T = K Q^T for both 32-key halves of a tile.  The schedule is pinned:
  // half 0's eight K fragments are read first, then each half-0 MFMA is
  // followed by the read of one half-1 fragment, then half 1's MFMAs; every
  // MFMA then finds its operand already in registers.
  auto qk_tile = [&](const uint8_t* kl, f32x16_t& sc0, f32x16_t& sc1) {
    const uint8_t* krow = kl + r32 * kKRow + hi * 16;
    u32x4_t kf0[kD / 16], kf1[kD / 16];
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks)
      kf0[ks] = *reinterpret_cast<const u32x4_t*>(krow + ks * 32);
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks)
      kf1[ks] = *reinterpret_cast<const u32x4_t*>(krow + 32 * kKRow + ks * 32);
#pragma unroll
    for (int r = 0; r < 16; ++r) sc0[r] = sc1[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) sc0 = mfma_qk<T>(kf0[ks], qf[ks], sc0);
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) sc1 = mfma_qk<T>(kf1[ks], qf[ks], sc1);
    __builtin_amdgcn_sched_group_barrier(0x100, kD / 16, 0);  // DS reads, half 0
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA, half 0
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // DS read, half 1
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kD / 16, 0);  // MFMAs, half 1
  };
  // Online-softmax update for one half; returns P (fp16) as two MFMA B
  // operands.  Element r of this lane is key kt*64 + mb*32 + 8*(r/4) +
  // 4*hi + r%4.
  auto softmax_half = [&](const f32x16_t& sc, int kt, int mb, auto mask_tag, u32x4_t* pf) {
    constexpr bool kMask = decltype(mask_tag)::value;
    bool vis[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if constexpr (kMask) {
        const int key = kt * kBN + mb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        vis[r] = key <= my_vis;
        tmax = fmaxf(tmax, vis[r] ? sc[r] : -INFINITY);
      } else {
        tmax = fmaxf(tmax, sc[r]);
      }
    }
    tmax = fmaxf(tmax, swap_halves(tmax));
    // Lazy rescale: raise the running max only when some row's new max is
    // more than kRescaleSlack above it (p = 2^(s*c - m) then stays < 2^8).
    const float m_cand = tmax * a.c;
    if (__builtin_amdgcn_ballot_w64(m_cand > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, m_cand);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_lane *= alpha;
#pragma unroll
      for (int md = 0; md < kD / 32; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[md][r] *= alpha;
    }
    const float neg_m = -m_run;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r0 = 8 * qq + 2 * j;
        float p0 = fast_exp2(fmaf(sc[r0], a.c, neg_m));
        float p1 = fast_exp2(fmaf(sc[r0 + 1], a.c, neg_m));
        if constexpr (kMask) {
          p0 = vis[r0] ? p0 : 0.f;
          p1 = vis[r0 + 1] ? p1 : 0.f;
        }
        const uint32_t pk = pack_f16(p0, p1);
        pf[qq][j] = pk;
        l_lane = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pk), ones, l_lane, false);
      }
  };
  // O^T += V^T P^T over one half's 32 keys.
  auto pv_half = [&](const uint8_t* vl, int mb, const u32x4_t* pf) {
    u32x4_t vf[kD / 32][2];
#pragma unroll
    for (int md = 0; md < kD / 32; ++md) {
      const int d = md * 32 + r32;
      const uint8_t* vrow = vl + d * kVRow;
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int kp = (mb * 32 + 16 * qq + 4 * hi) >> 1;
        const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vrow + vt_col(d, kp) * 4);
        const u32x2_t hv = *reinterpret_cast<const u32x2_t*>(vrow + vt_col(d, kp + 4) * 4);
        vf[md][qq] = u32x4_t{lo[0], lo[1], hv[0], hv[1]};
      }
    }
#pragma unroll
    for (int md = 0; md < kD / 32; ++md)
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) acc_o[md] = mfma_pv(vf[md][qq], pf[qq], acc_o[md]);
  };
  auto compute_tile = [&](int kt, int buf, auto mask_tag) {
    const uint8_t* kl = k_lds[buf];
    const uint8_t* vl = vt_lds[buf];
    f32x16_t sc0, sc1;
    qk_tile(kl, sc0, sc1);
    u32x4_t pf0[2], pf1[2];
    softmax_half(sc0, kt, 0, mask_tag, pf0);
    pv_half(vl, 0, pf0);
    softmax_half(sc1, kt, 1, mask_tag, pf1);
    pv_half(vl, 1, pf1);
  };

  // This workgroup's tiles: [kt0, kt1) (all of [0, ntk) without chunking).
  const int kt0 = min(ntk, chunk * a.chunk_tiles);
  const int kt1 = min(ntk, kt0 + a.chunk_tiles);
  if (kt0 < kt1) {
    load_tile(kt0);
    store_tile(kt0, kt0 & 1);
    if (kt0 + 1 < kt1) load_tile(kt0 + 1);
  }
  for (int kt = kt0; kt < kt1; ++kt) {
    __syncthreads();  // tile kt is in buffer kt & 1; buffer (kt+1) & 1 is free
    if (kt + 1 < kt1) {
      store_tile(kt + 1, (kt + 1) & 1);
      if (kt + 2 < kt1) load_tile(kt + 2);
    }
    if (kt < full) {
      compute_tile(kt, kt & 1, std::false_type{});
    } else if (kt <= last) {
      compute_tile(kt, kt & 1, std::true_type{});
    }
  }

  const float l_tot = l_lane + swap_halves(l_lane);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (a.part_o) {
    // Partial result of this key chunk: o / l and m + log2 l (log2 units of
    // the scaled scores; -inf when the chunk held no visible key), row by
    // row ([chunk][H][rows][d]; lane (r32, hi) holds columns md*32 + 8*rg +
    // 4*hi + 0..3 of its row).  The merge happens in the next kernel on the
    // stream, after this one's writes are complete.
    if (!row_ok) return;
    const float lse = l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY;
    const int64_t prow = ((int64_t)chunk * a.H + hq) * a.part_rows + q0 + my_i;
    float* po = a.part_o + prow * kD;
#pragma unroll
    for (int md = 0; md < kD / 32; ++md)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
        *reinterpret_cast<f32x4_t*>(po + md * 32 + 8 * rg + 4 * hi) =
            f32x4_t{acc_o[md][4 * rg] * inv, acc_o[md][4 * rg + 1] * inv,
                    acc_o[md][4 * rg + 2] * inv, acc_o[md][4 * rg + 3] * inv};
    if (hi == 0) a.part_lse[prow] = lse;
    return;
  }
  if (!row_ok) return;
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

template <class T, int G, int RW>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
  const int64_t blocks = a.wg_per_xcd * 8;
  return timed_launch("prefill", prefill_kernel<T, G, RW>, dim3((unsigned)blocks),
                      dim3(64 * RW * G), stream, a);
}

template <class T, int RW>
hipError_t dispatch_group(const PrefillPlan& pl, const PrefillArgs& a, hipStream_t stream) {
  switch (pl.G) {
    case 1: return launch_prefill_t<T, 1, RW>(a, stream);
    case 2: return launch_prefill_t<T, 2, RW>(a, stream);
    case 4:
    case 8: return launch_prefill_t<T, 4, RW>(a, stream);  // 8: two workgroups per KV head
    default: return hipErrorInvalidValue;
  }
}

template <class T>
hipError_t dispatch_rows(const PrefillPlan& pl, const PrefillArgs& a, hipStream_t stream) {
  switch (pl.row_waves) {
    case 1: return dispatch_group<T, 1>(pl, a, stream);
    case 2: return dispatch_group<T, 2>(pl, a, stream);
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
  a.MB = pl.MB;
  a.q_tiles = pl.q_tiles;
  a.bs_shift = __builtin_ctz(pl.B);
  a.tok_bytes = (int)(pl.pool.tok * 2);
  a.head_bytes = pl.pool.head * 2;
  a.causal = pl.causal;
  // A negative scale is applied by negating Q (exact in 16-bit formats) so
  // that the softmax always works with c >= 0.
  a.q_sign = pl.scale < 0.f ? 0x80008000u : 0u;
  a.c = (pl.scale < 0.f ? -pl.scale : pl.scale) * 1.4426950408889634f;
  a.fixed_L = pl.fixed_L;
  a.fixed_n = pl.fixed_n;
  a.n_chunks = pl.n_chunks;
  a.chunk_tiles = pl.chunk_tiles;
  a.H = pl.H;
  a.part_rows = pl.part_rows;
  a.part_o = pl.part_o;
  a.part_lse = pl.part_lse;
  a.kv_div = pl.G > 4 ? pl.G / 4 : 1;
  a.n_wg = (int64_t)pl.q_tiles * pl.Hkv * a.kv_div * pl.S * pl.n_chunks;
  a.wg_per_xcd = (a.n_wg + 7) / 8;
  if (a.n_wg == 0) return hipSuccess;
  switch (pl.dtype) {
    case PA_F16: return dispatch_rows<TF16>(pl, a, stream);
    case PA_BF16: return dispatch_rows<TBF16>(pl, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
