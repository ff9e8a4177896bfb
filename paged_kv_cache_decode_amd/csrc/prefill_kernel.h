// Device code of the prefill kernel (included by prefill.hip, and by
// shared_prefix.hip for the shared-prefix call's combined kernel).
//
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
//   a wave owns 16 query positions of one query head; a workgroup holds the
//   HG heads of one KV head (HG = G, or 4 when G = 8: then two workgroups
//   per KV head) times RW waves per head, i.e. 16 * RW positions.  Packed
//   prompts use workgroups of 16 waves (HG * RW = 16, 64 positions x 4
//   heads for G = 4), one per compute unit, at most 128 registers per wave:
//   every SIMD runs four waves whose loads, matrix products and
//   exponentials interleave.  K/V tiles of 64 keys are gathered once per
//   workgroup into LDS and feed all its waves.  Key tiles wholly above the
//   diagonal are never loaded.  LDS is double buffered (V^T triple buffered
//   in sixteen-wave workgroups): after computing on one tile a wave writes
//   its part of the next one, fetched during the previous step, to the free
//   buffers and fetches the tile after it, so there is one barrier per
//   tile.
//
// Per 64-key tile a wave computes, on 16x16x32 MFMAs:
//   S^T = K Q^T   (A = K from LDS, B = Q from registers; bf16/f16 inputs,
//                  fp32 accumulate).  Every score of query row r lands in
//                  the four lanes r, r + 16, r + 32, r + 48 (16 keys each),
//                  so a row's max and sum take two lane swaps.
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
// works through whole (head group, sequence) pairs, so that the tiles
// running together on an XCD share the same K/V in its L2.  Packed prompts
// (packed_item) take the pairs in order of decreasing context length and
// each pair's query tiles from the last, the longest, with no empty
// workgroup ahead of a real one; other shapes take a contiguous slice of
// (head group, sequence, query tile descending) per XCD.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace pa {
namespace {

constexpr int kBN = 64;                        // keys per tile
constexpr int kD = 128;                        // head size
constexpr int kKRow = kD * 2 + 32;             // K tile row in LDS (bytes, padded)
constexpr int kVRow = kBN * 2 + 32;            // V^T tile row in LDS (bytes, padded)
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
  // Packed prompts whose head groups split evenly over the 8 XCDs, at
  // most 64 (group, sequence) pairs per XCD: work items from packed_item.
  int packed_order;
};

template <class T>
__device__ __forceinline__ f32x4_t mfma_qk(u32x4_t a, u32x4_t b, f32x4_t c) {
  if constexpr (__is_same(T, TBF16))
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_pv(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
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

// The value of lane l ^ 16 / l ^ 32.  v_permlane16_swap exchanges the odd
// 16-lane rows of its first operand with the even rows of its second, and
// v_permlane32_swap the wave's halves, without LDS; with both operands the
// same register, a lane finds its partner's value in the result that its
// own row (half) did not keep, which is picked by the lane's position.
__device__ __forceinline__ float xor16(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const bool odd = (threadIdx.x & 16) != 0;
  return __builtin_bit_cast(float, odd ? r[0] : r[1]);
}
__device__ __forceinline__ float xor32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const bool upper = (threadIdx.x & 32) != 0;
  return __builtin_bit_cast(float, upper ? r[0] : r[1]);
}
// Max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the lanes that
// hold one query row's scores).
__device__ __forceinline__ float row4_max(float x) {
  x = fmaxf(x, xor16(x));
  return fmaxf(x, xor32(x));
}
__device__ __forceinline__ float row4_sum(float x) {
  x += xor16(x);
  return x + xor32(x);
}

// Work item of packed-prompt workgroup `bid` (its hardware number): head
// group `grp`, sequence `s` (query rows from q0, L of them, n keys), query
// tile `qt` of kRowsWG rows; false when the workgroup has none.  The (group, sequence) pairs are cut into 8 equal
// contiguous ranges, one per XCD (workgroup b runs on XCD b % 8), so that
// all query tiles of a pair share its K/V in one L2; with the number of
// groups a multiple of 8 every range holds whole groups and the same work.
// Within its range an XCD takes the pairs in order of decreasing context
// length (ties by position) and each pair's query tiles from the last,
// which visits the most keys: the longest tiles start first, the short
// ones of the short sequences fill the end, a pair's tiles run together
// while its K/V is in L2, and the workgroups with no tile come after every
// real one in dispatch order.  Lane i of every wave holds pair i of the
// range (at most 64).
template <int kRowsWG>
__device__ __forceinline__ bool packed_item(const PrefillArgs& a, int64_t bid, int& grp, int& s,
                                            int& qt, int& q0, int& L, int& n) {
  const int lane = threadIdx.x & 63;
  const int n_pairs = a.Hkv * a.kv_div * a.S;
  const int ppx = (n_pairs + 7) >> 3;
  const int p_lo = min(n_pairs, (int)(bid & 7) * ppx);
  const int np = min(n_pairs - p_lo, ppx);
  const int j = (int)(bid >> 3);
  int T = 0, lq0 = 0, lL = 0, ln = 0;
  if (lane < np) {
    const int ss = (p_lo + lane) % a.S;
    lq0 = a.qsl[ss];
    lL = a.qsl[ss + 1] - lq0;
    ln = a.cl[ss];
    T = lL > 0 ? min(a.q_tiles, (lL + kRowsWG - 1) / kRowsWG) : 0;
  }
  // Tiles of the pairs ahead of this lane's pair in the order.
  int start = 0;
  for (int p = 0; p < np; ++p) {
    const int np_ = __builtin_amdgcn_readlane(ln, p);
    const int tp = __builtin_amdgcn_readlane(T, p);
    start += (np_ > ln || (np_ == ln && p < lane)) ? tp : 0;
  }
  const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < np && start <= j && j < start + T);
  if (hit == 0) return false;
  const int src = __builtin_ctzll(hit);
  const int pair = p_lo + src;
  grp = pair / a.S;
  s = pair % a.S;
  qt = __builtin_amdgcn_readlane(T, src) - 1 - (j - __builtin_amdgcn_readlane(start, src));
  q0 = __builtin_amdgcn_readlane(lq0, src);
  L = __builtin_amdgcn_readlane(lL, src);
  n = __builtin_amdgcn_readlane(ln, src);
  return true;
}

// V^T in LDS: row d holds the tile's 64 keys as fp16, in an order that puts
// the 8 keys one lane feeds to a P.V MFMA next to each other.  The lane
// (row r16, group g4) of 32-key step s2 holds, as the MFMA's B operand, the
// P values of keys 32*s2 + {4*g4 + 0..3, 16 + 4*g4 + 0..3} (the keys its
// own S^T results cover), so within every 32 keys the key index bits
// (4, 3..2) become (2, 4..3): the lane's 8 keys form the 16-byte chunk
// 4*s2 + g4 of the row, read with one ds_read_b128.  The chunk index (0..7)
// is XORed with (d >> 4) & 7 and rows are 160 bytes apart; K rows are 288
// bytes apart.  Both strides were chosen by measuring the LDS bank-conflict
// counter on gfx950 for these exact access patterns: the K and V^T fragment
// reads then cost no conflict cycles and the transposing 4-byte writes of
// the staging step two per instruction (at the 272/144-byte strides that a
// 64-bank model predicts to be conflict-free, every fragment read cost
// four).
__device__ __forceinline__ int vt_pos(int key) {
  return (key & ~31) | (((key >> 2) & 3) << 3) | (((key >> 4) & 1) << 2) | (key & 3);
}

// LDS of one prefill workgroup of HG x RW waves: two K tiles and two V^T
// tiles, or three V^T tiles in sixteen-wave workgroups, where half of the
// waves compute a tile's P.V one step late (see the tile loop).
template <int HG, int RW>
struct PrefillLds {
  static constexpr bool kDelayPV = HG * RW == 16;
  static constexpr int kVBufs = kDelayPV ? 3 : 2;
  static constexpr int kBytes = 2 * kKBytes + kVBufs * kVBytes;
};

// Prefill workgroup `bid` (its hardware number, which fixes its XCD) of HG
// heads x RW waves of 16 query positions, with its LDS at `lds` (16-byte
// aligned, PrefillLds<HG, RW>::kBytes).  Called by every thread of the
// workgroup.
template <class T, int HG, int RW>
__device__ __forceinline__ void prefill_body(const PrefillArgs& a, int64_t bid, uint8_t* lds) {
  constexpr int kNT = 64 * HG * RW;  // threads
  constexpr int kRows = 16 * RW;     // query positions per workgroup
  constexpr int kKPer = kKChunks / kNT;
  // With 1024 threads the first 512 stage V (one unit each); on every SIMD
  // half of the workgroup's waves then do it.
  constexpr int kVPer = (kVUnits + kNT - 1) / kNT;
  constexpr bool kVAll = kVPer * kNT == kVUnits;
  static_assert(kKPer * kNT == kKChunks && (kVAll || kVPer == 1), "tile split");

  constexpr int kVBufs = PrefillLds<HG, RW>::kVBufs;
  auto k_lds = reinterpret_cast<uint8_t (*)[kKBytes]>(lds);
  auto vt_lds = reinterpret_cast<uint8_t (*)[kVBytes]>(lds + 2 * kKBytes);

  int g = 0, s = 0, qt = 0, chunk = 0, q0 = 0, L = 0, n = 0;
  if (a.packed_order) {
    if (!packed_item<kRows>(a, bid, g, s, qt, q0, L, n)) return;
  } else {
    // XCD-aware order: hardware workgroup b runs on XCD b % 8; each XCD
    // takes a contiguous slice of the logical order (g, s, query tile
    // descending, key chunk).
    const int64_t logical_c = (bid & 7) * a.wg_per_xcd + (bid >> 3);
    if (logical_c >= a.n_wg) return;
    chunk = (int)(logical_c % a.n_chunks);
    const int64_t logical = logical_c / a.n_chunks;
    const int per_g = a.S * a.q_tiles;
    g = (int)(logical / per_g);
    const int rem = (int)(logical % per_g);
    s = rem / a.q_tiles;
    qt = a.q_tiles - 1 - rem % a.q_tiles;
    const const_i32_ptr qsl = as_const(a.qsl);
    q0 = a.fixed_L >= 0 ? 0 : qsl[s];
    L = a.fixed_L >= 0 ? a.fixed_L : qsl[s + 1] - q0;
    n = a.fixed_L >= 0 ? a.fixed_n : as_const(a.cl)[s];
  }
  if (qt * kRows >= L) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hl = w % HG;  // head within the group
  const int rw = w / HG;  // which 16 of the workgroup's positions
  const int hq = g * HG + hl;
  const int r16 = lane & 15;
  const int g4 = lane >> 4;

  // This wave's rows: i = row0 + r16 (query index within the sequence).
  const int row0 = qt * kRows + rw * 16;
  const int my_i = row0 + r16;
  const bool row_ok = my_i < L;
  const int shift = n - L;  // absolute position of row i is shift + i

  // Keys the workgroup needs: [0, kend).
  int kend = n;
  if (a.causal) kend = min(n, shift + min(qt * kRows + kRows, L));
  const int ntk = (kend + kBN - 1) / kBN;
  // Per wave: tiles below `full` need no mask; tiles from `full` up to
  // `last` need one; later tiles hold no visible key for this wave.
  const bool wave_active = row0 < L;
  const int wave_last_i = min(row0 + 15, L - 1);
  const int vis_lo = a.causal ? shift + row0 : n - 1;         // first row's last key
  const int vis_hi = a.causal ? shift + wave_last_i : n - 1;  // last row's last key
  const int full = min(vis_lo + 1, n) / kBN;                  // fully visible tiles
  const int last = wave_active ? vis_hi / kBN : -1;
  const int my_vis = a.causal ? shift + my_i : n - 1;

  // Q^T as the MFMA B operand: lane (r16, g4) holds row r16, columns
  // 32*ks + 8*g4 .. +7.
  u32x4_t qf[kD / 32];
  {
    const uint8_t* qrow = a.q + (int64_t)(q0 + my_i) * a.q_st + (int64_t)hq * a.q_sh + g4 * 16;
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks) {
      qf[ks] = row_ok ? load16(qrow + ks * 64) : u32x4_t{0u, 0u, 0u, 0u};
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

  // Staging pieces.  K: one 16-byte chunk of key row kb + (lane >> 4) (four
  // keys per load instruction), stored as chunk c of the row-major tile.  V:
  // the same 16 bytes (8 columns) of two consecutive key rows, stored
  // transposed to fp16 (unit u: key pair u >> 4, columns (u & 15) * 8 ..).
  auto k_load = [&](int kt, int key_off) -> u32x4_t {
    const int kb = min(kt * kBN + key_off, kend_c);
    return load16(row_addr(kbase, kb) + k_lane);
  };
  auto k_store = [&](uint8_t* kl, int c, u32x4_t x) {
    *reinterpret_cast<u32x4_t*>(kl + (c >> 4) * kKRow + (c & 15) * 16) = x;
  };
  auto v_load = [&](int kt, int key_off, u32x4_t (&vr)[2]) {
    const int kb = min(kt * kBN + key_off, kend_c & ~7);
    const uint8_t* p = row_addr(vbase, kb) + v_lane;
    vr[0] = load16(p);
    vr[1] = load16(p + tok_stride);
  };
  // In the tile that reaches `kend`, V rows at or past it are zeroed first
  // (they may be clamped duplicates or unwritten slots; P is zero there, and
  // a zero row keeps the product finite).
  auto v_store = [&](int kt, uint8_t* vl, int u, u32x4_t (&vr)[2]) {
    if ((kt + 1) * kBN > kend) {
      const int key = kt * kBN + 2 * (u >> 4);
#pragma unroll
      for (int t = 0; t < 2; ++t)
        if (key + t >= kend) vr[t] = u32x4_t{0u, 0u, 0u, 0u};
    }
    const int pos = vt_pos(2 * (u >> 4));  // this key pair's place in a V^T row
    const int d0 = (u & 15) * 8;           // first of 8 columns
    // Rows d0 .. d0+7 share the swizzle (d0 >> 4) & 7.
    uint8_t* vp = vl + d0 * kVRow + (((pos >> 3) ^ ((d0 >> 4) & 7)) << 4) +
                  ((pos & 7) >> 1) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint32_t*>(vp + (2 * i) * kVRow) = pair_to_f16<T>(vr[0][i], vr[1][i], false);
      *reinterpret_cast<uint32_t*>(vp + (2 * i + 1) * kVRow) =
          pair_to_f16<T>(vr[0][i], vr[1][i], true);
    }
  };

  // O^T accumulators: acc_o[db][i] is column d = 16*db + 4*g4 + i of row r16.
  f32x4_t acc_o[kD / 16];
#pragma unroll
  for (int db = 0; db < kD / 16; ++db) acc_o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max of row r16, scaled (log2 units)
  float l_lane = 0.f;       // running sum of this lane's P values
  f32x4_t sc[4];            // S^T of the current tile: key kt*64 + 16*kb + 4*g4 + i
  u32x4_t pf[2];            // its P, as the B operands of the two 32-key steps

  f16x2_t ones;
  ones[0] = ones[1] = static_cast<_Float16>(1.f);
  // LDS fragment addresses.  K: row 16*kb + r16, bytes 64*ks + 16*g4.  V^T:
  // row d = 16*db + r16, chunk (4*s2 + g4) ^ (db & 7) = 4*(s2 ^ (db >> 2)) +
  // (g4 ^ (db & 3)), so a lane needs one base per value of db & 3.
  const int k_frag = r16 * kKRow + g4 * 16;
  int vt_frag[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) vt_frag[c] = r16 * kVRow + ((g4 ^ c) << 4);

  // S^T = K Q^T for tile kt (K in buffer kt & 1).
  auto qk_step = [&](int kt) {
    const uint8_t* kl = k_lds[kt & 1];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sc[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kD / 32; ++ks) {
        const u32x4_t kf =
            *reinterpret_cast<const u32x4_t*>(kl + k_frag + kb * 16 * kKRow + ks * 64);
        sc[kb] = mfma_qk<T>(kf, qf[ks], sc[kb]);
      }
    }
  };
  // Online-softmax update of row r16 over tile kt's 64 keys: sc -> pf.
  auto softmax_step = [&](int kt, auto mask_tag) {
    constexpr bool kMask = decltype(mask_tag)::value;
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (kMask) {
          const int key = kt * kBN + 16 * kb + 4 * g4 + i;
          if (key > my_vis) sc[kb][i] = -INFINITY;
        }
        tmax = fmaxf(tmax, sc[kb][i]);
      }
    tmax = row4_max(tmax);
    // Lazy rescale: raise the running max only when some row's new max is
    // more than kRescaleSlack above it (p = 2^(s*c - m) then stays < 2^8).
    const float m_cand = tmax * a.c;
    if (__builtin_amdgcn_ballot_w64(m_cand > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, m_cand);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_lane *= alpha;
#pragma unroll
      for (int db = 0; db < kD / 16; ++db) acc_o[db] *= alpha;
    }
    const float neg_m = -m_run;
    // P as the B operand of the two 32-key steps: step s2 holds keys
    // 32*s2 + {4*g4 + 0..3} (sc[2*s2]) then 32*s2 + 16 + {4*g4 + 0..3}
    // (sc[2*s2 + 1]).  Masked scores are -inf, so their P is 0.
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4_t& x = sc[2 * s2 + (j >> 1)];
        const float p0 = fast_exp2(fmaf(x[2 * (j & 1)], a.c, neg_m));
        const float p1 = fast_exp2(fmaf(x[2 * (j & 1) + 1], a.c, neg_m));
        const uint32_t pk = pack_f16(p0, p1);
        pf[s2][j] = pk;
        l_lane = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pk), ones, l_lane, false);
      }
  };
  auto softmax_tile = [&](int kt) {
    if (kt < full)
      softmax_step(kt, std::false_type{});
    else
      softmax_step(kt, std::true_type{});
  };
  // O^T += V^T P^T for tile kt (V^T in buffer kt & 1).
  auto pv_step = [&](int kt) {
    const uint8_t* vl = vt_lds[kt % kVBufs];
#pragma unroll
    for (int db = 0; db < kD / 16; ++db)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const u32x4_t vf = *reinterpret_cast<const u32x4_t*>(
            vl + vt_frag[db & 3] + db * 16 * kVRow + ((s2 ^ (db >> 2)) << 6));
        acc_o[db] = mfma_pv(vf, pf[s2], acc_o[db]);
      }
  };

  // This workgroup's tiles: [kt0, kt1) (all of [0, ntk) without chunking).
  const int kt0 = min(ntk, chunk * a.chunk_tiles);
  const int kt1 = min(ntk, kt0 + a.chunk_tiles);
  // One barrier per tile: after computing on tile kt a wave writes its part
  // of tile kt + 1 (fetched during step kt - 1) to the free buffers and
  // fetches tile kt + 2, which then has all of step kt + 1 to arrive.
  u32x4_t kreg[kKPer];
  u32x4_t vreg[kVPer][2];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int j = 0; j < kKPer; ++j) kreg[j] = k_load(kt, 4 * wu + j * (kNT / 16));
    if (kVAll || tid < kVUnits) {
#pragma unroll
      for (int j = 0; j < kVPer; ++j) v_load(kt, 8 * wu + j * (kNT / 8), vreg[j]);
    }
  };
  auto store_tile = [&](int kt) {
#pragma unroll
    for (int j = 0; j < kKPer; ++j) k_store(k_lds[kt & 1], tid + j * kNT, kreg[j]);
    if (kVAll || tid < kVUnits) {
#pragma unroll
      for (int j = 0; j < kVPer; ++j) v_store(kt, vt_lds[kt % kVBufs], tid + j * kNT, vreg[j]);
    }
  };
  if (kt0 < kt1) {
    load_tile(kt0);
    store_tile(kt0);
    if (kt0 + 1 < kt1) load_tile(kt0 + 1);
  }
  // With all waves leaving the barrier together, their QK^T, softmax and
  // P.V phases line up and the matrix cores idle during the softmax.  In
  // sixteen-wave workgroups two of the four waves on every SIMD therefore
  // run tile kt's P.V at the start of step kt + 1, beside the others'
  // QK^T, and their softmax beside the others' P.V (V^T then needs a third
  // buffer: tile kt - 1's is still read during step kt).  Measured: 1.5 %
  // faster on causal-bf16-prefill, same registers.
  const bool delayed = PrefillLds<HG, RW>::kDelayPV && ((w >> 2) & 1);
  for (int kt = kt0; kt < kt1; ++kt) {
    // Tile kt is in K buffer kt & 1 and V^T buffer kt % kVBufs; the buffers
    // of tile kt + 1 are free (tile kt - 1's K was last read in step
    // kt - 1, tile kt - 2's V^T in step kt - 1 at the latest; with two V^T
    // buffers, and no delayed P.V, tile kt - 1's V^T in step kt - 1).
    __syncthreads();
    if (delayed && kt > kt0 && kt - 1 <= last) pv_step(kt - 1);
    if (kt <= last) {
      qk_step(kt);
      softmax_tile(kt);
      if (!delayed) pv_step(kt);
    }
    if (kt + 1 < kt1) {
      store_tile(kt + 1);
      if (kt + 2 < kt1) load_tile(kt + 2);
    }
  }
  if (delayed && kt0 < kt1 && kt1 - 1 <= last) pv_step(kt1 - 1);

  const float l_tot = row4_sum(l_lane);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (a.part_o) {
    // Partial result of this key chunk: o / l and m + log2 l (log2 units of
    // the scaled scores; -inf when the chunk held no visible key), row by
    // row ([chunk][H][rows][d]; lane (r16, g4) holds columns 16*db + 4*g4 +
    // 0..3 of its row).  The merge happens in the next kernel on the
    // stream, after this one's writes are complete.
    if (!row_ok) return;
    const float lse = l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY;
    const int64_t prow = ((int64_t)chunk * a.H + hq) * a.part_rows + q0 + my_i;
    float* po = a.part_o + prow * kD + 4 * g4;
#pragma unroll
    for (int db = 0; db < kD / 16; ++db)
      *reinterpret_cast<f32x4_t*>(po + 16 * db) = acc_o[db] * inv;
    if (g4 == 0) a.part_lse[prow] = lse;
    return;
  }
  if (!row_ok) return;
  const int64_t obase = (int64_t)(q0 + my_i) * a.o_st + (int64_t)hq * a.o_sh + 4 * g4;
#pragma unroll
  for (int db = 0; db < kD / 16; ++db) {
    const f32x4_t o = acc_o[db] * inv;
    if (a.out_f32) {
      *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.out) + obase + 16 * db) = o;
    } else {
      uint16_t* op = static_cast<uint16_t*>(a.out) + obase + 16 * db;
      u32x2_t pk;
      if constexpr (__is_same(T, TBF16)) {
        pk[0] = (uint32_t)to_bf16_bits(o[0]) | ((uint32_t)to_bf16_bits(o[1]) << 16);
        pk[1] = (uint32_t)to_bf16_bits(o[2]) | ((uint32_t)to_bf16_bits(o[3]) << 16);
      } else {
        pk[0] = (uint32_t)to_f16_bits(o[0]) | ((uint32_t)to_f16_bits(o[1]) << 16);
        pk[1] = (uint32_t)to_f16_bits(o[2]) | ((uint32_t)to_f16_bits(o[3]) << 16);
      }
      *reinterpret_cast<u32x2_t*>(op) = pk;
    }
  }
}


// Kernel arguments of a planned prefill (host side).
inline PrefillArgs prefill_args(const PrefillPlan& pl) {
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
  const int64_t groups = (int64_t)pl.Hkv * a.kv_div;
  const int64_t ppx = (groups * pl.S + 7) / 8;
  a.packed_order = pl.fixed_L < 0 && pl.n_chunks == 1 && groups % 8 == 0 && ppx <= 64;
  if (a.packed_order) a.wg_per_xcd = ppx * pl.q_tiles;
  return a;
}

}  // namespace
}  // namespace pa
