// Device code of the decode partition kernel (included by decode.hip, and by
// shared_prefix.hip for the shared-prefix call's combined kernel).
//
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
// ceil(n_s / 16) tiles of 16 keys.  The units, KV-head major ((g, s)
// order), form one list in which a unit takes kUnitCost places for starting
// it (fetching Q, refilling the load pipeline, writing its result) and then
// one place per tile: `total` places.  The kernel launches W wavefronts
// ("workers", one workgroup of four per compute unit) and cuts each KV
// head's part of the list into W / Hkv equal slices (or, when Hkv does not
// divide W, the whole list into W equal slices), so every worker does about
// the same work whatever the mix of context lengths -- no tail of long
// partitions, no idle XCD; a worker that starts more units gets fewer
// tiles.  Slice j of every head covers the same sequences and tiles; two
// workers of one workgroup take slice j of two adjacent heads, so their
// waves read neighbouring 256-byte segments of the same token rows
// together.  Worker numbers are dealt so that each of the 8 XCDs (which
// receive workgroups round-robin) owns a contiguous run of them: with 8 KV
// heads an XCD serves one pair of heads over half of the sequences, and K/V
// blocks that several of those sequences share (a common prompt prefix)
// stay in its L2.
// The piece of a unit that one worker covers is a partition: a worker that
// covers a whole unit writes `out` directly; otherwise it writes a
// normalised partial output and its log2-sum-exp and counts itself in the
// unit's counter, and the worker that completes the count joins the
// partitions (log-sum-exp merge) and resets the counter to zero for the
// next call on the stream.  There is no second kernel.
//
// Per 16-key tile a worker:
//   * loads the K rows with the lane layout of the 16x16 MFMA B operand
//     (lane = key r16 and 16-byte column group c): every load instruction
//     reads 64 contiguous bytes of each of 16 rows (or, in the suffix step
//     after a shared prefix, whole rows like V, moved into that layout
//     through LDS);
//   * computes S = Q K^T on one MFMA chain; Q (the A operand) repeats the G
//     heads down its 16 rows, so every lane ends with the scores of its key
//     for all G heads (no transposes, no cross-lane traffic);
//   * does the online-softmax update with 16-lane DPP max reductions;
//   * loads the V rows with full-row coalescing (16 lanes x 16 bytes per
//     256-byte row) and accumulates p * v in fp32 on the VALU, reading the
//     probabilities of its key from a 256-byte per-wave LDS slot.
// Two register sets rotate: one tile's loads are in flight while the other
// tile is used.  (Three sets, two tiles in flight, measured slower once the
// slices account for unit starts: a shallower pipeline refills faster at a
// unit boundary, and 4 waves x 2 tiles x 8 KiB per CU still keep HBM busy.)
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace pa {
namespace {

#ifndef PA_DECODE_DEPTH
#define PA_DECODE_DEPTH 2
#endif
constexpr int kDecodeDepth = PA_DECODE_DEPTH;
#ifndef PA_DECODE_UNIT_COST
#define PA_DECODE_UNIT_COST 5
#endif
// What starting a unit costs a worker (its Q, the refilled load pipeline,
// the partial write-out), in 16-key tiles.  Slices are equal in tiles plus
// this cost per unit, so workers that cross many unit boundaries get fewer
// tiles.
constexpr int kUnitCost = PA_DECODE_UNIT_COST;

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
  float* part_o;    // [slots, G, D]
  float* part_lse;  // [slots, G] (log2 units)
  int* counters;    // [Hkv * S] finished partitions per unit (g-major); zero
                    // between calls
  int S, H, Hkv, W, bs_shift;
  // Pool layout: bytes between consecutive slots of a block, and between
  // KV heads (token-major: Hkv*d*e and d*e; head-major blocks: d*e and
  // B*d*e).  Blocks are Hkv*B*d*e bytes apart in both.
  uint32_t tok_bytes;
  int64_t head_bytes;
  float scale_log2;  // scale * log2(e)
  // Keys attended per sequence: [key_begin, n_s).  key_begin = 0 for plain
  // decode; the suffix step of a shared-prefix decode starts after the
  // prefix, whose keys another kernel attends.
  int key_begin;
  // Optional natural-log log-sum-exp per (s, query head): lse_out[s *
  // lse_ss + h], or nullptr.
  float* lse_out;
  int64_t lse_ss;
};

constexpr float kLn2 = 0.6931471805599453f;

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
// A unit's place in the work list: its tiles plus the start cost (none for
// a unit without keys).
__device__ __forceinline__ int cost_of(int n) { return n > 0 ? tiles_of(n) + kUnitCost : 0; }

// Partial results cross workgroups (and XCDs, whose L2 caches are not
// coherent with each other).  They are written and read at the coherent
// level (the sc1 bit) without flushing or invalidating the L2; a writer
// waits for its stores to complete before it counts its partition.  The
// log-sum-exp values use relaxed device-scope atomic accesses, which the
// compiler emits with sc1.
__device__ __forceinline__ void store_partial(float* p, float x) {
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The partial output rows use buffer instructions with sc1 set, so that one
// store instruction writes whole 16-byte pieces contiguous across lanes (a
// write-through store of 8-byte pieces at a 32-byte stride cost 3.4 times
// the DRAM writes).  kRawBuffer is the descriptor word of a raw (untyped,
// 32-bit element) buffer.
constexpr int kSc1 = 16;
constexpr int kRawBuffer = 0x00020000;
// Layout of one head's normalised partial row (D floats) in a slot: the
// kLPR lanes that hold the row own kE consecutive values each, and store j
// of lane i writes that lane's values 4j .. 4j+3 at row position
// j*4*kLPR + 4*i, so value d sits at position
//   ((d % kE) / 4) * 4 * kLPR + 4 * (d / kE) + d % 4.
template <int kE, int kLPR>
__device__ __forceinline__ int partial_pos(int d) {
  return ((d % kE) / 4) * 4 * kLPR + 4 * (d / kE) + d % 4;
}
template <int kE, int kLPR>
__device__ __forceinline__ void store_partial_row(float* row, int lane, const float* v,
                                                  float inv) {
  // `row` is the same for the whole wave; readfirstlane puts it in scalar
  // registers, as the descriptor needs.
  float* const row_u = reinterpret_cast<float*>(uniform_i64(reinterpret_cast<int64_t>(row)));
  const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(row_u, 0, kE * kLPR * 4, kRawBuffer);
#pragma unroll
  for (int j = 0; j < kE / 4; ++j) {
    const u32x4_t x = {__float_as_uint(v[4 * j] * inv), __float_as_uint(v[4 * j + 1] * inv),
                       __float_as_uint(v[4 * j + 2] * inv), __float_as_uint(v[4 * j + 3] * inv)};
    __builtin_amdgcn_raw_buffer_store_b128(x, rsrc, (j * 4 * kLPR + 4 * lane) * 4, 0, kSc1);
  }
}
// Values d0 .. d0+N-1 (original order, d0 a multiple of min(N, 4)) of a row
// stored by store_partial_row; `rsrc` covers the slot's G rows.
template <int N, int kE, int kLPR>
__device__ __forceinline__ void load_partial_vals(__amdgpu_buffer_rsrc_t rsrc, int row_off,
                                                  int d0, float* o) {
  if constexpr (N == 1) {
    o[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
        rsrc, (row_off + partial_pos<kE, kLPR>(d0)) * 4, 0, kSc1));
  } else if constexpr (N == 2) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b64(
        rsrc, (row_off + partial_pos<kE, kLPR>(d0)) * 4, 0, kSc1);
    o[0] = __uint_as_float(x[0]);
    o[1] = __uint_as_float(x[1]);
  } else {
    static_assert(N % 4 == 0, "whole 16-byte pieces");
#pragma unroll
    for (int m = 0; m < N; m += 4) {
      const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(
          rsrc, (row_off + partial_pos<kE, kLPR>(d0 + m)) * 4, 0, kSc1);
#pragma unroll
      for (int k = 0; k < 4; ++k) o[m + k] = __uint_as_float(x[k]);
    }
  }
}

__device__ __forceinline__ float load_partial(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Log-sum-exp merge of the np partitions of unit (g, s), held in slots
// slot0 .. slot0+np-1, by one wave:
//   out = sum_p 2^(lse_p - M) o_p / sum_p 2^(lse_p - M),  M = max_p lse_p,
// computed in one pass with a running maximum.  Lane l owns G*D/64
// consecutive values of the unit's [G][D] output.
template <class T, int D, int G>
__device__ __forceinline__ void merge_unit(const DecodeArgs& a, int g, int s, int64_t slot0,
                                           int np, int lane) {
  using Geo = DecodeGeom<T, D>;
  constexpr int kV = G * D / 64;
  static_assert(kV >= 1 && kV * 64 == G * D, "merge split");
  const int idx0 = lane * kV;
  const int h = idx0 / D, d0 = idx0 % D;
  auto slot_rsrc = [&](int64_t slot) {
    float* const base = a.part_o + uniform_i64(slot) * G * D;
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, G * D * 4, kRawBuffer);
  };
  float M = -INFINITY, wsum = 0.f, acc[kV];
#pragma unroll
  for (int e = 0; e < kV; ++e) acc[e] = 0.f;
  auto add = [&](float lse, const float* o) {
    if (lse == -INFINITY) return;  // a part with no keys
    const float mn = fmaxf(M, lse);
    const float sa = fast_exp2(M - mn), sb = fast_exp2(lse - mn);
    wsum = fmaf(wsum, sa, sb);
#pragma unroll
    for (int e = 0; e < kV; ++e) acc[e] = fmaf(acc[e], sa, sb * o[e]);
    M = mn;
  };
  constexpr int kU = 4;  // partitions whose loads are in flight together
  int p = 0;
  for (; p + kU <= np; p += kU) {
    float lse[kU], o[kU][kV];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t slot = slot0 + p + u;
      lse[u] = load_partial(a.part_lse + slot * G + h);
      load_partial_vals<kV, Geo::kE, Geo::kLPR>(slot_rsrc(slot), h * D, d0, o[u]);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) add(lse[u], o[u]);
  }
  for (; p < np; ++p) {
    const int64_t slot = slot0 + p;
    float lse, o[kV];
    lse = load_partial(a.part_lse + slot * G + h);
    load_partial_vals<kV, Geo::kE, Geo::kLPR>(slot_rsrc(slot), h * D, d0, o);
    add(lse, o);
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if (a.lse_out && d0 == 0)
    a.lse_out[(int64_t)s * a.lse_ss + g * G + h] = wsum > 0.f ? (M + __log2f(wsum)) * kLn2
                                                              : -INFINITY;
  const int64_t ob = (int64_t)s * a.o_ss + (int64_t)(g * G + h) * a.o_sh + d0;
#pragma unroll
  for (int e = 0; e < kV; ++e) store_out<T>(a.out, ob + e, acc[e] * inv, a.out_f32 != 0);
}

// Units with no key to attend here are in no worker's slice: their output
// is zero (and their log-sum-exp -inf).  Worker i writes units i, i + W, ...
// (after its own slice, so that the check is off the path to the first K/V
// loads).
template <class T, int D, int G>
__device__ __forceinline__ void zero_empty_units(const DecodeArgs& a, int worker, int lane) {
  for (int u = worker; u < a.S * a.Hkv; u += a.W) {
    const int su = u % a.S, gu = u / a.S;
    if (as_const(a.cl)[su] <= a.key_begin) {
      for (int i = lane; i < G * D; i += 64)
        store_out<T>(a.out, (int64_t)su * a.o_ss + (int64_t)(gu * G + i / D) * a.o_sh + i % D,
                     0.f, a.out_f32 != 0);
      if (a.lse_out && lane < G) a.lse_out[(int64_t)su * a.lse_ss + gu * G + lane] = -INFINITY;
    }
  }
}

// kKRows selects how K is read.  false: in the MFMA operand layout, 64
// bytes of 16 rows per load instruction, with normal caching.  true: whole
// rows per instruction like V, non-temporal, then moved into the operand
// layout through this wave's LDS slot (used for the suffix step after a
// shared prefix, where it measured faster; plain decode measured slower
// with it).
// LDS of one decode workgroup (per wave: the probabilities of a tile, Q of
// its heads, and with kKRows the K tile in the operand layout, rows padded
// by 16 bytes so that the 16 rows one read instruction covers start on
// different banks).
template <class T, int D, int G, bool kKRows>
struct DecodeLds {
  using Geo = DecodeGeom<T, D>;
  static constexpr int kPG = G > 4 ? G : 4;
  static constexpr int kKPad = Geo::kRowBytes + 16;
  static constexpr int kPBytes = kDecodeWaves * kTileKeys * kPG * 4;
  static constexpr int kQBytes = kDecodeWaves * G * Geo::kRowBytes;
  static constexpr int kKBytes = kKRows ? kTileKeys * kKPad : 16;
  static constexpr int kBytes = kPBytes + kQBytes + kDecodeWaves * kKBytes;
  static_assert(kPBytes % 16 == 0 && kQBytes % 16 == 0, "16-byte aligned parts");
};

// The decode workgroup `group` of `groups` (a multiple of 8; hardware
// workgroup b runs on XCD b % 8, and groups map to logical numbers that give
// each XCD a contiguous run of workers), with its LDS at `lds` (16-byte
// aligned, DecodeLds::kBytes).  Called by every thread of the workgroup.
template <class T, int D, int G, bool kKRows>
__device__ __forceinline__ void decode_body(const DecodeArgs& a, int group, int groups,
                                            uint8_t* lds) {
  using Geo = DecodeGeom<T, D>;
  using Lds = DecodeLds<T, D, G, kKRows>;
  constexpr int kDepth = kDecodeDepth;  // tiles whose loads are in flight per wave
  constexpr int kNW = kDecodeWaves;
  constexpr int kE = Geo::kE;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int logical = (group & 7) * (groups >> 3) + (group >> 3);
  const int worker = logical * kNW + w;
  if (worker >= a.W) return;

  auto p_lds = reinterpret_cast<float (*)[kTileKeys][Lds::kPG]>(lds);
  auto q_lds = reinterpret_cast<uint8_t (*)[G * Geo::kRowBytes]>(lds + Lds::kPBytes);
  auto k_lds = reinterpret_cast<uint8_t (*)[Lds::kKBytes]>(lds + Lds::kPBytes + Lds::kQBytes);
  constexpr int kKPad = Lds::kKPad;

  // ---- this worker's slice of the global tile list ----
  // Tiles per KV head over all sequences (the list is g-major).  With at
  // most 64 sequences one load of the lengths serves both passes.
  // Keys this kernel attends per sequence: n_s - key_begin.
  const int lane_len = lane < a.S ? max(as_const(a.cl)[lane] - a.key_begin, 0) : 0;
  const int lane_cost = cost_of(lane_len);
  int64_t t_all = wave_sum_i64(lane_cost);
  for (int c0 = 64; c0 < a.S; c0 += 64) {
    const int s = c0 + lane;
    t_all += wave_sum_i64(
        s < a.S ? (int64_t)cost_of(max(as_const(a.cl)[s] - a.key_begin, 0)) : 0);
  }
  // Positions below are in cost units: a unit occupies its start cost, then
  // one unit per tile.
  const int64_t total = t_all * a.Hkv;
  // When W is a multiple of Hkv, each KV head's sublist is cut into
  // wh = W / Hkv equal slices, so that slice j of every head covers the same
  // (sequence, tile) range.  Workers are dealt in pairs over adjacent heads
  // (worker 2i and 2i+1: slice j of heads 2p and 2p+1), so the two waves
  // read adjacent 256-byte head segments of the same token rows at about the
  // same time; consecutive pairs take consecutive j.  Slice number sl (which
  // names the partial-result slots) is head * wh + j.  Measured against one
  // head per run of workers: gqa-f16-decode 97.3 -> 91.9 us,
  // long-bf16-decode 273.5 -> 255 us (groups of all 8 heads per pair of
  // workgroups measured the same on those and lost more of the L2 reuse of
  // blocks shared between sequences).  With W not a multiple of Hkv, or an
  // odd Hkv, the list is cut into W equal slices in worker order.
  const bool aligned = a.W % a.Hkv == 0;
  const int wh = aligned ? a.W / a.Hkv : a.W;
  const int64_t per = aligned ? (t_all + wh - 1) / wh : (total + a.W - 1) / a.W;
  const int pair = a.Hkv % 2 == 0 ? 2 : 1;
  const int gw = (worker / (pair * wh)) * pair + worker % pair;  // this worker's head
  const int sl = aligned ? gw * wh + (worker / pair) % wh : worker;
  const int64_t hbase = aligned ? (int64_t)gw * t_all : 0;
  const int64_t hend = aligned ? hbase + t_all : total;
  const int64_t begin = aligned ? min(hend, hbase + (int64_t)(sl % wh) * per)
                                : (int64_t)worker * per;
  const int64_t end = min(hend, begin + per);
  if (begin >= end) {
    zero_empty_units<T, D, G>(a, worker, lane);
    return;
  }

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
          c0 == 0 ? lane_cost
                  : (ss < a.S ? (int64_t)cost_of(max(as_const(a.cl)[ss] - a.key_begin, 0)) : 0);
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
  const uint32_t tok_stride = a.tok_bytes;  // bytes between slots
  const int64_t blk_stride = ((int64_t)a.Hkv * Geo::kRowBytes) << a.bs_shift;
  const int v_row = lane / Geo::kLPR;
  const uint32_t k_off = (uint32_t)r16 * tok_stride + c * 16;
  const uint32_t v_off = (uint32_t)v_row * tok_stride + (lane % Geo::kLPR) * 16;
  uint8_t* my_q = q_lds[w];
  // Q as the MFMA A operand: its 16 rows repeat the heads of a chain.  Up to
  // 4 heads fit one 16x16 product (a lane's 4 results are heads 0..3); a
  // group of 8 takes two chains (heads 0..3 and 4..7) on the same K.
  constexpr int kChains = (G + 3) / 4;
  constexpr int kHC = G / kChains;  // heads per chain
  const uint8_t* q_frag = my_q + (r16 % kHC) * Geo::kRowBytes + c * 16;

  int64_t t = begin;
  while (t < end) {
    // Unit (g, s) starting at list position unit_first (its start cost,
    // then its tiles from tile0 on); t lies in or after it.
    // (readfirstlane marks the loop state wave-uniform for the compiler, so
    // table and length reads below become scalar loads.)
    s = uniform_i(s);
    g = uniform_i(g);
    // With at most 64 sequences every length is already in a register.
    const int n = a.S <= 64 ? __builtin_amdgcn_readlane(lane_len, s)
                            : max(as_const(a.cl)[s] - a.key_begin, 0);
    const int ts = tiles_of(n);
    const int64_t unit_len = cost_of(n);
    if (t >= unit_first + unit_len) {  // empty or finished unit: next sequence / head
      unit_first += unit_len;
      if (++s == a.S) {
        s = 0;
        ++g;
      }
      continue;
    }
    const int64_t tile0 = unit_first + kUnitCost;  // list position of tile 0
    if (tile0 >= end) break;  // the rest of this slice is the unit's start cost
    const int j0 = uniform_i((int)(max(t, tile0) - tile0));
    const int j1 = uniform_i((int)min((int64_t)ts, end - tile0));
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
    const uint8_t* kbase = a.k + (int64_t)g * a.head_bytes;
    const uint8_t* vbase = a.v + (int64_t)g * a.head_bytes;

    float m[G], l_lane[G], acc[G][kE];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
      l_lane[h] = 0.f;
#pragma unroll
      for (int e = 0; e < kE; ++e) acc[h][e] = 0.f;
    }
    static_assert(Geo::kKLoads == Geo::kVLoads, "a K row and a V row take the same loads");
    u32x4_t kr[kDepth][Geo::kKLoads], vr[kDepth][Geo::kVLoads];

    auto load_tile = [&](int k, u32x4_t* kd, u32x4_t* vd) {
      const int key0 = uniform_i(a.key_begin + (j0 + min(k, ntile - 1)) * kTileKeys);
      const int phys = bt_row[key0 >> a.bs_shift];
      const int64_t row0 = (int64_t)phys * blk_stride + (int64_t)(key0 & bmask) * tok_stride;
      const uint8_t* kb = kbase + row0;
      const uint8_t* vb = vbase + row0;
      if constexpr (kKRows) {
#pragma unroll
        for (int i = 0; i < Geo::kVLoads; ++i)
          kd[i] = load16_stream(kb + (int64_t)(i * Geo::kRPI) * tok_stride + v_off);
      } else {
#pragma unroll
        for (int i = 0; i < Geo::kKLoads; ++i) kd[i] = load16(kb + k_off + i * 64);
      }
      // V rows are read whole by one instruction each: non-temporal, so
      // streaming V does not push reusable lines out of the caches.  K rows
      // in the operand layout are read 64 bytes at a time by four
      // instructions, and the second half of each 128-byte line must still be
      // in L2 when it is needed, so they keep normal caching.
#pragma unroll
      for (int i = 0; i < Geo::kVLoads; ++i)
        vd[i] = load16_stream(vb + (int64_t)(i * Geo::kRPI) * tok_stride + v_off);
    };

    auto compute_tile = [&](int k, const u32x4_t* kf, const u32x4_t* vf) {
      const int valid = n - (j0 + k) * kTileKeys;  // keys of this tile below n (>= 1)
      u32x4_t kq[Geo::kKLoads];
      if constexpr (kKRows) {
        // Whole rows -> LDS -> operand layout (row r16, bytes i*64 + c*16).
        uint8_t* kl = k_lds[w];
#pragma unroll
        for (int i = 0; i < Geo::kVLoads; ++i)
          *reinterpret_cast<u32x4_t*>(kl + (i * Geo::kRPI + v_row) * kKPad +
                                      (lane % Geo::kLPR) * 16) = kf[i];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < Geo::kKLoads; ++i)
          kq[i] = *reinterpret_cast<const u32x4_t*>(kl + r16 * kKPad + i * 64 + c * 16);
      } else {
#pragma unroll
        for (int i = 0; i < Geo::kKLoads; ++i) kq[i] = kf[i];
      }
      f32x4_t sc[kChains];
#pragma unroll
      for (int ch = 0; ch < kChains; ++ch) {
        u32x4_t qf[Geo::kKLoads];
#pragma unroll
        for (int i = 0; i < Geo::kKLoads; ++i)
          qf[i] = *reinterpret_cast<const u32x4_t*>(q_frag + ch * kHC * Geo::kRowBytes + i * 64);
        sc[ch] = qk_tile<T, D>(qf, kq);
      }
      const bool key_ok = r16 < valid;
      float x[G], pr[G], mnew[G];
      bool grow = false;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        // Slots at or past n are selected away (they may hold NaN).
        x[h] = key_ok ? sc[h / kHC][h % kHC] * a.scale_log2 : -INFINITY;
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

    // kDepth-way rotation over this partition's tiles: the steady-state loop
    // issues one tile's loads per computed tile (fixed waits); an epilogue
    // finishes the last 1 .. 2*kDepth-1 tiles without loading past the end.
    // The first loads are clamped to the last tile of a short partition.
#pragma unroll
    for (int i = 0; i < kDepth; ++i) load_tile(i, kr[i], vr[i]);
#pragma unroll
    for (int j = 0; j < kQPer; ++j)
      if (lane + 64 * j < kQChunks) *reinterpret_cast<u32x4_t*>(my_q + (lane + 64 * j) * 16) = qreg[j];
    __builtin_amdgcn_wave_barrier();
    int k = 0;
    for (; k + 2 * kDepth - 1 < ntile; k += kDepth) {
#pragma unroll
      for (int i = 0; i < kDepth; ++i) {
        compute_tile(k + i, kr[i], vr[i]);
        load_tile(k + kDepth + i, kr[i], vr[i]);
      }
    }
    const int rest = ntile - k;  // 1 .. 2*kDepth-1; set i holds tile k + i
#pragma unroll
    for (int i = 0; i < kDepth; ++i) {
      if (i < rest) compute_tile(k + i, kr[i], vr[i]);
      if (kDepth + i < rest) load_tile(k + kDepth + i, kr[i], vr[i]);
    }
#pragma unroll
    for (int i = 0; i < kDepth - 1; ++i)
      if (kDepth + i < rest) compute_tile(k + kDepth + i, kr[i], vr[i]);

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
        if (whole) {
#pragma unroll
          for (int e = 0; e < kE; ++e)
            store_out<T>(a.out, (int64_t)s * a.o_ss + (int64_t)(hq0 + h) * a.o_sh + lane * kE + e,
                         acc[h][e] * inv, a.out_f32 != 0);
        } else {
          store_partial_row<kE, Geo::kLPR>(a.part_o + ((int64_t)(sl + u) * G + h) * D, lane,
                                           acc[h], inv);
        }
      }
    }
    if (whole && a.lse_out && lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h)
        a.lse_out[(int64_t)s * a.lse_ss + hq0 + h] = (m[h] + __log2f(l_lane[h])) * kLn2;
    }
    if (!whole) {
      if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
          store_partial(a.part_lse + (int64_t)(sl + u) * G + h, m[h] + __log2f(l_lane[h]));
      }
      // Slices first .. last hold the unit's partitions (slots first + u ..).
      const int64_t h0 = aligned ? (int64_t)g * t_all : 0;  // this head's sublist start
      const int sl0 = aligned ? g * wh : 0;
      const int first = sl0 + (int)((tile0 - h0) / per);
      const int last = sl0 + (int)((tile0 + ts - 1 - h0) / per);
      // Once this wave's partial stores have completed, count the partition;
      // the worker that brings the count to the number of partitions merges
      // them and leaves the counter at zero.
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      int done = 0;
      if (lane == 0) done = __hip_atomic_fetch_add(a.counters + u, 1, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      done = __builtin_amdgcn_readfirstlane(done);
      if (done == last - first) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        merge_unit<T, D, G>(a, g, s, (int64_t)first + u, last - first + 1, lane);
        if (lane == 0)
          __hip_atomic_store(a.counters + u, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    t = tile0 + j1;
  }
  zero_empty_units<T, D, G>(a, worker, lane);
}

// Kernel arguments of a planned decode whose workspace is `workspace`
// (host side).
inline DecodeArgs decode_args(const DecodePlan& pl, void* workspace) {
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
  // Workspace: counters [S*Hkv] int32 (padded to 256 bytes) | part_o | part_lse.
  a.counters = static_cast<int*>(workspace);
  a.part_o = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + pl.counter_bytes);
  a.part_lse = a.part_o + pl.slots * pl.G * pl.D;
  a.S = pl.S;
  a.H = pl.H;
  a.Hkv = pl.Hkv;
  a.W = pl.workers;
  a.bs_shift = __builtin_ctz(pl.B);
  a.tok_bytes = (uint32_t)(pl.pool.tok * e);
  a.head_bytes = pl.pool.head * e;
  a.scale_log2 = pl.scale * 1.4426950408889634f;
  a.key_begin = pl.key_begin;
  a.lse_out = pl.lse;
  a.lse_ss = pl.lse_ss;
  return a;
}

}  // namespace
}  // namespace pa
