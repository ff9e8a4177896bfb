// Host-side validation and launch planning for the paged-attention kernels.
//
// Pure C++: no HIP headers, no device access.  Every check here uses host
// shapes only, so a call that fails validation issues no GPU work.
#pragma once

#include <stdint.h>

#include <string>

#include "../../include/pa.h"

namespace pa {

// Decode geometry.  The decode kernel runs a fixed set of "workers" (one
// wavefront each, kDecodeWaves per workgroup); all (sequence, KV head)
// units' 16-key tiles form one list that is cut into equal contiguous
// slices, one per worker.  A worker's piece of one unit is a partition;
// the last worker to finish a split unit joins its partitions.
constexpr int kDecodeWaves = 4;

// Element strides of a pool's token and KV-head dimensions.  Pools are
// logically [NB, B, Hkv, d] in one of two layouts (the same for K and V):
//   token-major: fully contiguous, a token's Hkv rows adjacent (tok = Hkv*d,
//     head = d);
//   head-major within each block: strides (B*Hkv*d, d, B*d, 1), i.e. a
//     contiguous [NB, Hkv, B, d] buffer, a head's B rows adjacent (tok = d,
//     head = B*d).
struct PoolLayout {
  int64_t tok = 0;
  int64_t head = 0;
};
constexpr int kTileKeys = 16;
constexpr int kMaxWorkers = 1 << 20;

struct DecodePlan {
  int dtype = 0;      // pa_dtype of q / pools
  int out_dtype = 0;  // PA_F32 or dtype
  int S = 0, H = 0, Hkv = 0, G = 0, D = 0, B = 0, MB = 0;
  int64_t NB = 0;
  PoolLayout pool;
  int workers = 0;       // wavefronts launched
  int64_t slots = 0;     // partial-result slots: workers + S * Hkv
  int64_t grid[3] = {0, 0, 0};
  int block_threads = 0;
  int64_t counter_bytes = 0;  // per-unit counters at the start of the workspace
  int64_t ws_bytes = 0;       // counters, partial outputs and log-sum-exp
  // operands
  const void* q = nullptr;
  int64_t q_ss = 0, q_sh = 0;  // strides (elements) over sequence and head
  const void* k = nullptr;
  const void* v = nullptr;
  const int32_t* bt = nullptr;
  int64_t bt_ss = 0;
  const int32_t* cl = nullptr;
  void* out = nullptr;
  int64_t o_ss = 0, o_sh = 0;
  float scale = 0.f;
  // Keys attended per sequence: [key_begin, n_s) (the suffix step of
  // pa_decode_shared_prefix starts after the prefix; 0 otherwise).
  int key_begin = 0;
  // Optional natural-log log-sum-exp of each (sequence, query head),
  // lse[s * lse_ss + h] (pa_decode_lse).
  float* lse = nullptr;
  int64_t lse_ss = 0;
};

// pa_decode_noalloc runs on a fixed device array of kNoAllocScratchBytes per
// GPU instead of an allocated workspace.  Its first kNoAllocCounterBytes
// hold the per-unit counters of at most kNoAllocMaxUnits (sequence, KV head)
// pairs -- a region that never holds anything else, so the counters, which
// the kernel leaves at zero, stay zero between calls of any size -- and the
// partial results follow.
constexpr int64_t kNoAllocScratchBytes = (int64_t)32 << 20;
constexpr int64_t kNoAllocMaxUnits = (int64_t)1 << 16;
constexpr int64_t kNoAllocCounterBytes = kNoAllocMaxUnits * 4;

// Prefill workgroups: each wave owns 16 query positions of one head; a
// workgroup holds min(G, 4) heads of one KV head and row_waves waves per
// head.  Packed prompts use kPrefillWaves waves per workgroup (one workgroup
// per compute unit, four waves per SIMD), the shared-prefix step
// kPrefixStepWaves.
constexpr int kPrefillWaveRows = 16;
constexpr int kPrefillWaves = 16;
constexpr int kPrefixStepWaves = 4;

struct PrefillPlan {
  int dtype = 0, out_dtype = 0;
  int S = 0, T = 0, H = 0, Hkv = 0, G = 0, D = 0, B = 0, MB = 0;
  int64_t NB = 0;
  PoolLayout pool;
  int max_query_len = 0;
  int causal = 0;
  int row_waves = 0;  // waves per head: 16 * row_waves query rows per workgroup
  int q_tiles = 0;    // ceil(max_query_len / (16 * row_waves))
  int64_t grid[3] = {0, 0, 0};
  int block_threads = 0;
  const void* q = nullptr;
  int64_t q_st = 0, q_sh = 0;
  const void* k = nullptr;
  const void* v = nullptr;
  const int32_t* bt = nullptr;
  int64_t bt_ss = 0;
  const int32_t* cl = nullptr;
  const int32_t* qsl = nullptr;
  void* out = nullptr;
  int64_t o_st = 0, o_sh = 0;
  float scale = 0.f;
  // Shared-prefix attention (decode with a common prefix): one sequence given
  // by value and key chunks writing partial results, merged by the join
  // kernel; see prefill_kernel.h and shared_prefix.hip.
  int fixed_L = -1, fixed_n = 0;
  int n_chunks = 1, chunk_tiles = 1 << 30;
  int64_t part_rows = 0;
  float* part_o = nullptr;
  float* part_lse = nullptr;
};

// Most key chunks the shared-prefix step splits its keys into (the join
// kernel merges them keeping every chunk's part in registers).
constexpr int kMaxPrefixChunks = 4;

struct WriteKvPlan {
  int dtype = 0;
  int64_t N = 0, NB = 0;
  int B = 0, Hkv = 0, D = 0;
  PoolLayout pool;
  const void* kn = nullptr;
  const void* vn = nullptr;
  int64_t kn_s = 0, kn_h = 0, vn_s = 0, vn_h = 0;
  const int32_t* slots = nullptr;
  void* kp = nullptr;
  void* vp = nullptr;
};

// Merge of P partial attention states (pa_merge_states).
struct MergePlan {
  int P = 0, S = 0, H = 0, D = 0;
  const float* part_out = nullptr;  // [P, S, H, D], strides in elements
  int64_t po_p = 0, po_s = 0, po_h = 0;
  const float* part_lse = nullptr;  // [P, S, H]
  int64_t pl_p = 0, pl_s = 0, pl_h = 0;
  void* out = nullptr;              // [S, H, D]
  int out_dtype = 0;
  int64_t o_s = 0, o_h = 0;
  float* lse = nullptr;             // optional [S, H]
  int64_t l_s = 0, l_h = 0;
};

// Last step of pa_decode_shared_prefix: the prefix's key chunks
// (pre_o [n_pre, H, S, D], log2-sum-exp pre_lse [n_pre, H, S]) joined with
// the suffix step's state (suf_o [S, H, D] normalised, natural-log
// suf_lse [S, H]) into out.
struct PrefixJoinPlan {
  int S = 0, H = 0, D = 0, n_pre = 0;
  const float* pre_o = nullptr;
  const float* pre_lse = nullptr;
  const float* suf_o = nullptr;
  const float* suf_lse = nullptr;
  void* out = nullptr;
  int out_dtype = 0;
  int64_t o_ss = 0, o_sh = 0;
};

struct CopyBlocksPlan {
  int64_t N = 0;           // block pairs
  int64_t block_bytes = 0; // bytes of one block in one pool
  const int32_t* src = nullptr;
  const int32_t* dst = nullptr;
  void* kp = nullptr;
  void* vp = nullptr;
};

// Validates the decode arguments and sizes the launch for `workers`
// wavefronts (the device's resident capacity, or an override).
int plan_decode(const pa_tensor* q, const pa_tensor* k_pool, const pa_tensor* v_pool,
                const pa_tensor* block_table, const pa_tensor* context_lens, float scale,
                const pa_tensor* out, int workers, DecodePlan* plan, std::string* err);

int plan_prefill(const pa_tensor* q, const pa_tensor* k_pool, const pa_tensor* v_pool,
                 const pa_tensor* block_table, const pa_tensor* context_lens,
                 const pa_tensor* query_start_loc, int32_t max_query_len, float scale,
                 int32_t causal, const pa_tensor* out, PrefillPlan* plan, std::string* err);

int plan_write_kv(const pa_tensor* k_new, const pa_tensor* v_new,
                  const pa_tensor* slot_mapping, const pa_tensor* k_pool,
                  const pa_tensor* v_pool, WriteKvPlan* plan, std::string* err);

// Checks the optional log-sum-exp output of pa_decode_lse: f32 [S, H],
// not overlapping q, the pools or out.
int plan_decode_lse(const pa_tensor* lse, const pa_tensor* q, const pa_tensor* k_pool,
                    const pa_tensor* v_pool, const pa_tensor* out, DecodePlan* plan,
                    std::string* err);

int plan_merge(const pa_tensor* part_out, const pa_tensor* part_lse, const pa_tensor* out,
               const pa_tensor* lse, MergePlan* plan, std::string* err);

int plan_copy_blocks(const pa_tensor* k_pool, const pa_tensor* v_pool, const pa_tensor* src,
                     const pa_tensor* dst, CopyBlocksPlan* plan, std::string* err);

// Reads PA_DECODE_WORKERS (1 .. kMaxWorkers); 0 when unset, -1 when invalid.
int workers_override_from_env();

}  // namespace pa
