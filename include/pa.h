/*
 * pa.h -- paged-KV-cache attention on AMD MI355X (gfx950): the C ABI.
 *
 * What the library computes (cited by page title and section):
 *
 *   Exact attention softmax(q K^T * scale) V for every query row
 *   ("FlashAttention and PagedAttention: two fixes for two different
 *   bottlenecks", section "Why attention is expensive"), where the keys and
 *   values of each sequence are stored in fixed-size blocks of a shared pool
 *   and found through a per-sequence block table that maps logical blocks to
 *   physical ones (same page, "PagedAttention - How it works"; "Flash
 *   Attention vs Paged Attention", "Paged Attention: memory blocking",
 *   eq. (4)).  The kernels never build the score matrix: they stream K/V
 *   tiles and keep a running maximum and running sum per row (the online
 *   softmax of "FlashAttention - How it works"), which reaches the same
 *   result as the plain definition up to floating-point rounding.
 *
 * Conventions shared by every entry point:
 *
 *   - Every tensor is described by a pa_tensor: a device pointer, a dtype,
 *     a rank and per-dimension sizes and strides (strides in elements).
 *     The caller owns all memory; the library keeps no pointer after a call
 *     returns.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL means the
 *     default stream).  PA_OK means "validated and launched"; faults caused
 *     by bad device-side contents (see each call's contract) surface at the
 *     caller's next synchronisation, not as a status.
 *   - Every argument that can be checked on the host is checked before any
 *     GPU work is issued; on failure nothing is launched, a negative
 *     pa_status is returned and pa_last_error() describes the problem.
 *   - Layouts (names follow the pages' domain; S sequences, H query heads,
 *     Hkv KV heads, G = H / Hkv, d head size, B block size, NB pool blocks,
 *     MB table width, T packed query rows):
 *       k_pool, v_pool   [NB, B, Hkv, d]  the same layout for both, one of:
 *                        - token-major: fully contiguous (a token's Hkv
 *                          rows adjacent);
 *                        - head-major within each block: element strides
 *                          (B*Hkv*d, d, B*d, 1), i.e. a contiguous
 *                          [NB, Hkv, B, d] buffer viewed as [NB, B, Hkv, d]
 *                          (a KV head's B rows of a block adjacent).  On
 *                          MI355X decode reads this layout faster: a head's
 *                          rows then span all low address bits instead of
 *                          one 256-byte column of every 2 KiB token row.
 *                        Other strides return PA_ERR_STRIDE.
 *       block_table      int32 [S, MB]    last dim contiguous
 *       context_lens     int32 [S]        contiguous; n_s = keys of sequence s
 *     Logical token t of sequence s lives in physical block
 *     block_table[s][t / B], slot t % B.  Query head h reads KV head h / G.
 *   - Supported instances: dtype f32, f16 or bf16 (prefill: f16, bf16);
 *     d in {64, 128} (prefill: 128); B in {16, 32, 64, 128}; G in {1, 2, 4, 8}.
 *     Other shapes return PA_ERR_UNSUPPORTED.
 *   - Device-side contents the host cannot check without a synchronisation
 *     are the caller's contract: 0 <= n_s <= MB * B; block_table[s][j] in
 *     [0, NB) for j < ceil(n_s / B).  Entries at j >= ceil(n_s / B) and pool
 *     slots at or past n_s are never used (they may hold anything, NaN
 *     included).
 *   - Graph capture: pa_decode, pa_decode_shared_prefix, pa_prefill,
 *     pa_write_kv and pa_copy_blocks issue only kernel launches once a
 *     decode call's workspace exists, so they can be captured into a HIP
 *     graph and replayed (a replay reads the buffers' contents at replay
 *     time).  A decode call that would have to grow its stream's workspace
 *     during a capture returns PA_ERR_ALLOC instead: make one call of the
 *     same (or larger) size on that stream before capturing.  A graph uses
 *     the workspace of the stream it was captured on: a later call that
 *     grows that workspace keeps the captured buffer alive (it is freed by
 *     pa_workspace_release, which therefore invalidates such graphs), and
 *     a replay must not overlap another call that uses the same workspace
 *     (an eager decode on the capture stream, or a replay of another graph
 *     captured on it).  Dispatches recorded into a graph are not timed by
 *     the profiler.
 */
#ifndef PA_H_
#define PA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_dtype {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2,
  PA_I32 = 3
} pa_dtype;

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required tensor or data pointer is NULL      */
  PA_ERR_DTYPE = -2,       /* a dtype is not allowed for that argument       */
  PA_ERR_SHAPE = -3,       /* ranks or sizes are inconsistent                */
  PA_ERR_STRIDE = -4,      /* a layout/alignment requirement is not met      */
  PA_ERR_UNSUPPORTED = -5, /* valid, but no compiled instance for it         */
  PA_ERR_ALLOC = -6,       /* workspace allocation failed                    */
  PA_ERR_LAUNCH = -7,      /* the HIP runtime refused a launch or call       */
  PA_ERR_ARG = -8          /* a scalar argument is out of range              */
} pa_status;

typedef struct pa_tensor {
  void* data;        /* device pointer (host pointer never accepted)        */
  int32_t dtype;     /* pa_dtype                                            */
  int32_t ndim;      /* 1..4                                                */
  int64_t shape[4];  /* sizes; entries past ndim are ignored                */
  int64_t stride[4]; /* strides in elements; entries past ndim are ignored  */
} pa_tensor;

/*
 * pa_decode -- one query token per sequence attends to its paged KV cache.
 *
 * Defines: out[s][h] = sum_t p_t v_t with p = softmax_t(scale * q[s][h] . k_t)
 * over the n_s logical tokens t of sequence s, k_t / v_t read through the
 * block table (block-wise form: "Flash Attention vs Paged Attention",
 * eq. (4); gathering through the table: "How PagedAttention and
 * RadixAttention optimise KV-cache handling", "How PagedAttention works").
 *
 *   q            [S, H, d]   dtype f32/f16/bf16; last dim contiguous;
 *                            16-byte aligned rows
 *   k_pool       [NB, B, Hkv, d]  same dtype as q
 *   v_pool       same shape and dtype as k_pool
 *   block_table  int32 [S, MB]
 *   context_lens int32 [S]   n_s >= 0 (n_s = 0 gives a zero output row)
 *   scale        finite float (1/sqrt(d) for standard attention)
 *   out          [S, H, d]   dtype f32 or q's dtype; last dim contiguous;
 *                            must not alias any input
 *   stream       hipStream_t or NULL
 *
 * Work is balanced over a fixed set of W wavefronts (one workgroup of four
 * per compute unit, W = 1024 on an MI355X): the 16-key tiles of all
 * (sequence, KV head) pairs form one list, in which each pair also counts a
 * fixed start cost, cut into W contiguous slices of equal cost.  Long
 * contexts are so split into partitions processed in parallel and joined by
 * a log-sum-exp merge.
 * A wavefront that finishes the last partition of a split (sequence, KV
 * head) pair merges that pair's partitions itself: one kernel per call.
 *
 * Workspace: the library keeps one device buffer per (device, stream),
 * reused by every pa_decode call on that stream and grown when a call needs
 * more: about (W + S*Hkv) * G * (d + 1) * 4 + S * Hkv * 4 bytes (per-unit
 * counters, which the kernel leaves at zero, then partial results).  Growing
 * allocates (hipMallocAsync), zeroes the counters (hipMemsetAsync) and frees
 * the old buffer (hipFreeAsync), all on `stream` (a buffer that a graph
 * captured on the stream uses is kept instead; see "Graph capture" above).
 * Calls on one stream share the buffer safely; calls on different streams
 * use different buffers.  Release a stream's buffer with
 * pa_workspace_release before destroying the stream.
 * Returns PA_OK or a negative pa_status.
 */
int pa_decode(const pa_tensor* q, const pa_tensor* k_pool, const pa_tensor* v_pool,
              const pa_tensor* block_table, const pa_tensor* context_lens, float scale,
              const pa_tensor* out, void* stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, kernels and results as pa_decode
 * (bit for bit), but the workspace is a fixed device array of 32 MiB that
 * the library holds on each GPU it runs on until the process ends: no
 * hipMalloc, hipFree or other allocation happens in this call.  The first
 * call on a GPU also launches one small kernel on `stream` that zeroes the
 * array's counter region.
 * Limits: at most 65,536 (sequence, KV head) pairs, and at most
 * (32 MiB - 256 KiB) of partial results, i.e. (W + S*Hkv) * G * (d + 1) * 4
 * bytes with W the worker count (1024 on an MI355X) -- about 15,000 pairs
 * for G = 4, d = 128.  Larger calls return PA_ERR_ALLOC with nothing
 * launched.
 * All calls on one GPU share the array: calls that overlap in time on one
 * GPU (on different streams, or a graph replay next to an eager call) race
 * and give wrong results; order them on one stream.
 */
int pa_decode_noalloc(const pa_tensor* q, const pa_tensor* k_pool, const pa_tensor* v_pool,
                      const pa_tensor* block_table, const pa_tensor* context_lens, float scale,
                      const pa_tensor* out, void* stream);

/*
 * pa_decode_lse -- pa_decode that also returns each (sequence, query head)'s
 * log-sum-exp of the scaled scores, lse = ln sum_t e^(scale * q . k_t)
 * (-inf for n_s = 0).  With the normalised output it is the state the
 * online softmax carries ("FlashAttention and PagedAttention: two fixes for
 * two different bottlenecks", "FlashAttention - How it works": running
 * maximum and sum), so the attention over a context split into disjoint key
 * sets -- e.g. the contiguous block ranges that several GPUs each hold of a
 * very long context -- is recovered exactly by pa_merge_states.
 *   lse   f32 [S, H], last dim contiguous, 4-byte aligned, not aliasing
 *         q, the pools or out.  NULL returns PA_ERR_NULL.
 * Everything else as pa_decode.
 */
int pa_decode_lse(const pa_tensor* q, const pa_tensor* k_pool, const pa_tensor* v_pool,
                  const pa_tensor* block_table, const pa_tensor* context_lens, float scale,
                  const pa_tensor* out, const pa_tensor* lse, void* stream);

/*
 * pa_merge_states -- joins P partial attention states of every
 * (sequence, head), each over a disjoint set of keys (pa_decode_lse's out
 * and lse on each set):
 *   M = max_p lse_p,  w_p = e^(lse_p - M),
 *   out = sum_p w_p out_p / sum_p w_p,  lse = M + ln sum_p w_p,
 * the online softmax's rescaling applied to whole parts ("FlashAttention -
 * How it works").  Parts with lse_p = -inf hold no key and contribute
 * nothing; if every part is empty, out = 0 and lse = -inf.
 *   part_out   f32 [P, S, H, d], d in {64, 128}, last dim contiguous, P >= 1
 *   part_lse   f32 [P, S, H]
 *   out        [S, H, d], f32, f16 or bf16 (rounded to nearest even), last
 *              dim contiguous, rows 16-byte aligned
 *   lse        f32 [S, H] merged log-sum-exp, or NULL
 * Strides of the other dimensions are free.  out and lse must not alias the
 * parts.  Stream-ordered; no workspace.
 */
int pa_merge_states(const pa_tensor* part_out, const pa_tensor* part_lse, const pa_tensor* out,
                    const pa_tensor* lse, void* stream);

/*
 * pa_prefill -- packed query rows of several sequences attend to their paged
 * KV caches, optionally with a causal mask.
 *
 * Sequence s owns packed rows query_start_loc[s] .. query_start_loc[s+1]-1
 * (L_s rows).  Row i of sequence s sits at absolute position
 * n_s - L_s + i; with causal != 0 it sees keys t <= n_s - L_s + i
 * (bottom-right alignment; with L_s = n_s this is the usual lower-
 * triangular mask of "Flash Attention vs Paged Attention", fused causal
 * masking), otherwise all n_s keys.  Key tiles wholly above the diagonal
 * are skipped, never loaded.
 *
 *   q                [T, H, d]  f16 or bf16; last dim contiguous
 *   k_pool, v_pool   [NB, B, Hkv, d]  same dtype as q; the prompt's own
 *                    K/V must already be in the pool
 *   block_table      int32 [S, MB]
 *   context_lens     int32 [S]
 *   query_start_loc  int32 [S + 1], non-decreasing, query_start_loc[0] = 0,
 *                    query_start_loc[S] = T (device contents: contract)
 *   max_query_len    host-side upper bound on every L_s (not checked
 *                    against the device contents; rows past it are not
 *                    computed)
 *   scale            finite float
 *   causal           0 or 1
 *   out              [T, H, d]  f32 or q's dtype; must not alias inputs
 *
 * Contract: 0 <= L_s <= n_s.  The P.V product runs on fp16 matrix cores
 * with fp32 accumulation; bf16 V values must lie within the fp16 range
 * (|v| < 65504).
 */
int pa_prefill(const pa_tensor* q, const pa_tensor* k_pool, const pa_tensor* v_pool,
               const pa_tensor* block_table, const pa_tensor* context_lens,
               const pa_tensor* query_start_loc, int32_t max_query_len, float scale,
               int32_t causal, const pa_tensor* out, void* stream);

/*
 * pa_write_kv -- append new tokens' K and V rows to their pool slots.
 *
 * Blocks fill left to right and a sequence takes a new block only when its
 * last one is full ("Flash Attention vs Paged Attention", memory-management
 * paragraph; "How PagedAttention and RadixAttention optimise KV-cache
 * handling", "How PagedAttention works", on-demand growth).  The caller's
 * allocator chooses the slots; this call only moves the bytes.
 *
 *   k_new, v_new   [N, Hkv, d]  same dtype as the pools; last dim contiguous
 *   slot_mapping   int32 [N]; slot x means block x / B, position x % B;
 *                  x < 0 skips the row.  Slots must be distinct and below
 *                  NB * B (device contents: contract)
 *   k_pool, v_pool [NB, B, Hkv, d]  written in place
 */
int pa_write_kv(const pa_tensor* k_new, const pa_tensor* v_new,
                const pa_tensor* slot_mapping, const pa_tensor* k_pool,
                const pa_tensor* v_pool, void* stream);

/*
 * pa_decode_shared_prefix -- pa_decode for sequences whose first
 * prefix_len tokens are one shared prefix stored in the same physical
 * blocks ("FlashAttention and PagedAttention: two fixes for two different
 * bottlenecks", "PagedAttention - How it works": sequences with a common
 * prompt share its blocks).  The result is pa_decode's (same arguments and
 * the same math, up to floating-point rounding); the work is split so that
 * the prefix is read once per KV head instead of once per sequence:
 *   1. every sequence's G query heads attend to the prefix keys together,
 *      as one dense block on the matrix cores (prefill workgroups, keys
 *      split into at most 4 chunks), giving normalised partial outputs and
 *      log-sum-exps;
 *   2. alongside, in the same kernel, decode workgroups attend each
 *      sequence's own keys [prefix_len, n_s) and merge their parts as
 *      pa_decode does, into an f32 state (output and log-sum-exp) in the
 *      workspace;
 *   3. a second kernel merges, per (sequence, head), the prefix chunks with
 *      that state (log-sum-exp merge) and writes `out`.
 *
 *   prefix_len   host int, a multiple of the block size, 0 <= prefix_len
 *                <= MB * B.  0 is plain pa_decode.
 * Contract (device contents, not checked): n_s >= prefix_len for every s,
 * and block_table[s][j] == block_table[0][j] for j < prefix_len / B.
 * Supported: f16/bf16, d = 128 (other shapes return PA_ERR_UNSUPPORTED);
 * the same G, B and strides as pa_decode.  The workspace (see pa_decode)
 * also holds the prefix parts, n_chunks * S * H * (d + 1) * 4 bytes, where
 * n_chunks <= min(4, ceil(prefix_len / 64)), and the suffix state,
 * S * H * (d + 1) * 4 bytes.
 */
int pa_decode_shared_prefix(const pa_tensor* q, const pa_tensor* k_pool,
                            const pa_tensor* v_pool, const pa_tensor* block_table,
                            const pa_tensor* context_lens, int32_t prefix_len, float scale,
                            const pa_tensor* out, void* stream);

/*
 * pa_copy_blocks -- copy whole physical blocks src[i] -> dst[i] in both
 * pools (the copy-on-write step of "FlashAttention and PagedAttention: two
 * fixes for two different bottlenecks", "PagedAttention - How it works":
 * a block shared by several sequences is duplicated before one of them
 * writes to it).
 *
 *   k_pool, v_pool   [NB, B, Hkv, d]  written in place
 *   src, dst         int32 [N] device arrays of block ids in [0, NB); no dst
 *                    may equal any src or another dst (device contents:
 *                    contract)
 */
int pa_copy_blocks(const pa_tensor* k_pool, const pa_tensor* v_pool, const pa_tensor* src,
                   const pa_tensor* dst, void* stream);

/*
 * Host block manager: the logical-to-physical block tables the kernels
 * read, following the block-table management of "Flash Attention vs Paged
 * Attention" (blocks handed out on demand from a free list, returned when
 * no sequence holds them) and the sharing of "FlashAttention and
 * PagedAttention: two fixes for two different bottlenecks", "PagedAttention
 * - How it works" (a forked sequence shares its parent's blocks; a shared
 * block is copied when one of its sequences writes into it).  Host memory
 * only; every call is serialised by a lock inside the manager.  Functions
 * returning int return PA_OK (or a count) or a negative pa_status with
 * pa_last_error() set.
 *
 * pa_bm_create(num_blocks, block_size)  -- NULL on invalid sizes or no memory
 * pa_bm_destroy(bm)
 * pa_bm_num_free(bm)                    -- free blocks
 * pa_bm_refcount(bm, block)             -- sequences holding `block` (queued
 *                                          copies do not count)
 * pa_bm_add(bm, seq_id)                 -- new empty sequence (id >= 0)
 * pa_bm_fork(bm, parent, child)         -- child shares all of parent's
 *                                          blocks and tokens
 * pa_bm_append(bm, seq_id, n, slots_out)
 *     adds n tokens; slots_out[i] = block * B + position of the i-th new
 *     token (the slot_mapping of pa_write_kv).  Blocks are taken on demand.
 *     If the sequence's last, partly filled block is shared, it is first
 *     replaced by a fresh block and the pair (old, fresh) is queued: the
 *     caller copies it (pa_copy_blocks) before writing the new tokens.
 *     PA_ERR_ALLOC when too few blocks are free; PA_ERR_ARG when that shared
 *     block is itself the destination of a pair still queued (take and run
 *     the queued copies, and write the tokens appended so far, first).  On
 *     any error the sequence is unchanged.
 * pa_bm_take_copies(bm, src, dst, max)  -- moves up to max queued pairs out
 *     in queue order and returns how many.  A queued pair keeps both of its
 *     blocks out of the free list until it is taken, so no block of one
 *     batch is the source or destination of another pair of the same batch:
 *     a batch can run as one pa_copy_blocks call.  Order of work for the
 *     caller: run the copies, then write the tokens of the appends whose
 *     slots it holds; a sequence forked after an append shares that
 *     append's slots, so write them before forking.
 * pa_bm_free(bm, seq_id)                -- releases the sequence
 * pa_bm_block_table(bm, seq_ids, S, MB, table, lens)
 *     host int32 table[S * MB] (row s: the blocks of seq_ids[s], then -1)
 *     and lens[S] (tokens), ready to copy to the device for pa_decode /
 *     pa_prefill.  PA_ERR_SHAPE if a sequence holds more than MB blocks.
 */
typedef struct pa_block_manager pa_block_manager;
pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size);
void pa_bm_destroy(pa_block_manager* bm);
int32_t pa_bm_num_free(pa_block_manager* bm);
int32_t pa_bm_refcount(pa_block_manager* bm, int32_t block);
int pa_bm_add(pa_block_manager* bm, int64_t seq_id);
int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child);
int pa_bm_append(pa_block_manager* bm, int64_t seq_id, int32_t n, int32_t* slots_out);
int pa_bm_take_copies(pa_block_manager* bm, int32_t* src, int32_t* dst, int32_t max);
int pa_bm_free(pa_block_manager* bm, int64_t seq_id);
int pa_bm_block_table(pa_block_manager* bm, const int64_t* seq_ids, int32_t S, int32_t MB,
                      int32_t* table, int32_t* lens);

/*
 * pa_workspace_release -- frees (stream-ordered, hipFreeAsync) the decode
 * workspace kept for `stream` on the current device, including buffers that
 * graphs captured on the stream still referenced after the workspace grew:
 * graphs holding decode calls captured on `stream` must not be replayed
 * afterwards.  Later pa_decode calls on that stream allocate a new one.
 * Returns PA_OK (also when the stream has none) or PA_ERR_LAUNCH.
 */
int pa_workspace_release(void* stream);

/* Text for a pa_status value (static storage). */
const char* pa_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* pa_last_error(void);

/*
 * pa_decode_plan -- what pa_decode would launch for these arguments,
 * without launching anything (same validation as pa_decode).
 *
 *   workers           wavefronts W sharing the tile list
 *   waves_per_group   wavefronts per workgroup
 *   grid[3]           workgroups of the partition kernel
 *   block_threads     threads per workgroup
 *   workspace_bytes   workspace the call needs (counters and partials)
 *
 * The environment variable PA_DECODE_WORKERS (1 .. 2^20) overrides W; the
 * result is the same up to floating-point rounding for every W.
 */
typedef struct pa_decode_plan_info {
  int32_t workers;
  int32_t waves_per_group;
  int32_t block_threads;
  int32_t reserved;
  int64_t grid[3];
  int64_t workspace_bytes;
} pa_decode_plan_info;

int pa_decode_plan(const pa_tensor* q, const pa_tensor* k_pool, const pa_tensor* v_pool,
                   const pa_tensor* block_table, const pa_tensor* context_lens,
                   const pa_tensor* out, pa_decode_plan_info* info);

/*
 * Kernel timing.  While enabled, every kernel the library launches carries
 * a pair of HIP events bound to its dispatch (hipExtLaunchKernelGGL), so the
 * elapsed time is the kernel's own execution.
 * pa_profiler_read synchronises on the recorded events and adds their
 * elapsed times to per-kernel totals.  Kernel names: "decode_partitions",
 * "prefill", "shared_prefix" and "prefix_join" (pa_decode_shared_prefix's
 * two kernels), "merge_states", "write_kv", "copy_blocks".  Not meant for
 * concurrent use from several threads.
 */
int pa_profiler_enable(int on);
void pa_profiler_reset(void);
/* Returns PA_OK and fills total_ms / launches (0 if the name never ran). */
int pa_profiler_read(const char* kernel, double* total_ms, int64_t* launches);
/* Copies up to `max` of the kernel's per-launch durations (ms, launch order)
 * since the last reset into ms[]; returns how many (>= 0) or a PA_ERR_*. */
int64_t pa_profiler_samples(const char* kernel, float* ms, int64_t max);

/*
 * pa_clock_probe -- measures the shader clock while other work runs: one
 * wave on `stream` waits `ticks` ticks of the GPU's 100 MHz reference
 * counter (1 .. 10^8) and writes, to the device array out[2] (int64,
 * 8-byte aligned), the shader clock ticks (out[0]) and reference ticks
 * (out[1]) that passed; shader MHz = 100 * out[0] / out[1].  Asynchronous;
 * a measurement aid for the benchmark (the achieved fraction of the MFMA
 * peak at the clock the chip actually ran).
 */
int pa_clock_probe(int32_t ticks, int64_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
