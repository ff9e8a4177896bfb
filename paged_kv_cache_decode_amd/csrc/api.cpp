// The C ABI of libpa.so: validation (plan.cpp), stream-ordered workspace,
// kernel launches and error reporting.  See include/pa.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/pa.h"
#include "kernels.h"
#include "plan.h"

namespace {

thread_local std::string g_last_error;

int set_error(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int set_error(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

bool log_enabled() {
  static const bool on = [] {
    const char* s = std::getenv("PA_LOG");
    return s && *s && *s != '0';
  }();
  return on;
}

// Test hook: PA_TEST_FAIL_ALLOC=1 makes every workspace allocation fail.
bool forced_alloc_failure() {
  const char* s = std::getenv("PA_TEST_FAIL_ALLOC");
  return s && *s && *s != '0';
}

// ---- kernel timer state ---------------------------------------------------
std::mutex g_prof_mu;
bool g_prof_on = false;
struct PendingTiming {
  std::string name;
  hipEvent_t start, stop;
};
std::vector<PendingTiming> g_pending;
struct Total {
  double ms = 0;
  int64_t launches = 0;
  std::vector<float> samples;  // each launch's duration, in launch order
};
std::map<std::string, Total> g_totals;

void drain_pending_locked() {
  for (auto& p : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.stop) == hipSuccess &&
        hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
      Total& t = g_totals[p.name];
      t.ms += ms;
      t.launches += 1;
      t.samples.push_back(ms);
    }
    (void)hipEventDestroy(p.start);
    (void)hipEventDestroy(p.stop);
  }
  g_pending.clear();
}

}  // namespace

namespace pa {

void set_last_error(const char* msg) { g_last_error = msg; }

bool profiler_enabled() { return g_prof_on; }

// True when `stream` is being captured into a graph.  (A stream whose state
// cannot be read -- no device -- counts as not captured; the calls that
// follow report the real failure.)
bool capturing(hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(stream, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone;
}

KernelTimer::KernelTimer(const char* name, hipStream_t stream) : name_(name) {
  if (!g_prof_on) return;
  // A dispatch recorded into a graph is not timed: its events would be
  // recorded once, at capture, not at each replay.
  if (capturing(stream)) return;
  if (hipEventCreate(&start_) != hipSuccess) start_ = nullptr;
  if (start_ && hipEventCreate(&stop_) != hipSuccess) {
    (void)hipEventDestroy(start_);
    start_ = stop_ = nullptr;
  }
}

void KernelTimer::commit() {
  if (!start_) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_pending.push_back({name_, start_, stop_});
  start_ = stop_ = nullptr;
}

KernelTimer::~KernelTimer() {
  if (start_) (void)hipEventDestroy(start_);
  if (stop_) (void)hipEventDestroy(stop_);
}

}  // namespace pa

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_DTYPE: return "PA_ERR_DTYPE: dtype not allowed for this argument";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: inconsistent ranks or sizes";
    case PA_ERR_STRIDE: return "PA_ERR_STRIDE: layout or alignment requirement not met";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: no compiled instance for these shapes";
    case PA_ERR_ALLOC: return "PA_ERR_ALLOC: workspace allocation failed";
    case PA_ERR_LAUNCH: return "PA_ERR_LAUNCH: the HIP runtime refused a call";
    case PA_ERR_ARG: return "PA_ERR_ARG: scalar argument out of range";
    default: return "unknown pa_status";
  }
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

namespace {

// Workers for a decode call: PA_DECODE_WORKERS if set, else the device's
// resident capacity for the instance the shapes select.
int decode_workers(const pa_tensor* q, const pa_tensor* k_pool) {
  const int ov = pa::workers_override_from_env();
  if (ov != 0) return ov;  // -1 (invalid) is rejected by the planner
  if (!q || !k_pool) return 1;
  const int64_t H = q->shape[1], Hkv = k_pool->shape[2];
  const int G = (Hkv > 0 && H % Hkv == 0) ? (int)(H / Hkv) : 1;
  return pa::decode_worker_count(q->dtype, (int)q->shape[2], G);
}

}  // namespace

namespace {

// Decode workspaces, one per (device, stream), kept across calls and grown
// when a call needs more.  Layout: per-unit counters (zero between calls:
// the kernel resets every counter it uses) followed by the partial outputs.
// Calls on one stream run in order, so they can share the buffer; a grown
// buffer is allocated, its counters zeroed and the old one freed, all
// stream-ordered on that stream -- unless a graph captured on the stream
// holds the old buffer's address: such a buffer is kept (retired) until
// pa_workspace_release, so that the graph's replays keep working.
struct StreamWorkspace {
  void* ptr = nullptr;
  int64_t counter_bytes = 0;  // capacity of the counter region
  int64_t part_bytes = 0;     // capacity of the partial-result region
  bool captured = false;      // a capture on this stream recorded `ptr`
  std::vector<void*> retired; // superseded buffers that captured graphs use
};
std::mutex g_ws_mu;
std::map<std::pair<int, void*>, StreamWorkspace> g_ws;

int acquire_workspace(pa::DecodePlan* plan, hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  const int64_t need_c = plan->counter_bytes, need_p = plan->ws_bytes - plan->counter_bytes;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  StreamWorkspace& w = g_ws[{dev, static_cast<void*>(stream)}];
  if (w.ptr == nullptr || w.counter_bytes < need_c || w.part_bytes < need_p) {
    // Growing records an allocation and a memset; inside a graph capture
    // neither is wanted (a memset node's effect would not repeat at each
    // replay the way the kernels expect).  The buffer must be sized first.
    if (pa::capturing(stream))
      return set_error(PA_ERR_ALLOC, "the workspace of this stream must grow to %lld bytes, "
                       "which is not done during graph capture: make one call of this size "
                       "on the stream before capturing", (long long)plan->ws_bytes);
    if (forced_alloc_failure())
      return set_error(PA_ERR_ALLOC, "workspace of %lld bytes: allocation failure forced by "
                       "PA_TEST_FAIL_ALLOC", (long long)plan->ws_bytes);
    const int64_t cb = std::max(w.counter_bytes, need_c);
    const int64_t pb = std::max(w.part_bytes, need_p + need_p / 4);
    void* p = nullptr;
    hipError_t e = hipMallocAsync(&p, (size_t)(cb + pb), stream);
    if (e != hipSuccess)
      return set_error(PA_ERR_ALLOC, "hipMallocAsync(%lld bytes): %s", (long long)(cb + pb),
                       hipGetErrorString(e));
    e = hipMemsetAsync(p, 0, (size_t)cb, stream);
    if (e != hipSuccess) {
      (void)hipFreeAsync(p, stream);
      return set_error(PA_ERR_LAUNCH, "hipMemsetAsync: %s", hipGetErrorString(e));
    }
    if (w.ptr) {
      if (w.captured)
        w.retired.push_back(w.ptr);  // a graph may still replay with it
      else
        (void)hipFreeAsync(w.ptr, stream);
    }
    w.ptr = p;
    w.counter_bytes = cb;
    w.part_bytes = pb;
    w.captured = false;
  }
  if (pa::capturing(stream)) w.captured = true;
  plan->counter_bytes = w.counter_bytes;  // partials start after the counters
  *out = w.ptr;
  return PA_OK;
}

}  // namespace

int pa_decode_plan(const pa_tensor* q, const pa_tensor* k_pool, const pa_tensor* v_pool,
                   const pa_tensor* block_table, const pa_tensor* context_lens,
                   const pa_tensor* out, pa_decode_plan_info* info) {
  g_last_error.clear();
  if (!info) return set_error(PA_ERR_NULL, "info is NULL");
  pa::DecodePlan plan;
  int st = pa::plan_decode(q, k_pool, v_pool, block_table, context_lens, 1.0f, out, 1, &plan,
                           &g_last_error);
  if (st) return st;
  st = pa::plan_decode(q, k_pool, v_pool, block_table, context_lens, 1.0f, out,
                       decode_workers(q, k_pool), &plan, &g_last_error);
  if (st) return st;
  info->workers = plan.workers;
  info->waves_per_group = pa::kDecodeWaves;
  info->block_threads = plan.block_threads;
  info->reserved = 0;
  for (int i = 0; i < 3; ++i) info->grid[i] = plan.grid[i];
  info->workspace_bytes = plan.ws_bytes;
  return PA_OK;
}

namespace {

int decode_impl(const pa_tensor* q, const pa_tensor* k_pool, const pa_tensor* v_pool,
                const pa_tensor* block_table, const pa_tensor* context_lens, float scale,
                const pa_tensor* out, const pa_tensor* lse, void* stream_ptr) {
  g_last_error.clear();
  pa::DecodePlan plan;
  // Validate first (no device query for invalid arguments), then size.
  int st = pa::plan_decode(q, k_pool, v_pool, block_table, context_lens, scale, out, 1, &plan,
                           &g_last_error);
  if (st) return st;
  if (lse && (st = pa::plan_decode_lse(lse, q, k_pool, v_pool, out, &plan, &g_last_error)))
    return st;
  if (plan.S == 0) return PA_OK;
  st = pa::plan_decode(q, k_pool, v_pool, block_table, context_lens, scale, out,
                       decode_workers(q, k_pool), &plan, &g_last_error);
  if (st) return st;
  if (lse && (st = pa::plan_decode_lse(lse, q, k_pool, v_pool, out, &plan, &g_last_error)))
    return st;
  if (log_enabled())
    fprintf(stderr,
            "[pa] decode dtype=%d out=%d S=%d H=%d Hkv=%d d=%d B=%d MB=%d workers=%d "
            "groups=%lld ws=%lld\n",
            plan.dtype, plan.out_dtype, plan.S, plan.H, plan.Hkv, plan.D, plan.B, plan.MB,
            plan.workers, (long long)plan.grid[0], (long long)plan.ws_bytes);
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  void* ws = nullptr;
  st = acquire_workspace(&plan, stream, &ws);
  if (st) return st;
  const hipError_t e = pa::launch_decode(plan, ws, stream);
  if (e != hipSuccess) return set_error(PA_ERR_LAUNCH, "decode launch: %s", hipGetErrorString(e));
  return PA_OK;
}

}  // namespace

int pa_decode(const pa_tensor* q, const pa_tensor* k_pool, const pa_tensor* v_pool,
              const pa_tensor* block_table, const pa_tensor* context_lens, float scale,
              const pa_tensor* out, void* stream_ptr) {
  return decode_impl(q, k_pool, v_pool, block_table, context_lens, scale, out, nullptr,
                     stream_ptr);
}

int pa_decode_noalloc(const pa_tensor* q, const pa_tensor* k_pool, const pa_tensor* v_pool,
                      const pa_tensor* block_table, const pa_tensor* context_lens, float scale,
                      const pa_tensor* out, void* stream_ptr) {
  g_last_error.clear();
  pa::DecodePlan plan;
  int st = pa::plan_decode(q, k_pool, v_pool, block_table, context_lens, scale, out, 1, &plan,
                           &g_last_error);
  if (st) return st;
  if (plan.S == 0) return PA_OK;
  st = pa::plan_decode(q, k_pool, v_pool, block_table, context_lens, scale, out,
                       decode_workers(q, k_pool), &plan, &g_last_error);
  if (st) return st;
  // The fixed workspace: counters of at most kNoAllocMaxUnits units in their
  // own region, then the partial results.
  const int64_t units = (int64_t)plan.S * plan.Hkv;
  const int64_t part = plan.ws_bytes - plan.counter_bytes;
  const int64_t part_cap = pa::kNoAllocScratchBytes - pa::kNoAllocCounterBytes;
  if (units > pa::kNoAllocMaxUnits || part > part_cap)
    return set_error(PA_ERR_ALLOC, "pa_decode_noalloc: %lld (sequence, KV head) pairs and %lld "
                     "bytes of partial results exceed its fixed workspace (at most %lld pairs "
                     "and %lld bytes); use pa_decode", (long long)units, (long long)part,
                     (long long)pa::kNoAllocMaxUnits, (long long)part_cap);
  plan.counter_bytes = pa::kNoAllocCounterBytes;
  plan.ws_bytes = plan.counter_bytes + part;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  void* ws = nullptr;
  hipError_t e = pa::noalloc_workspace(stream, &ws);
  if (e != hipSuccess)
    return set_error(PA_ERR_LAUNCH, "pa_decode_noalloc workspace: %s", hipGetErrorString(e));
  e = pa::launch_decode(plan, ws, stream);
  if (e != hipSuccess) return set_error(PA_ERR_LAUNCH, "decode launch: %s", hipGetErrorString(e));
  return PA_OK;
}

int pa_decode_lse(const pa_tensor* q, const pa_tensor* k_pool, const pa_tensor* v_pool,
                  const pa_tensor* block_table, const pa_tensor* context_lens, float scale,
                  const pa_tensor* out, const pa_tensor* lse, void* stream_ptr) {
  if (!lse) {
    g_last_error.clear();
    return set_error(PA_ERR_NULL, "lse is NULL");
  }
  return decode_impl(q, k_pool, v_pool, block_table, context_lens, scale, out, lse,
                     stream_ptr);
}

int pa_merge_states(const pa_tensor* part_out, const pa_tensor* part_lse, const pa_tensor* out,
                    const pa_tensor* lse, void* stream_ptr) {
  g_last_error.clear();
  if (!part_out || !part_lse || !out) return set_error(PA_ERR_NULL, "a tensor is NULL");
  pa::MergePlan plan;
  const int st = pa::plan_merge(part_out, part_lse, out, lse, &plan, &g_last_error);
  if (st) return st;
  const hipError_t e = pa::launch_merge(plan, static_cast<hipStream_t>(stream_ptr));
  if (e != hipSuccess) return set_error(PA_ERR_LAUNCH, "merge launch: %s", hipGetErrorString(e));
  return PA_OK;
}

int pa_decode_shared_prefix(const pa_tensor* q, const pa_tensor* k_pool,
                            const pa_tensor* v_pool, const pa_tensor* block_table,
                            const pa_tensor* context_lens, int32_t prefix_len, float scale,
                            const pa_tensor* out, void* stream_ptr) {
  g_last_error.clear();
  pa::DecodePlan plan;
  int st = pa::plan_decode(q, k_pool, v_pool, block_table, context_lens, scale, out, 1, &plan,
                           &g_last_error);
  if (st) return st;
  if (prefix_len < 0 || prefix_len % plan.B != 0 || (int64_t)prefix_len > (int64_t)plan.MB * plan.B)
    return set_error(PA_ERR_ARG, "prefix_len %d must be a multiple of the block size %d in "
                     "[0, %lld]", prefix_len, plan.B, (long long)plan.MB * plan.B);
  if (prefix_len == 0 || plan.S == 0)
    return pa_decode(q, k_pool, v_pool, block_table, context_lens, scale, out, stream_ptr);
  if ((plan.dtype != PA_F16 && plan.dtype != PA_BF16) || plan.D != 128)
    return set_error(PA_ERR_UNSUPPORTED, "the shared-prefix path needs f16/bf16 and d = 128");
  st = pa::plan_decode(q, k_pool, v_pool, block_table, context_lens, scale, out,
                       decode_workers(q, k_pool), &plan, &g_last_error);
  if (st) return st;

  // Prefix step: the S query rows of every KV head against the prefix keys,
  // one pseudo-sequence of S rows and prefix_len keys read through row 0 of
  // the table, split into key chunks.  It runs in the same kernel as the
  // suffix step (the decode kernel on each sequence's own keys), as
  // workgroups of their own; a second kernel joins the two.
  pa::PrefillPlan pp;
  pp.dtype = plan.dtype;
  pp.out_dtype = PA_F32;
  pp.S = 1;
  pp.T = plan.S;
  pp.H = plan.H;
  pp.Hkv = plan.Hkv;
  pp.G = plan.G;
  pp.D = plan.D;
  pp.B = plan.B;
  pp.MB = plan.MB;
  pp.NB = plan.NB;
  pp.pool = plan.pool;
  pp.max_query_len = plan.S;
  pp.causal = 0;
  // Workgroups of four waves, like the decode workgroups they share compute
  // units with.
  const int hg = plan.G > 4 ? 4 : plan.G;
  pp.row_waves = pa::kPrefixStepWaves / hg;
  const int step_rows = pa::kPrefillWaveRows * pp.row_waves;
  pp.q_tiles = (plan.S + step_rows - 1) / step_rows;
  pp.q = plan.q;
  pp.q_st = plan.q_ss;
  pp.q_sh = plan.q_sh;
  pp.k = plan.k;
  pp.v = plan.v;
  pp.bt = plan.bt;  // row 0: the prefix blocks, common to all rows
  pp.bt_ss = 0;
  pp.scale = scale;
  pp.fixed_L = plan.S;
  pp.fixed_n = prefix_len;
  const int ptiles = (prefix_len + 63) / 64;
  const int base = pp.q_tiles * plan.Hkv;
  // Key chunks: enough for about 128 prefill workgroups (one per two CUs;
  // each CU also holds a decode workgroup), at most kMaxPrefixChunks.  More
  // chunks finish the prefix sooner but write more partial results, which
  // the join reads back: with 256 sequences and 8 KV heads one chunk (128
  // workgroups) measured 123 us per call, two chunks 127 us.
  const int chunks =
      std::max(1, std::min({ptiles, (128 + base - 1) / base, pa::kMaxPrefixChunks}));
  pp.chunk_tiles = (ptiles + chunks - 1) / chunks;
  pp.n_chunks = (ptiles + pp.chunk_tiles - 1) / pp.chunk_tiles;
  pp.part_rows = plan.S;
  // Workspace: the decode counters | decode partials | prefix chunk parts
  // [n_chunks, H, S] x (d + 1) floats | suffix state [S, H] x (d + 1) floats.
  auto up256 = [](int64_t x) { return (x + 255) / 256 * 256; };
  const int64_t dec_part = plan.ws_bytes - plan.counter_bytes;
  const int64_t chunk_rows = (int64_t)pp.n_chunks * plan.S * plan.H;
  const int64_t chunk_off = up256(dec_part);
  const int64_t suf_rows = (int64_t)plan.S * plan.H;
  const int64_t suf_off = chunk_off + up256(chunk_rows * (plan.D + 1) * 4);
  plan.ws_bytes = plan.counter_bytes + suf_off + suf_rows * (plan.D + 1) * 4;
  if (log_enabled())
    fprintf(stderr, "[pa] decode_shared_prefix S=%d prefix=%d chunks=%d x %d tiles workers=%d\n",
            plan.S, prefix_len, pp.n_chunks, pp.chunk_tiles, plan.workers);

  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  void* ws = nullptr;
  st = acquire_workspace(&plan, stream, &ws);
  if (st) return st;
  uint8_t* parts = static_cast<uint8_t*>(ws) + plan.counter_bytes;
  pp.part_o = reinterpret_cast<float*>(parts + chunk_off);
  pp.part_lse = pp.part_o + chunk_rows * plan.D;
  float* suf_o = reinterpret_cast<float*>(parts + suf_off);
  float* suf_lse = suf_o + suf_rows * plan.D;

  pa::PrefixJoinPlan jp;
  jp.S = plan.S;
  jp.H = plan.H;
  jp.D = plan.D;
  jp.n_pre = pp.n_chunks;
  jp.pre_o = pp.part_o;
  jp.pre_lse = pp.part_lse;
  jp.suf_o = suf_o;
  jp.suf_lse = suf_lse;
  jp.out = plan.out;
  jp.out_dtype = plan.out_dtype;
  jp.o_ss = plan.o_ss;
  jp.o_sh = plan.o_sh;

  // Suffix step: keys [prefix_len, n_s) of every unit, its result as an f32
  // state (normalised output and natural-log log-sum-exp) in the workspace.
  plan.key_begin = prefix_len;
  plan.out = suf_o;
  plan.out_dtype = PA_F32;
  plan.o_ss = (int64_t)plan.H * plan.D;
  plan.o_sh = plan.D;
  plan.lse = suf_lse;
  plan.lse_ss = plan.H;
  hipError_t e = pa::launch_shared_prefix(plan, ws, pp, stream);
  if (e != hipSuccess)
    return set_error(PA_ERR_LAUNCH, "shared-prefix launch: %s", hipGetErrorString(e));
  e = pa::launch_prefix_join(jp, stream);
  if (e != hipSuccess) return set_error(PA_ERR_LAUNCH, "join launch: %s", hipGetErrorString(e));
  return PA_OK;
}

int pa_workspace_release(void* stream_ptr) {
  g_last_error.clear();
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  auto it = g_ws.find({dev, stream_ptr});
  if (it == g_ws.end()) return PA_OK;
  const hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  hipError_t e = hipFreeAsync(it->second.ptr, stream);
  for (void* p : it->second.retired) {
    const hipError_t e2 = hipFreeAsync(p, stream);
    if (e == hipSuccess) e = e2;
  }
  g_ws.erase(it);
  if (e != hipSuccess) return set_error(PA_ERR_LAUNCH, "hipFreeAsync: %s", hipGetErrorString(e));
  return PA_OK;
}

int pa_prefill(const pa_tensor* q, const pa_tensor* k_pool, const pa_tensor* v_pool,
               const pa_tensor* block_table, const pa_tensor* context_lens,
               const pa_tensor* query_start_loc, int32_t max_query_len, float scale,
               int32_t causal, const pa_tensor* out, void* stream_ptr) {
  g_last_error.clear();
  pa::PrefillPlan plan;
  const int st = pa::plan_prefill(q, k_pool, v_pool, block_table, context_lens, query_start_loc,
                                  max_query_len, scale, causal, out, &plan, &g_last_error);
  if (st) return st;
  if (plan.S == 0 || plan.T == 0 || plan.max_query_len == 0) return PA_OK;
  if (log_enabled())
    fprintf(stderr, "[pa] prefill dtype=%d S=%d T=%d H=%d Hkv=%d B=%d max_q=%d causal=%d "
            "workgroups=%lld\n", plan.dtype, plan.S, plan.T, plan.H, plan.Hkv, plan.B,
            plan.max_query_len, plan.causal, (long long)plan.grid[0]);
  const hipError_t e = pa::launch_prefill(plan, static_cast<hipStream_t>(stream_ptr));
  if (e != hipSuccess)
    return set_error(PA_ERR_LAUNCH, "prefill launch: %s", hipGetErrorString(e));
  return PA_OK;
}

int pa_write_kv(const pa_tensor* k_new, const pa_tensor* v_new, const pa_tensor* slot_mapping,
                const pa_tensor* k_pool, const pa_tensor* v_pool, void* stream_ptr) {
  g_last_error.clear();
  pa::WriteKvPlan plan;
  const int st = pa::plan_write_kv(k_new, v_new, slot_mapping, k_pool, v_pool, &plan,
                                   &g_last_error);
  if (st) return st;
  const hipError_t e = pa::launch_write_kv(plan, static_cast<hipStream_t>(stream_ptr));
  if (e != hipSuccess)
    return set_error(PA_ERR_LAUNCH, "write_kv launch: %s", hipGetErrorString(e));
  return PA_OK;
}

int pa_copy_blocks(const pa_tensor* k_pool, const pa_tensor* v_pool, const pa_tensor* src,
                   const pa_tensor* dst, void* stream_ptr) {
  g_last_error.clear();
  pa::CopyBlocksPlan plan;
  const int st = pa::plan_copy_blocks(k_pool, v_pool, src, dst, &plan, &g_last_error);
  if (st) return st;
  const hipError_t e = pa::launch_copy_blocks(plan, static_cast<hipStream_t>(stream_ptr));
  if (e != hipSuccess)
    return set_error(PA_ERR_LAUNCH, "copy_blocks launch: %s", hipGetErrorString(e));
  return PA_OK;
}

int pa_clock_probe(int32_t ticks, int64_t* out, void* stream_ptr) {
  g_last_error.clear();
  if (!out) return set_error(PA_ERR_NULL, "out is NULL");
  if (ticks < 1 || ticks > 100000000)
    return set_error(PA_ERR_ARG, "ticks must be in 1 .. 10^8 (100 MHz reference ticks)");
  if ((reinterpret_cast<uintptr_t>(out) & 7u) != 0)
    return set_error(PA_ERR_STRIDE, "out must be 8-byte aligned");
  const hipError_t e = pa::launch_clock_probe(ticks, out, static_cast<hipStream_t>(stream_ptr));
  if (e != hipSuccess) return set_error(PA_ERR_LAUNCH, "clock probe: %s", hipGetErrorString(e));
  return PA_OK;
}

int pa_profiler_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return PA_OK;
}

void pa_profiler_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  drain_pending_locked();
  g_totals.clear();
}

int pa_profiler_read(const char* kernel, double* total_ms, int64_t* launches) {
  if (!kernel || !total_ms || !launches) return set_error(PA_ERR_NULL, "NULL argument");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  drain_pending_locked();
  auto it = g_totals.find(kernel);
  *total_ms = it == g_totals.end() ? 0.0 : it->second.ms;
  *launches = it == g_totals.end() ? 0 : it->second.launches;
  return PA_OK;
}

int64_t pa_profiler_samples(const char* kernel, float* ms, int64_t max) {
  if (!kernel || (max > 0 && !ms)) return set_error(PA_ERR_NULL, "NULL argument");
  if (max < 0) return set_error(PA_ERR_ARG, "max must be >= 0");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  drain_pending_locked();
  auto it = g_totals.find(kernel);
  if (it == g_totals.end()) return 0;
  const std::vector<float>& v = it->second.samples;
  const int64_t n = std::min<int64_t>(max, (int64_t)v.size());
  std::copy(v.begin(), v.begin() + n, ms);
  return n;
}

}  // extern "C"
