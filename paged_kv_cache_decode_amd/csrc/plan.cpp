// Host-side validation and launch planning (pure C++, no HIP).
#include "plan.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

namespace pa {
namespace {

int elem_bytes(int dtype) {
  switch (dtype) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
    case PA_I32: return 4;
    default: return 0;
  }
}

const char* dtype_name(int dtype) {
  switch (dtype) {
    case PA_F32: return "f32";
    case PA_F16: return "f16";
    case PA_BF16: return "bf16";
    case PA_I32: return "i32";
    default: return "?";
  }
}

int fail(std::string* err, int status, const char* fmt, ...)
    __attribute__((format(printf, 3, 4)));

int fail(std::string* err, int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (err) *err = buf;
  return status;
}

// Checks pointer, rank, non-negative sizes and the dtype set.
int check_basic(const pa_tensor* t, const char* name, int ndim, std::string* err,
                bool allow_empty_data) {
  if (!t) return fail(err, PA_ERR_NULL, "%s: tensor descriptor is NULL", name);
  if (t->ndim != ndim)
    return fail(err, PA_ERR_SHAPE, "%s: expected %d dimensions, got %d", name, ndim, t->ndim);
  int64_t numel = 1;
  for (int i = 0; i < ndim; ++i) {
    if (t->shape[i] < 0)
      return fail(err, PA_ERR_SHAPE, "%s: negative size %lld in dim %d", name,
                  (long long)t->shape[i], i);
    numel *= t->shape[i];
  }
  if (!t->data && !(allow_empty_data && numel == 0))
    return fail(err, PA_ERR_NULL, "%s: data pointer is NULL", name);
  if (elem_bytes(t->dtype) == 0)
    return fail(err, PA_ERR_DTYPE, "%s: unknown dtype %d", name, t->dtype);
  return PA_OK;
}

bool contiguous(const pa_tensor* t) {
  int64_t expect = 1;
  for (int i = t->ndim - 1; i >= 0; --i) {
    if (t->shape[i] != 1 && t->stride[i] != expect) return false;
    expect *= t->shape[i];
  }
  return true;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_float(int dt) { return dt == PA_F32 || dt == PA_F16 || dt == PA_BF16; }

bool supported_block(int64_t B) { return B == 16 || B == 32 || B == 64 || B == 128; }

bool supported_group(int64_t G) { return G == 1 || G == 2 || G == 4 || G == 8; }

// Pools: [NB, B, Hkv, d], same shape, dtype and layout (PoolLayout) for K
// and V.
int check_pools(const pa_tensor* k, const pa_tensor* v, std::string* err,
                PoolLayout* layout = nullptr) {
  int st;
  if ((st = check_basic(k, "k_pool", 4, err, false))) return st;
  if ((st = check_basic(v, "v_pool", 4, err, false))) return st;
  if (k->dtype != v->dtype)
    return fail(err, PA_ERR_DTYPE, "k_pool is %s but v_pool is %s", dtype_name(k->dtype),
                dtype_name(v->dtype));
  for (int i = 0; i < 4; ++i)
    if (k->shape[i] != v->shape[i])
      return fail(err, PA_ERR_SHAPE, "k_pool and v_pool shapes differ in dim %d", i);
  const int64_t B = k->shape[1], Hkv = k->shape[2], D = k->shape[3];
  auto layout_of = [&](const pa_tensor* t, PoolLayout* l) {
    if (contiguous(t)) {
      l->tok = Hkv * D;
      l->head = D;
      return true;
    }
    if (t->stride[3] == 1 && t->stride[2] == B * D && t->stride[1] == D &&
        (t->stride[0] == B * Hkv * D || t->shape[0] == 1)) {
      l->tok = D;
      l->head = B * D;
      return true;
    }
    return false;
  };
  PoolLayout lk, lv;
  if (!layout_of(k, &lk) || !layout_of(v, &lv))
    return fail(err, PA_ERR_STRIDE, "pools must be contiguous [NB, B, Hkv, d], or head-major "
                "within blocks (strides B*Hkv*d, d, B*d, 1)");
  if (lk.tok != lv.tok || lk.head != lv.head)
    return fail(err, PA_ERR_STRIDE, "k_pool and v_pool must have the same layout");
  if (layout) *layout = lk;
  if (!aligned16(k->data) || !aligned16(v->data))
    return fail(err, PA_ERR_STRIDE, "pool base pointers must be 16-byte aligned");
  if (k->data == v->data)
    return fail(err, PA_ERR_ARG, "k_pool and v_pool must not alias");
  return PA_OK;
}

int check_i32(const pa_tensor* t, const char* name, int ndim, std::string* err) {
  int st = check_basic(t, name, ndim, err, true);
  if (st) return st;
  if (t->dtype != PA_I32) return fail(err, PA_ERR_DTYPE, "%s must be int32", name);
  if (t->stride[ndim - 1] != 1 && t->shape[ndim - 1] > 1)
    return fail(err, PA_ERR_STRIDE, "%s: last dimension must be contiguous", name);
  if (t->data && (reinterpret_cast<uintptr_t>(t->data) & 3u))
    return fail(err, PA_ERR_STRIDE, "%s: data must be 4-byte aligned", name);
  return PA_OK;
}

// A [rows, H, d] activation (q or out) with a contiguous last dim and
// 16-byte aligned rows.
int check_rows(const pa_tensor* t, const char* name, std::string* err) {
  int st = check_basic(t, name, 3, err, true);
  if (st) return st;
  if (t->shape[2] > 1 && t->stride[2] != 1)
    return fail(err, PA_ERR_STRIDE, "%s: last dimension must be contiguous", name);
  const int64_t e = elem_bytes(t->dtype);
  if (t->data && t->shape[0] * t->shape[1] > 0) {
    if (!aligned16(t->data) || ((t->stride[0] * e) & 15) || ((t->stride[1] * e) & 15))
      return fail(err, PA_ERR_STRIDE, "%s: rows must be 16-byte aligned", name);
  }
  return PA_OK;
}

bool ranges_overlap(const pa_tensor* a, const pa_tensor* b) {
  if (!a->data || !b->data) return false;
  auto extent = [](const pa_tensor* t) {
    int64_t hi = 0;
    for (int i = 0; i < t->ndim; ++i)
      if (t->shape[i] > 0) hi += (t->shape[i] - 1) * t->stride[i];
    return (hi + 1) * (int64_t)elem_bytes(t->dtype);
  };
  const char* a0 = static_cast<const char*>(a->data);
  const char* b0 = static_cast<const char*>(b->data);
  return a0 < b0 + extent(b) && b0 < a0 + extent(a);
}

}  // namespace

int workers_override_from_env() {
  const char* s = std::getenv("PA_DECODE_WORKERS");
  if (!s || !*s) return 0;
  char* end = nullptr;
  long v = std::strtol(s, &end, 10);
  if (*end || v <= 0 || v > kMaxWorkers) return -1;
  return static_cast<int>(v);
}

int plan_decode(const pa_tensor* q, const pa_tensor* k_pool, const pa_tensor* v_pool,
                const pa_tensor* block_table, const pa_tensor* context_lens, float scale,
                const pa_tensor* out, int workers, DecodePlan* plan, std::string* err) {
  int st;
  if ((st = check_rows(q, "q", err))) return st;
  PoolLayout layout;
  if ((st = check_pools(k_pool, v_pool, err, &layout))) return st;
  if ((st = check_i32(block_table, "block_table", 2, err))) return st;
  if ((st = check_i32(context_lens, "context_lens", 1, err))) return st;
  if ((st = check_rows(out, "out", err))) return st;
  if (!is_float(q->dtype))
    return fail(err, PA_ERR_DTYPE, "q must be f32, f16 or bf16, got %s", dtype_name(q->dtype));
  if (k_pool->dtype != q->dtype)
    return fail(err, PA_ERR_DTYPE, "pools are %s but q is %s", dtype_name(k_pool->dtype),
                dtype_name(q->dtype));
  if (out->dtype != PA_F32 && out->dtype != q->dtype)
    return fail(err, PA_ERR_DTYPE, "out must be f32 or %s, got %s", dtype_name(q->dtype),
                dtype_name(out->dtype));
  const int64_t S = q->shape[0], H = q->shape[1], D = q->shape[2];
  const int64_t NB = k_pool->shape[0], B = k_pool->shape[1], Hkv = k_pool->shape[2];
  if (k_pool->shape[3] != D)
    return fail(err, PA_ERR_SHAPE, "pool head size %lld != q head size %lld",
                (long long)k_pool->shape[3], (long long)D);
  if (out->shape[0] != S || out->shape[1] != H || out->shape[2] != D)
    return fail(err, PA_ERR_SHAPE, "out must be [%lld, %lld, %lld]", (long long)S,
                (long long)H, (long long)D);
  if (block_table->shape[0] != S)
    return fail(err, PA_ERR_SHAPE, "block_table has %lld rows, expected %lld",
                (long long)block_table->shape[0], (long long)S);
  if (context_lens->shape[0] != S)
    return fail(err, PA_ERR_SHAPE, "context_lens has %lld entries, expected %lld",
                (long long)context_lens->shape[0], (long long)S);
  if (Hkv <= 0 || H <= 0 || H % Hkv)
    return fail(err, PA_ERR_SHAPE, "query heads %lld not a multiple of KV heads %lld",
                (long long)H, (long long)Hkv);
  if (!std::isfinite(scale)) return fail(err, PA_ERR_ARG, "scale must be finite");
  if (ranges_overlap(out, q) || ranges_overlap(out, k_pool) || ranges_overlap(out, v_pool))
    return fail(err, PA_ERR_ARG, "out must not alias q or the pools");
  const int64_t G = H / Hkv;
  if (!(D == 64 || D == 128))
    return fail(err, PA_ERR_UNSUPPORTED, "head size %lld not compiled (64, 128)", (long long)D);
  if (!supported_block(B))
    return fail(err, PA_ERR_UNSUPPORTED, "block size %lld not compiled (16/32/64/128)",
                (long long)B);
  if (!supported_group(G))
    return fail(err, PA_ERR_UNSUPPORTED, "group size H/Hkv = %lld not compiled (1/2/4/8)",
                (long long)G);
  const int64_t MB = block_table->shape[1];
  if (S > 0 && MB < 1) return fail(err, PA_ERR_SHAPE, "block_table has no columns");
  if (S > 65535 || Hkv > 65535)
    return fail(err, PA_ERR_UNSUPPORTED, "more than 65535 sequences or KV heads");
  if (MB * B > (int64_t)1 << 30)
    return fail(err, PA_ERR_UNSUPPORTED, "table covers more than 2^30 keys");
  if (B * Hkv * D * 4 >= ((int64_t)1 << 31))
    return fail(err, PA_ERR_UNSUPPORTED, "a pool block must be smaller than 2^31 bytes");
  if (workers <= 0 || workers > kMaxWorkers)
    return fail(err, PA_ERR_ARG, "decode worker count must be in 1..%d (PA_DECODE_WORKERS)",
                kMaxWorkers);
  const int64_t tiles_bound = S * Hkv * ((MB * B + kTileKeys - 1) / kTileKeys);
  if (tiles_bound >= ((int64_t)1 << 40))
    return fail(err, PA_ERR_UNSUPPORTED, "more than 2^40 key tiles");

  DecodePlan p;
  p.dtype = q->dtype;
  p.out_dtype = out->dtype;
  p.S = (int)S; p.H = (int)H; p.Hkv = (int)Hkv; p.G = (int)G; p.D = (int)D; p.B = (int)B;
  p.MB = (int)MB;
  p.NB = NB;
  p.workers = workers;
  p.slots = (int64_t)workers + S * Hkv;
  p.block_threads = 64 * kDecodeWaves;
  // Workgroups, rounded up to a multiple of the 8 XCDs (see the kernel).
  p.grid[0] = ((workers + kDecodeWaves - 1) / kDecodeWaves + 7) / 8 * 8;
  p.grid[1] = 1;
  p.grid[2] = 1;
  // counters [S*Hkv] int32, padded to 256 B | part_o [slots, G, D] f32 |
  // part_lse [slots, G] f32
  p.counter_bytes = ((int64_t)S * Hkv * 4 + 255) / 256 * 256;
  p.ws_bytes = p.counter_bytes + p.slots * G * D * 4 + p.slots * G * 4;
  p.q = q->data; p.q_ss = q->stride[0]; p.q_sh = q->stride[1];
  p.k = k_pool->data; p.v = v_pool->data;
  p.pool = layout;
  p.bt = static_cast<const int32_t*>(block_table->data); p.bt_ss = block_table->stride[0];
  p.cl = static_cast<const int32_t*>(context_lens->data);
  p.out = out->data; p.o_ss = out->stride[0]; p.o_sh = out->stride[1];
  p.scale = scale;
  *plan = p;
  return PA_OK;
}

int plan_prefill(const pa_tensor* q, const pa_tensor* k_pool, const pa_tensor* v_pool,
                 const pa_tensor* block_table, const pa_tensor* context_lens,
                 const pa_tensor* query_start_loc, int32_t max_query_len, float scale,
                 int32_t causal, const pa_tensor* out, PrefillPlan* plan, std::string* err) {
  int st;
  if ((st = check_rows(q, "q", err))) return st;
  PoolLayout layout;
  if ((st = check_pools(k_pool, v_pool, err, &layout))) return st;
  if ((st = check_i32(block_table, "block_table", 2, err))) return st;
  if ((st = check_i32(context_lens, "context_lens", 1, err))) return st;
  if ((st = check_i32(query_start_loc, "query_start_loc", 1, err))) return st;
  if ((st = check_rows(out, "out", err))) return st;
  if (!is_float(q->dtype))
    return fail(err, PA_ERR_DTYPE, "q must be f16 or bf16, got %s", dtype_name(q->dtype));
  if (k_pool->dtype != q->dtype)
    return fail(err, PA_ERR_DTYPE, "pools are %s but q is %s", dtype_name(k_pool->dtype),
                dtype_name(q->dtype));
  if (out->dtype != PA_F32 && out->dtype != q->dtype)
    return fail(err, PA_ERR_DTYPE, "out must be f32 or %s, got %s", dtype_name(q->dtype),
                dtype_name(out->dtype));
  const int64_t T = q->shape[0], H = q->shape[1], D = q->shape[2];
  const int64_t NB = k_pool->shape[0], B = k_pool->shape[1], Hkv = k_pool->shape[2];
  const int64_t S = context_lens->shape[0];
  if (k_pool->shape[3] != D)
    return fail(err, PA_ERR_SHAPE, "pool head size %lld != q head size %lld",
                (long long)k_pool->shape[3], (long long)D);
  if (out->shape[0] != T || out->shape[1] != H || out->shape[2] != D)
    return fail(err, PA_ERR_SHAPE, "out must be [%lld, %lld, %lld]", (long long)T,
                (long long)H, (long long)D);
  if (block_table->shape[0] != S)
    return fail(err, PA_ERR_SHAPE, "block_table has %lld rows, expected %lld",
                (long long)block_table->shape[0], (long long)S);
  if (query_start_loc->shape[0] != S + 1)
    return fail(err, PA_ERR_SHAPE, "query_start_loc must have S + 1 = %lld entries",
                (long long)(S + 1));
  if (Hkv <= 0 || H <= 0 || H % Hkv)
    return fail(err, PA_ERR_SHAPE, "query heads %lld not a multiple of KV heads %lld",
                (long long)H, (long long)Hkv);
  if (max_query_len < 0) return fail(err, PA_ERR_ARG, "max_query_len must be >= 0");
  if (causal != 0 && causal != 1) return fail(err, PA_ERR_ARG, "causal must be 0 or 1");
  if (!std::isfinite(scale)) return fail(err, PA_ERR_ARG, "scale must be finite");
  if (ranges_overlap(out, q) || ranges_overlap(out, k_pool) || ranges_overlap(out, v_pool))
    return fail(err, PA_ERR_ARG, "out must not alias q or the pools");
  const int64_t G = H / Hkv;
  if (q->dtype == PA_F32)
    return fail(err, PA_ERR_UNSUPPORTED, "prefill runs on 16-bit matrix cores (f16, bf16)");
  if (D != 128)
    return fail(err, PA_ERR_UNSUPPORTED, "prefill head size %lld not compiled (128)",
                (long long)D);
  if (!supported_block(B))
    return fail(err, PA_ERR_UNSUPPORTED, "block size %lld not compiled (16/32/64/128)",
                (long long)B);
  if (!supported_group(G))
    return fail(err, PA_ERR_UNSUPPORTED, "group size H/Hkv = %lld not compiled (1/2/4/8)",
                (long long)G);
  const int64_t MB = block_table->shape[1];
  if (S > 0 && MB < 1) return fail(err, PA_ERR_SHAPE, "block_table has no columns");
  if (MB * B > (int64_t)1 << 30)
    return fail(err, PA_ERR_UNSUPPORTED, "table covers more than 2^30 keys");
  if (T > ((int64_t)1 << 31) - 1) return fail(err, PA_ERR_UNSUPPORTED, "too many query rows");

  PrefillPlan p;
  p.dtype = q->dtype;
  p.out_dtype = out->dtype;
  p.S = (int)S; p.T = (int)T; p.H = (int)H; p.Hkv = (int)Hkv; p.G = (int)G; p.D = (int)D;
  p.B = (int)B; p.MB = (int)MB; p.NB = NB;
  p.max_query_len = max_query_len;
  p.causal = causal;
  // Groups of 8 heads run as two workgroups of 4 heads per KV head.
  const int64_t kv_div = G > 4 ? G / 4 : 1;
  const int hg = (int)(G / kv_div);
  p.row_waves = kPrefillWaves / hg;
  const int rows = kPrefillWaveRows * p.row_waves;
  p.q_tiles = (max_query_len + rows - 1) / rows;
  p.grid[0] = (int64_t)p.q_tiles * Hkv * kv_div * S;
  p.grid[1] = 1;
  p.grid[2] = 1;
  p.block_threads = 64 * p.row_waves * hg;  // 16 positions of one head per wave
  p.q = q->data; p.q_st = q->stride[0]; p.q_sh = q->stride[1];
  p.k = k_pool->data; p.v = v_pool->data;
  p.pool = layout;
  p.bt = static_cast<const int32_t*>(block_table->data); p.bt_ss = block_table->stride[0];
  p.cl = static_cast<const int32_t*>(context_lens->data);
  p.qsl = static_cast<const int32_t*>(query_start_loc->data);
  p.out = out->data; p.o_st = out->stride[0]; p.o_sh = out->stride[1];
  p.scale = scale;
  *plan = p;
  return PA_OK;
}

int plan_write_kv(const pa_tensor* k_new, const pa_tensor* v_new,
                  const pa_tensor* slot_mapping, const pa_tensor* k_pool,
                  const pa_tensor* v_pool, WriteKvPlan* plan, std::string* err) {
  int st;
  if ((st = check_rows(k_new, "k_new", err))) return st;
  if ((st = check_rows(v_new, "v_new", err))) return st;
  if ((st = check_i32(slot_mapping, "slot_mapping", 1, err))) return st;
  PoolLayout layout;
  if ((st = check_pools(k_pool, v_pool, err, &layout))) return st;
  if (k_new->dtype != k_pool->dtype || v_new->dtype != k_pool->dtype)
    return fail(err, PA_ERR_DTYPE, "new rows and pools must share a dtype");
  if (!is_float(k_pool->dtype)) return fail(err, PA_ERR_DTYPE, "pools must be f32/f16/bf16");
  const int64_t N = k_new->shape[0];
  const int64_t NB = k_pool->shape[0], B = k_pool->shape[1], Hkv = k_pool->shape[2],
                D = k_pool->shape[3];
  for (int i = 0; i < 3; ++i)
    if (k_new->shape[i] != v_new->shape[i])
      return fail(err, PA_ERR_SHAPE, "k_new and v_new shapes differ");
  if (k_new->shape[1] != Hkv || k_new->shape[2] != D)
    return fail(err, PA_ERR_SHAPE, "new rows must be [N, %lld, %lld]", (long long)Hkv,
                (long long)D);
  if (slot_mapping->shape[0] != N)
    return fail(err, PA_ERR_SHAPE, "slot_mapping has %lld entries, expected %lld",
                (long long)slot_mapping->shape[0], (long long)N);
  if ((D * elem_bytes(k_pool->dtype)) % 16)
    return fail(err, PA_ERR_UNSUPPORTED, "rows must be a multiple of 16 bytes");
  if (N > ((int64_t)1 << 31) - 1 || NB * B > ((int64_t)1 << 31) - 1)
    return fail(err, PA_ERR_UNSUPPORTED, "slot numbers must fit in int32");
  if (ranges_overlap(k_new, k_pool) || ranges_overlap(v_new, v_pool) ||
      ranges_overlap(k_new, v_pool) || ranges_overlap(v_new, k_pool))
    return fail(err, PA_ERR_ARG, "new rows must not alias the pools");
  WriteKvPlan p;
  p.dtype = k_pool->dtype;
  p.N = N; p.NB = NB; p.B = (int)B; p.Hkv = (int)Hkv; p.D = (int)D;
  p.kn = k_new->data; p.vn = v_new->data;
  p.kn_s = k_new->stride[0]; p.kn_h = k_new->stride[1];
  p.vn_s = v_new->stride[0]; p.vn_h = v_new->stride[1];
  p.slots = static_cast<const int32_t*>(slot_mapping->data);
  p.kp = k_pool->data; p.vp = v_pool->data;
  p.pool = layout;
  *plan = p;
  return PA_OK;
}

int plan_decode_lse(const pa_tensor* lse, const pa_tensor* q, const pa_tensor* k_pool,
                    const pa_tensor* v_pool, const pa_tensor* out, DecodePlan* plan,
                    std::string* err) {
  int st = check_basic(lse, "lse", 2, err, true);
  if (st) return st;
  if (lse->dtype != PA_F32) return fail(err, PA_ERR_DTYPE, "lse must be f32");
  if (lse->shape[0] != plan->S || lse->shape[1] != plan->H)
    return fail(err, PA_ERR_SHAPE, "lse must be [%d, %d]", plan->S, plan->H);
  if (lse->shape[1] > 1 && lse->stride[1] != 1)
    return fail(err, PA_ERR_STRIDE, "lse: last dimension must be contiguous");
  if (lse->data && (reinterpret_cast<uintptr_t>(lse->data) & 3u))
    return fail(err, PA_ERR_STRIDE, "lse must be 4-byte aligned");
  if (ranges_overlap(lse, q) || ranges_overlap(lse, k_pool) || ranges_overlap(lse, v_pool) ||
      ranges_overlap(lse, out))
    return fail(err, PA_ERR_ARG, "lse must not alias q, the pools or out");
  plan->lse = static_cast<float*>(lse->data);
  plan->lse_ss = lse->stride[0];
  return PA_OK;
}

int plan_merge(const pa_tensor* part_out, const pa_tensor* part_lse, const pa_tensor* out,
               const pa_tensor* lse, MergePlan* plan, std::string* err) {
  int st;
  if ((st = check_basic(part_out, "part_out", 4, err, true))) return st;
  if ((st = check_basic(part_lse, "part_lse", 3, err, true))) return st;
  if ((st = check_rows(out, "out", err))) return st;
  if (part_out->dtype != PA_F32 || part_lse->dtype != PA_F32)
    return fail(err, PA_ERR_DTYPE, "part_out and part_lse must be f32");
  if (!is_float(out->dtype)) return fail(err, PA_ERR_DTYPE, "out must be f32, f16 or bf16");
  const int64_t P = part_out->shape[0], S = part_out->shape[1], H = part_out->shape[2],
                D = part_out->shape[3];
  if (P < 1) return fail(err, PA_ERR_SHAPE, "at least one part is needed");
  if (part_lse->shape[0] != P || part_lse->shape[1] != S || part_lse->shape[2] != H)
    return fail(err, PA_ERR_SHAPE, "part_lse must be [%lld, %lld, %lld]", (long long)P,
                (long long)S, (long long)H);
  if (out->shape[0] != S || out->shape[1] != H || out->shape[2] != D)
    return fail(err, PA_ERR_SHAPE, "out must be [%lld, %lld, %lld]", (long long)S,
                (long long)H, (long long)D);
  if (!(D == 64 || D == 128))
    return fail(err, PA_ERR_UNSUPPORTED, "head size %lld (supported: 64, 128)", (long long)D);
  if (D > 1 && part_out->stride[3] != 1)
    return fail(err, PA_ERR_STRIDE, "part_out: last dimension must be contiguous");
  if (P * S * H > ((int64_t)1 << 31) - 1)
    return fail(err, PA_ERR_UNSUPPORTED, "too many parts");
  if (lse) {
    if ((st = check_basic(lse, "lse", 2, err, true))) return st;
    if (lse->dtype != PA_F32) return fail(err, PA_ERR_DTYPE, "lse must be f32");
    if (lse->shape[0] != S || lse->shape[1] != H)
      return fail(err, PA_ERR_SHAPE, "lse must be [%lld, %lld]", (long long)S, (long long)H);
    if (ranges_overlap(lse, part_out) || ranges_overlap(lse, part_lse) ||
        ranges_overlap(lse, out))
      return fail(err, PA_ERR_ARG, "lse must not alias the parts or out");
  }
  if (ranges_overlap(out, part_out) || ranges_overlap(out, part_lse))
    return fail(err, PA_ERR_ARG, "out must not alias the parts");
  MergePlan p;
  p.P = (int)P; p.S = (int)S; p.H = (int)H; p.D = (int)D;
  p.part_out = static_cast<const float*>(part_out->data);
  p.po_p = part_out->stride[0]; p.po_s = part_out->stride[1]; p.po_h = part_out->stride[2];
  p.part_lse = static_cast<const float*>(part_lse->data);
  p.pl_p = part_lse->stride[0]; p.pl_s = part_lse->stride[1]; p.pl_h = part_lse->stride[2];
  p.out = out->data; p.out_dtype = out->dtype;
  p.o_s = out->stride[0]; p.o_h = out->stride[1];
  if (lse) {
    p.lse = static_cast<float*>(lse->data);
    p.l_s = lse->stride[0]; p.l_h = lse->stride[1];
  }
  *plan = p;
  return PA_OK;
}

int plan_copy_blocks(const pa_tensor* k_pool, const pa_tensor* v_pool, const pa_tensor* src,
                     const pa_tensor* dst, CopyBlocksPlan* plan, std::string* err) {
  int st;
  if ((st = check_pools(k_pool, v_pool, err))) return st;
  if ((st = check_i32(src, "src", 1, err))) return st;
  if ((st = check_i32(dst, "dst", 1, err))) return st;
  if (!is_float(k_pool->dtype)) return fail(err, PA_ERR_DTYPE, "pools must be f32/f16/bf16");
  if (src->shape[0] != dst->shape[0])
    return fail(err, PA_ERR_SHAPE, "src has %lld entries, dst %lld", (long long)src->shape[0],
                (long long)dst->shape[0]);
  const int64_t block_bytes =
      k_pool->shape[1] * k_pool->shape[2] * k_pool->shape[3] * elem_bytes(k_pool->dtype);
  if (block_bytes % 16)
    return fail(err, PA_ERR_UNSUPPORTED, "a block must be a multiple of 16 bytes");
  if (src->shape[0] * (block_bytes / 16) > ((int64_t)1 << 38))
    return fail(err, PA_ERR_UNSUPPORTED, "copy too large");
  CopyBlocksPlan p;
  p.N = src->shape[0];
  p.block_bytes = block_bytes;
  p.src = static_cast<const int32_t*>(src->data);
  p.dst = static_cast<const int32_t*>(dst->data);
  p.kp = k_pool->data;
  p.vp = v_pool->data;
  *plan = p;
  return PA_OK;
}

}  // namespace pa
