// Host block manager: the logical-to-physical block tables the kernels read.
//
// Follows the block-table management of "Flash Attention vs Paged Attention"
// (section "Paged Attention: memory blocking" and its block-table paragraph:
// physical blocks are handed out on demand from a free list and returned
// when no longer needed) and the sharing rules of "FlashAttention and
// PagedAttention: two fixes for two different bottlenecks", section
// "PagedAttention - How it works" (sequences with a common prefix point at
// the same physical blocks; a shared block is copied only when one of its
// sequences writes to it -- copy-on-write).  Pure C++: no device access.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/pa.h"

namespace pa {
void set_last_error(const char* msg);
}

struct pa_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_list;  // stack; back() is handed out next
  std::vector<int32_t> refcount;   // per physical block: sequences holding it
  // Per physical block: queued copy pairs that name it (as source or
  // destination).  A block returns to the free list only when no sequence
  // holds it and no queued pair names it, so the blocks of a queued pair
  // cannot be handed out again before the caller has taken the pair.
  std::vector<int32_t> pending;
  std::vector<uint8_t> pending_dst;  // 1 while the block is a queued destination
  struct Seq {
    std::vector<int32_t> blocks;  // logical block j -> physical block
    int64_t tokens = 0;
  };
  std::unordered_map<int64_t, Seq> seqs;
  std::vector<int32_t> copy_src, copy_dst;  // queued copy-on-write pairs
  std::mutex mu;
};

namespace {

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  pa::set_last_error(buf);
  return status;
}

void maybe_free(pa_block_manager* bm, int32_t b) {
  if (bm->refcount[b] == 0 && bm->pending[b] == 0) bm->free_list.push_back(b);
}

void release_block(pa_block_manager* bm, int32_t b) {
  --bm->refcount[b];
  maybe_free(bm, b);
}

}  // namespace

extern "C" {

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size) {
  pa::set_last_error("");
  if (num_blocks <= 0 || block_size <= 0) {
    fail(PA_ERR_ARG, "num_blocks and block_size must be positive");
    return nullptr;
  }
  if ((int64_t)num_blocks * block_size > INT32_MAX) {
    fail(PA_ERR_ARG, "num_blocks * block_size must fit in int32 (slot numbers)");
    return nullptr;
  }
  pa_block_manager* bm = new (std::nothrow) pa_block_manager;
  if (!bm) {
    fail(PA_ERR_ALLOC, "out of host memory");
    return nullptr;
  }
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->refcount.assign(num_blocks, 0);
  bm->pending.assign(num_blocks, 0);
  bm->pending_dst.assign(num_blocks, 0);
  bm->free_list.reserve(num_blocks);
  for (int32_t b = num_blocks - 1; b >= 0; --b) bm->free_list.push_back(b);  // 0 first
  return bm;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int32_t pa_bm_num_free(pa_block_manager* bm) {
  if (!bm) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lk(bm->mu);
  return (int32_t)bm->free_list.size();
}

int pa_bm_add(pa_block_manager* bm, int64_t seq_id) {
  pa::set_last_error("");
  if (!bm) return fail(PA_ERR_NULL, "manager is NULL");
  std::lock_guard<std::mutex> lk(bm->mu);
  if (seq_id < 0) return fail(PA_ERR_ARG, "sequence ids must be >= 0");
  if (!bm->seqs.emplace(seq_id, pa_block_manager::Seq{}).second)
    return fail(PA_ERR_ARG, "sequence %lld exists", (long long)seq_id);
  return PA_OK;
}

int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
  pa::set_last_error("");
  if (!bm) return fail(PA_ERR_NULL, "manager is NULL");
  std::lock_guard<std::mutex> lk(bm->mu);
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return fail(PA_ERR_ARG, "no sequence %lld", (long long)parent);
  if (child < 0 || bm->seqs.count(child))
    return fail(PA_ERR_ARG, "child id %lld is negative or exists", (long long)child);
  pa_block_manager::Seq copy = it->second;
  for (int32_t b : copy.blocks) ++bm->refcount[b];
  bm->seqs.emplace(child, std::move(copy));
  return PA_OK;
}

int pa_bm_append(pa_block_manager* bm, int64_t seq_id, int32_t n, int32_t* slots_out) {
  pa::set_last_error("");
  if (!bm) return fail(PA_ERR_NULL, "manager is NULL");
  if (n < 0) return fail(PA_ERR_ARG, "n must be >= 0");
  if (n > 0 && !slots_out) return fail(PA_ERR_NULL, "slots_out is NULL");
  std::lock_guard<std::mutex> lk(bm->mu);
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return fail(PA_ERR_ARG, "no sequence %lld", (long long)seq_id);
  pa_block_manager::Seq& sq = it->second;
  const int64_t B = bm->block_size;
  const int64_t used = (sq.tokens + B - 1) / B;           // blocks holding tokens
  const int64_t need = (sq.tokens + n + B - 1) / B;       // blocks after the append
  const bool partial_last = sq.tokens % B != 0;
  const bool cow = n > 0 && partial_last && bm->refcount[sq.blocks[used - 1]] > 1;
  if (cow && bm->pending_dst[sq.blocks[used - 1]])
    return fail(PA_ERR_ARG, "sequence %lld: its last block %d is the destination of a queued "
                "copy and must be copied again; take and run the queued copies (and write "
                "the tokens appended so far) first", (long long)seq_id, sq.blocks[used - 1]);
  const int64_t fresh = (need - used) + (cow ? 1 : 0);
  if (fresh > (int64_t)bm->free_list.size())
    return fail(PA_ERR_ALLOC, "sequence %lld needs %lld free blocks, %zu left",
                (long long)seq_id, (long long)fresh, bm->free_list.size());
  if (cow) {
    // The last block is shared and will receive a token: give this
    // sequence its own copy first; the caller copies the contents.
    const int32_t old = sq.blocks[used - 1];
    const int32_t nb = bm->free_list.back();
    bm->free_list.pop_back();
    bm->refcount[nb] = 1;
    --bm->refcount[old];  // still > 0: another sequence holds it
    sq.blocks[used - 1] = nb;
    // The queued pair keeps both blocks out of the free list until taken.
    ++bm->pending[old];
    ++bm->pending[nb];
    bm->pending_dst[nb] = 1;
    bm->copy_src.push_back(old);
    bm->copy_dst.push_back(nb);
  }
  for (int64_t j = used; j < need; ++j) {
    const int32_t nb = bm->free_list.back();
    bm->free_list.pop_back();
    bm->refcount[nb] = 1;
    sq.blocks.push_back(nb);
  }
  for (int32_t i = 0; i < n; ++i) {
    const int64_t t = sq.tokens + i;
    slots_out[i] = (int32_t)(sq.blocks[t / B] * B + t % B);
  }
  sq.tokens += n;
  return PA_OK;
}

int pa_bm_take_copies(pa_block_manager* bm, int32_t* src, int32_t* dst, int32_t max) {
  pa::set_last_error("");
  if (!bm) return fail(PA_ERR_NULL, "manager is NULL");
  if (max < 0) return fail(PA_ERR_ARG, "max must be >= 0");
  std::lock_guard<std::mutex> lk(bm->mu);
  const int32_t k = (int32_t)std::min<size_t>(bm->copy_src.size(), (size_t)max);
  if (k > 0 && (!src || !dst)) return fail(PA_ERR_NULL, "src or dst is NULL");
  std::copy(bm->copy_src.begin(), bm->copy_src.begin() + k, src);
  std::copy(bm->copy_dst.begin(), bm->copy_dst.begin() + k, dst);
  for (int32_t i = 0; i < k; ++i) {
    const int32_t a = bm->copy_src[i], b = bm->copy_dst[i];
    bm->pending_dst[b] = 0;
    --bm->pending[a];
    --bm->pending[b];
    maybe_free(bm, a);
    maybe_free(bm, b);
  }
  bm->copy_src.erase(bm->copy_src.begin(), bm->copy_src.begin() + k);
  bm->copy_dst.erase(bm->copy_dst.begin(), bm->copy_dst.begin() + k);
  return k;
}

int pa_bm_free(pa_block_manager* bm, int64_t seq_id) {
  pa::set_last_error("");
  if (!bm) return fail(PA_ERR_NULL, "manager is NULL");
  std::lock_guard<std::mutex> lk(bm->mu);
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return fail(PA_ERR_ARG, "no sequence %lld", (long long)seq_id);
  for (int32_t b : it->second.blocks) release_block(bm, b);
  bm->seqs.erase(it);
  return PA_OK;
}

int pa_bm_block_table(pa_block_manager* bm, const int64_t* seq_ids, int32_t S, int32_t MB,
                      int32_t* table, int32_t* lens) {
  pa::set_last_error("");
  if (!bm) return fail(PA_ERR_NULL, "manager is NULL");
  if (S < 0 || MB < 0) return fail(PA_ERR_ARG, "S and MB must be >= 0");
  if (S > 0 && (!seq_ids || !lens || (MB > 0 && !table)))
    return fail(PA_ERR_NULL, "seq_ids, table or lens is NULL");
  std::lock_guard<std::mutex> lk(bm->mu);
  for (int32_t s = 0; s < S; ++s) {
    auto it = bm->seqs.find(seq_ids[s]);
    if (it == bm->seqs.end()) return fail(PA_ERR_ARG, "no sequence %lld", (long long)seq_ids[s]);
    if ((int64_t)it->second.blocks.size() > MB)
      return fail(PA_ERR_SHAPE, "sequence %lld holds %zu blocks, table width is %d",
                  (long long)seq_ids[s], it->second.blocks.size(), MB);
    if (it->second.tokens > INT32_MAX)
      return fail(PA_ERR_SHAPE, "sequence %lld is longer than int32", (long long)seq_ids[s]);
  }
  for (int32_t s = 0; s < S; ++s) {
    const pa_block_manager::Seq& sq = bm->seqs.find(seq_ids[s])->second;
    for (int32_t j = 0; j < MB; ++j)
      table[(int64_t)s * MB + j] = j < (int32_t)sq.blocks.size() ? sq.blocks[j] : -1;
    lens[s] = (int32_t)sq.tokens;
  }
  return PA_OK;
}

int32_t pa_bm_refcount(pa_block_manager* bm, int32_t block) {
  if (!bm) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lk(bm->mu);
  if (block < 0 || block >= bm->num_blocks) return PA_ERR_ARG;
  return bm->refcount[block];
}

}  // extern "C"
