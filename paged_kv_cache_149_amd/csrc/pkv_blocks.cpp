// Host-side physical block pool of a paged KV cache: which blocks are free,
// and a reference count for every block in use ("连续批处理与 PagedAttention
// 原理", section "块管理器": allocate, free and copy-on-write; "11.2 连续批处理
// 与 PagedAttention", section 11.2.3 "共享": several logical blocks may map to
// one physical block, and only a shared block that is not yet full is
// copied before a sequence writes into it).
//
// Free blocks form a stack: allocation pops the top, a block whose count
// drops to zero is pushed back on top, and a new pool holds 0 on top, then
// 1, 2, ... -- so allocation order is fully determined.
#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "pkv_internal.h"

struct pkv_block_pool {
  std::vector<int32_t> refcount;  // per block; 0 = free
  std::vector<int32_t> free_stack;  // top at the back
};

namespace {

bool valid(const pkv_block_pool_t *p, int64_t b) { return b >= 0 && b < (int64_t)p->refcount.size(); }

int32_t pop(pkv_block_pool_t *p) {
  const int32_t b = p->free_stack.back();
  p->free_stack.pop_back();
  p->refcount[b] = 1;
  return b;
}

void unref(pkv_block_pool_t *p, int32_t b) {
  if (--p->refcount[b] == 0) p->free_stack.push_back(b);
}

}  // namespace

extern "C" {

int pkv_block_pool_create(int64_t num_blocks, pkv_block_pool_t **pool) {
  if (!pool) return PKV_EINVAL;
  *pool = nullptr;
  if (num_blocks <= 0 || num_blocks > INT32_MAX) return PKV_ERANGE;
  pkv_block_pool_t *p = new (std::nothrow) pkv_block_pool_t;
  if (!p) return PKV_ERANGE;
  try {
    p->refcount.assign((size_t)num_blocks, 0);
    p->free_stack.resize((size_t)num_blocks);
  } catch (...) {
    delete p;
    return PKV_ERANGE;
  }
  for (int64_t i = 0; i < num_blocks; ++i) p->free_stack[(size_t)i] = (int32_t)(num_blocks - 1 - i);
  *pool = p;
  return PKV_OK;
}

void pkv_block_pool_destroy(pkv_block_pool_t *pool) { delete pool; }

int64_t pkv_block_pool_num_free(const pkv_block_pool_t *pool) {
  return pool ? (int64_t)pool->free_stack.size() : -1;
}

int32_t pkv_block_pool_refcount(const pkv_block_pool_t *pool, int32_t block) {
  return pool && valid(pool, block) ? pool->refcount[block] : -1;
}

int pkv_block_pool_allocate(pkv_block_pool_t *pool, int32_t n, int32_t *h_blocks) {
  if (!pool || n < 0 || (n > 0 && !h_blocks)) return PKV_EINVAL;
  if ((size_t)n > pool->free_stack.size()) return PKV_ERANGE;
  for (int32_t i = 0; i < n; ++i) h_blocks[i] = pop(pool);
  return PKV_OK;
}

int pkv_block_pool_share(pkv_block_pool_t *pool, const int32_t *h_blocks, int32_t n) {
  if (!pool || n < 0 || (n > 0 && !h_blocks)) return PKV_EINVAL;
  for (int32_t i = 0; i < n; ++i)
    if (!valid(pool, h_blocks[i]) || pool->refcount[h_blocks[i]] <= 0) return PKV_ERANGE;
  for (int32_t i = 0; i < n; ++i) ++pool->refcount[h_blocks[i]];
  return PKV_OK;
}

int pkv_block_pool_release(pkv_block_pool_t *pool, const int32_t *h_blocks, int32_t n) {
  if (!pool || n < 0 || (n > 0 && !h_blocks)) return PKV_EINVAL;
  // all-or-nothing: every block must hold at least as many references as
  // the list releases from it
  std::vector<int32_t> sorted(h_blocks, h_blocks + n);
  std::sort(sorted.begin(), sorted.end());
  for (int32_t i = 0; i < n;) {
    int32_t j = i;
    while (j < n && sorted[j] == sorted[i]) ++j;
    if (!valid(pool, sorted[i]) || pool->refcount[sorted[i]] < j - i) return PKV_ERANGE;
    i = j;
  }
  for (int32_t i = 0; i < n; ++i) unref(pool, h_blocks[i]);
  return PKV_OK;
}

int pkv_block_pool_append_slots(pkv_block_pool_t *pool, int32_t *h_table_row, int32_t capacity,
                                int32_t num_tokens, int32_t num_new, int32_t *h_copies,
                                int32_t *num_copies) {
  if (!pool || !h_table_row || !num_copies || capacity < 0 || num_tokens < 0 || num_new < 0) return PKV_EINVAL;
  *num_copies = 0;
  if (num_new == 0) return PKV_OK;
  const int64_t first = num_tokens / pkv::kBlock;                         // first logical block written
  const int64_t held = ((int64_t)num_tokens + pkv::kBlock - 1) / pkv::kBlock;  // blocks the row holds
  const int64_t need = ((int64_t)num_tokens + num_new + pkv::kBlock - 1) / pkv::kBlock;
  if (need > capacity) return PKV_ERANGE;
  for (int64_t lb = 0; lb < held; ++lb)
    if (!valid(pool, h_table_row[lb]) || pool->refcount[h_table_row[lb]] <= 0) return PKV_EINVAL;
  // a held block that the new tokens write into and that another sequence
  // also maps (count > 1) is copied first; at most one such block exists
  // (the partially filled last one)
  const bool cow = first < held && pool->refcount[h_table_row[first]] > 1;
  if (cow && !h_copies) return PKV_EINVAL;
  const int64_t fresh = need - held + (cow ? 1 : 0);
  if ((size_t)fresh > pool->free_stack.size()) return PKV_ERANGE;
  if (cow) {
    const int32_t old = h_table_row[first];
    const int32_t nb = pop(pool);
    unref(pool, old);
    h_table_row[first] = nb;
    h_copies[0] = old;
    h_copies[1] = nb;
    *num_copies = 1;
  }
  for (int64_t lb = held; lb < need; ++lb) h_table_row[lb] = pop(pool);
  return PKV_OK;
}

}  // extern "C"
