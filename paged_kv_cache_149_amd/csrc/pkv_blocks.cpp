// Host-side physical block pool of a paged KV cache: which blocks are free,
// and a reference count for every block in use ("连续批处理与 PagedAttention
// 原理", section "块管理器": allocate, free and copy-on-write; "11.2 连续批处理
// 与 PagedAttention", section 11.2.3 (sharing): several logical blocks may map to
// one physical block, and only a shared block that is not yet full is
// copied before a sequence writes into it).
//
// Free blocks form a stack: allocation pops the top, a block whose count
// drops to zero is pushed back on top, and a new pool holds 0 on top, then
// 1, 2, ... -- so allocation order is fully determined.
//
// Prefix caching ("11.2 连续批处理与 PagedAttention", section 11.2.4): a full
// block can be registered under a hash of its parent block's hash, its 16
// tokens and an extra key; a later prompt whose leading full blocks match
// maps the same physical blocks and skips their prefill.  A match is
// token-exact, not just hash-equal: a registered entry keeps its tokens, its
// extra key and the serial number of its parent entry (serials are never
// reused), and a lookup accepts an entry only if all three equal the
// prompt's block and the entry matched one block earlier.  A registered
// block whose count drops to zero is not freed but queued as evictable,
// oldest first; allocation takes free blocks first and then evicts the
// oldest evictable block, dropping its registration.
#include <algorithm>
#include <cstring>
#include <list>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv_internal.h"

namespace {
struct CachedBlock {
  uint64_t parent_serial, serial, extra;
  int32_t tokens[pkv::kBlock];
  int32_t block;
};
}  // namespace

struct pkv_block_pool {
  std::vector<int32_t> refcount;    // per block; 0 = free or evictable
  std::vector<int32_t> free_stack;  // top at the back
  std::unordered_map<uint64_t, CachedBlock> cache;  // registered full blocks by hash
  std::vector<uint64_t> hash_of;    // per block: its hash, if registered
  std::vector<char> registered;
  std::list<int32_t> evictable;     // registered blocks with count 0, oldest first
  std::vector<std::list<int32_t>::iterator> evict_pos;
  uint64_t next_serial = 1;         // 0 stands for "no parent"
};

namespace {

bool valid(const pkv_block_pool_t *p, int64_t b) { return b >= 0 && b < (int64_t)p->refcount.size(); }

size_t available(const pkv_block_pool_t *p) { return p->free_stack.size() + p->evictable.size(); }

// a block for a new owner: the top free block, else the oldest evictable one
int32_t pop(pkv_block_pool_t *p) {
  int32_t b;
  if (!p->free_stack.empty()) {
    b = p->free_stack.back();
    p->free_stack.pop_back();
  } else {
    b = p->evictable.front();
    p->evictable.pop_front();
    p->cache.erase(p->hash_of[b]);
    p->registered[b] = 0;
  }
  p->refcount[b] = 1;
  return b;
}

void unref(pkv_block_pool_t *p, int32_t b) {
  if (--p->refcount[b] != 0) return;
  if (p->registered[b])
    p->evict_pos[b] = p->evictable.insert(p->evictable.end(), b);
  else
    p->free_stack.push_back(b);
}

// one more reference; an evictable block leaves the queue
void ref(pkv_block_pool_t *p, int32_t b) {
  if (p->refcount[b] == 0) p->evictable.erase(p->evict_pos[b]);
  ++p->refcount[b];
}

// FNV-1a, 64 bits, over the little-endian bytes of parent, the block's 16
// token ids (4 bytes each) and extra
uint64_t fnv1a(uint64_t parent, const int32_t *tokens, uint64_t extra) {
  uint64_t h = 14695981039346656037ull;
  auto eat = [&](uint64_t v, int nbytes) {
    for (int i = 0; i < nbytes; ++i) {
      h ^= (v >> (8 * i)) & 0xFF;
      h *= 1099511628211ull;
    }
  };
  eat(parent, 8);
  for (int i = 0; i < pkv::kBlock; ++i) eat((uint32_t)tokens[i], 4);
  eat(extra, 8);
  return h;
}

bool same_block(const CachedBlock &e, uint64_t parent_serial, const int32_t *tokens, uint64_t extra) {
  return e.parent_serial == parent_serial && e.extra == extra &&
         std::memcmp(e.tokens, tokens, sizeof(e.tokens)) == 0;
}

// drop the registration of the entry under hash h; an evictable block
// becomes free
void unregister(pkv_block_pool_t *p, std::unordered_map<uint64_t, CachedBlock>::iterator it) {
  const int32_t b = it->second.block;
  p->registered[b] = 0;
  if (p->refcount[b] == 0) {
    p->evictable.erase(p->evict_pos[b]);
    p->free_stack.push_back(b);
  }
  p->cache.erase(it);
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
    p->hash_of.assign((size_t)num_blocks, 0);
    p->registered.assign((size_t)num_blocks, 0);
    p->evict_pos.resize((size_t)num_blocks);
  } catch (...) {
    delete p;
    return PKV_ERANGE;
  }
  for (int64_t i = 0; i < num_blocks; ++i) p->free_stack[(size_t)i] = (int32_t)(num_blocks - 1 - i);
  *pool = p;
  return PKV_OK;
}

void pkv_block_pool_destroy(pkv_block_pool_t *pool) { delete pool; }

int64_t pkv_block_pool_num_free(const pkv_block_pool_t *pool) { return pool ? (int64_t)available(pool) : -1; }

int64_t pkv_block_pool_num_cached(const pkv_block_pool_t *pool) { return pool ? (int64_t)pool->cache.size() : -1; }

int32_t pkv_block_pool_refcount(const pkv_block_pool_t *pool, int32_t block) {
  return pool && valid(pool, block) ? pool->refcount[block] : -1;
}

int pkv_block_pool_allocate(pkv_block_pool_t *pool, int32_t n, int32_t *h_blocks) {
  if (!pool || n < 0 || (n > 0 && !h_blocks)) return PKV_EINVAL;
  if ((size_t)n > available(pool)) return PKV_ERANGE;
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
  if ((size_t)fresh > available(pool)) return PKV_ERANGE;
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

uint64_t pkv_block_hash(uint64_t parent, const int32_t *h_tokens, uint64_t extra_key) {
  return h_tokens ? fnv1a(parent, h_tokens, extra_key) : 0;
}

int pkv_block_pool_match_prefix(pkv_block_pool_t *pool, const int32_t *h_tokens, int32_t num_tokens,
                                uint64_t extra_key, int32_t *h_table_row, int32_t capacity,
                                int32_t *num_cached_tokens) {
  if (!pool || !num_cached_tokens || num_tokens < 0 || capacity < 0 || (num_tokens > 0 && !h_tokens) ||
      (capacity > 0 && !h_table_row))
    return PKV_EINVAL;
  *num_cached_tokens = 0;
  // full blocks that leave at least one token to compute
  const int64_t nfull = std::min<int64_t>(num_tokens > 0 ? (num_tokens - 1) / pkv::kBlock : 0, capacity);
  uint64_t parent = 0, parent_serial = 0;
  int64_t hits = 0;
  for (; hits < nfull; ++hits) {
    const int32_t *t = h_tokens + hits * pkv::kBlock;
    const uint64_t h = fnv1a(parent, t, extra_key);
    auto it = pool->cache.find(h);
    if (it == pool->cache.end() || !same_block(it->second, parent_serial, t, extra_key)) break;
    h_table_row[hits] = it->second.block;
    parent = h;
    parent_serial = it->second.serial;
  }
  for (int64_t b = 0; b < hits; ++b) ref(pool, h_table_row[b]);
  *num_cached_tokens = (int32_t)(hits * pkv::kBlock);
  return PKV_OK;
}

int pkv_block_pool_register_prefix(pkv_block_pool_t *pool, const int32_t *h_tokens, int32_t num_tokens,
                                   uint64_t extra_key, const int32_t *h_table_row) {
  if (!pool || num_tokens < 0 || (num_tokens > 0 && (!h_tokens || !h_table_row))) return PKV_EINVAL;
  const int64_t nfull = num_tokens / pkv::kBlock;
  for (int64_t b = 0; b < nfull; ++b)
    if (!valid(pool, h_table_row[b]) || pool->refcount[h_table_row[b]] <= 0) return PKV_EINVAL;
  uint64_t parent = 0, parent_serial = 0;
  for (int64_t b = 0; b < nfull; ++b) {
    const int32_t *t = h_tokens + b * pkv::kBlock;
    const int32_t blk = h_table_row[b];
    // a block that is already this content's entry (a prefix hit) keeps its
    // hash: the same parent entry and tokens give the same hash
    if (pool->registered[blk]) {
      auto own = pool->cache.find(pool->hash_of[blk]);
      if (same_block(own->second, parent_serial, t, extra_key)) {
        parent_serial = own->second.serial;
        parent = own->first;
        continue;
      }
    }
    const uint64_t h = fnv1a(parent, t, extra_key);
    auto it = pool->cache.find(h);
    if (it != pool->cache.end() && same_block(it->second, parent_serial, t, extra_key)) {
      parent_serial = it->second.serial;  // already registered (this block or an equal one)
    } else {
      // a block registered under another hash holds other content: the
      // chain cannot go on through it
      if (pool->registered[blk]) break;
      // an entry under the same hash that is not this content (a collision,
      // or a child of an evicted parent) is replaced
      if (it != pool->cache.end()) unregister(pool, it);
      CachedBlock e;
      e.parent_serial = parent_serial;
      e.serial = pool->next_serial++;
      e.extra = extra_key;
      std::memcpy(e.tokens, t, sizeof(e.tokens));
      e.block = blk;
      pool->cache.emplace(h, e);
      pool->hash_of[blk] = h;
      pool->registered[blk] = 1;
      parent_serial = e.serial;
    }
    parent = h;
  }
  return PKV_OK;
}

}  // extern "C"
