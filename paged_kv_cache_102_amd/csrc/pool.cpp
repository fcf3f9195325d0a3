// Host block pool and slot planner of libpagedkv.
//
// "PagedAttention por dentro" (blog.lo0.es): "El pool de bloques" -- one
// global pool of fixed 16-token blocks, sized at start, O(1) allocation;
// the figure in "La tabla de paginas (block table)" -- blocks of a finished
// session return to the pool; the same section's append rule (write into
// the last block while it has room, otherwise take a new block and append
// it to the table); "Copy-on-write para sampling paralelo" -- shared blocks
// carry reference counts and are copied only when a sequence is about to
// write into one.
//
// The free list is a LIFO stack (std::vector, top at the back).  Every call
// validates before it mutates, so a failing call leaves the pool unchanged.
//
// Prefix caching ("Como funciona realmente vLLM", "Automatic Prefix
// Caching": instead of dropping a finished request's blocks, the engine
// indexes them by a hash of their content and a new request that starts
// with the same tokens reuses them directly): once enabled, full blocks are
// registered under (the registered block holding the previous 16 tokens,
// their 16 token ids), so a block is found only through the chain of
// blocks holding everything before it.  A registered block whose last
// reference is dropped stays indexed on a second free list, least recently
// freed first; allocation takes blocks holding nothing first (the LIFO
// stack) and only then evicts the least recently freed cached block.  An
// evicted block leaves the index with every block registered below it (they
// stay where they are on the free lists).  The hash only locates
// candidates; a hit is confirmed by comparing the parent and the tokens.
#include <algorithm>
#include <array>
#include <cstdint>
#include <list>
#include <new>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"

namespace {
struct CachedBlock {
  int32_t parent = -1;                        // registered block of the previous 16 tokens, -1 for the first
  std::vector<int32_t> children;              // blocks registered with this one as parent
  std::array<int32_t, PKV_BLOCK_SIZE> tokens{};
  uint64_t hash = 0;
  bool on = false;                            // registered
  std::list<int32_t>::iterator lru_it;        // valid while refcount 0 and registered
};

// FNV-1a (64-bit) over the parent id and the token ids, 4 bytes each, little end first.
uint64_t block_hash(int32_t parent, const int32_t* tokens) {
  uint64_t h = 0xcbf29ce484222325ull;
  auto mix = [&](uint32_t v) {
    for (int i = 0; i < 4; ++i) {
      h ^= (v >> (8 * i)) & 0xFFu;
      h *= 0x100000001b3ull;
    }
  };
  mix(static_cast<uint32_t>(parent));
  for (int i = 0; i < PKV_BLOCK_SIZE; ++i) mix(static_cast<uint32_t>(tokens[i]));
  return h;
}
}  // namespace

struct pkv_pool {
  int32_t num_blocks = 0;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> ref;         // 0 = free
  // prefix caching (off until pkv_prefix_cache_enable)
  bool prefix_on = false;
  std::vector<CachedBlock> cached;
  std::unordered_multimap<uint64_t, int32_t> index;
  std::list<int32_t> lru;           // cached blocks with refcount 0, least recently freed first
};

namespace {

bool live(const pkv_pool* p, int32_t id) {
  return id >= 0 && id < p->num_blocks && p->ref[id] > 0;
}

size_t num_free(const pkv_pool* p) { return p->free_stack.size() + p->lru.size(); }

// Removes `id` and everything registered below it from the index.
void unregister(pkv_pool* p, int32_t id) {
  std::vector<int32_t> todo{id};
  while (!todo.empty()) {
    const int32_t x = todo.back();
    todo.pop_back();
    CachedBlock& c = p->cached[x];
    if (!c.on) continue;
    auto range = p->index.equal_range(c.hash);
    for (auto it = range.first; it != range.second; ++it)
      if (it->second == x) {
        p->index.erase(it);
        break;
      }
    c.on = false;
    for (int32_t ch : c.children)
      if (p->cached[ch].on && p->cached[ch].parent == x) todo.push_back(ch);
    c.children.clear();
  }
}

// Hands out a free block (refcount 1): one holding nothing first, else the
// least recently freed cached block, which leaves the index.
int32_t pop_block(pkv_pool* p) {
  int32_t id;
  if (!p->free_stack.empty()) {
    id = p->free_stack.back();
    p->free_stack.pop_back();
  } else {
    id = p->lru.front();
    p->lru.pop_front();
    unregister(p, id);
  }
  p->ref[id] = 1;
  return id;
}

// The last reference of `id` is gone.
void release(pkv_pool* p, int32_t id) {
  if (p->prefix_on && p->cached[id].on) {
    p->lru.push_back(id);
    p->cached[id].lru_it = std::prev(p->lru.end());
  } else {
    p->free_stack.push_back(id);
  }
}

// The registered block matching (parent, tokens), or -1.
int32_t find_cached(const pkv_pool* p, int32_t parent, const int32_t* tokens) {
  const uint64_t h = block_hash(parent, tokens);
  auto range = p->index.equal_range(h);
  for (auto it = range.first; it != range.second; ++it) {
    const CachedBlock& c = p->cached[it->second];
    if (c.parent == parent && std::equal(c.tokens.begin(), c.tokens.end(), tokens))
      return it->second;
  }
  return -1;
}

}  // namespace

extern "C" {

const char* pkv_status_string(pkv_status s) {
  switch (s) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID: return "invalid argument";
    case PKV_ERR_OOM: return "out of free blocks";
    case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKV_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

pkv_status pkv_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* init_order,
                           pkv_pool** out_pool) {
  if (!out_pool) return PKV_ERR_INVALID;
  *out_pool = nullptr;
  if (block_size != PKV_BLOCK_SIZE) return PKV_ERR_UNSUPPORTED;
  if (num_blocks < 1) return PKV_ERR_INVALID;
  if (init_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t id = init_order[i];
      if (id < 0 || id >= num_blocks || seen[id]) return PKV_ERR_INVALID;
      seen[id] = 1;
    }
  }
  pkv_pool* p = new (std::nothrow) pkv_pool;
  if (!p) return PKV_ERR_OOM;
  p->num_blocks = num_blocks;
  p->ref.assign(num_blocks, 0);
  p->free_stack.resize(num_blocks);
  // The first allocation returns order[0]: it sits at the top (back).
  for (int32_t i = 0; i < num_blocks; ++i)
    p->free_stack[num_blocks - 1 - i] = init_order ? init_order[i] : i;
  *out_pool = p;
  return PKV_OK;
}

void pkv_pool_destroy(pkv_pool* pool) { delete pool; }

pkv_status kv_block_alloc(pkv_pool* p, int32_t n, int32_t* out_ids) {
  if (!p || n < 0 || (n > 0 && !out_ids)) return PKV_ERR_INVALID;
  if (static_cast<size_t>(n) > num_free(p)) return PKV_ERR_OOM;
  for (int32_t i = 0; i < n; ++i) out_ids[i] = pop_block(p);
  return PKV_OK;
}

pkv_status kv_block_share(pkv_pool* p, int32_t n, const int32_t* ids) {
  if (!p || n < 0 || (n > 0 && !ids)) return PKV_ERR_INVALID;
  for (int32_t i = 0; i < n; ++i)
    if (!live(p, ids[i])) return PKV_ERR_INVALID;
  for (int32_t i = 0; i < n; ++i) ++p->ref[ids[i]];
  return PKV_OK;
}

pkv_status kv_block_free(pkv_pool* p, int32_t n, const int32_t* ids) {
  if (!p || n < 0 || (n > 0 && !ids)) return PKV_ERR_INVALID;
  std::unordered_map<int32_t, int32_t> drops;
  for (int32_t i = 0; i < n; ++i) {
    int32_t id = ids[i];
    if (id < 0 || id >= p->num_blocks) return PKV_ERR_INVALID;
    if (++drops[id] > p->ref[id]) return PKV_ERR_INVALID;
  }
  for (int32_t i = 0; i < n; ++i) {
    int32_t id = ids[i];
    if (--p->ref[id] == 0) release(p, id);
  }
  return PKV_OK;
}

pkv_status kv_block_cow(pkv_pool* p, int32_t id, int32_t* out_id, int32_t* needs_copy) {
  if (!p || !out_id || !needs_copy || !live(p, id)) return PKV_ERR_INVALID;
  if (p->ref[id] == 1) {
    *out_id = id;
    *needs_copy = 0;
    return PKV_OK;
  }
  if (num_free(p) == 0) return PKV_ERR_OOM;
  int32_t fresh = pop_block(p);
  --p->ref[id];
  *out_id = fresh;
  *needs_copy = 1;
  return PKV_OK;
}

pkv_status kv_block_refcount(const pkv_pool* p, int32_t id, int32_t* out_refcount) {
  if (!p || !out_refcount || id < 0 || id >= p->num_blocks) return PKV_ERR_INVALID;
  *out_refcount = p->ref[id];
  return PKV_OK;
}

pkv_status kv_pool_stats(const pkv_pool* p, pkv_stats* s) {
  if (!p || !s) return PKV_ERR_INVALID;
  int32_t used = 0, shared = 0;
  int64_t refs = 0;
  for (int32_t r : p->ref) {
    used += r > 0;
    shared += r > 1;
    refs += r;
  }
  s->num_blocks = p->num_blocks;
  s->num_free = static_cast<int32_t>(num_free(p));
  s->num_used = used;
  s->num_shared = shared;
  s->num_refs = refs;
  s->usage_percent = 100.0 * used / p->num_blocks;
  return PKV_OK;
}

pkv_status kv_pool_free_list(const pkv_pool* p, int32_t capacity, int32_t* out_ids,
                             int32_t* out_n) {
  if (!p || !out_n || capacity < 0 || (capacity > 0 && !out_ids)) return PKV_ERR_INVALID;
  const int32_t ns = static_cast<int32_t>(p->free_stack.size());
  const int32_t n = static_cast<int32_t>(num_free(p));
  int32_t k = 0;
  for (int32_t i = 0; i < ns && k < capacity; ++i) out_ids[k++] = p->free_stack[ns - 1 - i];
  for (auto it = p->lru.begin(); it != p->lru.end() && k < capacity; ++it) out_ids[k++] = *it;
  *out_n = n;
  return PKV_OK;
}

pkv_status paged_kv_append_slots(pkv_pool* p, int32_t num_seqs, int32_t max_blocks_per_seq,
                                 int32_t* tables, int32_t* lens, const int32_t* num_new,
                                 int64_t* slot_mapping, int64_t slot_capacity,
                                 int32_t* table_updates, int32_t update_capacity,
                                 int32_t* num_updates, int32_t* cow_pairs, int32_t cow_capacity,
                                 int32_t* num_cow) {
  if (!p || num_seqs < 0 || max_blocks_per_seq < 1 || !num_updates || !num_cow)
    return PKV_ERR_INVALID;
  if (num_seqs > 0 && (!tables || !lens)) return PKV_ERR_INVALID;
  if (static_cast<int64_t>(num_seqs) * max_blocks_per_seq >= (int64_t(1) << 31))
    return PKV_ERR_INVALID;
  const int64_t cap_tokens = int64_t(max_blocks_per_seq) * PKV_BLOCK_SIZE;

  // Dry run: count what the real pass will need and validate every table
  // entry it will read, without touching the pool.  Only copy-on-write
  // changes existing refcounts inside one call (it drops one reference of
  // the shared block), tracked in `dropped`.
  int64_t slots = 0, allocs = 0, cows = 0;
  std::unordered_map<int32_t, int32_t> dropped;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t add = num_new ? num_new[s] : 1;
    const int64_t p0 = lens[s];
    if (add < 0 || p0 < 0 || p0 + add > cap_tokens) return PKV_ERR_INVALID;
    if (add == 0) continue;
    slots += add;
    // tokens p0 .. p0+add-1: a block starts at every p % 16 == 0
    const int64_t first_new = (p0 + PKV_BLOCK_SIZE - 1) / PKV_BLOCK_SIZE;  // first block index >= p0 boundary
    const int64_t last_blk = (p0 + add - 1) / PKV_BLOCK_SIZE;
    allocs += std::max<int64_t>(0, last_blk - first_new + 1);
    if (p0 % PKV_BLOCK_SIZE != 0) {
      // the first token lands in the existing, possibly shared, last block
      const int32_t old = tables[int64_t(s) * max_blocks_per_seq + p0 / PKV_BLOCK_SIZE];
      if (!live(p, old)) return PKV_ERR_INVALID;
      auto it = dropped.find(old);
      const int32_t refs = p->ref[old] - (it == dropped.end() ? 0 : it->second);
      if (refs > 1) {
        ++cows;
        ++allocs;
        ++dropped[old];
      }
    }
  }
  if (allocs > static_cast<int64_t>(num_free(p))) return PKV_ERR_OOM;
  if (slots > slot_capacity || allocs > update_capacity || cows > cow_capacity)
    return PKV_ERR_INVALID;
  if ((slots > 0 && !slot_mapping) || (allocs > 0 && !table_updates) || (cows > 0 && !cow_pairs))
    return PKV_ERR_INVALID;

  // Real pass: cannot fail any more.
  int64_t k = 0;
  int32_t nu = 0, nc = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t add = num_new ? num_new[s] : 1;
    int32_t* row = tables + int64_t(s) * max_blocks_per_seq;
    for (int32_t a = 0; a < add; ++a) {
      const int32_t pos = lens[s];
      const int32_t ti = pos / PKV_BLOCK_SIZE;
      if (pos % PKV_BLOCK_SIZE == 0) {
        const int32_t id = pop_block(p);
        row[ti] = id;
        table_updates[2 * nu] = s * max_blocks_per_seq + ti;
        table_updates[2 * nu + 1] = id;
        ++nu;
      } else if (p->ref[row[ti]] > 1) {
        const int32_t old = row[ti];
        const int32_t id = pop_block(p);
        --p->ref[old];
        row[ti] = id;
        table_updates[2 * nu] = s * max_blocks_per_seq + ti;
        table_updates[2 * nu + 1] = id;
        ++nu;
        cow_pairs[2 * nc] = old;
        cow_pairs[2 * nc + 1] = id;
        ++nc;
      }
      slot_mapping[k++] = int64_t(row[ti]) * PKV_BLOCK_SIZE + pos % PKV_BLOCK_SIZE;
      lens[s] = pos + 1;
    }
  }
  *num_updates = nu;
  *num_cow = nc;
  return PKV_OK;
}


pkv_status pkv_prefix_cache_enable(pkv_pool* p) {
  if (!p) return PKV_ERR_INVALID;
  if (!p->prefix_on) {
    p->prefix_on = true;
    p->cached.assign(p->num_blocks, CachedBlock{});
  }
  return PKV_OK;
}

pkv_status pkv_prefix_match(pkv_pool* p, const int32_t* tokens, int32_t num_tokens,
                            int32_t max_blocks, int32_t* out_ids, int32_t* out_num_blocks) {
  if (!p || !p->prefix_on || num_tokens < 0 || max_blocks < 0 || !out_num_blocks ||
      (num_tokens > 0 && !tokens) || (max_blocks > 0 && !out_ids))
    return PKV_ERR_INVALID;
  const int32_t full = std::min(num_tokens / PKV_BLOCK_SIZE, max_blocks);
  int32_t k = 0, parent = -1;
  for (; k < full; ++k) {
    const int32_t id = find_cached(p, parent, tokens + int64_t(k) * PKV_BLOCK_SIZE);
    if (id < 0) break;
    out_ids[k] = id;
    parent = id;
  }
  for (int32_t i = 0; i < k; ++i) {
    const int32_t id = out_ids[i];
    if (p->ref[id] == 0) p->lru.erase(p->cached[id].lru_it);
    ++p->ref[id];
  }
  *out_num_blocks = k;
  return PKV_OK;
}

pkv_status pkv_prefix_register(pkv_pool* p, const int32_t* tokens, int32_t num_tokens,
                               const int32_t* block_ids) {
  if (!p || !p->prefix_on || num_tokens < 0 || (num_tokens > 0 && (!tokens || !block_ids)))
    return PKV_ERR_INVALID;
  const int32_t full = num_tokens / PKV_BLOCK_SIZE;
  // Walk the chain: the parent of block i is the registered block holding
  // tokens [16(i-1), 16i) -- the sequence's own block, or an equal one
  // already indexed.  Validate first (live, distinct, and a registered block
  // must hold exactly this content), then register.
  for (int pass = 0; pass < 2; ++pass) {
    int32_t parent = -1;
    for (int32_t i = 0; i < full; ++i) {
      const int32_t id = block_ids[i];
      const int32_t* t = tokens + int64_t(i) * PKV_BLOCK_SIZE;
      if (pass == 0) {
        if (!live(p, id)) return PKV_ERR_INVALID;
        for (int32_t j = 0; j < i; ++j)
          if (block_ids[j] == id) return PKV_ERR_INVALID;
      }
      const int32_t found = parent < -1 ? -1 : find_cached(p, parent, t);
      CachedBlock& c = p->cached[id];
      if (c.on) {
        if (found != id) return PKV_ERR_INVALID;  // (pass 0 only: pass 1 sees the same state)
        parent = id;
      } else if (found >= 0) {
        parent = found;
      } else if (pass == 0) {
        parent = -2;  // registered in pass 1: nothing below it can be indexed yet
      } else {
        c.parent = parent;
        std::copy(t, t + PKV_BLOCK_SIZE, c.tokens.begin());
        c.hash = block_hash(parent, t);
        c.on = true;
        c.children.clear();
        p->index.emplace(c.hash, id);
        if (parent >= 0) p->cached[parent].children.push_back(id);
        parent = id;
      }
    }
  }
  return PKV_OK;
}

pkv_status kv_block_swap(pkv_pool* from, pkv_pool* to, int32_t n, const int32_t* ids,
                         int32_t* out_ids, int32_t* pairs, int32_t* num_pairs) {
  if (!from || !to || from == to || n < 0 || !num_pairs) return PKV_ERR_INVALID;
  if (n > 0 && (!ids || !out_ids || !pairs)) return PKV_ERR_INVALID;
  // references per distinct block, in first-seen order; validated first
  std::unordered_map<int32_t, int32_t> occ;
  std::vector<int32_t> order;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || id >= from->num_blocks) return PKV_ERR_INVALID;
    int32_t& c = occ[id];
    if (c == 0) order.push_back(id);
    if (++c > from->ref[id]) return PKV_ERR_INVALID;
  }
  if (order.size() > num_free(to)) return PKV_ERR_OOM;
  std::unordered_map<int32_t, int32_t> dest;
  for (size_t k = 0; k < order.size(); ++k) {
    const int32_t id = order[k];
    const int32_t nid = pop_block(to);
    to->ref[nid] = occ[id];
    dest[id] = nid;
    pairs[2 * k] = id;
    pairs[2 * k + 1] = nid;
  }
  for (int32_t i = 0; i < n; ++i) out_ids[i] = dest[ids[i]];
  for (int32_t i = 0; i < n; ++i)
    if (--from->ref[ids[i]] == 0) release(from, ids[i]);
  *num_pairs = static_cast<int32_t>(order.size());
  return PKV_OK;
}

pkv_status pkv_window_release(pkv_pool* p, int32_t num_seqs, int32_t max_blocks_per_seq,
                              int32_t* tables, const int32_t* context_lens, int32_t window,
                              int32_t* table_updates, int32_t update_capacity,
                              int32_t* num_updates) {
  if (!p || num_seqs < 0 || max_blocks_per_seq < 1 || window < 1 || !num_updates ||
      update_capacity < 0)
    return PKV_ERR_INVALID;
  if (num_seqs > 0 && (!tables || !context_lens)) return PKV_ERR_INVALID;
  if (static_cast<int64_t>(num_seqs) * max_blocks_per_seq >= (int64_t(1) << 31))
    return PKV_ERR_INVALID;
  const int64_t cap_tokens = int64_t(max_blocks_per_seq) * PKV_BLOCK_SIZE;
  // blocks wholly before the window start: i < max(0, L - window) / 16
  auto first_kept = [&](int32_t s) {
    return std::max<int32_t>(0, context_lens[s] - window) / PKV_BLOCK_SIZE;
  };
  std::unordered_map<int32_t, int32_t> drops;
  int64_t count = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (context_lens[s] < 0 || context_lens[s] > cap_tokens) return PKV_ERR_INVALID;
    const int32_t* row = tables + int64_t(s) * max_blocks_per_seq;
    for (int32_t i = 0; i < first_kept(s); ++i) {
      const int32_t id = row[i];
      if (id < 0) continue;  // released before
      if (id >= p->num_blocks || ++drops[id] > p->ref[id]) return PKV_ERR_INVALID;
      ++count;
    }
  }
  if (count > update_capacity || (count > 0 && !table_updates)) return PKV_ERR_INVALID;
  int32_t nu = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    int32_t* row = tables + int64_t(s) * max_blocks_per_seq;
    for (int32_t i = 0; i < first_kept(s); ++i) {
      const int32_t id = row[i];
      if (id < 0) continue;
      if (--p->ref[id] == 0) release(p, id);
      row[i] = -1;
      table_updates[2 * nu] = s * max_blocks_per_seq + i;
      table_updates[2 * nu + 1] = -1;
      ++nu;
    }
  }
  *num_updates = nu;
  return PKV_OK;
}

pkv_status pkv_prefix_stats(const pkv_pool* p, int32_t* num_cached, int32_t* num_cached_free) {
  if (!p || !num_cached || !num_cached_free) return PKV_ERR_INVALID;
  *num_cached = static_cast<int32_t>(p->index.size());
  *num_cached_free = static_cast<int32_t>(p->lru.size());
  return PKV_OK;
}

}  // extern "C"
