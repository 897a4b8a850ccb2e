// Host block pool: ids and reference counts of the fixed 16-slot KV blocks.
//
// Blocks are handed out on demand and go back to the pool when their last
// holder lets go ("PagedAttention for the professional", sections "Beginner's
// example: library shelves" and "The scientific explanation"); blocks of a
// shared prompt carry one reference per sharer and are copied when a sharer
// writes into them ("KV Cache and PagedAttention: why your LLM server slows
// down", section "How PagedAttention fixes this").
//
// The free list is a stack in a flat array: pushes and pops are O(1), a freed
// block is the next one handed out.
//
// Prefix cache: requests that start with the same tokens (one system prompt)
// reuse the blocks that hold them ("PagedAttention for the professional", the
// serve-command section on prefix caching), and cached blocks keep room in the
// pool until it is needed (same page, trade-offs section).  A full block is
// entered under the key (serial number of the entry of the block before it, 0
// for a sequence's first block; its 16 token ids).  Serial numbers are never
// reused, so a key stands for one exact token prefix -- the map compares whole
// keys, nothing is hashed away -- and the entries below an evicted block become
// unreachable instead of wrong.  A cached block whose count drops to 0 joins the
// tail of an intrusive LRU list; allocation pops the uncached stack first and
// then evicts the list's head.  Only registering allocates (hash-map nodes).
#include <array>
#include <cstdlib>
#include <cstring>
#include <new>
#include <unordered_map>

#include "pa.h"

namespace {

struct Key {
  uint64_t parent;
  std::array<int32_t, PA_BLOCK_SIZE> tokens;
  bool operator==(const Key& o) const { return parent == o.parent && tokens == o.tokens; }
};

struct KeyHash {
  size_t operator()(const Key& k) const {
    // FNV-1a over the parent serial and the token ids (bucket choice only)
    uint64_t h = 1469598103934665603ull;
    auto mix = [&h](uint64_t v) {
      for (int i = 0; i < 8; ++i) {
        h ^= (v >> (8 * i)) & 0xff;
        h *= 1099511628211ull;
      }
    };
    mix(k.parent);
    for (int32_t t : k.tokens) mix(static_cast<uint32_t>(t));
    return static_cast<size_t>(h);
  }
};

}  // namespace

struct pa_pool {
  int32_t num_blocks;
  int32_t top;         // number of ids on the free stack
  int64_t copies;
  int32_t* free_stack; // free_stack[top-1] is handed out next
  int32_t* refcount;
  // prefix cache
  uint64_t* serial;    // serial number of the block's cache entry, 0 = not cached
  Key* key;            // the block's key while cached
  int32_t* lru_prev;   // LRU list of cached blocks at count 0 (head = oldest)
  int32_t* lru_next;
  int32_t lru_head, lru_tail, lru_len;
  int32_t cached;
  uint64_t next_serial;
  int64_t prefix_hits;
  std::unordered_map<Key, int32_t, KeyHash>* index;
};

namespace {

inline int64_t blocks_for(int64_t tokens) { return (tokens + PA_BLOCK_SIZE - 1) / PA_BLOCK_SIZE; }

inline bool held(const pa_pool* p, int32_t b) {
  return b >= 0 && b < p->num_blocks && p->refcount[b] > 0;
}

void lru_unlink(pa_pool* p, int32_t b) {
  const int32_t pr = p->lru_prev[b], nx = p->lru_next[b];
  if (pr >= 0) p->lru_next[pr] = nx; else p->lru_head = nx;
  if (nx >= 0) p->lru_prev[nx] = pr; else p->lru_tail = pr;
  p->lru_prev[b] = p->lru_next[b] = -1;
  --p->lru_len;
}

void lru_push_back(pa_pool* p, int32_t b) {
  p->lru_prev[b] = p->lru_tail;
  p->lru_next[b] = -1;
  if (p->lru_tail >= 0) p->lru_next[p->lru_tail] = b; else p->lru_head = b;
  p->lru_tail = b;
  ++p->lru_len;
}

void uncache(pa_pool* p, int32_t b) {
  p->index->erase(p->key[b]);
  p->serial[b] = 0;
  --p->cached;
}

inline int32_t available(const pa_pool* p) { return p->top + p->lru_len; }

// caller has checked available(p) > 0
int32_t pop(pa_pool* p) {
  int32_t b;
  if (p->top > 0) {
    b = p->free_stack[--p->top];
  } else {
    b = p->lru_head;
    lru_unlink(p, b);
    uncache(p, b);
  }
  p->refcount[b] = 1;
  return b;
}

inline void drop(pa_pool* p, int32_t b) {
  if (--p->refcount[b] == 0) {
    if (p->serial[b] != 0) lru_push_back(p, b);
    else p->free_stack[p->top++] = b;
  }
}

inline void take_ref(pa_pool* p, int32_t b) {
  if (p->refcount[b] == 0) lru_unlink(p, b);
  ++p->refcount[b];
}

Key make_key(uint64_t parent, const int32_t* tokens) {
  Key k;
  k.parent = parent;
  std::memcpy(k.tokens.data(), tokens, sizeof(int32_t) * PA_BLOCK_SIZE);
  return k;
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_OUT_OF_BLOCKS: return "out of blocks";
    case PA_ERR_BAD_BLOCK: return "bad block id";
    case PA_ERR_UNSUPPORTED: return "unsupported";
    case PA_ERR_DEVICE: return "device error";
    case PA_ERR_WORKSPACE: return "workspace too small";
    case PA_ERR_HOST_MEMORY: return "host memory allocation failed";
    default: return "unknown status";
  }
}

pa_status pa_pool_create(int32_t num_blocks, const int32_t* free_order, pa_pool** out) {
  if (!out || num_blocks <= 0) return PA_ERR_INVALID_ARG;
  *out = nullptr;
  pa_pool* p = new (std::nothrow) pa_pool;
  if (!p) return PA_ERR_INVALID_ARG;
  const size_t nb = static_cast<size_t>(num_blocks);
  p->num_blocks = num_blocks;
  p->copies = 0;
  p->free_stack = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * nb));
  p->refcount = static_cast<int32_t*>(std::calloc(nb, sizeof(int32_t)));
  p->serial = static_cast<uint64_t*>(std::calloc(nb, sizeof(uint64_t)));
  p->key = static_cast<Key*>(std::malloc(sizeof(Key) * nb));
  p->lru_prev = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * nb));
  p->lru_next = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * nb));
  p->lru_head = p->lru_tail = -1;
  p->lru_len = 0;
  p->cached = 0;
  p->next_serial = 1;
  p->prefix_hits = 0;
  p->index = new (std::nothrow) std::unordered_map<Key, int32_t, KeyHash>();
  if (!p->free_stack || !p->refcount || !p->serial || !p->key || !p->lru_prev || !p->lru_next ||
      !p->index) {
    pa_pool_destroy(p);
    return PA_ERR_INVALID_ARG;
  }
  // stack bottom = last id of the order, top = first id; check it is a permutation
  for (int32_t i = 0; i < num_blocks; ++i) {
    int32_t b = free_order ? free_order[i] : i;
    if (b < 0 || b >= num_blocks || p->refcount[b] != 0) {
      pa_pool_destroy(p);
      return PA_ERR_INVALID_ARG;
    }
    p->refcount[b] = -1;  // seen marker
    p->free_stack[num_blocks - 1 - i] = b;
  }
  std::memset(p->refcount, 0, sizeof(int32_t) * nb);
  for (size_t b = 0; b < nb; ++b) p->lru_prev[b] = p->lru_next[b] = -1;
  p->top = num_blocks;
  *out = p;
  return PA_OK;
}

void pa_pool_destroy(pa_pool* p) {
  if (!p) return;
  std::free(p->free_stack);
  std::free(p->refcount);
  std::free(p->serial);
  std::free(p->key);
  std::free(p->lru_prev);
  std::free(p->lru_next);
  delete p->index;
  delete p;
}

pa_status pa_alloc(pa_pool* p, int32_t* block_out) {
  if (!p || !block_out) return PA_ERR_INVALID_ARG;
  if (available(p) == 0) return PA_ERR_OUT_OF_BLOCKS;
  *block_out = pop(p);
  return PA_OK;
}

pa_status pa_incref(pa_pool* p, int32_t b) {
  if (!p) return PA_ERR_INVALID_ARG;
  if (!held(p, b)) return PA_ERR_BAD_BLOCK;
  ++p->refcount[b];
  return PA_OK;
}

pa_status pa_free(pa_pool* p, int32_t b) {
  if (!p) return PA_ERR_INVALID_ARG;
  if (!held(p, b)) return PA_ERR_BAD_BLOCK;
  drop(p, b);
  return PA_OK;
}

pa_status pa_fork(pa_pool* p, const int32_t* table, int32_t n) {
  if (!p || n < 0 || (n > 0 && !table)) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (!held(p, table[i])) return PA_ERR_BAD_BLOCK;
  for (int32_t i = 0; i < n; ++i) ++p->refcount[table[i]];
  return PA_OK;
}

pa_status pa_free_table(pa_pool* p, const int32_t* table, int32_t n) {
  if (!p || n < 0 || (n > 0 && !table)) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) {
    pa_status st = pa_free(p, table[i]);
    if (st != PA_OK) return st;
  }
  return PA_OK;
}

pa_status pa_append_slots(pa_pool* p, int32_t* row, int32_t* nblocks, int32_t max_blocks,
                          int32_t pos, int32_t n, int64_t* slots, int32_t* cow_src,
                          int32_t* cow_dst) {
  if (!p || !nblocks || pos < 0 || n < 0 || max_blocks < 0) return PA_ERR_INVALID_ARG;
  if (*nblocks != blocks_for(pos) || *nblocks > max_blocks) return PA_ERR_INVALID_ARG;
  if (cow_src) *cow_src = -1;
  if (cow_dst) *cow_dst = -1;
  if (n == 0) return PA_OK;
  if (!row || !slots || !cow_src || !cow_dst) return PA_ERR_INVALID_ARG;
  const int64_t after = blocks_for((int64_t)pos + n);
  if (after > max_blocks) return PA_ERR_INVALID_ARG;
  const int32_t fresh = (int32_t)(after - *nblocks);
  const int32_t cur = pos / PA_BLOCK_SIZE;
  if (pos % PA_BLOCK_SIZE != 0 && !held(p, row[cur])) return PA_ERR_BAD_BLOCK;
  const bool cow = (pos % PA_BLOCK_SIZE) != 0 && p->refcount[row[cur]] > 1;
  if (available(p) < fresh + (cow ? 1 : 0)) return PA_ERR_OUT_OF_BLOCKS;
  if (cow) {
    const int32_t src = row[cur];
    const int32_t dst = pop(p);
    drop(p, src);  // still held by the other sharers
    row[cur] = dst;
    *cow_src = src;
    *cow_dst = dst;
    ++p->copies;
  }
  for (int32_t i = 0; i < fresh; ++i) row[(*nblocks)++] = pop(p);
  for (int32_t i = 0; i < n; ++i) {
    const int64_t q = (int64_t)pos + i;
    slots[i] = (int64_t)row[q / PA_BLOCK_SIZE] * PA_BLOCK_SIZE + q % PA_BLOCK_SIZE;
  }
  return PA_OK;
}

pa_status pa_swap_blocks(pa_pool* src, pa_pool* dst, const int32_t* blocks, int32_t n,
                         int64_t* pairs_out) {
  if (!src || !dst || src == dst || n < 0 || (n > 0 && (!blocks || !pairs_out)))
    return PA_ERR_INVALID_ARG;
  // every listed block must be held, one reference per listing: take the
  // references off tentatively, then put them back
  int32_t ok = 0;
  while (ok < n && held(src, blocks[ok])) --src->refcount[blocks[ok++]];
  for (int32_t i = 0; i < ok; ++i) ++src->refcount[blocks[i]];
  if (ok < n) return PA_ERR_BAD_BLOCK;
  if (available(dst) < n) return PA_ERR_OUT_OF_BLOCKS;
  for (int32_t i = 0; i < n; ++i) {
    pairs_out[2 * i] = blocks[i];
    pairs_out[2 * i + 1] = pop(dst);
  }
  for (int32_t i = 0; i < n; ++i) drop(src, blocks[i]);
  return PA_OK;
}

int32_t pa_refcount(const pa_pool* p, int32_t b) {
  if (!p || b < 0 || b >= p->num_blocks) return -1;
  return p->refcount[b];
}

int32_t pa_num_free(const pa_pool* p) { return p ? available(p) : -1; }

pa_status pa_pool_stats(const pa_pool* p, pa_pool_stats_t* out) {
  if (!p || !out) return PA_ERR_INVALID_ARG;
  int32_t used = 0, shared = 0;
  for (int32_t b = 0; b < p->num_blocks; ++b) {
    used += p->refcount[b] > 0;
    shared += p->refcount[b] > 1;
  }
  out->num_blocks = p->num_blocks;
  out->num_free = available(p);
  out->num_used = used;
  out->num_shared = shared;
  out->copies = p->copies;
  out->num_cached = p->cached;
  out->num_evictable = p->lru_len;
  out->prefix_hits = p->prefix_hits;
  return PA_OK;
}

pa_status pa_prefix_match(pa_pool* p, const int32_t* tokens, int32_t num_tokens,
                          int32_t* table_out, int32_t max_blocks, int32_t* num_matched) {
  if (!p || !num_matched || num_tokens < 0 || max_blocks < 0 || (num_tokens > 0 && !tokens))
    return PA_ERR_INVALID_ARG;
  *num_matched = 0;
  const int32_t chunks = num_tokens / PA_BLOCK_SIZE;
  if (chunks > 0 && max_blocks > 0 && !table_out) return PA_ERR_INVALID_ARG;
  uint64_t parent = 0;
  int32_t n = 0;
  while (n < chunks && n < max_blocks) {
    auto it = p->index->find(make_key(parent, tokens + (size_t)n * PA_BLOCK_SIZE));
    if (it == p->index->end()) break;
    const int32_t b = it->second;
    table_out[n++] = b;
    parent = p->serial[b];
  }
  for (int32_t i = 0; i < n; ++i) take_ref(p, table_out[i]);
  p->prefix_hits += n;
  *num_matched = n;
  return PA_OK;
}

pa_status pa_prefix_register(pa_pool* p, const int32_t* table_row, int32_t nblocks,
                             const int32_t* tokens, int32_t num_tokens, int32_t* num_added) {
  if (!p || nblocks < 0 || num_tokens < 0 || (num_tokens > 0 && !tokens)) return PA_ERR_INVALID_ARG;
  const int32_t chunks = num_tokens / PA_BLOCK_SIZE;
  if (chunks > nblocks || (chunks > 0 && !table_row)) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < chunks; ++i) {
    const int32_t b = table_row[i];
    if (!held(p, b)) return PA_ERR_BAD_BLOCK;
    if (p->serial[b] != 0 &&
        std::memcmp(p->key[b].tokens.data(), tokens + (size_t)i * PA_BLOCK_SIZE,
                    sizeof(int32_t) * PA_BLOCK_SIZE) != 0)
      return PA_ERR_INVALID_ARG;
  }
  int32_t added = 0;
  uint64_t parent = 0;
  const uint64_t first_serial = p->next_serial;
  for (int32_t i = 0; i < chunks; ++i) {
    const int32_t b = table_row[i];
    if (p->serial[b] == 0) {
      const Key k = make_key(parent, tokens + (size_t)i * PA_BLOCK_SIZE);
      auto it = p->index->find(k);
      if (it != p->index->end()) {  // same prefix cached in another block
        parent = p->serial[it->second];
        continue;
      }
      try {
        p->index->emplace(k, b);
      } catch (...) {  // out of host memory: undo this call's entries
        for (int32_t j = 0; j < i; ++j) {
          const int32_t c = table_row[j];
          if (p->serial[c] >= first_serial) uncache(p, c);
        }
        p->next_serial = first_serial;
        if (num_added) *num_added = 0;
        return PA_ERR_HOST_MEMORY;
      }
      p->key[b] = k;
      p->serial[b] = p->next_serial++;
      ++p->cached;
      ++added;
    }
    parent = p->serial[b];
  }
  if (num_added) *num_added = added;
  return PA_OK;
}

int64_t pa_blocks_for_bytes(int64_t bytes, int32_t layers, int32_t kv_heads, int32_t head_dim,
                            int32_t elem_bytes) {
  if (bytes <= 0 || layers <= 0 || kv_heads <= 0 || head_dim <= 0 || elem_bytes <= 0) return -1;
  const int64_t per_block =
      2LL * layers * PA_BLOCK_SIZE * (int64_t)kv_heads * head_dim * elem_bytes;
  return bytes / per_block;
}

pa_status pa_shared_prefix_groups(const int32_t* tables, const int32_t* nblocks, int32_t num_seqs,
                                  int32_t max_blocks, int32_t min_blocks, int32_t* prefix_seqs,
                                  int32_t* prefix_start, int32_t* prefix_blocks,
                                  int32_t* num_groups, int32_t* num_members) {
  if (num_seqs < 0 || max_blocks <= 0 || min_blocks < 1 || !num_groups || !num_members)
    return PA_ERR_INVALID_ARG;
  if (num_seqs > 0 && (!tables || !nblocks || !prefix_seqs || !prefix_start || !prefix_blocks))
    return PA_ERR_INVALID_ARG;
  *num_groups = 0;
  *num_members = 0;
  // sequences by their first block, in sequence order
  std::unordered_map<int32_t, int32_t> leader_of;  // first block -> first sequence holding it
  int32_t* next = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * (num_seqs > 0 ? num_seqs : 1)));
  int32_t* last = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * (num_seqs > 0 ? num_seqs : 1)));
  if (!next || !last) {
    std::free(next);
    std::free(last);
    return PA_ERR_HOST_MEMORY;
  }
  try {
    for (int32_t s = 0; s < num_seqs; ++s) {
      next[s] = -1;
      last[s] = s;
      const int32_t nb = nblocks[s];
      if (nb < 1 || nb > max_blocks) continue;
      const int32_t first = tables[static_cast<int64_t>(s) * max_blocks];
      auto it = leader_of.find(first);
      if (it == leader_of.end()) {
        leader_of.emplace(first, s);
      } else {
        const int32_t l = it->second;
        next[last[l]] = s;  // append to the leader's chain
        last[l] = s;
      }
    }
  } catch (...) {
    std::free(next);
    std::free(last);
    return PA_ERR_HOST_MEMORY;
  }
  int32_t g = 0, m = 0;
  for (int32_t l = 0; l < num_seqs; ++l) {
    const int32_t nb = nblocks[l];
    if (nb < 1 || nb > max_blocks || next[l] < 0) continue;
    const int32_t* lead = tables + static_cast<int64_t>(l) * max_blocks;
    // is l the head of its chain (the first sequence with its first block)?
    auto it = leader_of.find(lead[0]);
    if (it == leader_of.end() || it->second != l) continue;
    int32_t shared = nb;
    for (int32_t s = next[l]; s >= 0; s = next[s]) {
      const int32_t* row = tables + static_cast<int64_t>(s) * max_blocks;
      const int32_t lim = shared < nblocks[s] ? shared : nblocks[s];
      int32_t k = 0;
      while (k < lim && row[k] == lead[k]) ++k;
      shared = k;
    }
    if (shared < min_blocks) continue;
    prefix_start[g] = m;
    prefix_blocks[g] = shared;
    for (int32_t s = l; s >= 0; s = next[s]) prefix_seqs[m++] = s;
    ++g;
  }
  prefix_start[g] = m;
  std::free(next);
  std::free(last);
  *num_groups = g;
  *num_members = m;
  return PA_OK;
}

}  // extern "C"
