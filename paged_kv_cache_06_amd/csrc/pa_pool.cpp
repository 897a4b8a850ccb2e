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
// block is the next one handed out.  No call allocates after pa_pool_create.
#include <cstdlib>
#include <cstring>
#include <new>

#include "pa.h"

struct pa_pool {
  int32_t num_blocks;
  int32_t top;         // number of ids on the free stack
  int64_t copies;
  int32_t* free_stack; // free_stack[top-1] is handed out next
  int32_t* refcount;
};

namespace {

inline int64_t blocks_for(int64_t tokens) { return (tokens + PA_BLOCK_SIZE - 1) / PA_BLOCK_SIZE; }

inline bool held(const pa_pool* p, int32_t b) {
  return b >= 0 && b < p->num_blocks && p->refcount[b] > 0;
}

inline int32_t pop(pa_pool* p) {
  int32_t b = p->free_stack[--p->top];
  p->refcount[b] = 1;
  return b;
}

inline void drop(pa_pool* p, int32_t b) {
  if (--p->refcount[b] == 0) p->free_stack[p->top++] = b;
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
    default: return "unknown status";
  }
}

pa_status pa_pool_create(int32_t num_blocks, const int32_t* free_order, pa_pool** out) {
  if (!out || num_blocks <= 0) return PA_ERR_INVALID_ARG;
  *out = nullptr;
  pa_pool* p = new (std::nothrow) pa_pool;
  if (!p) return PA_ERR_INVALID_ARG;
  p->num_blocks = num_blocks;
  p->copies = 0;
  p->free_stack = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * (size_t)num_blocks));
  p->refcount = static_cast<int32_t*>(std::calloc((size_t)num_blocks, sizeof(int32_t)));
  if (!p->free_stack || !p->refcount) {
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
  std::memset(p->refcount, 0, sizeof(int32_t) * (size_t)num_blocks);
  p->top = num_blocks;
  *out = p;
  return PA_OK;
}

void pa_pool_destroy(pa_pool* p) {
  if (!p) return;
  std::free(p->free_stack);
  std::free(p->refcount);
  delete p;
}

pa_status pa_alloc(pa_pool* p, int32_t* block_out) {
  if (!p || !block_out) return PA_ERR_INVALID_ARG;
  if (p->top == 0) return PA_ERR_OUT_OF_BLOCKS;
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
  if (p->top < fresh + (cow ? 1 : 0)) return PA_ERR_OUT_OF_BLOCKS;
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

int32_t pa_refcount(const pa_pool* p, int32_t b) {
  if (!p || b < 0 || b >= p->num_blocks) return -1;
  return p->refcount[b];
}

int32_t pa_num_free(const pa_pool* p) { return p ? p->top : -1; }

pa_status pa_pool_stats(const pa_pool* p, pa_pool_stats_t* out) {
  if (!p || !out) return PA_ERR_INVALID_ARG;
  int32_t used = 0, shared = 0;
  for (int32_t b = 0; b < p->num_blocks; ++b) {
    used += p->refcount[b] > 0;
    shared += p->refcount[b] > 1;
  }
  out->num_blocks = p->num_blocks;
  out->num_free = p->top;
  out->num_used = used;
  out->num_shared = shared;
  out->copies = p->copies;
  return PA_OK;
}

int64_t pa_blocks_for_bytes(int64_t bytes, int32_t layers, int32_t kv_heads, int32_t head_dim,
                            int32_t elem_bytes) {
  if (bytes <= 0 || layers <= 0 || kv_heads <= 0 || head_dim <= 0 || elem_bytes <= 0) return -1;
  const int64_t per_block =
      2LL * layers * PA_BLOCK_SIZE * (int64_t)kv_heads * head_dim * elem_bytes;
  return bytes / per_block;
}

}  // extern "C"
