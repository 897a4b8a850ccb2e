// Writing the K and V of new tokens into their cache slots (only the new
// token's K/V are computed each step, everything older is read back: "KV
// Cache and PagedAttention: why your LLM server slows down", second article,
// section "What is the KV cache?").  Used by pa_reshape_and_cache and by the
// fused decode step, which writes the tokens in the same launch as it plans
// the decode.
#pragma once

#include "pa_common.h"

namespace pa {
namespace {

template <typename E>
struct CacheWriteArgs {
  const E* key;    // [T][Hkv][D]
  const E* value;
  E* k_cache;      // [NB][Hkv][D/X][16][X]
  E* v_cache;      // [NB][Hkv][D][16]
  const int64_t* slots;
  int32_t num_tokens;
  int64_t num_slots;
  int32_t hkv, head_dim;
};

template <typename E>
CacheWriteArgs<E> cache_write_args(const void* key, const void* value, void* k_cache,
                                   void* v_cache, const int64_t* slots, int32_t num_tokens,
                                   int64_t num_slots, int32_t hkv, int32_t head_dim) {
  return CacheWriteArgs<E>{static_cast<const E*>(key), static_cast<const E*>(value),
                           static_cast<E*>(k_cache), static_cast<E*>(v_cache), slots, num_tokens,
                           num_slots, hkv, head_dim};
}

// Thread gid moves one 16-byte chunk of D of one (token, head): a 16-byte K
// store (token rows of a chunk are contiguous) and X element stores of V
// (transposed within the block).  Threads past the end and skipped slots do
// nothing.
template <typename E>
__device__ __forceinline__ void write_token_chunk(const CacheWriteArgs<E>& w, int64_t gid) {
  constexpr int X = 16 / sizeof(E);
  const int chunks = w.head_dim / X;
  const int64_t total = static_cast<int64_t>(w.num_tokens) * w.hkv * chunks;
  if (gid >= total) return;
  const int c = static_cast<int>(gid % chunks);
  const int64_t th = gid / chunks;  // token * hkv + head
  const int h = static_cast<int>(th % w.hkv);
  const int64_t t = th / w.hkv;
  const int64_t slot = w.slots[t];
  if (slot < 0 || slot >= w.num_slots) return;
  const int64_t b = slot / kBlock;
  const int r = static_cast<int>(slot % kBlock);
  const int64_t src = th * w.head_dim + static_cast<int64_t>(c) * X;
  const int64_t head_base = (b * w.hkv + h) * static_cast<int64_t>(w.head_dim) * kBlock;

  const uint4 kv = *reinterpret_cast<const uint4*>(w.key + src);
  *reinterpret_cast<uint4*>(w.k_cache + head_base + (static_cast<int64_t>(c) * kBlock + r) * X) =
      kv;

  union {
    uint4 v;
    E e[X];
  } vv;
  vv.v = *reinterpret_cast<const uint4*>(w.value + src);
  E* vdst = w.v_cache + head_base + static_cast<int64_t>(c) * X * kBlock + r;
#pragma unroll
  for (int i = 0; i < X; ++i) vdst[i * kBlock] = vv.e[i];
}

}  // namespace
}  // namespace pa
