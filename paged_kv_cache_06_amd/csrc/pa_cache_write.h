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

// Threads are laid out token-fastest over windows of `window` consecutive
// tokens: thread gid takes token (gid / (window * chunks * hkv)) * window +
// gid % window, so the lanes that store one chunk or one dimension are
// consecutive tokens.  New tokens of one sequence fill consecutive rows of a
// block, so those lanes' stores land side by side (a K chunk's rows are
// contiguous, and so is a transposed V row) and combine into few memory
// transactions; token-major order would scatter them one lane per
// transaction (3.6x slower on 8,192 chunk tokens).  A decode step's tokens,
// one per sequence, share no block: window 1 keeps each token's loads
// contiguous instead.
constexpr int kWindowLog2 = 4;
constexpr int kWindow = 1 << kWindowLog2;

struct TokenChunk {
  int64_t t;  // token
  int h;      // KV head
  int c;      // chunk of the head's dimensions
};

__device__ __forceinline__ TokenChunk token_chunk(int64_t gid, int hkv, int chunks,
                                                  int window) {
  // window is 1 or kWindow: a mask and a shift, not a 64-bit division
  const int shift = window == kWindow ? kWindowLog2 : 0;
  const int i = static_cast<int>(gid & (window - 1));
  const int64_t rest = gid >> shift;
  const int c = static_cast<int>(rest % chunks);
  const int64_t wh = rest / chunks;  // window index * hkv + head
  return TokenChunk{(wh / hkv) * window + i, static_cast<int>(wh % hkv), c};
}

__host__ __device__ inline int64_t padded_tokens(int32_t num_tokens, int window) {
  if (window != kWindow) return num_tokens;  // window 1
  return (static_cast<int64_t>(num_tokens) + kWindow - 1) >> kWindowLog2 << kWindowLog2;
}

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
  int32_t window = kWindow;  // tokens a thread layout interleaves (above)
  __host__ __device__ int64_t threads() const {
    return padded_tokens(num_tokens, window) * hkv *
           (head_dim * static_cast<int>(sizeof(E)) / 16);
  }
  __device__ void write(int64_t gid) const;
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
// (transposed within the block), in the token-fastest order above.  Threads
// past the end and skipped slots do nothing.
template <typename E>
__device__ __forceinline__ void write_token_chunk(const CacheWriteArgs<E>& w, int64_t gid) {
  constexpr int X = 16 / sizeof(E);
  const int chunks = w.head_dim / X;
  if (gid >= w.threads()) return;
  const TokenChunk tc = token_chunk(gid, w.hkv, chunks, w.window);
  const int64_t t = tc.t;
  const int h = tc.h, c = tc.c;
  if (t >= w.num_tokens) return;
  const int64_t th = t * w.hkv + h;  // token * hkv + head
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

template <typename E>
__device__ __forceinline__ void CacheWriteArgs<E>::write(int64_t gid) const {
  write_token_chunk<E>(*this, gid);
}

// ---- INT8 cache ("KV Cache for the intermediate", section "KV Cache
// Quantization") ----

template <typename Tag>
struct CacheWriteI8Args {
  const typename Tag::Bits* key;  // [T][Hkv][D]
  const typename Tag::Bits* value;
  int8_t* k_cache;                // INT8 layout of include/pa.h
  int8_t* v_cache;
  const int64_t* slots;
  const float* k_scale;           // [Hkv][D]
  const float* v_scale;
  int32_t num_tokens;
  int64_t num_slots;
  int32_t hkv, head_dim;
  int32_t window = kWindow;  // tokens a thread layout interleaves (above)
  __host__ __device__ int64_t threads() const {
    return padded_tokens(num_tokens, window) * hkv * (head_dim / 16);
  }
  __device__ void write(int64_t gid) const;
};

// Thread gid quantizes one 16-dimension chunk of one (token, head), in the
// token-fastest order above: codes clamp(rint(x / s), -127, 127) in fp32
// (NaN -> 0); the 16 K codes are one 16-byte store, the 16 V codes land 16
// bytes apart (the V layout groups 4 tokens of 4 dimension slices per lane
// of the decode).
template <typename Tag>
__device__ __forceinline__ void CacheWriteI8Args<Tag>::write(int64_t gid) const {
  const int chunks = head_dim / 16;
  if (gid >= threads()) return;
  const TokenChunk tc = token_chunk(gid, hkv, chunks, window);
  const int64_t t = tc.t;
  const int h = tc.h, c = tc.c;
  if (t >= num_tokens) return;
  const int64_t th = t * hkv + h;  // token * hkv + head
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t b = slot / kBlock;
  const int r = static_cast<int>(slot % kBlock);
  const int64_t src = th * head_dim + static_cast<int64_t>(c) * 16;
  const float* ks = k_scale + static_cast<int64_t>(h) * head_dim + c * 16;
  const float* vs = v_scale + static_cast<int64_t>(h) * head_dim + c * 16;
  const int64_t slab = (b * hkv + h) * static_cast<int64_t>(head_dim) * kBlock + (c / 4) * 1024;

  auto code = [](float x, float s) {
    float y = rintf(__fdiv_rn(x, s));
    y = (y != y) ? 0.f : fminf(fmaxf(y, -127.f), 127.f);
    return static_cast<uint32_t>(static_cast<int32_t>(y)) & 0xFFu;
  };
  uint32_t kw[4] = {0, 0, 0, 0};
#pragma unroll
  for (int e = 0; e < 16; ++e) kw[e / 4] |= code(Tag::to_f32(key[src + e]), ks[e]) << (8 * (e % 4));
  *reinterpret_cast<uint4*>(k_cache + slab + ((c % 4) * 16 + r) * 16) =
      make_uint4(kw[0], kw[1], kw[2], kw[3]);
  int8_t* vdst = v_cache + slab + ((r / 4) * 16) * 16 + (c % 4) * 4 + r % 4;
#pragma unroll
  for (int e = 0; e < 16; ++e)
    vdst[e * 16] = static_cast<int8_t>(code(Tag::to_f32(value[src + e]), vs[e]));
}

}  // namespace
}  // namespace pa
