// Cache writes and block copies.
//
// reshape_and_cache stores the K and V of new tokens into their slots: only the
// new token's K/V are computed each step, everything older is read back ("KV
// Cache and PagedAttention: why your LLM server slows down", second article,
// section "What is the KV cache?").  copy_blocks duplicates shared blocks
// before a sharer writes into them (same page, section "How PagedAttention
// fixes this": shared prefix with copy-on-write).
//
// Both are small and memory-latency bound; every lane moves 16 bytes per
// access.  K rows keep the 16-byte chunks of one token contiguous (layout
// [blocks][Hkv][D/X][16][X]); V is stored transposed per block
// ([blocks][Hkv][D][16]) so that the decode kernel can feed the 16 token
// values of one dimension straight into the matrix cores.
#include "pa_cache_write.h"

namespace pa {
namespace {

// One thread per (token, head, 16-byte chunk of D).
template <typename E>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(CacheWriteArgs<E> w) {
  w.template write<false>(static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x);
}

// INT8 cache: one thread per (token, head, 16-dimension chunk).
template <typename Tag>
__global__ __launch_bounds__(256) void reshape_and_cache_i8_kernel(CacheWriteI8Args<Tag> w) {
  w.template write<false>(static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x);
}

// grid.x = pair * 2 + (0: K, 1: V); grid.y splits the block's bytes.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ k_cache,
                                                          uint4* __restrict__ v_cache,
                                                          const int64_t* __restrict__ pairs,
                                                          int32_t num_blocks, int64_t vec_per_block) {
  const int pair = blockIdx.x >> 1;
  uint4* cache = (blockIdx.x & 1) ? v_cache : k_cache;
  const int64_t src = pairs[2 * pair];
  const int64_t dst = pairs[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const uint4* s = cache + src * vec_per_block;
  uint4* d = cache + dst * vec_per_block;
  constexpr int kPerThread = 4;
  const int64_t base = static_cast<int64_t>(blockIdx.y) * 256 * kPerThread + threadIdx.x;
  uint4 tmp[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int64_t j = base + i * 256;
    if (j < vec_per_block) tmp[i] = s[j];
  }
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int64_t j = base + i * 256;
    if (j < vec_per_block) stream_store16(d + j, tmp[i]);
  }
}

// Blocks between two caches of the same shape, e.g. device memory and pinned
// host memory (moving blocks between tiers, "KV Cache and PagedAttention: why
// your LLM server slows down": fine-grained eviction of small pages to the CPU).
// grid.x = pair * 2 + (0: K, 1: V); grid.y splits the block's bytes.  Every
// thread keeps 4 loads of 16 bytes in flight, which the host link's latency
// needs.
__global__ __launch_bounds__(256) void transfer_blocks_kernel(
    const uint4* __restrict__ src_k, const uint4* __restrict__ src_v, uint4* __restrict__ dst_k,
    uint4* __restrict__ dst_v, const int64_t* __restrict__ pairs, int32_t src_blocks,
    int32_t dst_blocks, int64_t vec_per_block) {
  const int pair = blockIdx.x >> 1;
  const uint4* sc = (blockIdx.x & 1) ? src_v : src_k;
  uint4* dc = (blockIdx.x & 1) ? dst_v : dst_k;
  const int64_t src = pairs[2 * pair];
  const int64_t dst = pairs[2 * pair + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const uint4* s = sc + src * vec_per_block;
  uint4* d = dc + dst * vec_per_block;
  constexpr int kPerThread = 4;
  const int64_t base = static_cast<int64_t>(blockIdx.y) * 256 * kPerThread + threadIdx.x;
  uint4 tmp[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int64_t j = base + i * 256;
    if (j < vec_per_block) tmp[i] = s[j];
  }
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int64_t j = base + i * 256;
    if (j < vec_per_block) d[j] = tmp[i];
  }
}

// The address the device uses for `p`: device memory as it is, pinned host
// memory through its device mapping; nullptr for memory the device cannot
// reach (pageable host memory).
void* device_address(const void* p) {
  hipPointerAttribute_t attr;
  if (!p || hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the error the query leaves on pageable memory
    return nullptr;
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeHost) return nullptr;
  return attr.devicePointer;
}

bool cache_shape_ok(int32_t num_blocks, int32_t hkv, int32_t head_dim, pa_dtype dt) {
  if (dt == PA_I8) return num_blocks > 0 && hkv > 0 && head_dim > 0 && head_dim % 64 == 0 &&
                          head_dim <= 512;
  if (!valid_dtype(dt) || num_blocks <= 0 || hkv <= 0 || head_dim <= 0) return false;
  const int x = 16 / elem_bytes(dt);
  return head_dim % x == 0 && head_dim <= 512;
}

}  // namespace
}  // namespace pa

extern "C" {

pa_status pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                               const int64_t* slot_mapping, int32_t num_tokens,
                               int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                               pa_dtype dtype, void* stream) {
  using namespace pa;
  if (num_tokens < 0 || !cache_shape_ok(num_blocks, num_kv_heads, head_dim, dtype))
    return valid_dtype(dtype) ? PA_ERR_INVALID_ARG : PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * kBlock;
  const auto w32 = cache_write_args<float>(key, value, k_cache, v_cache, slot_mapping,
                                           num_tokens, num_slots, num_kv_heads, head_dim);
  const auto w16 = cache_write_args<uint16_t>(key, value, k_cache, v_cache, slot_mapping,
                                              num_tokens, num_slots, num_kv_heads, head_dim);
  const int64_t grid = ((dtype == PA_F32 ? w32.threads() : w16.threads()) + 255) / 256;
  if (grid > 0x7fffffff) return PA_ERR_INVALID_ARG;
  const dim3 g(static_cast<uint32_t>(grid)), b(256);
  if (dtype == PA_F32)
    return launch_kernel(PA_KERNEL_RESHAPE_AND_CACHE, reshape_and_cache_kernel<float>, g, b, 0,
                         st, w32);
  return launch_kernel(PA_KERNEL_RESHAPE_AND_CACHE, reshape_and_cache_kernel<uint16_t>, g, b, 0,
                       st, w16);
}

pa_status pa_reshape_and_cache_int8(const void* key, const void* value, void* k_cache,
                                    void* v_cache, const int64_t* slot_mapping,
                                    const float* k_scale, const float* v_scale,
                                    int32_t num_tokens, int32_t num_blocks,
                                    int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                                    void* stream) {
  using namespace pa;
  if (!valid_dtype(dtype)) return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || !cache_shape_ok(num_blocks, num_kv_heads, head_dim, PA_I8))
    return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping || !k_scale || !v_scale)
    return PA_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * kBlock;
  // thread count: every CacheWriteI8Args<Tag> of these sizes has the same one
  const int64_t threads = CacheWriteI8Args<F32T>{nullptr, nullptr, nullptr, nullptr, nullptr,
                                                 nullptr, nullptr, num_tokens, num_slots,
                                                 num_kv_heads, head_dim}
                              .threads();
  const int64_t grid = (threads + 255) / 256;
  if (grid > 0x7fffffff) return PA_ERR_INVALID_ARG;
  int8_t* kc = static_cast<int8_t*>(k_cache);
  int8_t* vc = static_cast<int8_t*>(v_cache);
  const dim3 g(static_cast<uint32_t>(grid)), b(256);
  constexpr int kKind = PA_KERNEL_RESHAPE_AND_CACHE;
  if (dtype == PA_F32)
    return launch_kernel(kKind, reshape_and_cache_i8_kernel<F32T>, g, b, 0, st,
                         CacheWriteI8Args<F32T>{static_cast<const float*>(key),
                                                static_cast<const float*>(value), kc, vc,
                                                slot_mapping, k_scale, v_scale, num_tokens,
                                                num_slots, num_kv_heads, head_dim});
  if (dtype == PA_BF16)
    return launch_kernel(kKind, reshape_and_cache_i8_kernel<BF16T>, g, b, 0, st,
                         CacheWriteI8Args<BF16T>{static_cast<const uint16_t*>(key),
                                                 static_cast<const uint16_t*>(value), kc, vc,
                                                 slot_mapping, k_scale, v_scale, num_tokens,
                                                 num_slots, num_kv_heads, head_dim});
  return launch_kernel(kKind, reshape_and_cache_i8_kernel<F16T>, g, b, 0, st,
                       CacheWriteI8Args<F16T>{static_cast<const uint16_t*>(key),
                                              static_cast<const uint16_t*>(value), kc, vc,
                                              slot_mapping, k_scale, v_scale, num_tokens,
                                              num_slots, num_kv_heads, head_dim});
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_pairs,
                         int32_t num_pairs, int32_t num_blocks, int32_t num_kv_heads,
                         int32_t head_dim, pa_dtype dtype, void* stream) {
  using namespace pa;
  if (num_pairs < 0 || !cache_shape_ok(num_blocks, num_kv_heads, head_dim, dtype))
    return valid_dtype(dtype) || dtype == PA_I8 ? PA_ERR_INVALID_ARG : PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_pairs) return PA_ERR_INVALID_ARG;
  if (num_pairs > (0x7fffffff >> 1)) return PA_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t bytes = static_cast<int64_t>(num_kv_heads) * kBlock * head_dim * elem_bytes(dtype);
  const int64_t vec = bytes / 16;
  const int64_t gy = (vec + 1023) / 1024;
  return launch_kernel(PA_KERNEL_COPY_BLOCKS, copy_blocks_kernel,
                       dim3(2 * num_pairs, static_cast<uint32_t>(gy)), dim3(256), 0, st,
                       static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), block_pairs,
                       num_blocks, vec);
}

pa_status pa_transfer_blocks(const void* src_k, const void* src_v, int32_t src_num_blocks,
                             void* dst_k, void* dst_v, int32_t dst_num_blocks,
                             const int64_t* block_pairs, int32_t num_pairs, int32_t num_kv_heads,
                             int32_t head_dim, pa_dtype dtype, void* stream) {
  using namespace pa;
  if (num_pairs < 0 || !cache_shape_ok(src_num_blocks, num_kv_heads, head_dim, dtype) ||
      dst_num_blocks <= 0)
    return valid_dtype(dtype) || dtype == PA_I8 ? PA_ERR_INVALID_ARG : PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (num_pairs > (0x7fffffff >> 1)) return PA_ERR_INVALID_ARG;
  const void* sk = device_address(src_k);
  const void* sv = device_address(src_v);
  void* dk = device_address(dst_k);
  void* dv = device_address(dst_v);
  const void* pr = device_address(block_pairs);
  if (!sk || !sv || !dk || !dv || !pr) return PA_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t bytes = static_cast<int64_t>(num_kv_heads) * kBlock * head_dim * elem_bytes(dtype);
  const int64_t vec = bytes / 16;
  const int64_t gy = (vec + 1023) / 1024;
  return launch_kernel(PA_KERNEL_TRANSFER_BLOCKS, transfer_blocks_kernel,
                       dim3(2 * num_pairs, static_cast<uint32_t>(gy)), dim3(256), 0, st,
                       static_cast<const uint4*>(sk), static_cast<const uint4*>(sv),
                       static_cast<uint4*>(dk), static_cast<uint4*>(dv),
                       static_cast<const int64_t*>(pr), src_num_blocks, dst_num_blocks, vec);
}

}  // extern "C"
