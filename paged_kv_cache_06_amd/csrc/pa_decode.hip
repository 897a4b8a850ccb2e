// Paged decode attention for gfx950 (CDNA4, wave64).
//
// One new query per head attends to every cached K/V of its sequence; K and V
// are gathered block by block through the sequence's block table ("KV Cache for
// the intermediate", section "Precise scientific definition"; "PagedAttention
// for the professional", section "The scientific explanation").  The query
// heads of one GQA group share a KV head ("KV Cache for the intermediate",
// section "Grouped Query Attention"), so one work item serves the whole group
// and every K/V byte is read from HBM once per step.
//
// Work items: (sequence, partition of P positions, KV head, group of up to 16
// query heads).  Sequences longer than P are cut into partitions whose partial
// results (running max m, sum l, unnormalised acc) are merged with the
// running-max rule (Milakov and Gimelshein 2018) -- on the matrix-core path by
// the last of a sequence's work-groups to finish (merge_if_last), on the VALU
// path by a second kernel; a sequence with one partition is normalised and
// written directly.  A work-group of 4
// waves (8 for the long partitions of long contexts) serves one item: the waves take the item's 16-token blocks
// round-robin and merge their partials through LDS at the end.
//
// Scheduling.  Item sizes vary by two orders of magnitude in a mixed batch
// (16 .. 8192 positions).  A one-work-group plan kernel turns the lengths into
// an item list ordered largest first -- every full partition, then the last
// partition of every sequence by size class -- plus the list of split
// sequences.  Work-group i of the decode kernel serves item i / (heads) of
// that list, so the hardware dispatcher hands out big items first and the
// last ones to start are the smallest: a short tail with no atomics and no
// idle work-groups besides the trailing ones past the list's end, which exit
// at once.  The VALU path's merge kernel walks only the split sequences.
// pa_decode_step builds the list in the same launch as it writes the step's
// new tokens into the cache (decode_prep_kernel).
//
// Matrix-core path (bf16/fp16, head_dim 64 or 128), per 16-token block:
//   scores[16 tok x 16 heads] = K[16 tok x D] . Q^T[D x 16 heads]
//       with v_mfma_f32_16x16x32_{bf16,f16}; lane l holds token l%16's 16-byte
//       K chunk (j*4 + l/16) so each of the D/32 loads reads 1 KiB contiguous;
//   online softmax in fp32 on the 4 scores each lane holds (one head, 4 tokens);
//   acc^T[D x 16 heads] += V^T[D x 16 tok] . P^T[16 tok x 16 heads]
//       with v_mfma_f32_16x16x16_{bf16,f16}; V is stored transposed per block,
//       so a lane's 4 token values of one dimension are 8 contiguous bytes and
//       each load reads 512 bytes contiguous.  P enters the matrix core as a
//       hi + lo pair in the storage dtype (two products), which keeps its
//       rounding error near 2^-16 relative; scores, exponentials, sums and the
//       accumulator stay fp32.
// Heads beyond the group's size occupy the idle columns of the 16-wide
// operands and are never stored.  Positions past the sequence end are masked
// by select (scores to -inf, V values to 0), never by multiplication, so stale
// or NaN bits in a block's tail cannot reach the result.
//
// Generic path (any supported dtype/head_dim, fp32 in particular): one
// work-group per query head, VALU dot products, 256-position chunks with the
// same online softmax and the same partial-result format.
#include "pa_decode_balanced.h"
#include "pa_decode_int8.h"
#include "pa_cache_write.h"
#include "pa_decode_common.h"
namespace pa {
namespace {

// ---- fixed partitions: work items from a plan ----

// Size class of a last partition: 0 (the largest) .. kClasses - 1 (an empty
// sequence).  Classes 0..5 are sixths of a partition, largest first; class 6
// holds slivers below 1/64 of a partition.
constexpr int kClasses = 8;
#ifndef PA_FUSED_MERGE
#define PA_FUSED_MERGE 1
#endif
constexpr bool kFusedMerge = PA_FUSED_MERGE != 0;
__device__ __forceinline__ int size_class(int tokens, int part_size) {
  if (tokens <= 0) return kClasses - 1;
  if (tokens * 64 < part_size) return kClasses - 2;
  return 6 - (tokens * 6 + part_size - 1) / part_size;
}

// Entries of the item list: every (sequence, partition), rounded up to a
// multiple of 32 and padded with end markers.
__host__ __device__ inline int plan_capacity(int num_seqs, int np_max) {
  return (num_seqs * np_max + 31) / 32 * 32;
}

struct PlanArgs {
  const int32_t* lens;
  // [num_seqs * np_max] (sequence, partition, length, partition size);
  // sequence -1 past the end
  int4* items;
  int* split;   // [num_seqs] sequences with more than one partition, then -1
  int* meta;    // [0] items, [1] split sequences
  int num_seqs, max_blocks, part_size, np_max;
  int* arrivals;     // per (sequence, head group): partials stored so far (zeroed here)
  int num_arrivals;
  int max_items;     // items the decode grid serves (see plan_partition)
};

__device__ __forceinline__ int plan_len(const PlanArgs& a, int i) {
  return min(max(a.lens[i], 0), a.max_blocks * kBlock);
}
__device__ __forceinline__ int plan_parts(const PlanArgs& a, int len, int part) {
  return min((len + part - 1) / part, a.np_max);
}

// The partition size of a list longer than max_items.  The decode grid is
// sized for max_items items -- the list's full capacity (every sequence at the
// longest length) would dispatch thousands of work-groups that find only an
// end marker -- so such a list takes part_size doubled, up to kDoublings
// times, until it fits, else one partition per sequence.  Larger partitions
// are fewer, longer items over the same blocks.  Sequences hold at least one
// item each (an empty one too), and max_items >= num_seqs.
constexpr int kDoublings = 6;

__device__ __forceinline__ int plan_partition(const PlanArgs& a, int* wave_tot) {
  const int S = a.num_seqs;
  const int whole = a.max_blocks * kBlock;
  const int per = (S + kThreads - 1) / kThreads;
  const int i0 = threadIdx.x * per;
  const int i1 = min(S, i0 + per);
  int cnt[kDoublings + 1];
#pragma unroll
  for (int k = 0; k <= kDoublings; ++k) cnt[k] = 0;
  for (int i = i0; i < i1; ++i) {
    const int len = plan_len(a, i);
#pragma unroll
    for (int k = 0; k <= kDoublings; ++k) {
      const int part = static_cast<int>(min(static_cast<int64_t>(a.part_size) << k,
                                            static_cast<int64_t>(whole)));
      cnt[k] += max(plan_parts(a, len, part), 1);
    }
  }
  int excl[kDoublings + 1], all[kDoublings + 1];
  block_scan<kDoublings + 1>(cnt, excl, all, wave_tot);
  __syncthreads();  // wave_tot is written again by the caller's scan
#pragma unroll
  for (int k = 0; k <= kDoublings; ++k)
    if (all[k] <= a.max_items)
      return static_cast<int>(min(static_cast<int64_t>(a.part_size) << k,
                                  static_cast<int64_t>(whole)));
  return whole;
}

// The item list, largest first (see the file header).  One work-group; each
// thread takes a run of consecutive sequences, so one exclusive scan of its
// per-class counts places every item, in sequence order within a class.
constexpr int kPlanVals = kClasses + 2;  // classes, full partitions, split sequences

// Per-class item counts of this thread's sequences i0 .. i1-1 at partition
// size `part`, then full partitions, then split sequences.
__device__ __forceinline__ void plan_count(const PlanArgs& a, int part, int i0, int i1,
                                           int* cnt) {
#pragma unroll
  for (int c = 0; c < kPlanVals; ++c) cnt[c] = 0;
  for (int i = i0; i < i1; ++i) {
    const int len = plan_len(a, i);
    const int np = plan_parts(a, len, part);
    const int cls = size_class(np > 0 ? len - (np - 1) * part : 0, part);
#pragma unroll
    for (int c = 0; c < kClasses; ++c) cnt[c] += cls == c;
    cnt[kClasses] += max(np - 1, 0);
    cnt[kClasses + 1] += np > 1;
  }
}

__device__ __forceinline__ void plan_body(const PlanArgs& a, int* wave_tot) {
  constexpr int kVals = kPlanVals;
  const int S = a.num_seqs;
  const int per = (S + kThreads - 1) / kThreads;
  const int i0 = threadIdx.x * per;
  const int i1 = min(S, i0 + per);
  int part = a.part_size;
  int cnt[kVals], excl[kVals], all[kVals];
  plan_count(a, part, i0, i1, cnt);
  block_scan<kVals>(cnt, excl, all, wave_tot);
  if (all[kClasses] + S > a.max_items) {  // the same on every thread
    __syncthreads();  // the scan's totals are read before they are rewritten
    part = plan_partition(a, wave_tot);
    plan_count(a, part, i0, i1, cnt);
    block_scan<kVals>(cnt, excl, all, wave_tot);
  }
  // item positions: full partitions from 0, then classes in order
  const int num_full = all[kClasses];
  int pos[kClasses];
  int run = num_full;
#pragma unroll
  for (int c = 0; c < kClasses; ++c) {
    pos[c] = run + excl[c];
    run += all[c];
  }
  int full_pos = excl[kClasses];
  int split_pos = excl[kClasses + 1];
  for (int i = i0; i < i1; ++i) {
    const int len = plan_len(a, i);
    const int np = plan_parts(a, len, part);
    for (int p = 0; p + 1 < np; ++p) a.items[full_pos++] = make_int4(i, p, len, part);
    const int cls = size_class(np > 0 ? len - (np - 1) * part : 0, part);
    int at = 0;
#pragma unroll
    for (int c = 0; c < kClasses; ++c)
      if (cls == c) at = pos[c]++;
    a.items[at] = make_int4(i, max(np - 1, 0), len, part);
    if (np > 1) a.split[split_pos++] = i;
  }
  const int total = num_full + S;
  const int cap = plan_capacity(S, a.np_max);
  for (int u = total + threadIdx.x; u < cap; u += kThreads) a.items[u] = make_int4(-1, 0, 0, 0);
  for (int i = all[kClasses + 1] + threadIdx.x; i < S; i += kThreads) a.split[i] = -1;
  if (threadIdx.x == 0) {
    a.meta[0] = total;
    a.meta[1] = all[kClasses + 1];
  }
  for (int i = threadIdx.x; i < a.num_arrivals; i += kThreads) a.arrivals[i] = 0;
}

__global__ __launch_bounds__(kThreads) void decode_plan_kernel(PlanArgs a) {
  __shared__ int wave_tot[kWaves * kPlanVals];
  plan_body(a, wave_tot);
}

// One decode step in fewer launches: work-group 0 builds the plan while the
// others write the step's new tokens into the cache (both only read their
// inputs, so they can run side by side); the decode kernels follow on the
// stream.
template <typename W>
__global__ __launch_bounds__(kThreads) void decode_prep_kernel(PlanArgs a, W w) {
  __shared__ int wave_tot[kWaves * kPlanVals];
  if (blockIdx.x == 0) {
    plan_body(a, wave_tot);
    return;
  }
  w.write(static_cast<int64_t>(blockIdx.x - 1) * kThreads + threadIdx.x);
}

// Merge of a split sequence's partials by the last of its work-groups to
// finish (running maximum / log-sum-exp rule, as decode_reduce_kernel): each
// work-group publishes its partial at device scope and counts itself in;
// the one that completes the count reads every partial back and writes the
// output rows, so no second launch is needed.
//
// Partials are written and read with device-scope (relaxed) atomic stores
// and loads, which go to and come from the device-coherent level instead of
// the XCD's L2, and every store has completed (s_waitcnt) before the
// arrival count moves; so no L2-wide write-back or invalidation is needed
// (device-scope fences, which do both, made the kernel twice as slow).
__device__ __forceinline__ void publish(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float fetch(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename Tag, int D, int W>
__device__ __forceinline__ void merge_if_last(const DecodeArgs& a, int s, int gh, int nparts,
                                              size_t row0, int nh) {
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are complete
  __syncthreads();                 // ... and every thread's
  if (threadIdx.x == 0) {
    const int heads = a.hkv * a.head_blocks;
    s_last = __hip_atomic_fetch_add(a.arrivals + static_cast<size_t>(s) * heads + gh, 1,
                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nparts - 1;
  }
  __syncthreads();
  if (!s_last) return;
  for (int e = threadIdx.x; e < nh * D; e += W * kWave) {
    const int h = e / D, d = e % D;
    const size_t row = row0 + h;
    const float* ml = a.ws_ml + row * a.np_max * 2;
    const float* acc = a.ws_acc + row * a.np_max * D + d;
    float M = -INFINITY;
    for (int i = 0; i < nparts; ++i) M = fmaxf(M, fetch(ml + 2 * i));
    float L = 0.f, A = 0.f;
    for (int i = 0; i < nparts; ++i) {
      const float wgt = fast_exp2(fetch(ml + 2 * i) - M);
      L = fmaf(wgt, fetch(ml + 2 * i + 1), L);
      A = fmaf(wgt, fetch(acc + static_cast<size_t>(i) * D), A);
    }
    a.out[row * D + d] = Tag::from_f32(L > 0.f ? A / L : 0.f);
  }
}

// The end of an item: the waves' partials are combined through LDS; a
// sequence with one partition is normalised and stored, a split one leaves
// its partial (m, l, acc) for the merge (in-kernel when a.arrivals is set,
// else by the merge kernel).  vs: INT8 cache only, the V scales of head g,
// applied to each combined accumulator.
template <typename Tag, int D, int W>
__device__ __forceinline__ void finish_item(const DecodeArgs& a, float* comb, int s, int p,
                                            int len, int part, int g, int h0, int nh, int gh,
                                            const float* vs) {
  const int nparts = min((len + part - 1) / part, a.np_max);
  const size_t row0 = static_cast<size_t>(s) * a.hq_total + g * a.group + h0;
  for (int e = threadIdx.x; e < nh * D; e += W * kWave) {
    const int h = e / D, d = e % D;
    float M, L, A;
    combine_waves<W>(comb, a.nh_max, D, h, d, M, L, A);
    if (vs) A *= vs[d];
    const size_t row = row0 + h;
    if (nparts <= 1) {
      a.out[row * D + d] = Tag::from_f32(L > 0.f ? A / L : 0.f);
    } else {
      const size_t part = row * a.np_max + p;
      if (a.arrivals) {  // merged in-kernel: stored where every XCD sees them
        publish(a.ws_acc + part * D + d, A);
        if (d == 0) {
          publish(a.ws_ml + 2 * part, M);
          publish(a.ws_ml + 2 * part + 1, L);
        }
      } else {
        a.ws_acc[part * D + d] = A;
        if (d == 0) {
          a.ws_ml[2 * part] = M;
          a.ws_ml[2 * part + 1] = L;
        }
      }
    }
  }
  if (nparts > 1 && a.arrivals) merge_if_last<Tag, D, W>(a, s, gh, nparts, row0, nh);
}

// Waves of a decode work-group: 4, or 8 for long partitions (item_waves).
__host__ __device__ constexpr int item_threads(int waves) { return waves * kWave; }

// One work item (sequence it.x, partition it.y of it.w positions, length
// it.z) for head group
// gh (KV head x query head block): the waves take the item's blocks
// round-robin, then finish_item.
template <typename Tag, int D, bool kInt8, int W>
__device__ __forceinline__ void decode_item(const DecodeArgs& a, int4 it, int gh, float* comb) {
  const int s = it.x, p = it.y, len = it.z, part = it.w;
  const int g = gh / a.head_blocks, h0 = (gh % a.head_blocks) * 16;
  const int nh = min(16, a.group - h0);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int start = p * part;
  const int end = min(len, start + part);
  const int nblk = max(end - start + kBlock - 1, 0) / kBlock;
  const int b_first = start / kBlock + wave;
  const int count = nblk > wave ? (nblk - wave + W - 1) / W : 0;
  const int32_t* trow = a.tables + static_cast<size_t>(s) * a.max_blocks;
  const int ids = load_ids<W>(trow, b_first, count);
  uint4 qf[D / 32];
  WaveState<D> st;
  st.reset();
  if constexpr (kInt8) {
    const float back = load_q_i8<Tag, D>(a, s, g, h0, nh, qf);
    attend_blocks_i8<D, W>(a, trow, ids, b_first, count, end, g, qf, a.scale_log2 * back, st);
  } else {
    load_q<D>(a, s, g, h0, nh, qf);
    attend_blocks<Tag, D, W>(a, trow, ids, b_first, count, end, g, qf, st);
  }
  stage_partials<D, W>(comb, a.nh_max, nh, st);
  __syncthreads();
  finish_item<Tag, D, W>(a, comb, s, p, len, part, g, h0, nh, gh,
                         kInt8 ? a.v_scale + static_cast<size_t>(g) * D : nullptr);
}

// Work-group b serves item b / heads of the plan for head group b % heads
// (heads = KV heads x query head blocks); work-groups past the list's end
// exit at once.  (A persistent form -- a resident-size grid taking items from
// a ticket counter -- measured slower on the mixed batch: the ticket's
// atomic sits between items, and the loop kept ~20 more registers live.)
template <typename Tag, int D, int W>
__global__ __launch_bounds__(item_threads(W), 4) void decode_items_kernel(
    DecodeArgs a, const int4* __restrict__ items) {
  extern __shared__ float comb[];
  const int heads = a.hkv * a.head_blocks;
  const int4 it = items[blockIdx.x / heads];
  if (it.x < 0) return;
  decode_item<Tag, D, false, W>(a, it, blockIdx.x % heads, comb);
}

// decode_items_kernel over an INT8 cache (same items, partitions and
// partials); the V scale multiplies each merged result before it is stored.
template <typename Tag, int D, int W>
__global__ __launch_bounds__(item_threads(W), 4) void decode_items_i8_kernel(
    DecodeArgs a, const int4* __restrict__ items) {
  extern __shared__ float comb[];
  const int heads = a.hkv * a.head_blocks;
  const int4 it = items[blockIdx.x / heads];
  if (it.x < 0) return;
  decode_item<Tag, D, true, W>(a, it, blockIdx.x % heads, comb);
}

// ---- generic VALU path ----

__device__ __forceinline__ float block_reduce_max(float x, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[wave] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_reduce_sum(float x, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[wave] = x;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) r += red[w];
  __syncthreads();
  return r;
}

template <typename Tag>
__global__ __launch_bounds__(kThreads) void decode_generic_kernel(
    const typename Tag::Bits* __restrict__ q, const typename Tag::Bits* __restrict__ k_cache,
    const typename Tag::Bits* __restrict__ v_cache, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ lens, float scale_log2, typename Tag::Bits* __restrict__ out,
    float* __restrict__ ws_ml, float* __restrict__ ws_acc, int num_seqs, int hq_total, int hkv,
    int group, int head_dim, int max_blocks, int part_size, int np_max) {
  using E = typename Tag::Bits;
  constexpr int X = 16 / sizeof(E);
  constexpr int kChunk = kThreads;  // positions per chunk
  __shared__ float qs[256];
  __shared__ float pw[kChunk];
  __shared__ float red[kWaves];

  int idx = blockIdx.x;
  const int hq = idx % hq_total;
  idx /= hq_total;
  const int s = idx % num_seqs;
  const int p = idx / num_seqs;
  const int len = min(max(lens[s], 0), max_blocks * kBlock);
  const int start = p * part_size;
  if (p > 0 && start >= len) return;
  const int g = hq / group;
  const int end = min(len, start + part_size);
  const int nparts = min((len + part_size - 1) / part_size, np_max);
  const int tid = threadIdx.x;
  const size_t row = static_cast<size_t>(s) * hq_total + hq;
  const size_t head_elems = static_cast<size_t>(head_dim) * kBlock;
  const int32_t* trow = tables + static_cast<size_t>(s) * max_blocks;

  for (int d = tid; d < head_dim; d += kThreads) qs[d] = Tag::to_f32(q[row * head_dim + d]);
  __syncthreads();

  float m_run = -INFINITY, l_run = 0.f, acc = 0.f;
  for (int c0 = start; c0 < end; c0 += kChunk) {
    const int t = c0 + tid;
    float x = -INFINITY;
    if (t < end) {
      const int phys = trow[t / kBlock];
      const int r = t % kBlock;
      const E* kb = k_cache + (static_cast<size_t>(phys) * hkv + g) * head_elems;
      float dot = 0.f;
      for (int c = 0; c < head_dim / X; ++c) {
        union {
          uint4 v;
          E e[X];
        } u;
        u.v = *reinterpret_cast<const uint4*>(kb + (c * kBlock + r) * X);
#pragma unroll
        for (int i = 0; i < X; ++i) dot = fmaf(qs[c * X + i], Tag::to_f32(u.e[i]), dot);
      }
      x = dot * scale_log2;
    }
    const float m_new = fmaxf(m_run, block_reduce_max(x, red));
    const float alpha = fast_exp2(m_run - m_new);
    const float w = (t < end) ? fast_exp2(x - m_new) : 0.f;
    pw[tid] = w;
    l_run = fmaf(l_run, alpha, block_reduce_sum(w, red));  // its barrier publishes pw
    m_run = m_new;
    if (tid < head_dim) {
      acc *= alpha;
      const int nt = min(kChunk, end - c0);
      for (int b0 = 0; b0 < nt; b0 += kBlock) {
        const int phys = trow[(c0 + b0) / kBlock];
        const E* vrow = v_cache + (static_cast<size_t>(phys) * hkv + g) * head_elems +
                        static_cast<size_t>(tid) * kBlock;
        const int rows = min(kBlock, nt - b0);
        for (int r = 0; r < rows; ++r) acc = fmaf(pw[b0 + r], Tag::to_f32(vrow[r]), acc);
      }
    }
    __syncthreads();  // pw is rewritten by the next chunk
  }

  if (tid < head_dim) {
    if (nparts <= 1) {
      out[row * head_dim + tid] = Tag::from_f32(l_run > 0.f ? acc / l_run : 0.f);
    } else {
      const size_t part = row * np_max + p;
      ws_acc[part * head_dim + tid] = acc;
      if (tid == 0) {
        ws_ml[2 * part] = m_run;
        ws_ml[2 * part + 1] = l_run;
      }
    }
  }
}

// Merge the partitions of one (sequence, query head): M = max m_p,
// out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p   (m in log2 units).
// Work-groups walk the rows of the split sequences of the plan.  Within a row,
// thread t reads 16-byte pieces d4 = t % (D/4) of the partitions
// p = t / (D/4) + k * (256 / (D/4)), so the row's loads are in flight
// together; the per-thread sums are merged through LDS.
template <typename Tag>
__global__ __launch_bounds__(kThreads) void decode_reduce_kernel(
    const float* __restrict__ ws_ml, const float* __restrict__ ws_acc,
    const int* __restrict__ split, const int* __restrict__ meta,
    const int32_t* __restrict__ lens, typename Tag::Bits* __restrict__ out, int hq_total,
    int head_dim, int max_blocks, int part_size, int np_max) {
  __shared__ float red[kWaves];
  __shared__ float4 part_sum[kThreads];
  const int rows = meta[1] * hq_total;
  const int tid = threadIdx.x;
  const int q4 = head_dim / 4;  // float4 pieces per row
  const int lanes_per_part = kThreads / q4;
  const int d4 = tid % q4, pr = tid / q4;
  for (int r = blockIdx.x; r < rows; r += gridDim.x) {
    const int s = split[r / hq_total];
    const size_t row = static_cast<size_t>(s) * hq_total + r % hq_total;
    const int len = min(max(lens[s], 0), max_blocks * kBlock);
    const int np = min((len + part_size - 1) / part_size, np_max);
    const float* ml = ws_ml + row * np_max * 2;
    float M = -INFINITY;
    for (int i = tid; i < np; i += kThreads) M = fmaxf(M, ml[2 * i]);
    M = block_reduce_max(M, red);
    float L = 0.f;
    for (int i = tid; i < np; i += kThreads) L = fmaf(fast_exp2(ml[2 * i] - M), ml[2 * i + 1], L);
    L = block_reduce_sum(L, red);
    float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
    if (pr < lanes_per_part) {
      const float4* acc = reinterpret_cast<const float4*>(ws_acc + row * np_max * head_dim);
      for (int i = pr; i < np; i += lanes_per_part) {
        const float wgt = fast_exp2(ml[2 * i] - M);
        const float4 v = acc[static_cast<size_t>(i) * q4 + d4];
        A.x = fmaf(wgt, v.x, A.x);
        A.y = fmaf(wgt, v.y, A.y);
        A.z = fmaf(wgt, v.z, A.z);
        A.w = fmaf(wgt, v.w, A.w);
      }
    }
    part_sum[tid] = A;
    __syncthreads();
    if (tid < q4) {
      float4 t = part_sum[tid];
      for (int k = 1; k < lanes_per_part; ++k) {
        const float4 u = part_sum[k * q4 + tid];
        t.x += u.x;
        t.y += u.y;
        t.z += u.z;
        t.w += u.w;
      }
      const float inv = 1.f / L;
      typename Tag::Bits* o = out + row * head_dim + 4 * tid;
      o[0] = Tag::from_f32(t.x * inv);
      o[1] = Tag::from_f32(t.y * inv);
      o[2] = Tag::from_f32(t.z * inv);
      o[3] = Tag::from_f32(t.w * inv);
    }
    __syncthreads();  // part_sum is reused by the next row
  }
}


// Automatic partition size.  Partitions of 1024 positions keep split overhead
// (partials, merge) near 1 % of the K/V bytes; shorter ones are used only when
// the batch would otherwise give fewer than ~2048 work items (a few long
// sequences), so that every CU has work.  Batches whose longest sequence fits
// one partition are not split.  Contexts of 16K positions and more take 2048
// when that still gives ~1024 items (one per resident work-group): their items
// are then mostly full partitions of one size, and fewer of them means less to
// merge (on MI355X: 32K-position batch of 8, 190 us against 194 us at 1024).
// An INT8 cache moves half the bytes per position, so every size above doubles
// and every item count halves (measured on MI355X: the mixed 70B-layer batch
// decodes in 62.7 us at 2048 against 63.6 us at 1024, the 32K batch in 99 us
// at 4096 against 103 us at 2048).
int auto_partition(int num_seqs, int hkv, int max_len, int kv_bytes = 2) {
  const int k = kv_bytes == 1 ? 2 : 1;
  if (max_len <= 1024 * k) return PA_PARTITION_NONE;
  const int long_part = 2048 * k;
  if (max_len >= 16384 &&
      static_cast<int64_t>(num_seqs) * ((max_len + long_part - 1) / long_part) * hkv >= 1024 / k)
    return long_part;
  int ps = 1024 * k;
  while (ps > 256 &&
         static_cast<int64_t>(num_seqs) * ((max_len + ps - 1) / ps) * hkv < 2048 / k)
    ps /= 2;
  return ps;
}

bool resolve_split(int partition_size, int num_seqs, int hkv, int max_len, Split* out,
                   int kv_bytes = 2) {
  int ps = partition_size;
  if (ps == PA_PARTITION_AUTO) ps = auto_partition(num_seqs, hkv, max_len, kv_bytes);
  if (ps < 0 || ps % kBlock != 0) return false;
  if (ps == PA_PARTITION_NONE) ps = max(kBlock, (max_len + kBlock - 1) / kBlock * kBlock);
  out->part = ps;
  out->np = max(1, (max_len + ps - 1) / ps);
  return true;
}

// Workspace of the fixed-partition path: [plan: meta (256 B), items, split
// list] [m, l of every partial] [acc of every partial]; the partial areas
// exist only when some sequence is split.

Layout workspace_layout(int num_seqs, int hq, int head_dim, const Split& sp) {
  Layout l;
  const size_t cap = static_cast<size_t>(plan_capacity(num_seqs, sp.np));
  l.meta = 0;
  l.items = kAlign;
  l.split = l.items + align_up(cap * sizeof(int4));
  l.ml = l.split + align_up(static_cast<size_t>(num_seqs) * sizeof(int));
  l.acc = l.ml;
  l.total = l.ml;
  l.arrivals = l.total;
  if (sp.np > 1) {
    const size_t parts = static_cast<size_t>(num_seqs) * sp.np * hq;
    l.acc = l.ml + align_up(parts * 2 * sizeof(float));
    l.arrivals = l.acc + align_up(parts * head_dim * sizeof(float));
    l.total = l.arrivals + align_up(static_cast<size_t>(num_seqs) * hq * sizeof(int));
  }
  return l;
}

template <typename Tag, typename W = CacheWriteArgs<typename Tag::Bits>>
pa_status launch(const void* q, const void* k_cache, const void* v_cache, const int32_t* tables,
                 const int32_t* lens, float scale_log2, void* out, int num_seqs, int hq, int hkv,
                 int head_dim, int max_blocks, const Split& sp, char* ws, bool use_mfma,
                 hipStream_t st, const float* k_scale = nullptr, const float* v_scale = nullptr,
                 const W* write = nullptr) {
  using E = typename Tag::Bits;
  const int group = hq / hkv;
  const int head_blocks = use_mfma ? (group + 15) / 16 : 1;
  if (static_cast<int64_t>(sp.np) * num_seqs * hq > 0x7fffffff / 2) return PA_ERR_INVALID_ARG;
  // the matrix-core path's grid: items for two per sequence and at least 2048
  // work-groups, or the list's whole capacity when that is smaller; a longer
  // list takes larger partitions (plan_partition).  The merge kernel of the
  // other paths reads partitions of sp.part, so their plan keeps it.
  const bool fused_merge = use_mfma && sp.np > 1 && kFusedMerge;
  const int cap = plan_capacity(num_seqs, sp.np);
  const int heads = hkv * head_blocks;
  const int item_grid =
      fused_merge ? std::min(cap, std::max(2 * num_seqs, (2048 + heads - 1) / heads)) : cap;
  const int64_t grid = use_mfma ? static_cast<int64_t>(item_grid) * heads
                                : static_cast<int64_t>(sp.np) * num_seqs * hq;
  const Layout lay = workspace_layout(num_seqs, hq, head_dim, sp);
  int* meta = reinterpret_cast<int*>(ws + lay.meta);
  int4* items = reinterpret_cast<int4*>(ws + lay.items);
  int* split = reinterpret_cast<int*>(ws + lay.split);
  float* ws_ml = reinterpret_cast<float*>(ws + lay.ml);
  float* ws_acc = reinterpret_cast<float*>(ws + lay.acc);
  // the matrix-core kernels merge split sequences themselves (merge_if_last)
  int* arrivals = fused_merge ? reinterpret_cast<int*>(ws + lay.arrivals) : nullptr;
  if (use_mfma || sp.np > 1) {
    PlanArgs pa{lens, items, split, meta, num_seqs, max_blocks, sp.part, sp.np, arrivals,
                fused_merge ? num_seqs * hkv * head_blocks : 0,  // one per (sequence, head group)
                item_grid};
    if (write) {  // the step's cache writes ride along with the plan
      const int64_t wgs = 1 + (write->threads() + kThreads - 1) / kThreads;
      const int pslot = timing_start(PA_KERNEL_DECODE_PLAN, st);
      decode_prep_kernel<W><<<dim3(static_cast<uint32_t>(wgs)), dim3(kThreads), 0, st>>>(pa, *write);
      const pa_status ps = launch_status();
      timing_stop(pslot, st);
      if (ps != PA_OK) return ps;
    } else {
      const int pslot = timing_start(PA_KERNEL_DECODE_PLAN, st);
      decode_plan_kernel<<<dim3(1), dim3(kThreads), 0, st>>>(pa);
      const pa_status ps = launch_status();
      timing_stop(pslot, st);
      if (ps != PA_OK) return ps;
    }
  }
  int slot = timing_start(PA_KERNEL_DECODE, st);
  pa_status status = PA_OK;
  if (use_mfma) {
    if constexpr (sizeof(E) == 2) {
      DecodeArgs a = mfma_args<Tag>(q, k_cache, v_cache, tables, lens, scale_log2, out,
                                    num_seqs, hq, hkv, max_blocks, sp, ws_ml, ws_acc);
      a.k_scale = k_scale;
      a.v_scale = v_scale;
      a.arrivals = arrivals;
      // 8 waves per item for the partitions chosen for long contexts (>= 2048
      // positions, INT8 >= 4096): each wave then still streams many blocks, and
      // the 32K context decodes ~4 % faster; 4 otherwise (mixed batches of
      // short items lose 8 % at 8 waves on the INT8 cache)
      const int waves = sp.part >= (k_scale ? 4096 : 2048) ? 8 : 4;
      const size_t lds = comb_floats(waves, a.nh_max, head_dim) * sizeof(float);
      const dim3 g3(static_cast<uint32_t>(grid)), b3(item_threads(waves));
      if (k_scale) {  // INT8 cache
        if (head_dim == 128) {
          if (waves == 8)
            decode_items_i8_kernel<Tag, 128, 8><<<g3, b3, lds, st>>>(a, items);
          else
            decode_items_i8_kernel<Tag, 128, 4><<<g3, b3, lds, st>>>(a, items);
        } else if (waves == 8) {
          decode_items_i8_kernel<Tag, 64, 8><<<g3, b3, lds, st>>>(a, items);
        } else {
          decode_items_i8_kernel<Tag, 64, 4><<<g3, b3, lds, st>>>(a, items);
        }
      } else if (head_dim == 128) {
        if (waves == 8)
          decode_items_kernel<Tag, 128, 8><<<g3, b3, lds, st>>>(a, items);
        else
          decode_items_kernel<Tag, 128, 4><<<g3, b3, lds, st>>>(a, items);
      } else if (waves == 8) {
        decode_items_kernel<Tag, 64, 8><<<g3, b3, lds, st>>>(a, items);
      } else {
        decode_items_kernel<Tag, 64, 4><<<g3, b3, lds, st>>>(a, items);
      }
      status = launch_status();
    }
  } else {
    decode_generic_kernel<Tag><<<dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0, st>>>(
        static_cast<const E*>(q), static_cast<const E*>(k_cache), static_cast<const E*>(v_cache),
        tables, lens, scale_log2, static_cast<E*>(out), ws_ml, ws_acc, num_seqs, hq, hkv, group,
        head_dim, max_blocks, sp.part, sp.np);
    status = launch_status();
  }
  timing_stop(slot, st);
  if (status != PA_OK || sp.np <= 1 || fused_merge) return status;
  slot = timing_start(PA_KERNEL_DECODE_REDUCE, st);
  const int rows = static_cast<int>(std::min<int64_t>(static_cast<int64_t>(num_seqs) * hq, 2048));
  decode_reduce_kernel<Tag><<<dim3(rows), dim3(kThreads), 0, st>>>(
      ws_ml, ws_acc, split, meta, lens, static_cast<E*>(out), hq, head_dim, max_blocks, sp.part,
      sp.np);
  status = launch_status();
  timing_stop(slot, st);
  return status;
}
}  // namespace
}  // namespace pa

extern "C" {

int32_t pa_decode_auto_partition(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len, pa_dtype dtype) {
  (void)num_q_heads;
  (void)head_dim;
  return pa::auto_partition(num_seqs, num_kv_heads, max_context_len,
                            dtype == PA_I8 ? 1 : pa::elem_bytes(dtype));
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size) {
  pa::Split sp;
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0) return 0;
  if (partition_size == PA_PARTITION_BALANCED)
    return pa::balanced_split_workspace_bytes(
        num_q_heads, head_dim, pa::balanced_split_ranges(num_seqs, num_q_heads, max_context_len));
  // the automatic choice shrinks partitions for fewer KV heads, so sizing with
  // one KV head covers every head count
  if (!pa::resolve_split(partition_size, num_seqs, 1, max_context_len, &sp)) return 0;
  const size_t fixed = pa::workspace_layout(num_seqs, num_q_heads, head_dim, sp).total;
  return fixed;
}

}  // extern "C"

namespace pa {
namespace {

// Thread layout of a fused step's cache writes: one new token per sequence
// (plain decode) shares no block with another, so window 1; more tokens than
// sequences (a sequence appending a run) interleave windows of tokens.
inline int step_window(int32_t num_tokens, int32_t num_seqs) {
  return num_tokens <= num_seqs ? 1 : kWindow;
}

// The new tokens of a fused decode step (pa_decode_step); key == nullptr: none.
struct StepWrite {
  const void* key;
  const void* value;
  const int64_t* slots;
  int32_t num_tokens;
  int32_t num_blocks;
};

pa_status decode_impl(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t max_blocks_per_seq, int32_t max_context_len,
                      int32_t partition_size, void* workspace, size_t workspace_bytes,
                      pa_dtype dtype, void* stream, const StepWrite& wr) {
  if (!valid_dtype(dtype)) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_blocks_per_seq <= 0 || max_context_len < 0)
    return PA_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (head_dim % (16 / elem_bytes(dtype)) != 0 || head_dim > 256) return PA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * kBlock)
    return PA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return PA_ERR_INVALID_ARG;
  const bool use_mfma = mfma_path(dtype, head_dim);
  if (partition_size == PA_PARTITION_BALANCED && !use_mfma) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return PA_ERR_INVALID_ARG;
  const bool balanced = use_mfma && partition_size == PA_PARTITION_BALANCED;
  Split sp{kBlock, 1};
  size_t need;
  int64_t ranges = 0;
  if (balanced) {
    // block indices of the balanced split stay below 2^30
    const int64_t units = static_cast<int64_t>(num_kv_heads) * ((num_q_heads / num_kv_heads + 15) / 16);
    if (static_cast<int64_t>(num_seqs) * units * max_blocks_per_seq >= (int64_t{1} << 30))
      return PA_ERR_INVALID_ARG;
    ranges = balanced_split_ranges(num_seqs, num_q_heads, max_context_len);
    need = balanced_split_workspace_bytes(num_q_heads, head_dim, ranges);
  } else {
    if (!resolve_split(partition_size, num_seqs, num_kv_heads, max_context_len, &sp))
      return PA_ERR_INVALID_ARG;
    need = workspace_layout(num_seqs, num_q_heads, head_dim, sp).total;
  }
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return PA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  const float scale_log2 = scale * kLog2e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool fused = wr.key != nullptr && wr.num_tokens > 0 && use_mfma && !balanced;
  if (wr.key != nullptr && wr.num_tokens > 0 && !fused) {  // write first, then decode
    const pa_status ws_st =
        pa_reshape_and_cache(wr.key, wr.value, const_cast<void*>(k_cache),
                             const_cast<void*>(v_cache), wr.slots, wr.num_tokens, wr.num_blocks,
                             num_kv_heads, head_dim, dtype, stream);
    if (ws_st != PA_OK) return ws_st;
  }
  if (balanced)
    return launch_balanced_split(dtype, q, k_cache, v_cache, block_tables, context_lens,
                                 scale_log2, out, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                 max_blocks_per_seq, ranges, ws, st);
  const int64_t num_slots = static_cast<int64_t>(wr.num_blocks) * kBlock;
  switch (dtype) {
    case PA_BF16: {
      auto w = cache_write_args<uint16_t>(wr.key, wr.value, const_cast<void*>(k_cache),
                                          const_cast<void*>(v_cache), wr.slots, wr.num_tokens,
                                          num_slots, num_kv_heads, head_dim);
      w.window = step_window(wr.num_tokens, num_seqs);
      return launch<BF16T>(q, k_cache, v_cache, block_tables, context_lens, scale_log2, out,
                           num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, sp,
                           ws, use_mfma, st, nullptr, nullptr, fused ? &w : nullptr);
    }
    case PA_F16: {
      auto w = cache_write_args<uint16_t>(wr.key, wr.value, const_cast<void*>(k_cache),
                                          const_cast<void*>(v_cache), wr.slots, wr.num_tokens,
                                          num_slots, num_kv_heads, head_dim);
      w.window = step_window(wr.num_tokens, num_seqs);
      return launch<F16T>(q, k_cache, v_cache, block_tables, context_lens, scale_log2, out,
                          num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, sp,
                          ws, use_mfma, st, nullptr, nullptr, fused ? &w : nullptr);
    }
    default:
      return launch<F32T>(q, k_cache, v_cache, block_tables, context_lens, scale_log2, out,
                          num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, sp,
                          ws, false, st);
  }
}

pa_status decode_int8_impl(const void* q, const void* k_cache, const void* v_cache,
                           const float* k_scale, const float* v_scale,
                           const int32_t* block_tables, const int32_t* context_lens, float scale,
                           void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t max_blocks_per_seq, int32_t max_context_len,
                           int32_t partition_size, void* workspace, size_t workspace_bytes,
                           pa_dtype dtype, void* stream, const StepWrite& wr) {
  if (dtype != PA_BF16 && dtype != PA_F16) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (partition_size == PA_PARTITION_BALANCED) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
      max_context_len < 0)
    return PA_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * kBlock)
    return PA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !k_scale || !v_scale || !block_tables || !context_lens || !out)
    return PA_ERR_INVALID_ARG;
  Split sp;
  if (!resolve_split(partition_size, num_seqs, num_kv_heads, max_context_len, &sp, 1))
    return PA_ERR_INVALID_ARG;
  const size_t need = workspace_layout(num_seqs, num_q_heads, head_dim, sp).total;
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return PA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  const float scale_log2 = scale * kLog2e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool fused = wr.key != nullptr && wr.num_tokens > 0;
  const int64_t num_slots = static_cast<int64_t>(wr.num_blocks) * kBlock;
  int8_t* kc = static_cast<int8_t*>(const_cast<void*>(k_cache));
  int8_t* vc = static_cast<int8_t*>(const_cast<void*>(v_cache));
  if (dtype == PA_BF16) {
    CacheWriteI8Args<BF16T> w{static_cast<const uint16_t*>(wr.key),
                              static_cast<const uint16_t*>(wr.value), kc, vc, wr.slots,
                              k_scale, v_scale, wr.num_tokens, num_slots, num_kv_heads,
                              head_dim};
    w.window = step_window(wr.num_tokens, num_seqs);
    return launch<BF16T>(q, k_cache, v_cache, block_tables, context_lens, scale_log2, out,
                         num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, sp,
                         ws, true, st, k_scale, v_scale, fused ? &w : nullptr);
  }
  CacheWriteI8Args<F16T> w{static_cast<const uint16_t*>(wr.key),
                           static_cast<const uint16_t*>(wr.value), kc, vc, wr.slots, k_scale,
                           v_scale, wr.num_tokens, num_slots, num_kv_heads, head_dim};
  w.window = step_window(wr.num_tokens, num_seqs);
  return launch<F16T>(q, k_cache, v_cache, block_tables, context_lens, scale_log2, out, num_seqs,
                      num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, sp, ws, true, st,
                      k_scale, v_scale, fused ? &w : nullptr);
}

}  // namespace
}  // namespace pa

extern "C" {

pa_status pa_paged_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    float scale, void* out, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t max_blocks_per_seq, int32_t max_context_len,
                                    int32_t partition_size, void* workspace,
                                    size_t workspace_bytes, pa_dtype dtype, void* stream) {
  return pa::decode_impl(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs,
                         num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                         max_context_len, partition_size, workspace, workspace_bytes, dtype,
                         stream, pa::StepWrite{nullptr, nullptr, nullptr, 0, 0});
}

pa_status pa_decode_step(const void* key, const void* value, const int64_t* slot_mapping,
                         int32_t num_new_tokens, int32_t num_blocks, const void* q, void* k_cache,
                         void* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens, float scale, void* out, int32_t num_seqs,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t max_blocks_per_seq, int32_t max_context_len,
                         int32_t partition_size, void* workspace, size_t workspace_bytes,
                         pa_dtype dtype, void* stream) {
  using namespace pa;
  // the write's own checks, as pa_reshape_and_cache makes them
  if (!valid_dtype(dtype)) return PA_ERR_UNSUPPORTED;
  if (num_new_tokens < 0 || num_blocks <= 0 || head_dim % (16 / elem_bytes(dtype)) != 0 ||
      head_dim > 512)
    return PA_ERR_INVALID_ARG;
  if (num_new_tokens > 0 && (!key || !value || !slot_mapping)) return PA_ERR_INVALID_ARG;
  if ((static_cast<int64_t>(num_new_tokens) * num_kv_heads * head_dim + 255) / 256 > 0x7fffffff)
    return PA_ERR_INVALID_ARG;
  if (num_seqs == 0)  // nothing to attend: only the write
    return pa_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, num_new_tokens,
                                num_blocks, num_kv_heads, head_dim, dtype, stream);
  return decode_impl(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, max_context_len,
                     partition_size, workspace, workspace_bytes, dtype, stream,
                     StepWrite{key, value, slot_mapping, num_new_tokens, num_blocks});
}

pa_status pa_paged_attention_decode_int8(const void* q, const void* k_cache, const void* v_cache,
                                         const float* k_scale, const float* v_scale,
                                         const int32_t* block_tables,
                                         const int32_t* context_lens, float scale, void* out,
                                         int32_t num_seqs, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t max_blocks_per_seq, int32_t max_context_len,
                                         int32_t partition_size, void* workspace,
                                         size_t workspace_bytes, pa_dtype dtype, void* stream) {
  return pa::decode_int8_impl(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                              scale, out, num_seqs, num_q_heads, num_kv_heads, head_dim,
                              max_blocks_per_seq, max_context_len, partition_size, workspace,
                              workspace_bytes, dtype, stream,
                              pa::StepWrite{nullptr, nullptr, nullptr, 0, 0});
}

pa_status pa_decode_step_int8(const void* key, const void* value, const int64_t* slot_mapping,
                              int32_t num_new_tokens, int32_t num_blocks, const void* q,
                              void* k_cache, void* v_cache, const float* k_scale,
                              const float* v_scale, const int32_t* block_tables,
                              const int32_t* context_lens, float scale, void* out,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t max_blocks_per_seq,
                              int32_t max_context_len, int32_t partition_size, void* workspace,
                              size_t workspace_bytes, pa_dtype dtype, void* stream) {
  using namespace pa;
  if (num_new_tokens < 0 || num_blocks <= 0) return PA_ERR_INVALID_ARG;
  if (num_new_tokens > 0 && (!key || !value || !slot_mapping)) return PA_ERR_INVALID_ARG;
  if ((static_cast<int64_t>(num_new_tokens) * num_kv_heads * head_dim / 16 + 255) / 256 >
      0x7fffffff)
    return PA_ERR_INVALID_ARG;
  if (num_seqs == 0)  // nothing to attend: only the write
    return pa_reshape_and_cache_int8(key, value, k_cache, v_cache, slot_mapping, k_scale, v_scale,
                                     num_new_tokens, num_blocks, num_kv_heads, head_dim, dtype,
                                     stream);
  return decode_int8_impl(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                          scale, out, num_seqs, num_q_heads, num_kv_heads, head_dim,
                          max_blocks_per_seq, max_context_len, partition_size, workspace,
                          workspace_bytes, dtype, stream,
                          StepWrite{key, value, slot_mapping, num_new_tokens, num_blocks});
}

}  // extern "C"
