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
// results (running max m, sum l, unnormalised acc) are merged by a second
// kernel with the running-max rule (Milakov and Gimelshein 2018); a sequence
// with one partition is normalised and written directly.  A work-group of 4
// waves serves one item: the waves take the item's 16-token blocks
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
// at once.  The merge kernel walks only the split sequences.
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
#include <algorithm>
#include <cmath>

#include "pa_common.h"

namespace pa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename Tag>
struct Mfma;

template <>
struct Mfma<BF16T> {
  __device__ static f32x4_t qk(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  __device__ static f32x4_t pv(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                     __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
  }
  __device__ static uint2 pack(float a, float b, float c, float d) {
    bf16x4_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b), static_cast<__bf16>(c),
                  static_cast<__bf16>(d)};
    return __builtin_bit_cast(uint2, v);
  }
  // the two packed values of a 32-bit word, widened exactly
  __device__ static float lo(uint32_t w) { return __uint_as_float(w << 16); }
  __device__ static float hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
};

template <>
struct Mfma<F16T> {
  __device__ static f32x4_t qk(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  __device__ static f32x4_t pv(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  }
  __device__ static uint2 pack(float a, float b, float c, float d) {
    f16x4_t v = {static_cast<_Float16>(a), static_cast<_Float16>(b), static_cast<_Float16>(c),
                 static_cast<_Float16>(d)};
    return __builtin_bit_cast(uint2, v);
  }
  __device__ static float lo(uint32_t w) { return f16_to_f32(static_cast<uint16_t>(w)); }
  __device__ static float hi(uint32_t w) { return f16_to_f32(static_cast<uint16_t>(w >> 16)); }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Arguments shared by the kernels of the matrix-core path.
struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* tables;
  const int32_t* lens;
  uint16_t* out;
  float* ws_ml;
  float* ws_acc;
  float scale_log2;
  int num_seqs, hq_total, hkv, group, head_blocks, max_blocks, part_size, np_max;
  int nh_max;  // query heads of the largest head group (<= 16): LDS rows per wave
};

__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int len) {
  // lengths beyond the table width are cut to it, so a bad length cannot read
  // past the table row
  return min(max(len, 0), a.max_blocks * kBlock);
}

// The loads that start a work item (its block ids and its q rows), issued
// before the item runs so that they can overlap earlier work.
template <int D>
struct ItemPrep {
  int s, p, g, hb, len;
  int ids;              // lane j: id of this wave's j-th block (first 64)
  uint4 qf[D / 32];     // B operand of the QK products: head lane%16, k-group lane/16
};

template <typename Tag, int D, int W>
__device__ __forceinline__ void prep_item(const DecodeArgs& a, int s, int p, int g, int hb,
                                          int len, ItemPrep<D>& it) {
  constexpr int kSteps = D / 32;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int n = lane & 15;
  const int kg = lane >> 4;
  it.s = s;
  it.p = p;
  it.g = g;
  it.hb = hb;
  it.len = len;
  const int h0 = hb * 16;
  const int nh = min(16, a.group - h0);
  const int start = p * a.part_size;
  const int end = min(len, start + a.part_size);
  const int nblk = max(end - start + kBlock - 1, 0) / kBlock;
  const int my_blocks = nblk > wave ? (nblk - wave + W - 1) / W : 0;
  const int32_t* trow =
      a.tables + static_cast<size_t>(s) * a.max_blocks + start / kBlock + wave;
  it.ids = lane < my_blocks ? trow[W * lane] : 0;
  if (n < nh) {
    const uint16_t* qp = a.q + (static_cast<size_t>(s) * a.hq_total + g * a.group + h0 + n) * D;
#pragma unroll
    for (int j = 0; j < kSteps; ++j)
      it.qf[j] = *reinterpret_cast<const uint4*>(qp + (j * 4 + kg) * 8);
  } else {
#pragma unroll
    for (int j = 0; j < kSteps; ++j) it.qf[j] = make_uint4(0, 0, 0, 0);
  }
}

// One work item: positions [p*P, min(len, (p+1)*P)) of sequence s against KV
// head g for query heads h0 .. h0+nh-1 of its group, served by W waves; each
// wave issues the loads of B of its blocks before using any of them.  `comb`
// is LDS of comb_floats(W, nh_max, D) floats.  Ends with the result stored;
// the caller must __syncthreads() before reusing `comb`.
template <typename Tag, int D, int W, int B>
__device__ void run_item(const DecodeArgs& a, const ItemPrep<D>& it, float* comb) {
  constexpr int kSteps = D / 32;   // QK k-steps of 32 dims
  constexpr int kSlices = D / 16;  // PV output slices of 16 dims
  const int s = it.s, p = it.p, g = it.g, hb = it.hb, len = it.len;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int n = lane & 15;   // token row (K, scores) / head column (Q, P, acc)
  const int kg = lane >> 4;  // k-group of the MFMA operands
  const int h0 = hb * 16;
  const int nh = min(16, a.group - h0);
  const int start = p * a.part_size;
  const int end = min(len, start + a.part_size);
  const int nblk = max(end - start + kBlock - 1, 0) / kBlock;
  const int blk0 = start / kBlock;
  const int nparts = min((len + a.part_size - 1) / a.part_size, a.np_max);
  // this wave's blocks: blk0 + wave + W * j, j < my_blocks
  const int my_blocks = nblk > wave ? (nblk - wave + W - 1) / W : 0;
  const int32_t* trow = a.tables + static_cast<size_t>(s) * a.max_blocks + blk0 + wave;
  int ids = it.ids;
  const uint4* qf = it.qf;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t acc[kSlices];
#pragma unroll
  for (int i = 0; i < kSlices; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const size_t head_elems = static_cast<size_t>(D) * kBlock;
  const uint16_t* kbase = a.k_cache + static_cast<size_t>(g) * head_elems;
  const uint16_t* vbase = a.v_cache + static_cast<size_t>(g) * head_elems;
  const size_t block_stride = static_cast<size_t>(a.hkv) * head_elems;

  for (int j0 = 0; j0 < my_blocks; j0 += B) {
    if (j0 > 0 && (j0 & 63) < B) {  // the batch starts in the next 64 block ids
      const int jj = (j0 & ~63) + lane;
      ids = jj < my_blocks ? trow[W * jj] : 0;
    }
    uint4 kf[B][kSteps];
    uint2 vf[B][kSlices];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (j0 + b < my_blocks) {
        const int phys = __builtin_amdgcn_readlane(ids, (j0 + b) & 63);
        const uint16_t* kb = kbase + static_cast<size_t>(phys) * block_stride;
        const uint16_t* vb = vbase + static_cast<size_t>(phys) * block_stride;
#pragma unroll
        for (int t = 0; t < kSteps; ++t)
          kf[b][t] = *reinterpret_cast<const uint4*>(kb + t * 512 + lane * 8);
#pragma unroll
        for (int sl = 0; sl < kSlices; ++sl)
          vf[b][sl] = *reinterpret_cast<const uint2*>(vb + (sl * 16 + n) * kBlock + kg * 4);
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (j0 + b >= my_blocks) break;
      f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < kSteps; ++t) sc = Mfma<Tag>::qk(kf[b][t], qf[t], sc);

      const int blk = blk0 + wave + W * (j0 + b);
      const int pos0 = blk * kBlock + kg * 4;  // position of this lane's first score
      float s4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) s4[r] = (pos0 + r < end) ? sc[r] * a.scale_log2 : -INFINITY;
      float mx = fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      float p4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p4[r] = fast_exp2(s4[r] - m_new);
      l_run = fmaf(l_run, alpha, (p4[0] + p4[1]) + (p4[2] + p4[3]));
      m_run = m_new;
#pragma unroll
      for (int sl = 0; sl < kSlices; ++sl) acc[sl] *= alpha;

      if ((blk + 1) * kBlock > end) {  // tail block: zero V of masked positions
        const uint32_t lo =
            (pos0 + 0 < end ? 0x0000FFFFu : 0u) | (pos0 + 1 < end ? 0xFFFF0000u : 0u);
        const uint32_t hi =
            (pos0 + 2 < end ? 0x0000FFFFu : 0u) | (pos0 + 3 < end ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int sl = 0; sl < kSlices; ++sl) {
          vf[b][sl].x &= lo;
          vf[b][sl].y &= hi;
        }
      }
      // P as hi + lo in the storage dtype: two products, near-fp32 weights
      const uint2 ph = Mfma<Tag>::pack(p4[0], p4[1], p4[2], p4[3]);
      const uint2 pl = Mfma<Tag>::pack(p4[0] - Mfma<Tag>::lo(ph.x), p4[1] - Mfma<Tag>::hi(ph.x),
                                       p4[2] - Mfma<Tag>::lo(ph.y), p4[3] - Mfma<Tag>::hi(ph.y));
#pragma unroll
      for (int sl = 0; sl < kSlices; ++sl) {
        acc[sl] = Mfma<Tag>::pv(vf[b][sl], ph, acc[sl]);
        acc[sl] = Mfma<Tag>::pv(vf[b][sl], pl, acc[sl]);
      }
    }
  }

  // per-wave partials to LDS: comb = [m: W][nh_max] [l: W][nh_max] [acc: W][nh_max][D]
  const int nhm = a.nh_max;
  float* cm = comb;
  float* cl = comb + W * nhm;
  float* ca = comb + 2 * W * nhm;
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (n < nh) {
    if (kg == 0) {
      cm[wave * nhm + n] = m_run;
      cl[wave * nhm + n] = l_tot;
    }
#pragma unroll
    for (int sl = 0; sl < kSlices; ++sl)
      *reinterpret_cast<f32x4_t*>(&ca[(wave * nhm + n) * D + sl * 16 + kg * 4]) = acc[sl];
  }
  __syncthreads();

  const size_t row0 = static_cast<size_t>(s) * a.hq_total + g * a.group + h0;
  for (int e = threadIdx.x; e < nh * D; e += W * kWave) {
    const int h = e / D, d = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, cm[w * nhm + h]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float f = fast_exp2(cm[w * nhm + h] - M);
        L = fmaf(f, cl[w * nhm + h], L);
        A = fmaf(f, ca[(w * nhm + h) * D + d], A);
      }
    }
    const size_t row = row0 + h;
    if (nparts <= 1) {
      a.out[row * D + d] = Tag::from_f32(L > 0.f ? A / L : 0.f);
    } else {
      const size_t part = row * a.np_max + p;
      a.ws_acc[part * D + d] = A;
      if (d == 0) {
        a.ws_ml[2 * part] = M;
        a.ws_ml[2 * part + 1] = L;
      }
    }
  }
}

__host__ __device__ inline size_t comb_floats(int waves, int nh_max, int head_dim) {
  return static_cast<size_t>(waves) * nh_max * (2 + head_dim);
}

// Waves per decode work-group and blocks each wave loads together.
#ifndef PA_ITEM_WAVES
#define PA_ITEM_WAVES 4
#endif
#ifndef PA_ITEM_BATCH
#define PA_ITEM_BATCH 1
#endif
#ifndef PA_ITEMS_PER_GROUP
#define PA_ITEMS_PER_GROUP 1
#endif
constexpr int kItemWaves = PA_ITEM_WAVES;
constexpr int kItemBatch = PA_ITEM_BATCH;
constexpr int kItemsPerGroup = PA_ITEMS_PER_GROUP;  // work items per work-group
constexpr int kItemThreads = kItemWaves * kWave;

// Size class of a last partition: 0 (the largest) .. kClasses - 1 (an empty
// sequence).  Classes 0..5 are sixths of a partition, largest first; class 6
// holds slivers below 1/64 of a partition.
constexpr int kClasses = 8;
__device__ __forceinline__ int size_class(int tokens, int part_size) {
  if (tokens <= 0) return kClasses - 1;
  if (tokens * 64 < part_size) return kClasses - 2;
  return 6 - (tokens * 6 + part_size - 1) / part_size;
}

// Entries of the item list: every (sequence, partition), rounded up to a
// multiple of 32 (a whole number of work-groups' items) and padded with end
// markers.
__host__ __device__ inline int plan_capacity(int num_seqs, int np_max) {
  return (num_seqs * np_max + 31) / 32 * 32;
}

struct PlanArgs {
  const int32_t* lens;
  int4* items;  // [num_seqs * np_max] (sequence, partition, length, 0); sequence -1 past the end
  int* split;   // [num_seqs] sequences with more than one partition, then -1
  int* meta;    // [0] items, [1] split sequences
  int num_seqs, max_blocks, part_size, np_max;
};

__device__ __forceinline__ int plan_len(const PlanArgs& a, int i) {
  return min(max(a.lens[i], 0), a.max_blocks * kBlock);
}
__device__ __forceinline__ int plan_parts(const PlanArgs& a, int len) {
  return min((len + a.part_size - 1) / a.part_size, a.np_max);
}

// The item list, largest first (see the file header).  One work-group; each
// thread takes a run of consecutive sequences, so one exclusive scan of its
// per-class counts places every item, in sequence order within a class.
__global__ __launch_bounds__(kThreads) void decode_plan_kernel(PlanArgs a) {
  constexpr int kVals = kClasses + 2;  // classes, full partitions, split sequences
  __shared__ int wave_tot[kWaves][kVals];
  const int S = a.num_seqs;
  const int per = (S + kThreads - 1) / kThreads;
  const int i0 = threadIdx.x * per;
  const int i1 = min(S, i0 + per);
  int cnt[kVals];
#pragma unroll
  for (int c = 0; c < kVals; ++c) cnt[c] = 0;
  for (int i = i0; i < i1; ++i) {
    const int len = plan_len(a, i);
    const int np = plan_parts(a, len);
    const int cls = size_class(np > 0 ? len - (np - 1) * a.part_size : 0, a.part_size);
#pragma unroll
    for (int c = 0; c < kClasses; ++c) cnt[c] += cls == c;
    cnt[kClasses] += max(np - 1, 0);
    cnt[kClasses + 1] += np > 1;
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  int excl[kVals];
#pragma unroll
  for (int c = 0; c < kVals; ++c) {
    int x = cnt[c];
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    excl[c] = x - cnt[c];
    if (lane == kWave - 1) wave_tot[wv][c] = x;
  }
  __syncthreads();
  int all[kVals];
#pragma unroll
  for (int c = 0; c < kVals; ++c) {
    int before = 0, sum = 0;
    for (int w = 0; w < kWaves; ++w) {
      before += w < wv ? wave_tot[w][c] : 0;
      sum += wave_tot[w][c];
    }
    excl[c] += before;
    all[c] = sum;
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
    const int np = plan_parts(a, len);
    for (int p = 0; p + 1 < np; ++p) a.items[full_pos++] = make_int4(i, p, len, 0);
    const int cls = size_class(np > 0 ? len - (np - 1) * a.part_size : 0, a.part_size);
    int at = 0;
#pragma unroll
    for (int c = 0; c < kClasses; ++c)
      if (cls == c) at = pos[c]++;
    a.items[at] = make_int4(i, max(np - 1, 0), len, 0);
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
}

// Work-group i serves item i / heads of the plan (heads = KV heads x query
// head groups); work-groups past the list's end exit at once.
template <typename Tag, int D>
__global__ __launch_bounds__(kItemThreads, 16 / kItemWaves) void decode_items_kernel(
    DecodeArgs a, const int4* __restrict__ items) {
  extern __shared__ float comb[];
  const int heads = a.hkv * a.head_blocks;
  // items u0 .. u0 + kItemsPerGroup - 1 (neighbours in the list, so of similar
  // size), all for head gh; the later items' block ids and q are loaded
  // up front so their start overlaps the earlier items
  const int u0 = (blockIdx.x / heads) * kItemsPerGroup;
  const int gh = blockIdx.x % heads;
  ItemPrep<D> prep[kItemsPerGroup];
  int valid = 0;
#pragma unroll
  for (int k = 0; k < kItemsPerGroup; ++k) {
    const int4 it = items[u0 + k];
    if (it.x < 0) break;
    prep_item<Tag, D, kItemWaves>(a, it.x, it.y, gh / a.head_blocks, gh % a.head_blocks, it.z,
                                  prep[k]);
    ++valid;
  }
#pragma unroll
  for (int k = 0; k < kItemsPerGroup; ++k) {
    if (k >= valid) break;
    if (k > 0) __syncthreads();  // comb is reused
    run_item<Tag, D, kItemWaves, kItemBatch>(a, prep[k], comb);
  }
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

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Resolved partition size (a positive multiple of 16) and partition count.
struct Split {
  int part;
  int np;
};

// Partitions of 1024 positions keep split overhead (partials, merge) near 1 %
// of the K/V bytes; shorter ones are used only when the batch would otherwise
// give fewer than ~2048 work items (a few long sequences), so that every CU
// has work.  Batches whose longest sequence fits one partition are not split.
int auto_partition(int num_seqs, int hkv, int max_len) {
  if (max_len <= 1024) return PA_PARTITION_NONE;
  int ps = 1024;
  while (ps > 256 &&
         static_cast<int64_t>(num_seqs) * ((max_len + ps - 1) / ps) * hkv < 2048)
    ps /= 2;
  return ps;
}

bool resolve_split(int partition_size, int num_seqs, int hkv, int max_len, Split* out) {
  int ps = partition_size;
  if (ps == PA_PARTITION_AUTO) ps = auto_partition(num_seqs, hkv, max_len);
  if (ps < 0 || ps % kBlock != 0) return false;
  if (ps == PA_PARTITION_NONE) ps = max(kBlock, (max_len + kBlock - 1) / kBlock * kBlock);
  out->part = ps;
  out->np = max(1, (max_len + ps - 1) / ps);
  return true;
}

// Workspace: [plan: meta (256 B), items, split list] [m, l of every partial]
// [acc of every partial]; the partial areas exist only when some sequence is
// split.  Every call rewrites what it reads.
struct Layout {
  size_t meta, items, split, ml, acc, total;
};

Layout workspace_layout(int num_seqs, int hq, int head_dim, const Split& sp) {
  Layout l;
  const size_t cap = static_cast<size_t>(plan_capacity(num_seqs, sp.np));
  l.meta = 0;
  l.items = kAlign;
  l.split = l.items + align_up(cap * sizeof(int4));
  l.ml = l.split + align_up(static_cast<size_t>(num_seqs) * sizeof(int));
  l.acc = l.ml;
  l.total = l.ml;
  if (sp.np > 1) {
    const size_t parts = static_cast<size_t>(num_seqs) * sp.np * hq;
    l.acc = l.ml + align_up(parts * 2 * sizeof(float));
    l.total = l.acc + align_up(parts * head_dim * sizeof(float));
  }
  return l;
}

bool mfma_path(pa_dtype dt, int head_dim) {
  return (dt == PA_BF16 || dt == PA_F16) && (head_dim == 64 || head_dim == 128);
}

template <typename Tag>
pa_status launch(const void* q, const void* k_cache, const void* v_cache, const int32_t* tables,
                 const int32_t* lens, float scale_log2, void* out, int num_seqs, int hq, int hkv,
                 int head_dim, int max_blocks, const Split& sp, char* ws, bool use_mfma,
                 hipStream_t st) {
  using E = typename Tag::Bits;
  const int group = hq / hkv;
  const int head_blocks = use_mfma ? (group + 15) / 16 : 1;
  if (static_cast<int64_t>(sp.np) * num_seqs * hq > 0x7fffffff / 2) return PA_ERR_INVALID_ARG;
  const int64_t grid = use_mfma ? static_cast<int64_t>(plan_capacity(num_seqs, sp.np)) /
                                      kItemsPerGroup * hkv * head_blocks
                                : static_cast<int64_t>(sp.np) * num_seqs * hq;
  const Layout lay = workspace_layout(num_seqs, hq, head_dim, sp);
  int* meta = reinterpret_cast<int*>(ws + lay.meta);
  int4* items = reinterpret_cast<int4*>(ws + lay.items);
  int* split = reinterpret_cast<int*>(ws + lay.split);
  float* ws_ml = reinterpret_cast<float*>(ws + lay.ml);
  float* ws_acc = reinterpret_cast<float*>(ws + lay.acc);
  if (use_mfma || sp.np > 1) {
    PlanArgs pa{lens, items, split, meta, num_seqs, max_blocks, sp.part, sp.np};
    const int pslot = timing_start(PA_KERNEL_DECODE_PLAN, st);
    decode_plan_kernel<<<dim3(1), dim3(kThreads), 0, st>>>(pa);
    const pa_status ps = launch_status();
    timing_stop(pslot, st);
    if (ps != PA_OK) return ps;
  }
  int slot = timing_start(PA_KERNEL_DECODE, st);
  pa_status status = PA_OK;
  if (use_mfma) {
    if constexpr (sizeof(E) == 2) {
      DecodeArgs a;
      a.q = static_cast<const uint16_t*>(q);
      a.k_cache = static_cast<const uint16_t*>(k_cache);
      a.v_cache = static_cast<const uint16_t*>(v_cache);
      a.tables = tables;
      a.lens = lens;
      a.out = static_cast<uint16_t*>(out);
      a.ws_ml = ws_ml;
      a.ws_acc = ws_acc;
      a.scale_log2 = scale_log2;
      a.num_seqs = num_seqs;
      a.hq_total = hq;
      a.hkv = hkv;
      a.group = group;
      a.head_blocks = head_blocks;
      a.max_blocks = max_blocks;
      a.part_size = sp.part;
      a.np_max = sp.np;
      a.nh_max = std::min(16, group);
      const size_t lds = comb_floats(kItemWaves, a.nh_max, head_dim) * sizeof(float);
      const dim3 g3(static_cast<uint32_t>(grid)), b3(kItemThreads);
      if (head_dim == 128)
        decode_items_kernel<Tag, 128><<<g3, b3, lds, st>>>(a, items);
      else
        decode_items_kernel<Tag, 64><<<g3, b3, lds, st>>>(a, items);
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
  if (status != PA_OK || sp.np <= 1) return status;
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
  (void)dtype;
  return pa::auto_partition(num_seqs, num_kv_heads, max_context_len);
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size) {
  pa::Split sp;
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0) return 0;
  // the automatic choice shrinks partitions for fewer KV heads, so sizing with
  // one KV head covers every head count
  if (!pa::resolve_split(partition_size, num_seqs, 1, max_context_len, &sp)) return 0;
  return pa::workspace_layout(num_seqs, num_q_heads, head_dim, sp).total;
}

pa_status pa_paged_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    float scale, void* out, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t max_blocks_per_seq, int32_t max_context_len,
                                    int32_t partition_size, void* workspace,
                                    size_t workspace_bytes, pa_dtype dtype, void* stream) {
  using namespace pa;
  if (!valid_dtype(dtype)) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_blocks_per_seq <= 0 || max_context_len < 0)
    return PA_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (head_dim % (16 / elem_bytes(dtype)) != 0 || head_dim > 256) return PA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * kBlock)
    return PA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return PA_ERR_INVALID_ARG;
  Split sp;
  if (!resolve_split(partition_size, num_seqs, num_kv_heads, max_context_len, &sp))
    return PA_ERR_INVALID_ARG;
  const size_t need = workspace_layout(num_seqs, num_q_heads, head_dim, sp).total;
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return PA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  const float scale_log2 = scale * kLog2e;
  const bool use_mfma = mfma_path(dtype, head_dim);
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case PA_BF16:
      return launch<BF16T>(q, k_cache, v_cache, block_tables, context_lens, scale_log2, out,
                           num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, sp,
                           ws, use_mfma, st);
    case PA_F16:
      return launch<F16T>(q, k_cache, v_cache, block_tables, context_lens, scale_log2, out,
                          num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, sp,
                          ws, use_mfma, st);
    default:
      return launch<F32T>(q, k_cache, v_cache, block_tables, context_lens, scale_log2, out,
                          num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, sp,
                          ws, false, st);
  }
}

}  // extern "C"
