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

// Loads through a buffer resource: a wave-uniform base and byte range in
// scalar registers, 32-bit lane offsets, and 0 for every byte outside the
// range (which is how rows past a head group or blocks past a wave's count
// read as zero without a branch).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kBufferConfig = 0x00020000;  // raw 32-bit data, gfx9 buffer resource word 3

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferConfig);
}
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 buffer_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t buffer_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

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

// A wave-uniform read of read-only data through the constant address space, so
// that it is a scalar load: a vector load here would make the wave wait for all
// of its K/V loads in flight.
__device__ __forceinline__ int uniform_load(const int32_t* p, int i) {
  typedef const __attribute__((address_space(4))) int32_t* ConstPtr;
  return ((ConstPtr)p)[i];
}

__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int len) {
  // lengths beyond the table width are cut to it, so a bad length cannot read
  // past the table row
  return min(max(len, 0), a.max_blocks * kBlock);
}

// Waves per decode work-group.
constexpr int kItemWaves = 4;
constexpr int kItemThreads = kItemWaves * kWave;

// Running softmax state of one wave: m (log2 units) and l per head column,
// acc^T[D x 16 heads] as D/16 MFMA accumulators.
template <int D>
struct WaveState {
  float m, l;
  f32x4_t acc[D / 16];
  __device__ void reset() {
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
};

// B operand of the QK products for query heads h0 .. h0+nh-1 of KV head g:
// lane l holds head l%16, dims (j*4 + l/16)*8 .. +7 of k-step j; idle columns 0.
template <int D>
__device__ __forceinline__ void load_q(const DecodeArgs& a, int s, int g, int h0, int nh,
                                       uint4* qf) {
  const uint32_t lane = threadIdx.x & (kWave - 1);
  const uint32_t n = lane & 15, kg = lane >> 4;
  const auto rq = buffer_of(a.q + (static_cast<size_t>(s) * a.hq_total + g * a.group + h0) * D,
                            static_cast<uint32_t>(nh) * D * 2);  // rows past nh read 0
  const uint32_t off = (n * D + kg * 8) * 2;
#pragma unroll
  for (int j = 0; j < D / 32; ++j) qf[j] = buffer_load16(rq, off + j * 64);
}

// Physical ids of a wave's blocks b_first + W*i, i < count: lane i holds
// block i (the first 64; attend_blocks reloads for later ones).
template <int W>
__device__ __forceinline__ int load_ids(const int32_t* trow, int b_first, int count) {
  const uint32_t lane = threadIdx.x & (kWave - 1);
  if (count <= 0) return 0;
  // lanes at or past count fall outside the range and read 0
  const auto rt = buffer_of(trow + b_first, static_cast<uint32_t>((count - 1) * W + 1) * 4);
  return static_cast<int>(buffer_load4(rt, lane * (4 * W)));
}

// K and V of one block of KV head g as MFMA operands: kf[t] is the A operand
// of QK k-step t (lane l: token l%16, 16-byte chunk t*4 + l/16), vf[sl] the A
// operand of PV slice sl (lane l: dim sl*16 + l%16, tokens 4*(l/16) .. +3).
template <int D>
struct BlockRegs {
  uint4 kf[D / 32];
  uint2 vf[D / 16];
};

template <int D>
__device__ __forceinline__ void load_block(const DecodeArgs& a, int g, int phys,
                                           BlockRegs<D>& r) {
  const uint32_t lane = threadIdx.x & (kWave - 1);
  constexpr uint32_t kBytes = D * kBlock * 2;  // one KV head of one block
  const size_t off = (static_cast<size_t>(phys) * a.hkv + g) * (D * kBlock);
  const auto rk = buffer_of(a.k_cache + off, kBytes);
  const auto rv = buffer_of(a.v_cache + off, kBytes);
  const uint32_t ko = lane * 16;
  const uint32_t vo = ((lane & 15) * kBlock + (lane >> 4) * 4) * 2;
#pragma unroll
  for (int t = 0; t < D / 32; ++t) r.kf[t] = buffer_load16(rk, ko + t * 1024);
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) r.vf[sl] = buffer_load8(rv, vo + sl * 512);
}

// One block (logical index blk) into the running state: positions at or past
// `len` are masked.
// `qf(t)` gives the B operand of QK k-step t (registers or LDS).
template <typename Tag, int D, typename QOperand>
__device__ __forceinline__ void attend_block(const DecodeArgs& a, BlockRegs<D>& r, int blk,
                                             int len, const QOperand& qf, WaveState<D>& st) {
  constexpr int kSteps = D / 32;   // QK k-steps of 32 dims
  constexpr int kSlices = D / 16;  // PV output slices of 16 dims
  const int lane = threadIdx.x & (kWave - 1);
  const int kg = lane >> 4;  // k-group of the MFMA operands
  f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < kSteps; ++t) sc = Mfma<Tag>::qk(r.kf[t], qf(t), sc);

  const int pos0 = blk * kBlock + kg * 4;  // position of this lane's first score
  float s4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s4[i] = (pos0 + i < len) ? sc[i] * a.scale_log2 : -INFINITY;
  float mx = fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3]));
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(st.m, mx);
  const float alpha = fast_exp2(st.m - m_new);
  float p4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p4[i] = fast_exp2(s4[i] - m_new);
  st.l = fmaf(st.l, alpha, (p4[0] + p4[1]) + (p4[2] + p4[3]));
  st.m = m_new;
#pragma unroll
  for (int sl = 0; sl < kSlices; ++sl) st.acc[sl] *= alpha;

  if ((blk + 1) * kBlock > len) {  // tail block: zero V of masked positions
    const uint32_t lo = (pos0 + 0 < len ? 0x0000FFFFu : 0u) | (pos0 + 1 < len ? 0xFFFF0000u : 0u);
    const uint32_t hi = (pos0 + 2 < len ? 0x0000FFFFu : 0u) | (pos0 + 3 < len ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int sl = 0; sl < kSlices; ++sl) {
      r.vf[sl].x &= lo;
      r.vf[sl].y &= hi;
    }
  }
  // P as hi + lo in the storage dtype: two products, near-fp32 weights
  const uint2 ph = Mfma<Tag>::pack(p4[0], p4[1], p4[2], p4[3]);
  const uint2 pl = Mfma<Tag>::pack(p4[0] - Mfma<Tag>::lo(ph.x), p4[1] - Mfma<Tag>::hi(ph.x),
                                   p4[2] - Mfma<Tag>::lo(ph.y), p4[3] - Mfma<Tag>::hi(ph.y));
#pragma unroll
  for (int sl = 0; sl < kSlices; ++sl) {
    st.acc[sl] = Mfma<Tag>::pv(r.vf[sl], ph, st.acc[sl]);
    st.acc[sl] = Mfma<Tag>::pv(r.vf[sl], pl, st.acc[sl]);
  }
}

// Attends one wave's blocks b_first + W*i (i < count) of the sequence whose
// table row is trow: positions at or past `len` are masked.  `ids` comes from
// load_ids for the same blocks.  Updates st.
template <typename Tag, int D, int W>
__device__ __forceinline__ void attend_blocks(const DecodeArgs& a, const int32_t* trow, int ids,
                                              int b_first, int count, int len, int g,
                                              const uint4* qf, WaveState<D>& st) {
  for (int j = 0; j < count; ++j) {
    if (j > 0 && (j & 63) == 0) ids = load_ids<W>(trow, b_first + W * j, count - j);
    BlockRegs<D> r;
    load_block<D>(a, g, __builtin_amdgcn_readlane(ids, j & 63), r);
    attend_block<Tag, D>(a, r, b_first + W * j, len, [&](int t) { return qf[t]; }, st);
  }
}

__host__ __device__ inline size_t comb_floats(int waves, int nh_max, int head_dim) {
  return static_cast<size_t>(waves) * nh_max * (2 + head_dim);
}

// Per-wave partials to LDS: comb = [m: W][nh_max] [l: W][nh_max] [acc: W][nh_max][D].
template <int D, int W>
__device__ __forceinline__ void stage_partials(float* comb, int nhm, int nh,
                                               const WaveState<D>& st) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int n = lane & 15, kg = lane >> 4;
  float* cm = comb;
  float* cl = comb + W * nhm;
  float* ca = comb + 2 * W * nhm;
  float l_tot = st.l + __shfl_xor(st.l, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (n < nh) {
    if (kg == 0) {
      cm[wave * nhm + n] = st.m;
      cl[wave * nhm + n] = l_tot;
    }
#pragma unroll
    for (int sl = 0; sl < D / 16; ++sl)
      *reinterpret_cast<f32x4_t*>(&ca[(wave * nhm + n) * D + sl * 16 + kg * 4]) = st.acc[sl];
  }
}

// Merge of the W waves' partials of head h, dimension d (after a barrier that
// publishes stage_partials): M = max m_w, L = sum 2^(m_w-M) l_w,
// A = sum 2^(m_w-M) acc_w.
template <int W>
__device__ __forceinline__ void combine_waves(const float* comb, int nhm, int D, int h, int d,
                                              float& M, float& L, float& A) {
  const float* cm = comb;
  const float* cl = comb + W * nhm;
  const float* ca = comb + 2 * W * nhm;
  M = -INFINITY;
#pragma unroll
  for (int w = 0; w < W; ++w) M = fmaxf(M, cm[w * nhm + h]);
  L = 0.f;
  A = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float f = fast_exp2(cm[w * nhm + h] - M);
      L = fmaf(f, cl[w * nhm + h], L);
      A = fmaf(f, ca[(w * nhm + h) * D + d], A);
    }
  }
}

// ---- fixed partitions: work items from a plan ----

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
// multiple of 32 and padded with end markers.
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

// Exclusive scan over the 256 threads of a work-group of kVals counters at
// once; all[] receives the totals.  `tot` is LDS of kWaves * kVals ints.
template <int kVals>
__device__ __forceinline__ void block_scan(const int* cnt, int* excl, int* all, int* tot) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
#pragma unroll
  for (int c = 0; c < kVals; ++c) {
    int x = cnt[c];
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    excl[c] = x - cnt[c];
    if (lane == kWave - 1) tot[wv * kVals + c] = x;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kVals; ++c) {
    int before = 0, sum = 0;
    for (int w = 0; w < kWaves; ++w) {
      before += w < wv ? tot[w * kVals + c] : 0;
      sum += tot[w * kVals + c];
    }
    excl[c] += before;
    all[c] = sum;
  }
}

// The item list, largest first (see the file header).  One work-group; each
// thread takes a run of consecutive sequences, so one exclusive scan of its
// per-class counts places every item, in sequence order within a class.
__global__ __launch_bounds__(kThreads) void decode_plan_kernel(PlanArgs a) {
  constexpr int kVals = kClasses + 2;  // classes, full partitions, split sequences
  __shared__ int wave_tot[kWaves * kVals];
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
  int excl[kVals], all[kVals];
  block_scan<kVals>(cnt, excl, all, wave_tot);
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
// head groups); work-groups past the list's end exit at once.  The waves take
// the item's blocks round-robin and merge through LDS; a sequence with one
// partition is normalised and stored, a split one leaves its partial (m, l,
// acc) for the merge kernel.
template <typename Tag, int D>
__global__ __launch_bounds__(kItemThreads, 16 / kItemWaves) void decode_items_kernel(
    DecodeArgs a, const int4* __restrict__ items) {
  constexpr int W = kItemWaves;
  extern __shared__ float comb[];
  const int heads = a.hkv * a.head_blocks;
  const int4 it = items[blockIdx.x / heads];
  if (it.x < 0) return;
  const int gh = blockIdx.x % heads;
  const int s = it.x, p = it.y, len = it.z;
  const int g = gh / a.head_blocks, h0 = (gh % a.head_blocks) * 16;
  const int nh = min(16, a.group - h0);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int start = p * a.part_size;
  const int end = min(len, start + a.part_size);
  const int nblk = max(end - start + kBlock - 1, 0) / kBlock;
  const int b_first = start / kBlock + wave;
  const int count = nblk > wave ? (nblk - wave + W - 1) / W : 0;
  const int32_t* trow = a.tables + static_cast<size_t>(s) * a.max_blocks;
  const int ids = load_ids<W>(trow, b_first, count);
  uint4 qf[D / 32];
  load_q<D>(a, s, g, h0, nh, qf);
  WaveState<D> st;
  st.reset();
  attend_blocks<Tag, D, W>(a, trow, ids, b_first, count, end, g, qf, st);
  stage_partials<D, W>(comb, a.nh_max, nh, st);
  __syncthreads();

  const int nparts = min((len + a.part_size - 1) / a.part_size, a.np_max);
  const size_t row0 = static_cast<size_t>(s) * a.hq_total + g * a.group + h0;
  for (int e = threadIdx.x; e < nh * D; e += W * kWave) {
    const int h = e / D, d = e % D;
    float M, L, A;
    combine_waves<W>(comb, a.nh_max, D, h, d, M, L, A);
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

// ---- balanced split: every work-group gets the same amount of work ----
//
// The work of a call is laid out as one row of "units" -- (sequence, KV head,
// query-head group), sequence-major.  A unit of a sequence of length len has
// nb = max(1, ceil(len/16)) blocks (a sequence of length 0 keeps one empty
// block so that its output is written) and costs kUnitCost + nb: the fixed
// part stands for what starting a unit takes (its q and first blocks arrive
// with nothing else in flight, the merge of its waves).  Of C cost in all,
// work-group k takes [k*q, (k+1)*q), q = ceil(C/G) for a grid of G resident
// work-groups; a range boundary inside a unit's fixed part moves to the
// unit's first block.  So range k runs from start[k] to start[k+1], each a
// (sequence, unit, first block) triple.  The k-th block of a range goes to
// wave k % 4, so the waves' shares differ by at most one block whatever the
// unit boundaries.  A unit that lies wholly in one range is normalised and
// stored; a unit cut by range boundaries leaves one partial per piece, merged
// by decode_balanced_merge_kernel.  Work-group k writes at most two partials:
// slot 0 for a unit that began before its range, slot 1 for a unit that
// begins in its range and runs past its end.
#ifndef PA_UNIT_COST
#define PA_UNIT_COST 4
#endif
constexpr int kUnitCost = PA_UNIT_COST;  // fixed cost of a unit, in blocks
constexpr int kMinQuota = 16;            // cost per work-group at least (> kUnitCost)
constexpr int kMaxBalancedGroups = 2048;
static_assert(kUnitCost < kMinQuota, "a range must reach past a unit's fixed part");

struct BalanceArgs {
  const int32_t* lens;
  int4* start;  // [G + 1] range starts (sequence, unit in sequence, first block, 0); the last
                // one after the end (num_seqs, 0, 0, 0)
  int* meta;    // [0] C, [1] q, [2] work-groups with work
  int num_seqs, max_blocks, units, groups;
};

// One work-group: unit costs per sequence, their exclusive scan, and the
// start of every work-group's range.
__global__ __launch_bounds__(kThreads) void decode_balance_kernel(BalanceArgs a) {
  __shared__ int wave_tot[kWaves];
  const int S = a.num_seqs;
  const int per = (S + kThreads - 1) / kThreads;
  const int i0 = threadIdx.x * per;
  const int i1 = min(S, i0 + per);
  int cnt = 0;
  for (int i = i0; i < i1; ++i) {
    const int len = min(max(a.lens[i], 0), a.max_blocks * kBlock);
    cnt += kUnitCost + max(1, (len + kBlock - 1) / kBlock);
  }
  int excl, all;
  block_scan<1>(&cnt, &excl, &all, wave_tot);
  const int C = all * a.units;
  const int q = max(kMinQuota, (C + a.groups - 1) / a.groups);
  const int nwg = (C + q - 1) / q;
  for (int i = i0; i < i1; ++i) {
    const int len = min(max(a.lens[i], 0), a.max_blocks * kBlock);
    const int uc = kUnitCost + max(1, (len + kBlock - 1) / kBlock);  // cost of one unit
    const int x = excl * a.units;  // cost offset of the sequence's unit 0
    for (int k = (x + q - 1) / q; k * q < x + uc * a.units; ++k) {
      const int rel = k * q - x;
      const int r = rel % uc;
      a.start[k] = make_int4(i, rel / uc, r < kUnitCost ? 0 : r - kUnitCost, 0);
    }
    excl += uc;
  }
  if (threadIdx.x == 0) {
    a.start[nwg] = make_int4(S, 0, 0, 0);
    a.meta[0] = C;
    a.meta[1] = q;
    a.meta[2] = nwg;
  }
}

// The part of one unit that a work-group's range holds, as one wave sees it.
struct Unit {
  int s, j, o, e;      // blocks [o, e) of unit j of sequence s
  int len, nb;         // sequence length; blocks the schedule gives the unit
  int g, h0, nh;       // KV head, first query head of the group, query heads
  int b_first, count;  // this wave's blocks: b_first + W*i, i < count
  int xb;              // index of block o among the range's blocks
  bool last;           // the range ends in this unit
};

// Unit j of sequence s from block o, in the range that ends at `end` (the
// next range's start); xb blocks of the range come before it.
template <int W>
__device__ __forceinline__ Unit make_unit(const DecodeArgs& a, int s, int j, int o, int len,
                                          int xb, int4 end) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  Unit u;
  u.s = s;
  u.j = j;
  u.o = o;
  u.len = len;
  const int nbr = (len + kBlock - 1) / kBlock;
  u.nb = max(1, nbr);
  u.last = s == end.x && j == end.y;
  u.e = u.last ? end.z : u.nb;
  u.g = j / a.head_blocks;
  u.h0 = (j % a.head_blocks) * 16;
  u.nh = min(16, a.group - u.h0);
  u.b_first = o + (wave - xb % W + W) % W;  // block o belongs to wave xb % W
  const int e_real = min(u.e, nbr);
  u.count = u.b_first < e_real ? (e_real - u.b_first + W - 1) / W : 0;
  u.xb = xb;
  return u;
}

// Per-wave partials of a unit to LDS for a head group of at most NH rows:
// comb = [m: W][NH] [l: W][NH] [acc: W][NH][D] (rows past the group hold the
// idle columns and are never stored).
template <int D, int W, int NH>
__device__ __forceinline__ void stage_rows(float* comb, const WaveState<D>& st) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int n = lane & 15, kg = lane >> 4;
  float* cm = comb;
  float* cl = comb + W * NH;
  float* ca = comb + 2 * W * NH;
  float l_tot = st.l + __shfl_xor(st.l, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (n < NH) {
    if (kg == 0) {
      cm[wave * NH + n] = st.m;
      cl[wave * NH + n] = l_tot;
    }
#pragma unroll
    for (int sl = 0; sl < D / 16; ++sl)
      *reinterpret_cast<f32x4_t*>(&ca[(wave * NH + n) * D + sl * 16 + kg * 4]) = st.acc[sl];
  }
}

// Work-group k: the units of blocks [k*q, (k+1)*q), for head groups of at
// most NH query heads.  While a unit's blocks are in use, the block ids of
// the next unit are in flight; its q and first block are loaded right after
// the unit's rows are stored.
template <typename Tag, int D, int NH>
__global__ __launch_bounds__(kItemThreads, 16 / kItemWaves) void decode_balanced_kernel(
    DecodeArgs a, const int4* __restrict__ start, const int* __restrict__ meta,
    float* __restrict__ part_ml, float* __restrict__ part_acc) {
  constexpr int W = kItemWaves;
  constexpr int kIters = (NH * D + kItemThreads - 1) / kItemThreads;  // merge passes
  extern __shared__ float comb[];
  const int k = blockIdx.x;
  if (k >= meta[2]) return;
  const int units = a.hkv * a.head_blocks;
  const int4 st0 = start[k];
  const int4 end = start[k + 1];
  Unit cur = make_unit<W>(a, st0.x, st0.y, st0.z, clamp_len(a, uniform_load(a.lens, st0.x)), 0,
                          end);
  const int32_t* trow = a.tables + static_cast<size_t>(cur.s) * a.max_blocks;
  int ids = load_ids<W>(trow, cur.b_first, cur.count);
  uint4 qf[D / 32];
  load_q<D>(a, cur.s, cur.g, cur.h0, cur.nh, qf);
  BlockRegs<D> r;
  if (cur.count > 0) load_block<D>(a, cur.g, __builtin_amdgcn_readfirstlane(ids), r);
  for (;;) {
    // the next unit, and its block ids
    int sn = cur.s, jn = cur.j + 1;
    if (jn == units) {
      jn = 0;
      ++sn;
    }
    const bool has_next = !cur.last && !(sn == end.x && jn == end.y && end.z == 0);
    Unit nxt = cur;
    int ids_next = 0;
    const int32_t* trow_next = trow;
    if (has_next) {
      const int len = sn == cur.s ? cur.len : clamp_len(a, uniform_load(a.lens, sn));
      nxt = make_unit<W>(a, sn, jn, 0, len, cur.xb + (cur.e - cur.o), end);
      trow_next = a.tables + static_cast<size_t>(sn) * a.max_blocks;
      ids_next = load_ids<W>(trow_next, nxt.b_first, nxt.count);
    }

    WaveState<D> st;
    st.reset();
    for (int jj = 0; jj < cur.count; ++jj) {
      if (jj > 0) {
        if ((jj & 63) == 0) ids = load_ids<W>(trow, cur.b_first + W * jj, cur.count - jj);
        load_block<D>(a, cur.g, __builtin_amdgcn_readlane(ids, jj & 63), r);
      }
      attend_block<Tag, D>(a, r, cur.b_first + W * jj, cur.len, [&](int t) { return qf[t]; }, st);
    }
    // first block of the next unit (its ids arrived during the loop above)
    const int first_next = __builtin_amdgcn_readfirstlane(ids_next);
    stage_rows<D, W, NH>(comb, st);
    __syncthreads();

    // the unit's rows: out rows when the range holds it whole, else a partial
    // slot (0: the unit began before this range, 1: it begins in it); stores
    // go through buffer ranges of exactly the unit's rows
    const bool whole = cur.o == 0 && cur.e == cur.nb;
    const int slot = cur.o > 0 ? 0 : 1;
    const int prow0 = (k * 2 + slot) * NH;
    const auto rout = buffer_of(
        a.out + (static_cast<size_t>(cur.s) * a.hq_total + cur.g * a.group + cur.h0) * D,
        static_cast<uint32_t>(cur.nh) * D * 2);
    const auto racc = buffer_of(part_acc + static_cast<size_t>(prow0) * D,
                                static_cast<uint32_t>(cur.nh) * D * 4);
    const auto rml = buffer_of(part_ml + 2 * prow0, static_cast<uint32_t>(cur.nh) * 8);
    const float* cm = comb;
    const float* cl = comb + W * NH;
    const float* ca = comb + 2 * W * NH;
#pragma unroll 1  // unrolled, the merge's LDS loads raise register use past 128
    for (int i = 0; i < kIters; ++i) {
      const int el = threadIdx.x + i * kItemThreads;  // row h = el / D, dim el % D
      if ((NH * D) % kItemThreads != 0 && el >= NH * D) break;
      const int h = el / D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < W; ++w) M = fmaxf(M, cm[w * NH + h]);
      float L = 0.f, A = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < W; ++w) {
          const float f = fast_exp2(cm[w * NH + h] - M);
          L = fmaf(f, cl[w * NH + h], L);
          A = fmaf(f, ca[w * NH * D + el], A);
        }
      }
      if (whole) {
        __builtin_amdgcn_raw_buffer_store_b16(Tag::from_f32(L > 0.f ? A / L : 0.f), rout,
                                              el * 2, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(A), racc, el * 4, 0, 0);
        if (el % D == 0) {
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(M), rml, h * 8, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(L), rml, h * 8 + 4, 0, 0);
        }
      }
    }
    if (!has_next) break;
    // the next unit's q and first block go out behind the stores (loads and
    // stores complete in issue order)
    load_q<D>(a, nxt.s, nxt.g, nxt.h0, nxt.nh, qf);
    if (nxt.count > 0) load_block<D>(a, nxt.g, first_next, r);
    __syncthreads();  // comb is rewritten by the next unit
    cur = nxt;
    trow = trow_next;
    ids = ids_next;
  }
}

// Merge of the units cut by range boundaries.  Work-group k looks at the
// start of range k; when it cuts a unit that began in range k-1 (boundary k
// is that unit's first cut), it merges the unit's pieces -- range k-1, then
// ranges k, k+1, .. while they start inside the unit -- and stores the unit's
// rows: M = max m_p, out = sum 2^(m_p-M) acc_p / sum 2^(m_p-M) l_p.  Pieces
// go in chunks of kMergeChunk: their (m, l) are staged in LDS, then each
// thread folds one 4-float column of a row over the chunk with a running
// maximum, the column loads of a chunk all in flight.
constexpr int kMergeChunk = 32;

template <typename Tag>
__global__ __launch_bounds__(kThreads) void decode_balanced_merge_kernel(
    const int4* __restrict__ start, const int* __restrict__ meta,
    const float* __restrict__ part_ml, const float* __restrict__ part_acc,
    typename Tag::Bits* __restrict__ out, int hq_total, int group, int head_blocks, int head_dim,
    int nhm) {
  __shared__ float sm[kMergeChunk][16], sl[kMergeChunk][16];
  const int k = blockIdx.x;
  const int nwg = meta[2];
  if (k == 0 || k >= nwg) return;
  const int4 st = start[k];
  if (st.z == 0) return;  // range k starts at a unit's first block: no cut
  const int4 prev = start[k - 1];
  if (prev.x == st.x && prev.y == st.y && prev.z > 0) return;  // an earlier cut merges it
  int k_last = k;
  while (k_last + 1 < nwg && start[k_last + 1].x == st.x && start[k_last + 1].y == st.y)
    ++k_last;
  const int s = st.x;
  const int k_first = k - 1;
  const int g = st.y / head_blocks, h0 = (st.y % head_blocks) * 16;
  const int nh = min(16, group - h0);
  const int q4 = head_dim / 4;  // 4-float columns per row
  const int cols = nh * q4;     // <= 16 * 32: at most two per thread
  float M[2] = {-INFINITY, -INFINITY}, L[2] = {0.f, 0.f};
  float4 A[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
  auto prow = [&](int p, int h) {  // partial row of piece p
    return (static_cast<size_t>(p) * 2 + (p == k_first ? 1 : 0)) * nhm + h;
  };
  for (int c0 = k_first; c0 <= k_last; c0 += kMergeChunk) {
    const int n = min(kMergeChunk, k_last + 1 - c0);
    for (int t = threadIdx.x; t < n * nh; t += kThreads) {
      const int i = t / nh, h = t % nh;
      const size_t pr = prow(c0 + i, h);
      sm[i][h] = part_ml[2 * pr];
      sl[i][h] = part_ml[2 * pr + 1];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = threadIdx.x + u * kThreads;
      if (c >= cols) break;
      const int h = c / q4, d4 = c % q4;
      float cm = M[u];
      for (int i = 0; i < n; ++i) cm = fmaxf(cm, sm[i][h]);
      if (cm == -INFINITY) continue;  // nothing attended yet
      const float rescale = fast_exp2(M[u] - cm);
      float4 acc = make_float4(A[u].x * rescale, A[u].y * rescale, A[u].z * rescale,
                               A[u].w * rescale);
      float l = L[u] * rescale;
      for (int i = 0; i < n; ++i) {
        const float f = fast_exp2(sm[i][h] - cm);
        const float4 v =
            *reinterpret_cast<const float4*>(part_acc + prow(c0 + i, h) * head_dim + 4 * d4);
        l = fmaf(f, sl[i][h], l);
        acc.x = fmaf(f, v.x, acc.x);
        acc.y = fmaf(f, v.y, acc.y);
        acc.z = fmaf(f, v.z, acc.z);
        acc.w = fmaf(f, v.w, acc.w);
      }
      M[u] = cm;
      L[u] = l;
      A[u] = acc;
    }
    __syncthreads();  // sm, sl are rewritten by the next chunk
  }
  const size_t row0 = static_cast<size_t>(s) * hq_total + g * group + h0;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = threadIdx.x + u * kThreads;
    if (c >= cols) break;
    const int h = c / q4, d4 = c % q4;
    const float inv = L[u] > 0.f ? 1.f / L[u] : 0.f;
    typename Tag::Bits* o4 = out + (row0 + h) * head_dim + 4 * d4;
    o4[0] = Tag::from_f32(A[u].x * inv);
    o4[1] = Tag::from_f32(A[u].y * inv);
    o4[2] = Tag::from_f32(A[u].z * inv);
    o4[3] = Tag::from_f32(A[u].w * inv);
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

inline int pow2_at_least(int n) {
  int p = 1;
  while (p < n) p *= 2;
  return p;
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Resolved partition size (a positive multiple of 16) and partition count.
struct Split {
  int part;
  int np;
};

// Fixed partitions for the paths that have no balanced split.  Partitions of
// 1024 positions keep split overhead (partials, merge) near 1 % of the K/V
// bytes; shorter ones are used only when the batch would otherwise give fewer
// than ~2048 work items (a few long sequences), so that every CU has work.
// Batches whose longest sequence fits one partition are not split.
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

bool mfma_path(pa_dtype dt, int head_dim) {
  return (dt == PA_BF16 || dt == PA_F16) && (head_dim == 64 || head_dim == 128);
}

// Workspace of the fixed-partition path: [plan: meta (256 B), items, split
// list] [m, l of every partial] [acc of every partial]; the partial areas
// exist only when some sequence is split.
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

// Workspace of the balanced path: meta (256 B), range starts, and two partial
// slots per work-group of min(16, hq) rows (rounded up to a power of two)
// each.  Independent of the lengths.
Layout balanced_layout(int hq, int head_dim) {
  Layout l;
  const size_t rows = static_cast<size_t>(kMaxBalancedGroups) * 2 * pow2_at_least(std::min(16, hq));
  l.meta = 0;
  l.items = kAlign;  // range starts
  l.split = l.items;
  l.ml = l.items + align_up(static_cast<size_t>(kMaxBalancedGroups + 1) * sizeof(int4));
  l.acc = l.ml + align_up(rows * 2 * sizeof(float));
  l.total = l.acc + align_up(rows * head_dim * sizeof(float));
  return l;
}

int resident_groups(const void* kernel, size_t lds);

// Cap on the balanced grid set by pa_decode_set_max_groups (0: none).
int g_max_groups = 0;

// Work-groups of the balanced grid: the resident count of `kernel` on the
// current device (CUs x occupancy, cached per device and kernel), at most
// kMaxBalancedGroups and the cap.
int balanced_groups(const void* kernel, size_t lds) {
  const int n = resident_groups(kernel, lds);
  return n > 0 && g_max_groups > 0 ? std::min(n, g_max_groups) : n;
}

int resident_groups(const void* kernel, size_t lds) {
  struct Entry {
    int dev;
    const void* fn;
    size_t lds;
    int n;
  };
  static Entry cache[32];
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  for (int i = 0; i < used; ++i)
    if (cache[i].dev == dev && cache[i].fn == kernel && cache[i].lds == lds) return cache[i].n;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kItemThreads, lds) !=
          hipSuccess)
    return -1;
  const int n = std::max(1, std::min(kMaxBalancedGroups, cus * std::max(per_cu, 1)));
  if (used < 32) cache[used++] = Entry{dev, kernel, lds, n};
  return n;
}

template <typename Tag>
DecodeArgs mfma_args(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* tables, const int32_t* lens, float scale_log2, void* out,
                     int num_seqs, int hq, int hkv, int max_blocks, const Split& sp, float* ws_ml,
                     float* ws_acc) {
  DecodeArgs a;
  const int group = hq / hkv;
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
  a.head_blocks = (group + 15) / 16;
  a.max_blocks = max_blocks;
  a.part_size = sp.part;
  a.np_max = sp.np;
  a.nh_max = std::min(16, group);
  return a;
}

// The balanced decode kernel for a head size and head-group rows (1 .. 16).
template <typename Tag>
const void* balanced_kernel_for(int head_dim, int nh) {
#define PA_BALANCED_CASE(DIM, NH)                                                  \
  if (head_dim == DIM && nh == NH)                                                 \
    return reinterpret_cast<const void*>(&decode_balanced_kernel<Tag, DIM, NH>);
  PA_BALANCED_CASE(128, 1) PA_BALANCED_CASE(128, 2) PA_BALANCED_CASE(128, 4)
  PA_BALANCED_CASE(128, 8) PA_BALANCED_CASE(128, 16)
  PA_BALANCED_CASE(64, 1) PA_BALANCED_CASE(64, 2) PA_BALANCED_CASE(64, 4)
  PA_BALANCED_CASE(64, 8) PA_BALANCED_CASE(64, 16)
#undef PA_BALANCED_CASE
  return nullptr;
}

// Balanced path: balance plan, decode over equal block ranges, merge of the
// cut units.
template <typename Tag>
pa_status launch_balanced(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* tables, const int32_t* lens, float scale_log2, void* out,
                          int num_seqs, int hq, int hkv, int head_dim, int max_blocks, char* ws,
                          hipStream_t st) {
  const Layout lay = balanced_layout(hq, head_dim);
  int* meta = reinterpret_cast<int*>(ws + lay.meta);
  int4* start = reinterpret_cast<int4*>(ws + lay.items);
  float* part_ml = reinterpret_cast<float*>(ws + lay.ml);
  float* part_acc = reinterpret_cast<float*>(ws + lay.acc);
  DecodeArgs a = mfma_args<Tag>(q, k_cache, v_cache, tables, lens, scale_log2, out, num_seqs, hq,
                                hkv, max_blocks, Split{kBlock, 1}, nullptr, nullptr);
  a.nh_max = pow2_at_least(a.nh_max);  // LDS and partial rows per head group
  const size_t lds = comb_floats(kItemWaves, a.nh_max, head_dim) * sizeof(float);
  const void* kernel = balanced_kernel_for<Tag>(head_dim, a.nh_max);
  if (!kernel) return PA_ERR_UNSUPPORTED;
  const int groups = balanced_groups(kernel, lds);
  if (groups <= 0) return PA_ERR_DEVICE;

  BalanceArgs ba{lens, start, meta, num_seqs, max_blocks, hkv * a.head_blocks, groups};
  int slot = timing_start(PA_KERNEL_DECODE_PLAN, st);
  decode_balance_kernel<<<dim3(1), dim3(kThreads), 0, st>>>(ba);
  pa_status status = launch_status();
  timing_stop(slot, st);
  if (status != PA_OK) return status;

  slot = timing_start(PA_KERNEL_DECODE, st);
  const dim3 g3(static_cast<uint32_t>(groups)), b3(kItemThreads);
  void* args[] = {&a, &start, &meta, &part_ml, &part_acc};
  status = hipLaunchKernel(kernel, g3, b3, args, lds, st) == hipSuccess ? PA_OK : PA_ERR_DEVICE;
  timing_stop(slot, st);
  if (status != PA_OK) return status;

  slot = timing_start(PA_KERNEL_DECODE_REDUCE, st);
  decode_balanced_merge_kernel<Tag><<<g3, dim3(kThreads), 0, st>>>(
      start, meta, part_ml, part_acc, static_cast<typename Tag::Bits*>(out), hq, a.group,
      a.head_blocks, head_dim, a.nh_max);
  status = launch_status();
  timing_stop(slot, st);
  return status;
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
  const int64_t grid = use_mfma ? static_cast<int64_t>(plan_capacity(num_seqs, sp.np)) * hkv *
                                      head_blocks
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
      const DecodeArgs a = mfma_args<Tag>(q, k_cache, v_cache, tables, lens, scale_log2, out,
                                          num_seqs, hq, hkv, max_blocks, sp, ws_ml, ws_acc);
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

pa_status pa_decode_set_max_groups(int32_t max_groups) {
  if (max_groups < 0) return PA_ERR_INVALID_ARG;
  pa::g_max_groups = max_groups;
  return PA_OK;
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size) {
  pa::Split sp;
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0) return 0;
  const size_t balanced = pa::balanced_layout(num_q_heads, head_dim).total;
  if (partition_size == PA_PARTITION_BALANCED) return balanced;
  // the automatic choice shrinks partitions for fewer KV heads, so sizing with
  // one KV head covers every head count
  if (!pa::resolve_split(partition_size, num_seqs, 1, max_context_len, &sp)) return 0;
  const size_t fixed = pa::workspace_layout(num_seqs, num_q_heads, head_dim, sp).total;
  return fixed;
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
  const bool use_mfma = mfma_path(dtype, head_dim);
  if (partition_size == PA_PARTITION_BALANCED && !use_mfma) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return PA_ERR_INVALID_ARG;
  const bool balanced = use_mfma && partition_size == PA_PARTITION_BALANCED;
  Split sp{kBlock, 1};
  size_t need;
  if (balanced) {
    // block indices of the balanced split stay below 2^30
    const int64_t units = static_cast<int64_t>(num_kv_heads) * ((num_q_heads / num_kv_heads + 15) / 16);
    if (static_cast<int64_t>(num_seqs) * units * max_blocks_per_seq >= (int64_t{1} << 30))
      return PA_ERR_INVALID_ARG;
    need = balanced_layout(num_q_heads, head_dim).total;
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
  switch (dtype) {
    case PA_BF16:
      if (balanced)
        return launch_balanced<BF16T>(q, k_cache, v_cache, block_tables, context_lens, scale_log2,
                                      out, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                      max_blocks_per_seq, ws, st);
      return launch<BF16T>(q, k_cache, v_cache, block_tables, context_lens, scale_log2, out,
                           num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, sp,
                           ws, use_mfma, st);
    case PA_F16:
      if (balanced)
        return launch_balanced<F16T>(q, k_cache, v_cache, block_tables, context_lens, scale_log2,
                                     out, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                     max_blocks_per_seq, ws, st);
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
