// Paged decode attention for gfx950 (CDNA4, wave64).
//
// One new query per head attends to every cached K/V of its sequence; K and V
// are gathered block by block through the sequence's block table ("KV Cache for
// the intermediate", section "Precise scientific definition"; "PagedAttention
// for the professional", section "The scientific explanation").  The query
// heads of one GQA group share a KV head ("KV Cache for the intermediate",
// section "Grouped Query Attention"), so a work-group serves the whole group
// and every K/V byte is read from HBM once per step.
//
// Work split: one work-group (4 waves) per (sequence, KV head, partition of P
// positions, group of up to 16 query heads).  Sequences longer than P are cut
// into partitions whose partial results (running max m, sum l, unnormalised
// acc) are merged by a second kernel with the running-max rule (Milakov and
// Gimelshein 2018); a sequence with a single partition is normalised and
// written directly.  Waves of a work-group take the partition's 16-token
// blocks round-robin and merge their partials through LDS at the end.
//
// Matrix-core path (bf16/fp16, head_dim 64 or 128), per 16-token block:
//   scores[16 tok x 16 heads] = K[16 tok x D] . Q^T[D x 16 heads]
//       with v_mfma_f32_16x16x32_{bf16,f16}; lane l holds token l%16's 16-byte
//       K chunk (j*4 + l/16) so each of the D/32 loads reads 1 KiB contiguous;
//   online softmax in fp32 on the 4 scores each lane holds (one head, 4 tokens);
//   acc^T[D x 16 heads] += V^T[D x 16 tok] . P^T[16 tok x 16 heads]
//       with v_mfma_f32_16x16x16_{bf16,f16}; V is stored transposed per block,
//       so a lane's 4 token values of one dimension are 8 contiguous bytes and
//       each load reads 512 bytes contiguous.  P enters the matrix core in the
//       storage dtype (bf16 or fp16); scores, exponentials, sums and the
//       accumulator stay fp32.
// Heads beyond the group's size occupy the idle columns of the 16-wide
// operands and are never stored.  Positions past the sequence end are masked
// by select (scores to -inf, V values to 0), never by multiplication, so stale
// or NaN bits in a block's tail cannot reach the result.
//
// Generic path (any supported dtype/head_dim, fp32 in particular): one
// work-group per query head, VALU dot products, 256-position chunks with the
// same online softmax and the same partial-result format.
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
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Merge the per-wave partials in LDS and store the work-group's result: the
// normalised output when the sequence has one partition, else the partial.
template <typename Tag, int D, int H>
__device__ __forceinline__ void store_result(const float (&sm_m)[kWaves][H],
                                             const float (&sm_l)[kWaves][H],
                                             const float (&sm_acc)[kWaves][H][D], int nh,
                                             size_t row0, int p, int nparts, int np_max,
                                             typename Tag::Bits* __restrict__ out,
                                             float* __restrict__ ws_ml,
                                             float* __restrict__ ws_acc) {
  for (int e = threadIdx.x; e < nh * D; e += kThreads) {
    const int h = e / D, d = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = fast_exp2(sm_m[w][h] - M);
        L = fmaf(f, sm_l[w][h], L);
        A = fmaf(f, sm_acc[w][h][d], A);
      }
    }
    const size_t row = row0 + h;
    if (nparts <= 1) {
      out[row * D + d] = Tag::from_f32(L > 0.f ? A / L : 0.f);
    } else {
      const size_t part = row * np_max + p;
      ws_acc[part * D + d] = A;
      if (d == 0) {
        ws_ml[2 * part] = M;
        ws_ml[2 * part + 1] = L;
      }
    }
  }
}

template <typename Tag, int D>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ lens, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ ws_ml, float* __restrict__ ws_acc, int num_seqs, int hq_total, int hkv,
    int group, int head_blocks, int max_blocks, int part_size, int np_max) {
  constexpr int kSteps = D / 32;   // QK k-steps of 32 dims
  constexpr int kSlices = D / 16;  // PV output slices of 16 dims
  __shared__ float sm_m[kWaves][16];
  __shared__ float sm_l[kWaves][16];
  __shared__ float sm_acc[kWaves][16][D];

  int idx = blockIdx.x;
  const int hb = idx % head_blocks;
  idx /= head_blocks;
  const int g = idx % hkv;
  idx /= hkv;
  const int s = idx % num_seqs;
  const int p = idx / num_seqs;
  // lengths beyond the table width are cut to it, so a bad length cannot read
  // past the table row
  const int len = min(max(lens[s], 0), max_blocks * kBlock);
  const int start = p * part_size;
  if (p > 0 && start >= len) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int n = lane & 15;  // token row (K, scores) / head column (Q, P, acc)
  const int kg = lane >> 4; // k-group of the MFMA operands
  const int h0 = hb * 16;
  const int nh = min(16, group - h0);
  const int end = min(len, start + part_size);
  const int nblk = (end - start + kBlock - 1) / kBlock;
  const int blk0 = start / kBlock;
  const int nparts = min((len + part_size - 1) / part_size, np_max);

  uint4 qf[kSteps];
  if (n < nh) {
    const uint16_t* qp = q + (static_cast<size_t>(s) * hq_total + g * group + h0 + n) * D;
#pragma unroll
    for (int j = 0; j < kSteps; ++j) qf[j] = *reinterpret_cast<const uint4*>(qp + (j * 4 + kg) * 8);
  } else {
#pragma unroll
    for (int j = 0; j < kSteps; ++j) qf[j] = make_uint4(0, 0, 0, 0);
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t acc[kSlices];
#pragma unroll
  for (int i = 0; i < kSlices; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int32_t* trow = tables + static_cast<size_t>(s) * max_blocks + blk0;
  const size_t head_elems = static_cast<size_t>(D) * kBlock;
  for (int i = wave; i < nblk; i += kWaves) {
    const int phys = trow[i];
    const size_t base = (static_cast<size_t>(phys) * hkv + g) * head_elems;
    const uint16_t* kb = k_cache + base;
    const uint16_t* vb = v_cache + base;
    uint4 kf[kSteps];
#pragma unroll
    for (int j = 0; j < kSteps; ++j) kf[j] = *reinterpret_cast<const uint4*>(kb + j * 512 + lane * 8);
    uint2 vf[kSlices];
#pragma unroll
    for (int sl = 0; sl < kSlices; ++sl)
      vf[sl] = *reinterpret_cast<const uint2*>(vb + (sl * 16 + n) * kBlock + kg * 4);

    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kSteps; ++j) sc = Mfma<Tag>::qk(kf[j], qf[j], sc);

    const int pos0 = (blk0 + i) * kBlock + kg * 4;  // position of this lane's first score
    float s4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) s4[r] = (pos0 + r < end) ? sc[r] * scale_log2 : -INFINITY;
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

    if ((blk0 + i + 1) * kBlock > end) {  // tail block: zero V of masked positions
      const uint32_t lo = (pos0 + 0 < end ? 0x0000FFFFu : 0u) | (pos0 + 1 < end ? 0xFFFF0000u : 0u);
      const uint32_t hi = (pos0 + 2 < end ? 0x0000FFFFu : 0u) | (pos0 + 3 < end ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int sl = 0; sl < kSlices; ++sl) {
        vf[sl].x &= lo;
        vf[sl].y &= hi;
      }
    }
    const uint2 pf = Mfma<Tag>::pack(p4[0], p4[1], p4[2], p4[3]);
#pragma unroll
    for (int sl = 0; sl < kSlices; ++sl) acc[sl] = Mfma<Tag>::pv(vf[sl], pf, acc[sl]);
  }

  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (kg == 0) {
    sm_m[wave][n] = m_run;
    sm_l[wave][n] = l_tot;
  }
#pragma unroll
  for (int sl = 0; sl < kSlices; ++sl)
    *reinterpret_cast<f32x4_t*>(&sm_acc[wave][n][sl * 16 + kg * 4]) = acc[sl];
  __syncthreads();

  const size_t row0 = static_cast<size_t>(s) * hq_total + g * group + h0;
  store_result<Tag, D, 16>(sm_m, sm_l, sm_acc, nh, row0, p, nparts, np_max, out, ws_ml, ws_acc);
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
template <typename Tag>
__global__ __launch_bounds__(kWave) void decode_reduce_kernel(
    const float* __restrict__ ws_ml, const float* __restrict__ ws_acc,
    const int32_t* __restrict__ lens, typename Tag::Bits* __restrict__ out, int hq_total,
    int head_dim, int max_blocks, int part_size, int np_max) {
  const size_t row = blockIdx.x;
  const int len = min(max(lens[row / hq_total], 0), max_blocks * kBlock);
  const int np = min((len + part_size - 1) / part_size, np_max);
  if (np <= 1) return;
  const float* ml = ws_ml + row * np_max * 2;
  float M = -INFINITY;
  for (int i = 0; i < np; ++i) M = fmaxf(M, ml[2 * i]);
  float L = 0.f;
  for (int i = 0; i < np; ++i) L = fmaf(fast_exp2(ml[2 * i] - M), ml[2 * i + 1], L);
  const float* acc = ws_acc + row * np_max * head_dim;
  for (int d = threadIdx.x; d < head_dim; d += kWave) {
    float A = 0.f;
    for (int i = 0; i < np; ++i) A = fmaf(fast_exp2(ml[2 * i] - M), acc[i * head_dim + d], A);
    out[row * head_dim + d] = Tag::from_f32(A / L);
  }
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Resolved partition size (a positive multiple of 16) and partition count.
struct Split {
  int part;
  int np;
};

int auto_partition(int num_seqs, int hkv, int max_len) {
  (void)num_seqs;
  (void)hkv;
  return max_len <= 512 ? 0 : 512;
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

size_t workspace_bytes(int num_seqs, int hq, int head_dim, const Split& sp) {
  if (sp.np <= 1) return 0;
  const size_t parts = static_cast<size_t>(num_seqs) * hq * sp.np;
  return align_up(parts * 2 * sizeof(float)) + align_up(parts * head_dim * sizeof(float));
}

bool mfma_path(pa_dtype dt, int head_dim) {
  return (dt == PA_BF16 || dt == PA_F16) && (head_dim == 64 || head_dim == 128);
}

template <typename Tag>
pa_status launch(const void* q, const void* k_cache, const void* v_cache, const int32_t* tables,
                 const int32_t* lens, float scale_log2, void* out, int num_seqs, int hq, int hkv,
                 int head_dim, int max_blocks, const Split& sp, float* ws_ml, float* ws_acc,
                 bool use_mfma, hipStream_t st) {
  using E = typename Tag::Bits;
  const int group = hq / hkv;
  const int head_blocks = use_mfma ? (group + 15) / 16 : 1;
  const int64_t grid = use_mfma ? static_cast<int64_t>(sp.np) * num_seqs * hkv * head_blocks
                                : static_cast<int64_t>(sp.np) * num_seqs * hq;
  if (grid > 0x7fffffff) return PA_ERR_INVALID_ARG;
  const dim3 grid3(static_cast<uint32_t>(grid)), block3(kThreads);
  int slot = timing_start(PA_KERNEL_DECODE, st);
  if (use_mfma) {
    if constexpr (sizeof(E) == 2) {
      if (head_dim == 128)
        decode_mfma_kernel<Tag, 128><<<grid3, block3, 0, st>>>(
            static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
            static_cast<const uint16_t*>(v_cache), tables, lens, scale_log2,
            static_cast<uint16_t*>(out), ws_ml, ws_acc, num_seqs, hq, hkv, group, head_blocks,
            max_blocks, sp.part, sp.np);
      else
        decode_mfma_kernel<Tag, 64><<<grid3, block3, 0, st>>>(
            static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
            static_cast<const uint16_t*>(v_cache), tables, lens, scale_log2,
            static_cast<uint16_t*>(out), ws_ml, ws_acc, num_seqs, hq, hkv, group, head_blocks,
            max_blocks, sp.part, sp.np);
    }
  } else {
    decode_generic_kernel<Tag><<<grid3, block3, 0, st>>>(
        static_cast<const E*>(q), static_cast<const E*>(k_cache), static_cast<const E*>(v_cache),
        tables, lens, scale_log2, static_cast<E*>(out), ws_ml, ws_acc, num_seqs, hq, hkv, group,
        head_dim, max_blocks, sp.part, sp.np);
  }
  pa_status status = launch_status();
  timing_stop(slot, st);
  if (status != PA_OK || sp.np <= 1) return status;
  slot = timing_start(PA_KERNEL_DECODE_REDUCE, st);
  decode_reduce_kernel<Tag><<<dim3(static_cast<uint32_t>(num_seqs * hq)), dim3(kWave), 0, st>>>(
      ws_ml, ws_acc, lens, static_cast<E*>(out), hq, head_dim, max_blocks, sp.part, sp.np);
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
  // the auto choice does not depend on the KV head count today; pass 1
  if (!pa::resolve_split(partition_size, num_seqs, 1, max_context_len, &sp)) return 0;
  return pa::workspace_bytes(num_seqs, num_q_heads, head_dim, sp);
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
  const size_t need = pa::workspace_bytes(num_seqs, num_q_heads, head_dim, sp);
  if (need > 0 && (!workspace || workspace_bytes < need ||
                   reinterpret_cast<uintptr_t>(workspace) % kAlign != 0))
    return PA_ERR_WORKSPACE;
  float* ws_ml = static_cast<float*>(workspace);
  float* ws_acc = nullptr;
  if (need > 0) {
    const size_t parts = static_cast<size_t>(num_seqs) * num_q_heads * sp.np;
    ws_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                      align_up(parts * 2 * sizeof(float)));
  }
  const float scale_log2 = scale * kLog2e;
  const bool use_mfma = mfma_path(dtype, head_dim);
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case PA_BF16:
      return launch<BF16T>(q, k_cache, v_cache, block_tables, context_lens, scale_log2, out,
                           num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, sp,
                           ws_ml, ws_acc, use_mfma, st);
    case PA_F16:
      return launch<F16T>(q, k_cache, v_cache, block_tables, context_lens, scale_log2, out,
                          num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, sp,
                          ws_ml, ws_acc, use_mfma, st);
    default:
      return launch<F32T>(q, k_cache, v_cache, block_tables, context_lens, scale_log2, out,
                          num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, sp,
                          ws_ml, ws_acc, false, st);
  }
}

}  // extern "C"
