// Device pieces shared by the decode and prefill kernels (matrix-core
// operands, block loads, the online softmax of one block, the merge of waves)
// and the host helpers of the decode path.  Included by pa_decode.hip (items
// kernels, generic path, the decode entry points) and pa_prefill.hip.
#pragma once

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
// The same loads with the non-temporal hint (cache policy bit nt), for data
// read once per call -- the cached K/V.  Streamed past the caches this way,
// a random gather of 4 KiB pieces measured 6.3-6.4 TB/s on MI355X against
// 5.5-5.6 TB/s with the default policy (same kernel, same addresses).
constexpr int kNonTemporal = 2;
__device__ __forceinline__ uint4 stream_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 stream_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNonTemporal);
  return make_uint2(v.x, v.y);
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
  const float* k_scale;  // INT8 cache only: [Hkv][D] per-channel scales
  const float* v_scale;
  int* arrivals;         // split sequences merged in-kernel: [S][heads] counters, else null
  // shared prefixes (pfx_seqs null: none): the caller's member list and
  // group starts, and the plan's group of each sequence, partial count of
  // each sequence and a member of each group whose row holds its blocks
  const int* pfx_seqs;
  const int* pfx_start;
  const int* grp_of;
  const int* nparts_of;
  const int* grp_leader;
  int num_members, members_per_tile;
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
  for (int t = 0; t < D / 32; ++t) r.kf[t] = stream_load16(rk, ko + t * 1024);
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) r.vf[sl] = stream_load8(rv, vo + sl * 512);
}

// Softmax update and PV product of one block (logical index blk) whose raw
// scores sc (lane l: head l%16, tokens 4*(l/16) .. +3) are known: scores are
// multiplied by sl2 (the softmax scale in log2 units), positions at or past
// `len` are masked, vf holds the block's V as PV A operands.
// `lim` (per lane, at most len): scores of positions at or past it are masked
// (a causal limit per column); `len` bounds the V rows that hold data.
template <typename Tag, int D>
__device__ __forceinline__ void block_update_lim(uint2* vf, f32x4_t sc, float sl2, int blk,
                                                 int len, int lim, WaveState<D>& st) {
  constexpr int kSlices = D / 16;  // PV output slices of 16 dims
  const int lane = threadIdx.x & (kWave - 1);
  const int kg = lane >> 4;  // k-group of the MFMA operands
  const int pos0 = blk * kBlock + kg * 4;  // position of this lane's first score
  float s4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s4[i] = (pos0 + i < lim) ? sc[i] * sl2 : -INFINITY;
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
      vf[sl].x &= lo;
      vf[sl].y &= hi;
    }
  }
  // P as hi + lo in the storage dtype: two products, near-fp32 weights
  const uint2 ph = Mfma<Tag>::pack(p4[0], p4[1], p4[2], p4[3]);
  const uint2 pl = Mfma<Tag>::pack(p4[0] - Mfma<Tag>::lo(ph.x), p4[1] - Mfma<Tag>::hi(ph.x),
                                   p4[2] - Mfma<Tag>::lo(ph.y), p4[3] - Mfma<Tag>::hi(ph.y));
#pragma unroll
  for (int sl = 0; sl < kSlices; ++sl) {
    st.acc[sl] = Mfma<Tag>::pv(vf[sl], ph, st.acc[sl]);
    st.acc[sl] = Mfma<Tag>::pv(vf[sl], pl, st.acc[sl]);
  }
}

template <typename Tag, int D>
__device__ __forceinline__ void block_update(uint2* vf, f32x4_t sc, float sl2, int blk, int len,
                                             WaveState<D>& st) {
  block_update_lim<Tag, D>(vf, sc, sl2, blk, len, len, st);
}

// One block (logical index blk) into the running state: positions at or past
// `len` are masked.
// `qf(t)` gives the B operand of QK k-step t (registers or LDS).
template <typename Tag, int D, typename QOperand>
__device__ __forceinline__ void attend_block(const DecodeArgs& a, BlockRegs<D>& r, int blk,
                                             int len, const QOperand& qf, WaveState<D>& st) {
  constexpr int kSteps = D / 32;   // QK k-steps of 32 dims
  f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < kSteps; ++t) sc = Mfma<Tag>::qk(r.kf[t], qf(t), sc);
  block_update<Tag, D>(r.vf, sc, a.scale_log2, blk, len, st);
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

// Inclusive prefix sum over the 64 lanes of a wave from DPP moves, which are
// ALU operations, where a shuffle is a round trip through the LDS crossbar:
// Hillis-Steele steps of 1, 2, 4 and 8 lanes within each row of 16, then
// lane 15 of rows 0 and 2 added into rows 1 and 3 (row_bcast:15) and lane 31
// into rows 2 and 3 (row_bcast:31).  A lane whose source lies outside its
// row, or whose row the mask leaves out, adds the 0 passed as the old value.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2, 3
  return x;
}

// Exclusive scan over the 256 threads of a work-group of kVals counters at
// once; all[] receives the totals.  `tot` is LDS of kWaves * kVals ints.
template <int kVals>
__device__ __forceinline__ void block_scan(const int* cnt, int* excl, int* all, int* tot) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
#pragma unroll
  for (int c = 0; c < kVals; ++c) {
    const int x = wave_inclusive_sum(cnt[c]);
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

// ---- host helpers ----

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
  bool long_context = false;  // the longest context has >= 16K positions
  int waves = kItemWaves;     // waves per work-group of the matrix-core items kernels
  int max_len = 0;            // the call's bound on every length
  bool auto_part = false;     // part is the automatic choice (the plan may double it)
};

// Shared prefixes of a decode call: groups of sequences whose tables begin
// with the same blocks (device arrays; none when num_groups is 0).
struct SharedPrefix {
  const int32_t* seqs = nullptr;    // [num_members] sequences, group by group
  const int32_t* start = nullptr;   // [num_groups + 1]
  const int32_t* blocks = nullptr;  // [num_groups] shared leading table entries
  int num_groups = 0, num_members = 0;
};

// Byte offsets of a decode workspace's areas.
struct Layout {
  size_t meta, items, split, grp_of, nparts_of, grp_tokens, grp_leader, ml, acc, arrivals, total;
  int np_slots;  // partial slots per (sequence, query head)
};

inline bool mfma_path(pa_dtype dt, int head_dim) {
  return (dt == PA_BF16 || dt == PA_F16) && (head_dim == 64 || head_dim == 128);
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
  a.k_scale = nullptr;
  a.v_scale = nullptr;
  a.arrivals = nullptr;
  a.pfx_seqs = a.pfx_start = a.grp_of = a.nparts_of = a.grp_leader = nullptr;
  a.num_members = a.members_per_tile = 0;
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

}  // namespace
}  // namespace pa
