// Balanced split of the paged decode for gfx950: every wave gets the same
// amount of K/V work, whatever the mix of sequence lengths (see the section
// comments below).  Entry points for pa_decode.hip are declared in
// pa_decode_balanced.h; pa_decode_set_max_groups is defined here.
#include "pa_decode_balanced.h"
#include "pa_decode_common.h"

#include <mutex>

namespace pa {
namespace {

// ---- balanced split: every wave gets the same amount of work ----
//
// The work of a call is laid out as one row of "units" -- (sequence, KV head,
// query-head group), sequence-major.  A unit of a sequence of length len has
// nb = max(1, ceil(len/16)) blocks (a sequence of length 0 keeps one empty
// block so that its output is written) and costs kUnitCost + nb: the fixed
// part stands for what moving to another unit takes.  Of C cost in all, range
// k is [k*q, (k+1)*q) with q = ceil(C/G) for G resident waves (at most
// kStreamRangeCap, so that a range's block ids fit the wave's LDS; then there
// are more ranges than waves and the waves take them in turn); a range
// boundary inside a unit's fixed part moves to the unit's first block.  So
// range k runs from start[k] to start[k+1], each a (sequence, unit, first
// block) triple.  A unit that lies wholly in one range is normalised and
// stored; a unit cut by range boundaries leaves one partial per piece, merged
// by decode_balanced_merge_kernel.  Range k writes at most two partials: slot
// 0 for a unit that began before it, slot 1 for a unit that begins in it and
// runs past its end.
#ifndef PA_UNIT_COST
#define PA_UNIT_COST 2
#endif
constexpr int kUnitCost = PA_UNIT_COST;  // fixed cost of a unit, in blocks
constexpr int kMinQuota = 16;            // cost per work-group at least (> kUnitCost)
#ifndef PA_MAX_BALANCED_GROUPS
#define PA_MAX_BALANCED_GROUPS 2048
#endif
constexpr int kMaxBalancedGroups = PA_MAX_BALANCED_GROUPS;
static_assert(kUnitCost < kMinQuota, "a range must reach past a unit's fixed part");

struct BalanceArgs {
  const int32_t* lens;
  int4* start;  // [ranges + 1] range starts (sequence, unit in sequence, first block, 0); the
                // last one after the end (num_seqs, 0, 0, 0)
  int* meta;    // [0] C, [1] q, [2] ranges
  int num_seqs, max_blocks, units, groups;
  int max_q;       // largest range cost (0: none); more ranges than groups then
  int max_ranges;  // ranges the workspace holds
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
  int q = max(kMinQuota, (C + a.groups - 1) / a.groups);
  if (a.max_q > 0) q = min(q, a.max_q);
  // lengths past the caller's bound could ask for more ranges than the
  // workspace holds: then fewer, longer ones
  if ((C + q - 1) / q > a.max_ranges) q = (C + a.max_ranges - 1) / a.max_ranges;
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

// Merge of the units cut by range boundaries.  For each range boundary k
// (work-groups take them in a grid-stride loop) it looks at the start of
// range k; when it cuts a unit that began in range k-1 (boundary k
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
  const int nwg = meta[2];
  for (int k = blockIdx.x + 1; k < nwg; k += gridDim.x) {
  const int4 st = start[k];
  if (st.z == 0) continue;  // range k starts at a unit's first block: no cut
  const int4 prev = start[k - 1];
  if (prev.x == st.x && prev.y == st.y && prev.z > 0) continue;  // an earlier cut merges it
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
  __syncthreads();  // sm, sl are rewritten by the next unit
  }
}

// ---- the balanced split's decode kernel: one wave per range ----
//
// A range belongs to one wave, which takes every block of its units itself:
// no merge of waves and no barrier.  K and V go from HBM straight into a ring
// of kDepth block stages in the wave's LDS (buffer loads with the LDS
// destination), the wave refilling each stage as soon as it has read it, so
// kDepth blocks stay in flight across unit boundaries.  q of each unit goes
// into a ring of q slots the same way, and the block ids of the whole range
// into LDS when the range starts.  The wave waits for a stage by counting the
// loads issued after it (vector memory loads complete in issue order), and
// reads the stages with LDS loads written out here, so that no
// compiler-inserted wait drains the ring.  Rows that a unit finishes are
// parked in registers and stored when the range ends (a store among the loads
// in flight would break the count).

// One unit as the streamed kernel walks it: blocks [o, e) of unit j of
// sequence s, of which [o, min(e, nbr)) hold positions.
struct SUnit {
  int s, j, o, e, nbr, nb, len;
  int g, h0, nh;
  bool last;  // the range ends in this unit
  __device__ int end_real() const { return min(e, nbr); }
  __device__ bool empty() const { return end_real() <= o; }
  __device__ int blocks() const { return max(end_real() - o, 0); }
};

// Lengths of sequences base .. base+63 in one register (lane i: base + i).
struct LenWindow {
  int base, v;
  __device__ void load(const DecodeArgs& a, int b) {
    const uint32_t lane = threadIdx.x & (kWave - 1);
    base = b;
    const int n = min(64, a.num_seqs - b);
    const auto r = buffer_of(a.lens + b, static_cast<uint32_t>(max(n, 0)) * 4);
    v = min(max(static_cast<int>(buffer_load4(r, lane * 4)), 0), a.max_blocks * kBlock);
  }
  __device__ int get(const DecodeArgs& a, int s) {
    if (s - base >= 64) load(a, s);
    return __builtin_amdgcn_readlane(v, s - base);
  }
};

__device__ __forceinline__ SUnit stream_unit(const DecodeArgs& a, LenWindow& lw, int s, int j,
                                             int o, int4 end) {
  SUnit u;
  u.s = s;
  u.j = j;
  u.o = o;
  u.len = lw.get(a, s);
  u.nbr = (u.len + kBlock - 1) / kBlock;
  u.nb = max(1, u.nbr);
  u.last = s == end.x && j == end.y;
  u.e = u.last ? end.z : u.nb;
  u.g = j / a.head_blocks;
  u.h0 = (j % a.head_blocks) * 16;
  u.nh = min(16, a.group - u.h0);
  return u;
}

// The unit after u in the range, if any.
__device__ __forceinline__ bool stream_next(const DecodeArgs& a, LenWindow& lw, const SUnit& u,
                                            int4 end, SUnit& nx) {
  if (u.last) return false;
  int s = u.s, j = u.j + 1;
  if (j == a.hkv * a.head_blocks) {
    j = 0;
    ++s;
  }
  if (s == end.x && j == end.y && end.z == 0) return false;
  nx = stream_unit(a, lw, s, j, 0, end);
  return true;
}

typedef __attribute__((address_space(3))) void* lds_void_t;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// s_waitcnt vmcnt(n) (gfx9 encoding: vmcnt low bits [3:0], high bits [15:14];
// expcnt and lgkmcnt left unwaited)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Per-wave LDS of the streamed kernel.
template <int D, int NH, int DEPTH>
struct StreamLds {
  static constexpr int kBlk = 2 * D * kBlock * 2;           // K then V of one block-head
  static constexpr int kQSlots = DEPTH + 1;                 // units the ring can span
  // q rows of one unit, padded to whole 1 KiB load-to-LDS rounds (a round
  // writes 16 bytes for every lane, in range or not)
  static constexpr int kQBytes = (NH * D * 2 + 1023) / 1024 * 1024;
  static constexpr int kIds = 512;                          // block ids of one range
  static constexpr int kRing = 0;
  static constexpr int kQ = kRing + DEPTH * kBlk;
  static constexpr int kZero = kQ + kQSlots * kQBytes;      // a zero q row (idle columns)
  static constexpr int kIdsOff = kZero + D * 2;
  static constexpr int kBytes = kIdsOff + (kIds + kWave) * 4;  // a round writes 64 ids
};

#ifndef PA_STREAM_WG_WAVES
#define PA_STREAM_WG_WAVES 4
#endif
#ifndef PA_STREAM_RANGE_MULT
#define PA_STREAM_RANGE_MULT 1
#endif
constexpr int kStreamWaves = PA_STREAM_WG_WAVES;       // waves (ranges) per work-group
constexpr int kStreamThreads = kStreamWaves * kWave;
constexpr int kStreamRangeMult = PA_STREAM_RANGE_MULT;  // ranges per resident wave

template <int D, int NH, int DEPTH>
constexpr int stream_waves_lds() {
  return kStreamWaves * StreamLds<D, NH, DEPTH>::kBytes;
}

// Finished rows parked in registers: lane (n, kg) holds, per 16-dim slice,
// dims 4kg .. 4kg+3 of row n packed in the storage dtype.
template <int D>
struct Parked {
  uint32_t v[D / 8];
  int s, j;
};

template <typename Tag, int D>
__device__ __forceinline__ void park_rows(Parked<D>& p, const SUnit& u, const WaveState<D>& st) {
  float l_tot = st.l + __shfl_xor(st.l, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) {
    const f32x4_t v = st.acc[sl];
    p.v[2 * sl] = static_cast<uint32_t>(Tag::from_f32(v[0] * inv)) |
                  (static_cast<uint32_t>(Tag::from_f32(v[1] * inv)) << 16);
    p.v[2 * sl + 1] = static_cast<uint32_t>(Tag::from_f32(v[2] * inv)) |
                      (static_cast<uint32_t>(Tag::from_f32(v[3] * inv)) << 16);
  }
  p.s = u.s;
  p.j = u.j;
}

template <int D>
__device__ __forceinline__ void store_rows(const DecodeArgs& a, const Parked<D>& p) {
  const uint32_t lane = threadIdx.x & (kWave - 1);
  const uint32_t n = lane & 15, kg = lane >> 4;
  const int g = p.j / a.head_blocks, h0 = (p.j % a.head_blocks) * 16;
  const int nh = min(16, a.group - h0);
  // rows past the group fall outside the range and are dropped
  const auto r = buffer_of(a.out + (static_cast<size_t>(p.s) * a.hq_total + g * a.group + h0) * D,
                           static_cast<uint32_t>(nh) * D * 2);
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl)
    __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{p.v[2 * sl], p.v[2 * sl + 1]}, r,
                                          (n * D + sl * 16 + kg * 4) * 2, 0, 0);
}

// A partial (m, l, acc) of a cut unit into partial slot `slot` of range k.
template <int D, int NH>
__device__ __forceinline__ void store_partial(const SUnit& u, int k, int slot,
                                              const WaveState<D>& st, float* part_ml,
                                              float* part_acc) {
  const uint32_t lane = threadIdx.x & (kWave - 1);
  const uint32_t n = lane & 15, kg = lane >> 4;
  float l_tot = st.l + __shfl_xor(st.l, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const int prow0 = (k * 2 + slot) * NH;
  const auto r = buffer_of(part_acc + static_cast<size_t>(prow0) * D,
                           static_cast<uint32_t>(u.nh) * D * 4);
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) {
    const f32x4_t v = st.acc[sl];
    __builtin_amdgcn_raw_buffer_store_b128(
        u32x4_t{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                __float_as_uint(v[3])},
        r, (n * D + sl * 16 + kg * 4) * 4, 0, 0);
  }
  const auto rm = buffer_of(part_ml + 2 * prow0, static_cast<uint32_t>(u.nh) * 8);
  if (kg == 0)
    __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{__float_as_uint(st.m), __float_as_uint(l_tot)},
                                          rm, n * 8, 0, 0);
}

// One stage's MFMA operands and the unit's q from LDS, in one block of LDS
// loads that ends with their wait (K: 16 bytes per lane per k-step, 1 KiB
// apart; V: 8 bytes per lane per slice, 512 bytes apart; q: 16 bytes per lane
// per k-step, 64 bytes apart).
template <int D>
__device__ __forceinline__ void read_stage(uint32_t ka, uint32_t va, uint32_t qa, BlockRegs<D>& r,
                                           uint4* qf);

template <>
__device__ __forceinline__ void read_stage<128>(uint32_t ka, uint32_t va, uint32_t qa,
                                                BlockRegs<128>& r, uint4* qf) {
  asm volatile(
      "ds_read_b128 %0, %16\n"
      "ds_read_b128 %1, %16 offset:1024\n"
      "ds_read_b128 %2, %16 offset:2048\n"
      "ds_read_b128 %3, %16 offset:3072\n"
      "ds_read_b64 %4, %17\n"
      "ds_read_b64 %5, %17 offset:512\n"
      "ds_read_b64 %6, %17 offset:1024\n"
      "ds_read_b64 %7, %17 offset:1536\n"
      "ds_read_b64 %8, %17 offset:2048\n"
      "ds_read_b64 %9, %17 offset:2560\n"
      "ds_read_b64 %10, %17 offset:3072\n"
      "ds_read_b64 %11, %17 offset:3584\n"
      "ds_read_b128 %12, %18\n"
      "ds_read_b128 %13, %18 offset:64\n"
      "ds_read_b128 %14, %18 offset:128\n"
      "ds_read_b128 %15, %18 offset:192\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.kf[0]), "=&v"(r.kf[1]), "=&v"(r.kf[2]), "=&v"(r.kf[3]), "=&v"(r.vf[0]),
        "=&v"(r.vf[1]), "=&v"(r.vf[2]), "=&v"(r.vf[3]), "=&v"(r.vf[4]), "=&v"(r.vf[5]),
        "=&v"(r.vf[6]), "=&v"(r.vf[7]), "=&v"(qf[0]), "=&v"(qf[1]), "=&v"(qf[2]), "=&v"(qf[3])
      : "v"(ka), "v"(va), "v"(qa)
      : "memory");
}

template <>
__device__ __forceinline__ void read_stage<64>(uint32_t ka, uint32_t va, uint32_t qa,
                                               BlockRegs<64>& r, uint4* qf) {
  asm volatile(
      "ds_read_b128 %0, %8\n"
      "ds_read_b128 %1, %8 offset:1024\n"
      "ds_read_b64 %2, %9\n"
      "ds_read_b64 %3, %9 offset:512\n"
      "ds_read_b64 %4, %9 offset:1024\n"
      "ds_read_b64 %5, %9 offset:1536\n"
      "ds_read_b128 %6, %10\n"
      "ds_read_b128 %7, %10 offset:64\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.kf[0]), "=&v"(r.kf[1]), "=&v"(r.vf[0]), "=&v"(r.vf[1]), "=&v"(r.vf[2]),
        "=&v"(r.vf[3]), "=&v"(qf[0]), "=&v"(qf[1])
      : "v"(ka), "v"(va), "v"(qa)
      : "memory");
}

#ifndef PA_STREAM_DEPTH
#define PA_STREAM_DEPTH 3
#endif
constexpr int kParked = 4;  // finished units held in registers
constexpr int kStreamLdsMax = 160 * 1024 * kStreamWaves / 4;  // a CU's LDS over 4 waves

// Blocks in flight per wave: PA_STREAM_DEPTH, or fewer where the four waves'
// LDS would not fit one CU.
template <int D, int NH>
constexpr int stream_depth() {
  return stream_waves_lds<D, NH, PA_STREAM_DEPTH>() <= kStreamLdsMax ? PA_STREAM_DEPTH
         : stream_waves_lds<D, NH, 2>() <= kStreamLdsMax             ? 2
                                                                     : 1;
}

template <typename Tag, int D, int NH>
__global__ __launch_bounds__(kStreamThreads, 1) void decode_stream_kernel(
    DecodeArgs a, const int4* __restrict__ start, const int* __restrict__ meta,
    float* __restrict__ part_ml, float* __restrict__ part_acc) {
  constexpr int kDepth = stream_depth<D, NH>();
  using L = StreamLds<D, NH, kDepth>;
  constexpr int kSteps = D / 32;
  extern __shared__ char stream_lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t lane = threadIdx.x & (kWave - 1);
  const uint32_t qn_lane = lane & 15, qkg = lane >> 4;
  char* my = stream_lds + wave * L::kBytes;
  const int nranges = meta[2];
  const int workers = gridDim.x * kStreamWaves;

  // the zero q row read by head columns past the group
  if (NH < 16 && lane < D / 8) reinterpret_cast<uint4*>(my + L::kZero)[lane] = make_uint4(0, 0, 0, 0);

  for (int k = blockIdx.x * kStreamWaves + wave; k < nranges; k += workers) {
    const int4 st0 = start[k];
    const int4 end = start[k + 1];
    LenWindow lw;
    lw.load(a, st0.x);

    // block ids of the range into LDS, unit after unit
    {
      LenWindow lwl = lw;
      SUnit u = stream_unit(a, lwl, st0.x, st0.y, st0.z, end);
      int at = 0;
      for (;;) {
        const int nblk = u.blocks();
        const int32_t* row = a.tables + static_cast<size_t>(u.s) * a.max_blocks + u.o;
        for (int c = 0; c < nblk && at < L::kIds; c += kWave) {
          const int n = min(min(kWave, nblk - c), L::kIds - at);
          const auto r = buffer_of(row + c, static_cast<uint32_t>(n) * 4);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t)(my + L::kIdsOff + at * 4), 4,
                                                   lane * 4, 0, 0, 0);
          at += n;
        }
        SUnit nx;
        if (!stream_next(a, lwl, u, end, nx)) break;
        u = nx;
      }
    }
    wait_vm<0>();  // the ids (and the length window) are in

    // issue side: unit iu, its next block ib; r_issue: index of that block
    // among the range's blocks (its id's slot); q_ord: q slot of iu
    LenWindow lwi = lw;
    SUnit iu = stream_unit(a, lwi, st0.x, st0.y, st0.z, end);
    int ib = iu.o, r_issue = 0, iu_ord = 0;
    bool issue_live = true;
    auto load_q_lds = [&](const SUnit& u, int ord) {
      const auto rq = buffer_of(a.q + (static_cast<size_t>(u.s) * a.hq_total + u.g * a.group + u.h0) * D,
                                static_cast<uint32_t>(u.nh) * D * 2);
      char* dst = my + L::kQ + (ord % L::kQSlots) * L::kQBytes;
#pragma unroll
      for (int c = 0; c < NH * D * 2; c += kWave * 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void_t)(dst + c), 16, lane * 16 + c, 0, 0,
                                                 0);
    };
    // move the issue side onto the next unit with positions (its q loads
    // first), or mark the range's loads done
    auto issue_enter = [&]() {
      while (ib >= iu.end_real()) {
        SUnit nx;
        if (!stream_next(a, lwi, iu, end, nx)) {
          issue_live = false;
          return;
        }
        iu = nx;
        ib = iu.o;
        if (!iu.empty()) {
          ++iu_ord;
          load_q_lds(iu, iu_ord);
        }
      }
    };
    if (!iu.empty()) load_q_lds(iu, 0);
    issue_enter();
    auto issue = [&](int stage) {
      // the block's id from LDS
      int id;
      asm volatile("ds_read_b32 %0, %1\n s_waitcnt lgkmcnt(0)"
                   : "=&v"(id)
                   : "v"(lds_addr(my + L::kIdsOff + min(r_issue, L::kIds - 1) * 4)));
      id = __builtin_amdgcn_readfirstlane(id);
      const size_t off = (static_cast<size_t>(id) * a.hkv + iu.g) * (D * kBlock);
      const auto rk = buffer_of(a.k_cache + off, D * kBlock * 2);
      const auto rv = buffer_of(a.v_cache + off, D * kBlock * 2);
      char* dst = my + L::kRing + stage * L::kBlk;
#pragma unroll
      for (int c = 0; c < D * kBlock * 2; c += kWave * 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t)(dst + c), 16, lane * 16 + c, 0, 0,
                                                 0);
#pragma unroll
      for (int c = 0; c < D * kBlock * 2; c += kWave * 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t)(dst + D * kBlock * 2 + c), 16,
                                                 lane * 16 + c, 0, 0, 0);
      ++ib;
      ++r_issue;
      issue_enter();
    };
    constexpr int kLoadsPerBlock = 2 * (D * kBlock * 2) / (kWave * 16);  // DMA ops per stage

    // compute side: unit cu, next block cb, q slot cu_ord
    LenWindow lwc = lw;
    SUnit cu = stream_unit(a, lwc, st0.x, st0.y, st0.z, end);
    int cb = cu.o, cu_ord = 0;
    WaveState<D> st;
    st.reset();
    Parked<D> park[kParked];
    int used = 0;
    WaveState<D> first_part;
    SUnit first_unit = cu;
    bool has_first_part = false;
    bool drain = false;  // stores were issued: the next wait must be for all loads
    auto flush = [&]() {
#pragma unroll
      for (int i = 0; i < kParked; ++i)
        if (i < used) store_rows<D>(a, park[i]);
      used = 0;
      drain = true;
    };
    // finish unit cu: park its rows, or store it as a partial
    auto finish = [&]() {
      const bool whole = cu.o == 0 && cu.e == cu.nb;
      if (whole) {
        if (used == kParked) flush();
#pragma unroll
        for (int i = 0; i < kParked; ++i)
          if (i == used) park_rows<Tag, D>(park[i], cu, st);
        ++used;
      } else if (cu.o > 0) {
        // the range's first unit, cut: its partial waits in registers until
        // the range ends (no loads are in flight then)
        first_part = st;
        first_unit = cu;
        has_first_part = true;
      } else {
        // the range's last unit, cut: nothing is in flight after it
        store_partial<D, NH>(cu, k, 1, st, part_ml, part_acc);
        drain = true;
      }
    };
    // move the compute side to the next unit with positions, finishing the
    // units without positions on the way; false at the range's end
    auto compute_enter = [&]() {
      for (;;) {
        SUnit nx;
        if (!stream_next(a, lwc, cu, end, nx)) return false;
        cu = nx;
        st.reset();
        if (!cu.empty()) break;
        finish();
      }
      cb = cu.o;
      ++cu_ord;
      return true;
    };
    bool compute_live = true;
    if (cu.empty()) {
      finish();
      compute_live = compute_enter();
    }

    int inflight = 0, cpos = 0, ipos = 0;
    // every pass uses a block; a range holds at most kIds blocks
    int passes_left = L::kIds + 16;
    while (compute_live && --passes_left > 0) {
      while (inflight < kDepth && issue_live) {  // refill the ring
        issue(ipos);
        ++inflight;
        ipos = ipos + 1 == kDepth ? 0 : ipos + 1;
      }
      if (inflight == 0) break;  // nothing left to load or use (not reached)
      // stage cpos holds the oldest block: wait until at most the later
      // stages' loads are outstanding (after stores: until none are)
      const int later = drain ? 0 : inflight - 1;
      if (kDepth > 3 && later >= 3) wait_vm<(3 * kLoadsPerBlock < 64 ? 3 * kLoadsPerBlock : 63)>();
      else if (kDepth > 2 && later >= 2) wait_vm<(2 * kLoadsPerBlock < 64 ? 2 * kLoadsPerBlock : 63)>();
      else if (later >= 1) wait_vm<kLoadsPerBlock>();
      else wait_vm<0>();
      drain = false;
      const char* src = my + L::kRing + cpos * L::kBlk;
      const char* qs = my + L::kQ + (cu_ord % L::kQSlots) * L::kQBytes;
      const uint32_t qrow = (NH < 16 && qn_lane >= NH) ? lds_addr(my + L::kZero)
                                                       : lds_addr(qs + qn_lane * D * 2);
      BlockRegs<D> r;
      uint4 qf[kSteps];
      read_stage<D>(lds_addr(src) + lane * 16,
                    lds_addr(src + D * kBlock * 2) + (qn_lane * kBlock + qkg * 4) * 2,
                    qrow + qkg * 16, r, qf);
      // the stage is read: load the next block into it before computing
      --inflight;
      const int freed = cpos;
      cpos = cpos + 1 == kDepth ? 0 : cpos + 1;
      if (ipos == freed && issue_live) {
        issue(freed);
        ++inflight;
        ipos = ipos + 1 == kDepth ? 0 : ipos + 1;
      }
      attend_block<Tag, D>(a, r, cb, cu.len, [&](int t) { return qf[t]; }, st);
      if (++cb == cu.end_real()) {
        finish();
        compute_live = compute_enter();
      }
    }
    flush();
    if (has_first_part) store_partial<D, NH>(first_unit, k, 0, first_part, part_ml, part_acc);
    wait_vm<0>();  // the next range reuses the LDS
  }
}

// Ranges the balanced split may use for these sizes: one per resident
// work-group or wave (at most kMaxBalancedGroups), or more when a range of the
// streamed kernel would exceed kStreamRangeCap cost.
constexpr int kStreamRangeCap = 512;  // = the streamed kernel's block-id room per range
int64_t balanced_ranges(int num_seqs, int hq, int max_len) {
  const int64_t blocks = std::max(1, (max_len + kBlock - 1) / kBlock);
  const int64_t cost = static_cast<int64_t>(num_seqs) * hq * (kUnitCost + blocks);
  return std::max<int64_t>(kMaxBalancedGroups, (cost + kStreamRangeCap - 1) / kStreamRangeCap);
}

// Workspace of the balanced path: meta (256 B), range starts (one more than
// the ranges), and two partial slots per range of min(16, hq) rows (rounded up
// to a power of two) each.
Layout balanced_layout(int hq, int head_dim, int64_t ranges) {
  Layout l;
  const size_t rows = static_cast<size_t>(ranges) * 2 * pow2_at_least(std::min(16, hq));
  l.meta = 0;
  l.items = kAlign;  // range starts
  l.split = l.items;
  l.ml = l.items + align_up(static_cast<size_t>(ranges + 1) * sizeof(int4));
  l.acc = l.ml + align_up(rows * 2 * sizeof(float));
  l.total = l.acc + align_up(rows * head_dim * sizeof(float));
  l.arrivals = l.total;  // unused by the balanced split
  return l;
}

int resident_groups(const void* kernel, int threads, size_t lds);

// Cap on the balanced grid set by pa_decode_set_max_groups (0: none).
int g_max_groups = 0;

// Work-groups of the balanced grid: the resident count of `kernel` on the
// current device (CUs x occupancy, cached per device and kernel), at most
// kMaxBalancedGroups and the cap.
int balanced_groups(const void* kernel, size_t lds, int threads = kItemThreads) {
  const int n = resident_groups(kernel, threads, lds);
  return n > 0 && g_max_groups > 0 ? std::min(n, g_max_groups) : n;
}

int resident_groups(const void* kernel, int threads, size_t lds) {
  struct Entry {
    int dev;
    const void* fn;
    size_t lds;
    int n;
  };
  static std::mutex mu;  // host threads may launch concurrently
  static Entry cache[32];
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (cache[i].dev == dev && cache[i].fn == kernel && cache[i].lds == lds) return cache[i].n;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) !=
          hipSuccess)
    return -1;
  const int n = std::max(1, std::min(kMaxBalancedGroups, cus * std::max(per_cu, 1)));
  if (used < 32) cache[used++] = Entry{dev, kernel, lds, n};
  return n;
}

// The streamed decode kernel for a head size and head-group rows (1 .. 16).
template <typename Tag>
const void* stream_kernel_for(int head_dim, int nh) {
#define PA_STREAM_CASE(DIM, NH)                                                    \
  if (head_dim == DIM && nh == NH)                                                 \
    return reinterpret_cast<const void*>(&decode_stream_kernel<Tag, DIM, NH>);
  PA_STREAM_CASE(128, 1) PA_STREAM_CASE(128, 2) PA_STREAM_CASE(128, 4)
  PA_STREAM_CASE(128, 8) PA_STREAM_CASE(128, 16)
  PA_STREAM_CASE(64, 1) PA_STREAM_CASE(64, 2) PA_STREAM_CASE(64, 4)
  PA_STREAM_CASE(64, 8) PA_STREAM_CASE(64, 16)
#undef PA_STREAM_CASE
  return nullptr;
}

size_t stream_lds_for(int head_dim, int nh) {
#define PA_STREAM_LDS(DIM, NH) \
  if (head_dim == DIM && nh == NH)  \
    return stream_waves_lds<DIM, NH, stream_depth<DIM, NH>()>();
  PA_STREAM_LDS(128, 1) PA_STREAM_LDS(128, 2) PA_STREAM_LDS(128, 4) PA_STREAM_LDS(128, 8)
  PA_STREAM_LDS(128, 16) PA_STREAM_LDS(64, 1) PA_STREAM_LDS(64, 2) PA_STREAM_LDS(64, 4)
  PA_STREAM_LDS(64, 8) PA_STREAM_LDS(64, 16)
#undef PA_STREAM_LDS
  return 0;
}

// Streamed balanced path: balance plan over one range per wave (ranges of at
// most kStreamRangeCap cost), the streamed kernel, merge of the cut units.
template <typename Tag>
pa_status launch_stream(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* tables, const int32_t* lens, float scale_log2, void* out,
                        int num_seqs, int hq, int hkv, int head_dim, int max_blocks,
                        int64_t ranges, char* ws, hipStream_t st) {
  const Layout lay = balanced_layout(hq, head_dim, ranges);
  int* meta = reinterpret_cast<int*>(ws + lay.meta);
  int4* start = reinterpret_cast<int4*>(ws + lay.items);
  float* part_ml = reinterpret_cast<float*>(ws + lay.ml);
  float* part_acc = reinterpret_cast<float*>(ws + lay.acc);
  DecodeArgs a = mfma_args<Tag>(q, k_cache, v_cache, tables, lens, scale_log2, out, num_seqs, hq,
                                hkv, max_blocks, Split{kBlock, 1}, nullptr, nullptr);
  a.nh_max = pow2_at_least(a.nh_max);
  const void* kernel = stream_kernel_for<Tag>(head_dim, a.nh_max);
  if (!kernel) return PA_ERR_UNSUPPORTED;
  const size_t lds = stream_lds_for(head_dim, a.nh_max);
  static const void* lds_set[32];
  static int lds_set_n = 0;
  bool known = false;
  for (int i = 0; i < lds_set_n; ++i) known = known || lds_set[i] == kernel;
  if (!known) {
    if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds)) != hipSuccess)
      return PA_ERR_DEVICE;
    if (lds_set_n < 32) lds_set[lds_set_n++] = kernel;
  }
  int wgs = balanced_groups(kernel, lds, kStreamThreads);  // resident work-groups
  if (wgs <= 0) return PA_ERR_DEVICE;
  wgs = std::max(1, std::min(wgs * kStreamRangeMult, kMaxBalancedGroups / kStreamWaves));
  const int groups = wgs * kStreamWaves;  // one range per wave

  BalanceArgs ba{lens, start, meta, num_seqs, max_blocks, hkv * a.head_blocks, groups,
                 kStreamRangeCap, static_cast<int>(std::min<int64_t>(ranges, 0x7fffffff))};
  int slot = timing_start(PA_KERNEL_DECODE_PLAN, st);
  decode_balance_kernel<<<dim3(1), dim3(kThreads), 0, st>>>(ba);
  pa_status status = launch_status();
  timing_stop(slot, st);
  if (status != PA_OK) return status;

  slot = timing_start(PA_KERNEL_DECODE, st);
  void* args[] = {&a, &start, &meta, &part_ml, &part_acc};
  status = hipLaunchKernel(kernel, dim3(wgs), dim3(kStreamThreads), args, lds, st) == hipSuccess
               ? PA_OK
               : PA_ERR_DEVICE;
  timing_stop(slot, st);
  if (status != PA_OK) return status;

  slot = timing_start(PA_KERNEL_DECODE_REDUCE, st);
  decode_balanced_merge_kernel<Tag><<<dim3(groups), dim3(kThreads), 0, st>>>(
      start, meta, part_ml, part_acc, static_cast<typename Tag::Bits*>(out), hq, a.group,
      a.head_blocks, head_dim, a.nh_max);
  status = launch_status();
  timing_stop(slot, st);
  return status;
}

}  // namespace

int64_t balanced_split_ranges(int num_seqs, int hq, int max_len) {
  return balanced_ranges(num_seqs, hq, max_len);
}

size_t balanced_split_workspace_bytes(int hq, int head_dim, int64_t ranges) {
  return balanced_layout(hq, head_dim, ranges).total;
}

pa_status launch_balanced_split(pa_dtype dtype, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* tables, const int32_t* lens,
                                float scale_log2, void* out, int num_seqs, int hq, int hkv,
                                int head_dim, int max_blocks, int64_t ranges, char* ws,
                                hipStream_t st) {
  switch (dtype) {
    case PA_BF16:
      return launch_stream<BF16T>(q, k_cache, v_cache, tables, lens, scale_log2, out, num_seqs,
                                  hq, hkv, head_dim, max_blocks, ranges, ws, st);
    case PA_F16:
      return launch_stream<F16T>(q, k_cache, v_cache, tables, lens, scale_log2, out, num_seqs, hq,
                                 hkv, head_dim, max_blocks, ranges, ws, st);
    default:
      return PA_ERR_UNSUPPORTED;
  }
}

}  // namespace pa

extern "C" pa_status pa_decode_set_max_groups(int32_t max_groups) {
  if (max_groups < 0) return PA_ERR_INVALID_ARG;
  pa::g_max_groups = max_groups;
  return PA_OK;
}
