// Chunked-prefill paged attention: a chunk of new tokens per sequence, each
// attending causally to every cached position up to its own (every token
// needs the K and V of all tokens before it: "KV Cache and PagedAttention:
// why your LLM server slows down", second article, section "What is the KV
// cache?").  The chunk's K/V are in the cache before the call, as for decode,
// so one token per sequence is exactly decode.
//
// A tile is 32 matrix-core columns: (query, head) pairs of consecutive chunk
// queries of one sequence and KV head, query-major, so with G query heads per
// KV head (G <= 32) a tile holds 32 / G queries and every K/V position is
// multiplied against 32 query rows at once.  Per 32-position round (two
// 16-token blocks) and tile:
//   scores[32 pos x 32 cols] = K . Q^T          (MFMA 32x32x16, K as A)
//   online softmax per column, masked causally: position t counts for the
//   column of the query at position p iff t <= p
//   acc^T[D x 32 cols] += V^T . P^T             (MFMA 32x32x16, per block)
// A work-group (4 waves, one tile each) walks the rounds its tiles need
// through an LDS ring that each round enters once, software-pipelined so
// that one round's QK products run beside the previous round's softmax.  The
// longest sequences are handed out first, the work-groups of one sequence
// together, so that those sharing its K/V share one XCD's L2.
#include "pa_decode_common.h"

namespace pa {
namespace {

struct PrefillArgs {
  const uint16_t* q;        // [T][Hq][D]
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* tables;    // [S][max_blocks]
  const int32_t* qstart;    // [S + 1]
  const int32_t* lens;      // [S]
  uint16_t* out;            // [T][Hq][D]
  float scale_log2;
  int num_seqs, hq, hkv, group, head_blocks, max_blocks;
  int cols_heads;           // query heads per tile: min(G, 32)
  int qpw;                  // queries per wave: 32 / cols_heads
  int groups_max;           // query runs of the longest chunk: ceil(max_chunk / qpw)
  int longest_first;        // longest sequence first (num_seqs <= kOrderMaxSeqs)
};

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

constexpr int kPrefillWaves = 4;  // one 32-column tile each

// ---- operand layout ----
//
// With a 32-column tile and 32-position rounds each lane holds 16 scores of
// one column, so the per-score vector work (scale, mask, running maximum,
// exponential, sum, packing) is amortised over 32x32x16 products.
//   QK: rows = the round's 32 tokens, columns = the tile (A = K, B = Q^T).
//       Row r carries token pi(r), r with bits 2 and 3 swapped, so that lane
//       l (column l%32, rows 8j + 4(l/32) + i) ends up holding, for block b,
//       the scores of tokens 8(l/32) + e, e < 8, as elements 8b + e;
//   PV: per block b and 32-dimension slice dt, A = V^T (lane l: dimension
//       dt*32 + l%32, tokens 8(l/32)..+7: one 16-byte piece of a transposed V
//       row) and B = P^T (lane l: column l%32, elements 8b..8b+7).
// The V copy into LDS places the piece lane l reads at 16*l within the slice
// (the DMA lanes gather rows' halves), so the wave's V reads are one
// contiguous KiB per slice, as its K reads are 256 contiguous bytes per
// 16 lanes: no bank conflicts.
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <typename Tag>
struct Mfma32;

template <>
struct Mfma32<BF16T> {
  __device__ static f32x16_t mma(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};

template <>
struct Mfma32<F16T> {
  __device__ static f32x16_t mma(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
};

// K operands of one round (D / 16 k-steps, 512 bytes apart) from LDS, one
// block of reads ending with its wait.
template <int D>
__device__ __forceinline__ void read_k32(uint32_t ka, uint4* kf);

template <>
__device__ __forceinline__ void read_k32<128>(uint32_t ka, uint4* kf) {
  asm volatile(
      "ds_read_b128 %0, %8\n"
      "ds_read_b128 %1, %8 offset:512\n"
      "ds_read_b128 %2, %8 offset:1024\n"
      "ds_read_b128 %3, %8 offset:1536\n"
      "ds_read_b128 %4, %8 offset:2048\n"
      "ds_read_b128 %5, %8 offset:2560\n"
      "ds_read_b128 %6, %8 offset:3072\n"
      "ds_read_b128 %7, %8 offset:3584\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kf[0]), "=&v"(kf[1]), "=&v"(kf[2]), "=&v"(kf[3]), "=&v"(kf[4]), "=&v"(kf[5]),
        "=&v"(kf[6]), "=&v"(kf[7])
      : "v"(ka)
      : "memory");
}

template <>
__device__ __forceinline__ void read_k32<64>(uint32_t ka, uint4* kf) {
  asm volatile(
      "ds_read_b128 %0, %4\n"
      "ds_read_b128 %1, %4 offset:512\n"
      "ds_read_b128 %2, %4 offset:1024\n"
      "ds_read_b128 %3, %4 offset:1536\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kf[0]), "=&v"(kf[1]), "=&v"(kf[2]), "=&v"(kf[3])
      : "v"(ka)
      : "memory");
}

// K operands of the next round and V operands of the current one (two blocks,
// D / 32 slices each: vf[b * D / 32 + dt]), one block of reads ending with
// its wait.
template <int D>
__device__ __forceinline__ void read_kv32(uint32_t ka, uint32_t va, uint4* kf, uint4* vf);

template <>
__device__ __forceinline__ void read_kv32<128>(uint32_t ka, uint32_t va, uint4* kf, uint4* vf) {
  asm volatile(
      "ds_read_b128 %0, %16\n"
      "ds_read_b128 %1, %16 offset:512\n"
      "ds_read_b128 %2, %16 offset:1024\n"
      "ds_read_b128 %3, %16 offset:1536\n"
      "ds_read_b128 %4, %16 offset:2048\n"
      "ds_read_b128 %5, %16 offset:2560\n"
      "ds_read_b128 %6, %16 offset:3072\n"
      "ds_read_b128 %7, %16 offset:3584\n"
      "ds_read_b128 %8, %17\n"
      "ds_read_b128 %9, %17 offset:1024\n"
      "ds_read_b128 %10, %17 offset:2048\n"
      "ds_read_b128 %11, %17 offset:3072\n"
      "ds_read_b128 %12, %17 offset:4096\n"
      "ds_read_b128 %13, %17 offset:5120\n"
      "ds_read_b128 %14, %17 offset:6144\n"
      "ds_read_b128 %15, %17 offset:7168\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kf[0]), "=&v"(kf[1]), "=&v"(kf[2]), "=&v"(kf[3]), "=&v"(kf[4]), "=&v"(kf[5]),
        "=&v"(kf[6]), "=&v"(kf[7]), "=&v"(vf[0]), "=&v"(vf[1]), "=&v"(vf[2]), "=&v"(vf[3]),
        "=&v"(vf[4]), "=&v"(vf[5]), "=&v"(vf[6]), "=&v"(vf[7])
      : "v"(ka), "v"(va)
      : "memory");
}

template <>
__device__ __forceinline__ void read_kv32<64>(uint32_t ka, uint32_t va, uint4* kf, uint4* vf) {
  asm volatile(
      "ds_read_b128 %0, %8\n"
      "ds_read_b128 %1, %8 offset:512\n"
      "ds_read_b128 %2, %8 offset:1024\n"
      "ds_read_b128 %3, %8 offset:1536\n"
      "ds_read_b128 %4, %9\n"
      "ds_read_b128 %5, %9 offset:1024\n"
      "ds_read_b128 %6, %9 offset:2048\n"
      "ds_read_b128 %7, %9 offset:3072\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kf[0]), "=&v"(kf[1]), "=&v"(kf[2]), "=&v"(kf[3]), "=&v"(vf[0]), "=&v"(vf[1]),
        "=&v"(vf[2]), "=&v"(vf[3])
      : "v"(ka), "v"(va)
      : "memory");
}

template <typename Tag>
__device__ __forceinline__ uint4 pack8(const float* p) {
  const uint2 lo = Mfma<Tag>::pack(p[0], p[1], p[2], p[3]);
  const uint2 hi = Mfma<Tag>::pack(p[4], p[5], p[6], p[7]);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// ---- work-group order: longest sequence first, its groups together ----
//
// A work-group covers query group rg (queries rg*pw .. rg*pw + pw - 1 of its
// chunk, pw = 4 * qpw) of sequence s for one KV head, and walks 32-position
// rounds up to its last query's position.  Its K/V are a prefix of the
// sequence's, shared by every group of (s, head).  Work-groups are dispatched
// in index order, round-robin over the XCDs, and consecutive indices differ in
// the KV head first; so an order that keeps the groups of one sequence
// together keeps the work-groups of one (sequence, head) on one XCD at the
// same time, where they walk the same blocks and all but the first read hit
// that XCD's L2 (measured: HBM reads 1.55x -> 1.0x the bytes read once).
// Sequences go by the rounds of their last group, W(s) = (c_s + n_s - 1)/32 + 1
// (c_s = tokens before the chunk, n_s = its length), longest first, ties by
// index; within a sequence the top (longest) group first.  The number of
// groups in sequences with W >= V has a closed form per sequence; searched
// over V it gives the pair of any rank.  Longest first keeps the long
// work-groups from starting last.
constexpr int kOrderMaxSeqs = 256;   // sequences one wave ranks (4 per lane)

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = max(x, __shfl_xor(x, off));
  return x;
}

// Pair (s, rg) of rank q, or false if q is past the last non-empty group.
// Wave-uniform; every wave of the work-group computes the same answer.
__device__ bool longest_first(const PrefillArgs& a, int q, int R, int pw, int& s_out,
                              int& rg_out) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int kPer = kOrderMaxSeqs / kWave;
  int G[kPer], W[kPer];
  int total = 0, vmax = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int s = lane + k * kWave;
    G[k] = 0, W[k] = 0;
    if (s < a.num_seqs) {
      const int q0 = a.qstart[s], q1 = a.qstart[s + 1];
      const int len = min(max(a.lens[s], q1 - q0), a.max_blocks * kBlock);
      const int n = max(0, min(q1 - q0, len));
      G[k] = min((n + pw - 1) / pw, R);
      if (G[k] > 0) W[k] = (len - 1) / 32 + 1;  // the last query sits at len - 1
      vmax = max(vmax, W[k]);
    }
    total += G[k];
  }
  total = wave_sum(total);
  if (q >= total) return false;
  vmax = wave_max(vmax);
  auto count = [&](int V) {  // groups in sequences with W >= V
    int x = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) x += W[k] >= V ? G[k] : 0;
    return wave_sum(x);
  };
  int lo = 1, hi = vmax + 1;  // count(lo) > q >= count(hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (count(mid) > q)
      lo = mid;
    else
      hi = mid;
  }
  int r = q - count(lo + 1);  // rank among the groups of sequences with W == lo
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int e = W[k] == lo ? G[k] : 0;
    int incl = e;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(incl > r);
    if (hit != 0) {
      const int f = static_cast<int>(__builtin_ctzll(hit));
      s_out = f + k * kWave;
      rg_out = __builtin_amdgcn_readlane(G[k] - 1 - (r - (incl - e)), f);
      return true;
    }
    r -= __builtin_amdgcn_readlane(incl, kWave - 1);
  }
  return false;  // not reached: the ranks below total are all covered
}

// Rounds in the LDS ring: the one being multiplied, the next (its QK
// products run in the same iteration) and three in flight.  80 KiB at D = 128:
// two work-groups (8 waves, 2 per SIMD at up to 256 registers) fill a CU.
constexpr int kRingDepth = 5;

template <typename Tag, int D>
__global__ __launch_bounds__(kPrefillWaves * kWave, 2) void prefill_kernel(PrefillArgs a) {
  constexpr int kBlk = D * kBlock * 2;      // K (or V) of one block-head
  constexpr int kStage = 4 * kBlk;          // [K b0][K b1][V b0][V b1]
  constexpr int kChunks = kBlk / 1024;      // 1 KiB loads per block part = per wave
  constexpr int kSteps = D / 16;            // QK k-steps
  constexpr int kSlices = D / 32;           // PV dimension slices
  constexpr float kSlack = 8.f;             // log2 units
  __shared__ __attribute__((aligned(1024))) char ring[kRingDepth * kStage];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane & 31, h = lane >> 5;
  const int inner = a.hkv * a.head_blocks;  // work-groups of one (sequence, query group)
  const int u = blockIdx.x;
  const int run_groups = (a.groups_max + kPrefillWaves - 1) / kPrefillWaves;
  const int g = (u % inner) / a.head_blocks;
  const int hb = u % a.head_blocks;
  int s, rg;
  if (a.longest_first) {
    if (!longest_first(a, u / inner, run_groups, kPrefillWaves * a.qpw, s, rg)) return;
    s = __builtin_amdgcn_readfirstlane(s);
    rg = __builtin_amdgcn_readfirstlane(rg);
  } else {  // sequences in index order, each one's groups together, top first
    s = (u / inner) / run_groups;
    rg = run_groups - 1 - (u / inner) % run_groups;
  }
  const int q0 = uniform_load(a.qstart, s), q1 = uniform_load(a.qstart, s + 1);
  const int len = min(max(uniform_load(a.lens, s), q1 - q0), a.max_blocks * kBlock);
  const int nchunk = min(q1 - q0, len);
  const int i_wg = rg * kPrefillWaves * a.qpw;
  if (i_wg >= nchunk) return;  // uniform over the work-group
  const int i0 = i_wg + wave * a.qpw;
  const int nq = max(0, min(a.qpw, nchunk - i0));
  const int h_base = hb * 32;
  const int nh = min(a.cols_heads, a.group - h_base);
  const int ci = c / a.cols_heads, ch = c % a.cols_heads;
  const bool col_ok = ci < nq && ch < nh;
  const int first_pos = nq > 0 ? len - nchunk + i0 : 0;
  const int col_pos = nq > 0 ? first_pos + (col_ok ? ci : nq - 1) : 0;
  const int wave_last = nq > 0 ? first_pos + nq - 1 : 0;
  const int wg_last = len - nchunk + min(nchunk, i_wg + kPrefillWaves * a.qpw) - 1;
  const int nblk = wg_last / kBlock + 1;
  const int my_rounds = nq > 0 ? wave_last / (2 * kBlock) + 1 : 0;

  uint4 qf[kSteps];
#pragma unroll
  for (int st = 0; st < kSteps; ++st) qf[st] = make_uint4(0, 0, 0, 0);
  if (col_ok) {
    const size_t row = static_cast<size_t>(q0 + i0 + ci) * a.hq + g * a.group + h_base + ch;
    const uint4* qrow = reinterpret_cast<const uint4*>(a.q + row * D);
#pragma unroll
    for (int st = 0; st < kSteps; ++st) qf[st] = qrow[2 * st + h];
  }
  float m = -INFINITY, l = 0.f;
  f32x16_t acc[kSlices];
#pragma unroll
  for (int dt = 0; dt < kSlices; ++dt) acc[dt] = f32x16_t{};

  const int32_t* trow = a.tables + static_cast<size_t>(s) * a.max_blocks;
  const int tok = (c & 0x13) | ((c & 4) << 1) | ((c & 8) >> 1);  // token of row c
  const uint32_t k_lane = ((tok >> 4) * kBlk) + ((h * 16 + (tok & 15)) * 16);
  const uint32_t v_lane = 2 * kBlk + lane * 16;
  // source offset of this lane's 16 bytes within a KiB: K pieces stay in
  // place, V pieces (dimension lane%32, half lane/32) are gathered
  const uint32_t dma_lane = wave < 2 ? lane * 16 : c * 32 + h * 16;
  const bool pos_scale = a.scale_log2 >= 0.f;
  const int total = wg_last / (2 * kBlock) + 1;  // rounds of the work-group
  // Wave w moves part w of each round (K of its first block, K of its
  // second, V of its first, V of its second) into the ring; blocks past the
  // work-group's last are issued with an empty range (they write zeros), so
  // that every issue counts the same in vmcnt.  The block id of the wave's
  // next issue is loaded one issue ahead.
  int next_id = wave % 2 < nblk ? uniform_load(trow, wave % 2) : 0;
  auto issue = [&](int j) {
    const int b = 2 * j + (wave & 1);
    const size_t off = (static_cast<size_t>(next_id) * a.hkv + g) * (D * kBlock);
    const auto rsrc = buffer_of((wave < 2 ? a.k_cache : a.v_cache) + off, b < nblk ? kBlk : 0u);
    char* dst = ring + (j % kRingDepth) * kStage + wave * kBlk;
#pragma unroll
    for (int q = 0; q < kChunks; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t)(dst + q * 1024), 16,
                                               dma_lane + q * 1024, 0, 0, 0);
    // scalar loads return out of order: issued after this one's use, so that
    // waiting for it never waits for the next
    next_id = b + 2 < nblk ? uniform_load(trow, b + 2) : 0;
  };
  auto qk = [&](const uint4* kf) {
    f32x16_t sc = f32x16_t{};
#pragma unroll
    for (int st = 0; st < kSteps; ++st) sc = Mfma32<Tag>::mma(kf[st], qf[st], sc);
    return sc;
  };
  auto grow = [&](float own) {  // lazy running maximum: rescale only when it moves by > slack
    if (__builtin_amdgcn_ballot_w64(own > m + kSlack) != 0) {
      const float m_new = fmaxf(m, fmaxf(own, __shfl_xor(own, 32)));
      const float alpha = fast_exp2(m - m_new);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < kSlices; ++dt) acc[dt] *= alpha;
      m = m_new;
    }
  };
  auto pv = [&](const uint4* vf, const float* p) {
    const uint4 pb0 = pack8<Tag>(p), pb1 = pack8<Tag>(p + 8);
#pragma unroll
    for (int dt = 0; dt < kSlices; ++dt) acc[dt] = Mfma32<Tag>::mma(vf[dt], pb0, acc[dt]);
#pragma unroll
    for (int dt = 0; dt < kSlices; ++dt)
      acc[dt] = Mfma32<Tag>::mma(vf[kSlices + dt], pb1, acc[dt]);
  };

  // Software pipeline: iteration j reads round j+1's K and round j's V,
  // issues round j+1's QK products and, beside them, round j's softmax, then
  // round j's PV products.  The ring holds rounds j and j+1, rounds j+2 and
  // j+3 in flight, and the stage of round j-1, refilled with round j+4 once
  // every wave is past iteration j-1.
#pragma unroll
  for (int j = 0; j < kRingDepth - 1; ++j) issue(j);
  // Each wave waits for its own copies (vmcnt counts them in issue order) and
  // the barrier for everyone's.  A bare s_barrier: __syncthreads would also
  // wait for every copy still in flight.
  wait_vm<(kRingDepth - 2) * kChunks>();  // round 0 in, for this wave ...
  __builtin_amdgcn_s_barrier();           // ... and for every other
  f32x16_t sc_cur = f32x16_t{};
  if (my_rounds > 0) {
    uint4 kf[kSteps];
    read_k32<D>(lds_addr(ring) + k_lane, kf);
    sc_cur = qk(kf);
  }
  for (int j = 0; j < total; ++j) {
    wait_vm<(kRingDepth - 3) * kChunks>();  // round j+1 in
    __builtin_amdgcn_s_barrier();
    issue(j + kRingDepth - 1);  // into the stage of round j-1
    if (j >= my_rounds) continue;
    const char* cur = ring + (j % kRingDepth) * kStage;
    const char* nxt = ring + ((j + 1) % kRingDepth) * kStage;
    uint4 kf[kSteps], vf[2 * kSlices];
    read_kv32<D>(lds_addr(nxt) + k_lane, lds_addr(cur) + v_lane, kf, vf);
    const int base = j * 2 * kBlock;  // position of the round's first token
    if (base + 2 * kBlock > len) {    // zero V of positions past the end (stale bits)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int rem = len - base - b * kBlock - 8 * h;  // this lane's tokens below the end
        const uint32_t m0 = (0 < rem ? 0x0000FFFFu : 0u) | (1 < rem ? 0xFFFF0000u : 0u);
        const uint32_t m1 = (2 < rem ? 0x0000FFFFu : 0u) | (3 < rem ? 0xFFFF0000u : 0u);
        const uint32_t m2 = (4 < rem ? 0x0000FFFFu : 0u) | (5 < rem ? 0xFFFF0000u : 0u);
        const uint32_t m3 = (6 < rem ? 0x0000FFFFu : 0u) | (7 < rem ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int dt = 0; dt < kSlices; ++dt) {
          uint4& v = vf[b * kSlices + dt];
          v.x &= m0;
          v.y &= m1;
          v.z &= m2;
          v.w &= m3;
        }
      }
    }
    // element e of sc_cur is the score of position base + 16(e/8) + 8h + e%8;
    // its exponent is sc_cur[e] * mul - m
    float mul, own;
    if (base + 2 * kBlock - 1 <= first_pos) {
      // every position is real and in range: no masks, scale inside the exponent
      float hi = sc_cur[0];
      if (pos_scale) {
#pragma unroll
        for (int e = 1; e < 16; ++e) hi = fmaxf(hi, sc_cur[e]);
      } else {
#pragma unroll
        for (int e = 1; e < 16; ++e) hi = fminf(hi, sc_cur[e]);
      }
      own = hi * a.scale_log2;
      mul = a.scale_log2;
    } else {
      const int lim = col_pos - base - 8 * h;  // element e is in range if its offset <= lim
#pragma unroll
      for (int e = 0; e < 16; ++e)
        sc_cur[e] = 16 * (e >> 3) + (e & 7) <= lim ? sc_cur[e] * a.scale_log2 : -INFINITY;
      own = sc_cur[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) own = fmaxf(own, sc_cur[e]);
      mul = 1.f;
    }
    grow(own);
    // round j+1's QK products with round j's exponentials beside them, then
    // round j's PV products
    float p[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) p[e] = fast_exp2(fmaf(sc_cur[e], mul, -m));
    sc_cur = qk(kf);
#pragma unroll
    for (int e = 0; e < 16; ++e) l += p[e];
    pv(vf, p);
  }
  wait_vm<0>();
  const float l_tot = l + __shfl_xor(l, 32);
  if (!col_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  uint16_t* orow = a.out + (static_cast<size_t>(q0 + i0 + ci) * a.hq + g * a.group + h_base + ch) * D;
#pragma unroll
  for (int dt = 0; dt < kSlices; ++dt)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const f32x16_t& v = acc[dt];
      const uint2 packed = Mfma<Tag>::pack(v[4 * j4] * inv, v[4 * j4 + 1] * inv,
                                           v[4 * j4 + 2] * inv, v[4 * j4 + 3] * inv);
      *reinterpret_cast<uint2*>(orow + dt * 32 + 8 * j4 + 4 * h) = packed;
    }
}

template <typename Tag>
pa_status launch_prefill(const PrefillArgs& a, int head_dim, int64_t units, hipStream_t st) {
  const dim3 g3(static_cast<uint32_t>(units)), b3(kPrefillWaves * kWave);
  if (head_dim == 128)  // the ring is static LDS
    return launch_kernel(PA_KERNEL_PREFILL, prefill_kernel<Tag, 128>, g3, b3, 0, st, a);
  return launch_kernel(PA_KERNEL_PREFILL, prefill_kernel<Tag, 64>, g3, b3, 0, st, a);
}

}  // namespace
}  // namespace pa

extern "C" {

pa_status pa_paged_attention_prefill(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, const int32_t* query_start,
                                     const int32_t* context_lens, float scale, void* out,
                                     int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t max_blocks_per_seq,
                                     int32_t max_chunk_len, pa_dtype dtype, void* stream) {
  using namespace pa;
  if (dtype != PA_BF16 && dtype != PA_F16) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
      max_chunk_len < 0)
    return PA_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0 || max_chunk_len == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !query_start || !context_lens || !out)
    return PA_ERR_INVALID_ARG;
  PrefillArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.tables = block_tables;
  a.qstart = query_start;
  a.lens = context_lens;
  a.out = static_cast<uint16_t*>(out);
  a.scale_log2 = scale * kLog2e;
  a.num_seqs = num_seqs;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.head_blocks = (a.group + 31) / 32;
  a.max_blocks = max_blocks_per_seq;
  a.cols_heads = std::min(a.group, 32);
  a.qpw = 32 / a.cols_heads;
  a.groups_max = (max_chunk_len + a.qpw - 1) / a.qpw;
  a.longest_first = num_seqs <= kOrderMaxSeqs;
  const int64_t units = static_cast<int64_t>((a.groups_max + kPrefillWaves - 1) / kPrefillWaves) *
                        num_seqs * num_kv_heads * a.head_blocks;
  if (units > 0x7fffffff) return PA_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return dtype == PA_BF16 ? launch_prefill<BF16T>(a, head_dim, units, st)
                          : launch_prefill<F16T>(a, head_dim, units, st);
}

}  // extern "C"
