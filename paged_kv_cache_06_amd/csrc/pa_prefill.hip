// Chunked-prefill paged attention: a chunk of new tokens per sequence, each
// attending causally to every cached position up to its own (every token
// needs the K and V of all tokens before it: "KV Cache and PagedAttention:
// why your LLM server slows down", second article, section "What is the KV
// cache?").  The chunk's K/V are in the cache before the call, as for decode,
// so one token per sequence is exactly decode.
//
// A tile is a run of consecutive chunk queries of one (sequence, KV head,
// group of up to 16 query heads); the 16 columns of its matrix-core products
// are (query, head) pairs, query-major: with G query heads per KV head
// (G <= 16) a tile holds 16 / G queries of that KV head, so every K/V block
// is multiplied against 16 query rows at once.  Per 16-token block and tile:
//   scores[16 tok x 16 cols] = K . Q^T          (MFMA 16x16x32, K as A)
//   online softmax per column, masked causally: token t counts for the column
//   of the query at position p iff t <= p
//   acc^T[D x 16 cols] += V^T . P^T             (MFMA 16x16x16)
// A work-group (4 waves x 2 tiles each) walks the K/V blocks its 8 tiles
// need through an LDS ring that every block enters once (prefill_kernel);
// work-groups with the latest queries (the most positions) start first.
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
  int cols_heads;           // query heads per column group: min(G, 16)
  int qpw;                  // queries per wave: 16 / cols_heads
  int groups_max;           // query runs of the longest chunk: ceil(max_chunk / qpw)
  int largest_first;        // order work-groups by their work (num_seqs <= kOrderMaxSeqs)
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

constexpr int kPrefillWaves = 4;
#ifndef PA_PREFILL_ROUND
#define PA_PREFILL_ROUND 1
#endif
// blocks per barrier (2 measured 4 % slower on MI355X: fewer barriers, but
// the waves then wait on longer rounds) and LDS stages: a round in use and
// at least two blocks loading
constexpr int kPrefillRound = PA_PREFILL_ROUND;
constexpr int kPrefillDepth = kPrefillRound == 1 ? 4 : 3 * kPrefillRound;
#ifndef PA_PREFILL_TILES
#define PA_PREFILL_TILES 2
#endif
constexpr int kPrefillTiles = PA_PREFILL_TILES;  // 16-column tiles per wave
#ifndef PA_PREFILL_32
#define PA_PREFILL_32 1
#endif
constexpr bool kPrefill32 = PA_PREFILL_32 != 0;  // 32-column tiles (prefill32_kernel)

// One block's MFMA operands from an LDS stage (K: 16 bytes per lane per
// k-step, 1 KiB apart; V: 8 bytes per lane per slice, 512 bytes apart), in one
// block of LDS reads that ends with their wait.
template <int D>
__device__ __forceinline__ void read_block(uint32_t ka, uint32_t va, BlockRegs<D>& r);

template <>
__device__ __forceinline__ void read_block<128>(uint32_t ka, uint32_t va, BlockRegs<128>& r) {
  asm volatile(
      "ds_read_b128 %0, %12\n"
      "ds_read_b128 %1, %12 offset:1024\n"
      "ds_read_b128 %2, %12 offset:2048\n"
      "ds_read_b128 %3, %12 offset:3072\n"
      "ds_read_b64 %4, %13\n"
      "ds_read_b64 %5, %13 offset:512\n"
      "ds_read_b64 %6, %13 offset:1024\n"
      "ds_read_b64 %7, %13 offset:1536\n"
      "ds_read_b64 %8, %13 offset:2048\n"
      "ds_read_b64 %9, %13 offset:2560\n"
      "ds_read_b64 %10, %13 offset:3072\n"
      "ds_read_b64 %11, %13 offset:3584\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.kf[0]), "=&v"(r.kf[1]), "=&v"(r.kf[2]), "=&v"(r.kf[3]), "=&v"(r.vf[0]),
        "=&v"(r.vf[1]), "=&v"(r.vf[2]), "=&v"(r.vf[3]), "=&v"(r.vf[4]), "=&v"(r.vf[5]),
        "=&v"(r.vf[6]), "=&v"(r.vf[7])
      : "v"(ka), "v"(va)
      : "memory");
}

template <>
__device__ __forceinline__ void read_block<64>(uint32_t ka, uint32_t va, BlockRegs<64>& r) {
  asm volatile(
      "ds_read_b128 %0, %6\n"
      "ds_read_b128 %1, %6 offset:1024\n"
      "ds_read_b64 %2, %7\n"
      "ds_read_b64 %3, %7 offset:512\n"
      "ds_read_b64 %4, %7 offset:1024\n"
      "ds_read_b64 %5, %7 offset:1536\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.kf[0]), "=&v"(r.kf[1]), "=&v"(r.vf[0]), "=&v"(r.vf[1]), "=&v"(r.vf[2]),
        "=&v"(r.vf[3])
      : "v"(ka), "v"(va)
      : "memory");
}

// Online-softmax step of one block for the prefill kernel.  Two departures
// from decode's block_update, both for the matrix cores' sake (prefill is
// bound by arithmetic, not by HBM): P enters PV as one value in the storage
// dtype (decode's hi + lo pair doubles the PV products), and the running
// maximum is raised only when a score exceeds it by more than 2^8 (the
// weights then stay below 2^8, which fp32 sums and bf16/fp16 weights hold),
// so that the accumulator is rescaled on few blocks instead of on every one.
// `masked`: some position of the block may lie past a column's limit (the
// caller knows when none can, and the comparisons are skipped).  The cross-
// lane maximum is only formed when some lane's own scores outgrow the
// running maximum by the slack; otherwise the block needs no exchange.
template <typename Tag, int D>
__device__ __forceinline__ void prefill_update(uint2* vf, f32x4_t sc, float sl2, int blk, int len,
                                               int lim, bool masked, WaveState<D>& st) {
  constexpr int kSlices = D / 16;
  constexpr float kSlack = 8.f;  // log2 units
  const int lane = threadIdx.x & (kWave - 1);
  const int kg = lane >> 4;
  const int pos0 = blk * kBlock + kg * 4;
  float s4[4];
  if (masked) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s4[i] = (pos0 + i < lim) ? sc[i] * sl2 : -INFINITY;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) s4[i] = sc[i] * sl2;
  }
  const float own = fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3]));
  if (__builtin_amdgcn_ballot_w64(own > st.m + kSlack) != 0) {  // some column outgrew its max
    float mx = fmaxf(own, __shfl_xor(own, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(st.m, mx);
    const float alpha = fast_exp2(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int sl = 0; sl < kSlices; ++sl) st.acc[sl] *= alpha;
    st.m = m_new;
  }
  float p4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p4[i] = fast_exp2(s4[i] - st.m);
  st.l += (p4[0] + p4[1]) + (p4[2] + p4[3]);
  if ((blk + 1) * kBlock > len) {  // last block: zero V of positions past the end
    const uint32_t lo = (pos0 + 0 < len ? 0x0000FFFFu : 0u) | (pos0 + 1 < len ? 0xFFFF0000u : 0u);
    const uint32_t hi = (pos0 + 2 < len ? 0x0000FFFFu : 0u) | (pos0 + 3 < len ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int sl = 0; sl < kSlices; ++sl) {
      vf[sl].x &= lo;
      vf[sl].y &= hi;
    }
  }
  const uint2 ph = Mfma<Tag>::pack(p4[0], p4[1], p4[2], p4[3]);
#pragma unroll
  for (int sl = 0; sl < kSlices; ++sl) st.acc[sl] = Mfma<Tag>::pv(vf[sl], ph, st.acc[sl]);
}

// Work-group = 4 waves x kPrefillTiles consecutive runs of chunk queries of
// one (sequence, KV head, head block).  They walk the same K/V blocks, so
// each block is brought into LDS once for all of them by direct
// buffer-to-LDS loads (each wave moves 1/4 of it) through a ring of
// kPrefillDepth stages; every wave reads the block's operands from there once
// and multiplies them against its kPrefillTiles column tiles.
template <typename Tag, int D>
__global__ __launch_bounds__(kPrefillWaves * kWave, 2) void prefill_kernel(PrefillArgs a) {
  constexpr int kStage = 2 * D * kBlock * 2;         // K then V of one block-head
  constexpr int kChunksPerWave = D / 64;              // 1 KiB loads per wave per stage
  constexpr int T = kPrefillTiles;
  extern __shared__ char ring[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const int n = lane & 15, kg = lane >> 4;
  // unit = (run group, sequence, KV head, head block), from the last runs
  const int per_run = a.num_seqs * a.hkv * a.head_blocks;
  const int u = blockIdx.x;
  const int runs_per_wg = kPrefillWaves * T;
  const int run_groups = (a.groups_max + runs_per_wg - 1) / runs_per_wg;
  const int rg = run_groups - 1 - u / per_run;
  const int r = u % per_run;
  const int s = r / (a.hkv * a.head_blocks);
  const int g = (r / a.head_blocks) % a.hkv;
  const int hb = r % a.head_blocks;
  const int q0 = uniform_load(a.qstart, s), q1 = uniform_load(a.qstart, s + 1);
  const int len = min(max(uniform_load(a.lens, s), q1 - q0), a.max_blocks * kBlock);
  const int nchunk = min(q1 - q0, len);
  const int i_wg = rg * runs_per_wg * a.qpw;  // first query of the work-group
  if (i_wg >= nchunk) return;                  // uniform over the work-group
  const int h_base = hb * 16;
  const int nh = min(a.cols_heads, a.group - h_base);
  const int ci = n / a.cols_heads, ch = n % a.cols_heads;
  // tile t of this wave: queries i0[t] .. i0[t] + nq[t] - 1
  int i0[T], col_pos[T], first_pos[T];
  bool col_ok[T];
  int wave_last = 0;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    i0[t] = i_wg + (wave * T + t) * a.qpw;
    const int nq = max(0, min(a.qpw, nchunk - i0[t]));
    col_ok[t] = ci < nq && ch < nh;
    first_pos[t] = nq > 0 ? len - nchunk + i0[t] : 0;
    col_pos[t] = nq > 0 ? first_pos[t] + (col_ok[t] ? ci : nq - 1) : 0;
    if (nq > 0) wave_last = first_pos[t] + nq - 1;
  }
  const int wg_last = len - nchunk + min(nchunk, i_wg + runs_per_wg * a.qpw) - 1;
  const int nblk = wg_last / kBlock + 1;     // blocks the work-group walks
  const int my_blk = wave_last / kBlock + 1;  // blocks this wave needs

  uint4 qf[T][D / 32];
#pragma unroll
  for (int t = 0; t < T; ++t) {
#pragma unroll
    for (int j = 0; j < D / 32; ++j) qf[t][j] = make_uint4(0, 0, 0, 0);
    if (col_ok[t]) {
      const size_t row = static_cast<size_t>(q0 + i0[t] + ci) * a.hq + g * a.group + h_base + ch;
      const uint4* qrow = reinterpret_cast<const uint4*>(a.q + row * D);
#pragma unroll
      for (int j = 0; j < D / 32; ++j) qf[t][j] = qrow[j * 4 + kg];
    }
  }

  WaveState<D> st[T];
#pragma unroll
  for (int t = 0; t < T; ++t) st[t].reset();
  const int32_t* trow = a.tables + static_cast<size_t>(s) * a.max_blocks;
  const uint32_t va_lane = ((lane & 15) * kBlock + (lane >> 4) * 4) * 2;
  for (int c0 = 0; c0 < nblk; c0 += 64) {
    const int cn = min(64, nblk - c0);
    const int ids = load_ids<1>(trow, c0, cn);
    // this wave's share of block j of the chunk into its stage; blocks past
    // the chunk are issued with an empty range (they write zeros), so that
    // every wave always has the same number of loads in flight
    auto issue = [&](int j) {
      const bool real = j < cn;
      const int phys = __builtin_amdgcn_readlane(ids, real ? j : 0);
      const size_t off = (static_cast<size_t>(phys) * a.hkv + g) * (D * kBlock);
      const uint32_t range = real ? D * kBlock * 2 : 0u;
      const auto rk = buffer_of(a.k_cache + off, range);
      const auto rv = buffer_of(a.v_cache + off, range);
      char* dst = ring + (j % kPrefillDepth) * kStage;
#pragma unroll
      for (int c = 0; c < kChunksPerWave; ++c) {
        const int chunk = wave * kChunksPerWave + c;  // of the stage's 2 * D / 32 KiBs
        const bool is_v = chunk >= D / 32;
        const int byte = (is_v ? chunk - D / 32 : chunk) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(is_v ? rv : rk,
                                                 (lds_void_t)(dst + (is_v ? D * kBlock * 2 : 0) + byte),
                                                 16, lane * 16 + byte, 0, 0, 0);
      }
    };
    // rounds of kPrefillRound blocks: one wait and one barrier per round
    constexpr int R = kPrefillRound;
#pragma unroll
    for (int j = 0; j < kPrefillDepth - R; ++j) issue(j);
    for (int j = 0; j < cn; j += R) {
      wait_vm<(kPrefillDepth - 2 * R) * kChunksPerWave>();  // this wave's part of the round
      // ... and every other wave's: a bare barrier (a fenced one would wait for
      // every load in flight); the loads are counted in by the waits, and LDS
      // reads of earlier rounds end with their own wait
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int i = 0; i < R; ++i) issue(j + kPrefillDepth - R + i);  // stages read last round
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int blk = c0 + j + i;
        if (j + i < cn && blk < my_blk) {
          const char* stg = ring + ((j + i) % kPrefillDepth) * kStage;
          BlockRegs<D> rb;
          read_block<D>(lds_addr(stg) + lane * 16, lds_addr(stg + D * kBlock * 2) + va_lane, rb);
#pragma unroll
          for (int t = 0; t < T; ++t) {
            f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < D / 32; ++k) sc = Mfma<Tag>::qk(rb.kf[k], qf[t][k], sc);
            // every position of the block is at or before the tile's first query
            const bool masked = (blk + 1) * kBlock > first_pos[t] + 1;
            prefill_update<Tag, D>(rb.vf, sc, a.scale_log2, blk, len, col_pos[t] + 1, masked,
                                   st[t]);
          }
        }
      }
    }
    wait_vm<0>();
    __builtin_amdgcn_s_barrier();  // the next chunk's first stages may be overwritten
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    float l_tot = st[t].l + __shfl_xor(st[t].l, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (!col_ok[t]) continue;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow =
        a.out + (static_cast<size_t>(q0 + i0[t] + ci) * a.hq + g * a.group + h_base + ch) * D;
#pragma unroll
    for (int sl = 0; sl < D / 16; ++sl) {
      const f32x4_t v = st[t].acc[sl];
      const uint2 packed = Mfma<Tag>::pack(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
      *reinterpret_cast<uint2*>(orow + sl * 16 + kg * 4) = packed;
    }
  }
}

// ---- 32-column tiles ----
//
// The same computation on v_mfma_f32_32x32x16: a wave's tile is 32 (query,
// head) columns and a round is 32 positions (two blocks), so each lane holds
// 16 scores of one column and the per-score vector work (scale, mask, running
// maximum, exponential, sum, packing) is amortised over twice the products.
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

// ---- largest-first work-group order ----
//
// A work-group of the 32-column kernel covers query group rg (queries
// rg*pw .. rg*pw + pw - 1 of its chunk, pw = 4 * qpw) of sequence s for one
// KV head, and walks 32-position rounds up to its last query's position,
// c_s + min(n_s, (rg + 1) * pw) - 1 (c_s = tokens before the chunk, n_s = its
// length).  That count W(s, rg) grows with rg, so the groups of s with W >= V
// are the top ones and their number has a closed form; summed over the
// sequences and searched over V, it gives the pair of any rank in the order
// of decreasing W (ties by sequence, then group).  Work-groups are
// dispatched in index order, so handing out the longest first keeps the
// long ones from starting last.
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

// groups rg < G of one sequence whose round count is at least V (V >= 1)
__device__ __forceinline__ int groups_at_least(int c, int n, int G, int pw, int V) {
  const int t = 32 * (V - 1) - c + 1;  // the group must reach min(n, (rg+1)pw) >= t
  if (t <= 1) return G;
  if (n < t) return 0;
  return max(0, G - max(0, (t + pw - 1) / pw - 1));
}

// Pair (s, rg) of rank q, or false if q is past the last non-empty group.
// Wave-uniform; every wave of the work-group computes the same answer.
__device__ bool largest_first(const PrefillArgs& a, int q, int R, int pw, int& s_out,
                              int& rg_out) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int kPer = kOrderMaxSeqs / kWave;
  int c[kPer], n[kPer], G[kPer];
  int total = 0, vmax = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int s = lane + k * kWave;
    c[k] = 0, n[k] = 0, G[k] = 0;
    if (s < a.num_seqs) {
      const int q0 = a.qstart[s], q1 = a.qstart[s + 1];
      const int len = min(max(a.lens[s], q1 - q0), a.max_blocks * kBlock);
      n[k] = max(0, min(q1 - q0, len));
      c[k] = len - n[k];
      G[k] = min((n[k] + pw - 1) / pw, R);
      if (G[k] > 0) vmax = max(vmax, (c[k] + n[k] - 1) / 32 + 1);
    }
    total += G[k];
  }
  total = wave_sum(total);
  if (q >= total) return false;
  vmax = wave_max(vmax);
  auto count = [&](int V) {
    int x = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) x += groups_at_least(c[k], n[k], G[k], pw, V);
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
  int r = q - count(lo + 1);  // rank among the pairs of exactly lo rounds
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int at = groups_at_least(c[k], n[k], G[k], pw, lo);
    const int e = at - groups_at_least(c[k], n[k], G[k], pw, lo + 1);
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
      rg_out = __builtin_amdgcn_readlane(G[k] - at + r - (incl - e), f);
      return true;
    }
    r -= __builtin_amdgcn_readlane(incl, kWave - 1);
  }
  return false;  // not reached: the ranks below total are all covered
}

#ifndef PA_PREFILL32_OCC
#define PA_PREFILL32_OCC 2
#endif
constexpr int kPrefill32Depth = 4;  // rounds (pairs of blocks) in the LDS ring

template <typename Tag, int D>
__global__ __launch_bounds__(kPrefillWaves * kWave, PA_PREFILL32_OCC) void prefill32_kernel(PrefillArgs a) {
  constexpr int kBlk = D * kBlock * 2;      // K (or V) of one block-head
  constexpr int kStage = 4 * kBlk;          // [K b0][K b1][V b0][V b1]
  constexpr int kChunks = kBlk / 1024;      // 1 KiB loads per block part = per wave
  constexpr int kSteps = D / 16;            // QK k-steps
  constexpr int kSlices = D / 32;           // PV dimension slices
  constexpr float kSlack = 8.f;             // log2 units
  extern __shared__ char ring[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane & 31, h = lane >> 5;
  const int inner = a.hkv * a.head_blocks;  // work-groups of one (sequence, query group)
  const int u = blockIdx.x;
  const int run_groups = (a.groups_max + kPrefillWaves - 1) / kPrefillWaves;
  const int g = (u % inner) / a.head_blocks;
  const int hb = u % a.head_blocks;
  int s, rg;
  if (a.largest_first) {
    if (!largest_first(a, u / inner, run_groups, kPrefillWaves * a.qpw, s, rg)) return;
    s = __builtin_amdgcn_readfirstlane(s);
    rg = __builtin_amdgcn_readfirstlane(rg);
  } else {  // later query groups (more positions) first
    rg = run_groups - 1 - u / (a.num_seqs * inner);
    s = (u / inner) % a.num_seqs;
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
    char* dst = ring + (j % kPrefill32Depth) * kStage + wave * kBlk;
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
  // round j's PV products.  The ring holds rounds j-1 (free once every wave
  // is past iteration j-1), j, j+1 and j+2 in flight.
#pragma unroll
  for (int j = 0; j < kPrefill32Depth - 1; ++j) issue(j);
  wait_vm<(kPrefill32Depth - 2) * kChunks>();  // round 0 in, for this wave ...
  __builtin_amdgcn_s_barrier();                // ... and every other (bare: see above)
  f32x16_t sc_cur = f32x16_t{};
  if (my_rounds > 0) {
    uint4 kf[kSteps];
    read_k32<D>(lds_addr(ring) + k_lane, kf);
    sc_cur = qk(kf);
  }
  for (int j = 0; j < total; ++j) {
    wait_vm<(kPrefill32Depth - 3) * kChunks>();  // round j+1 in
    __builtin_amdgcn_s_barrier();
    issue(j + kPrefill32Depth - 1);  // into the stage of round j-1
    if (j >= my_rounds) continue;
    const char* cur = ring + (j % kPrefill32Depth) * kStage;
    const char* nxt = ring + ((j + 1) % kPrefill32Depth) * kStage;
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
  if (kPrefill32) {
    const size_t lds = static_cast<size_t>(kPrefill32Depth) * 4 * head_dim * kBlock * 2;
    if (head_dim == 128)
      prefill32_kernel<Tag, 128><<<g3, b3, lds, st>>>(a);
    else
      prefill32_kernel<Tag, 64><<<g3, b3, lds, st>>>(a);
    return launch_status();
  }
  const size_t lds = static_cast<size_t>(kPrefillDepth) * 2 * head_dim * kBlock * 2;
  if (head_dim == 128)
    prefill_kernel<Tag, 128><<<g3, b3, lds, st>>>(a);
  else
    prefill_kernel<Tag, 64><<<g3, b3, lds, st>>>(a);
  return launch_status();
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
  const int cols = kPrefill32 ? 32 : 16;  // columns of a tile
  a.head_blocks = (a.group + cols - 1) / cols;
  a.max_blocks = max_blocks_per_seq;
  a.cols_heads = std::min(a.group, cols);
  a.qpw = cols / a.cols_heads;
  a.groups_max = (max_chunk_len + a.qpw - 1) / a.qpw;
  a.largest_first = kPrefill32 && num_seqs <= kOrderMaxSeqs;
  const int runs_per_wg = kPrefillWaves * (kPrefill32 ? 1 : kPrefillTiles);
  const int64_t units = static_cast<int64_t>((a.groups_max + runs_per_wg - 1) / runs_per_wg) *
                        num_seqs * num_kv_heads * a.head_blocks;
  if (units > 0x7fffffff) return PA_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int slot = timing_start(PA_KERNEL_PREFILL, st);
  const pa_status s = dtype == PA_BF16 ? launch_prefill<BF16T>(a, head_dim, units, st)
                                       : launch_prefill<F16T>(a, head_dim, units, st);
  timing_stop(slot, st);
  return s;
}

}  // extern "C"
