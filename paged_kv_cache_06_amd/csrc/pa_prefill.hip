// Chunked-prefill paged attention: a chunk of new tokens per sequence, each
// attending causally to every cached position up to its own (every token
// needs the K and V of all tokens before it: "KV Cache and PagedAttention:
// why your LLM server slows down", second article, section "What is the KV
// cache?").  The chunk's K/V are in the cache before the call, as for decode,
// so one token per sequence is exactly decode.
//
// One wave per unit of work = (sequence, KV head, group of up to 16 query
// heads, a run of consecutive chunk queries); the 16 columns of its matrix-
// core products are (query, head) pairs, query-major: with G query heads per
// KV head (G <= 16) a wave serves 16 / G queries of that KV head at once, so
// every K/V block it loads is multiplied against 16 query rows.  Per 16-token
// block, as in decode:
//   scores[16 tok x 16 cols] = K . Q^T          (MFMA 16x16x32, K as A)
//   online softmax per column, masked causally: token t counts for the column
//   of the query at position p iff t <= p
//   acc^T[D x 16 cols] += V^T . P^T             (MFMA 16x16x16, P as hi + lo)
// Units are ordered so that the queries with the most positions start first.
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
};

template <typename Tag, int D>
__global__ __launch_bounds__(kWave, 4) void prefill_kernel(PrefillArgs a) {
  const int lane = threadIdx.x;
  const int n = lane & 15, kg = lane >> 4;
  // unit = (run, sequence, KV head, head block), run-major from the last run
  const int per_run = a.num_seqs * a.hkv * a.head_blocks;
  const int u = blockIdx.x;
  const int run = a.groups_max - 1 - u / per_run;
  const int r = u % per_run;
  const int s = r / (a.hkv * a.head_blocks);
  const int g = (r / a.head_blocks) % a.hkv;
  const int hb = r % a.head_blocks;
  const int q0 = uniform_load(a.qstart, s), q1 = uniform_load(a.qstart, s + 1);
  // a length below the chunk reads as the chunk; both stop at the table's width
  const int len = min(max(uniform_load(a.lens, s), q1 - q0), a.max_blocks * kBlock);
  const int nchunk = min(q1 - q0, len);
  const int i0 = run * a.qpw;
  if (i0 >= nchunk) return;
  const int nq = min(a.qpw, nchunk - i0);
  const int h_base = hb * 16;
  const int nh = min(a.cols_heads, a.group - h_base);
  // this lane's column: query i, head h
  const int ci = n / a.cols_heads, ch = n % a.cols_heads;
  const bool col_ok = ci < nq && ch < nh;
  const int first_pos = len - nchunk + i0;  // position of the run's first query
  const int col_pos = first_pos + (col_ok ? ci : nq - 1);
  const int last_pos = first_pos + nq - 1;
  const int nblk = last_pos / kBlock + 1;

  // query operand: column n's row, dims (j*4 + kg)*8 .. +7 of k-step j; idle
  // columns are 0
  uint4 qf[D / 32];
#pragma unroll
  for (int j = 0; j < D / 32; ++j) qf[j] = make_uint4(0, 0, 0, 0);
  if (col_ok) {
    const size_t row = static_cast<size_t>(q0 + i0 + ci) * a.hq + g * a.group + h_base + ch;
    const uint4* qrow = reinterpret_cast<const uint4*>(a.q + row * D);
#pragma unroll
    for (int j = 0; j < D / 32; ++j) qf[j] = qrow[j * 4 + kg];
  }
  DecodeArgs da;  // the fields the block loads use
  da.k_cache = a.k_cache;
  da.v_cache = a.v_cache;
  da.hkv = a.hkv;

  WaveState<D> st;
  st.reset();
  const int32_t* trow = a.tables + static_cast<size_t>(s) * a.max_blocks;
  for (int c0 = 0; c0 < nblk; c0 += 64) {
    const int ids = load_ids<1>(trow, c0, nblk - c0);
    const int cn = min(64, nblk - c0);
    for (int j = 0; j < cn; ++j) {
      const int blk = c0 + j;
      BlockRegs<D> rb;
      load_block<D>(da, g, __builtin_amdgcn_readlane(ids, j), rb);
      f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < D / 32; ++t) sc = Mfma<Tag>::qk(rb.kf[t], qf[t], sc);
      // causal limit of this lane's column: positions after the query's own
      // are masked; V rows past the sequence's end are zeroed on its last block
      block_update_lim<Tag, D>(rb.vf, sc, a.scale_log2, blk, len, col_pos + 1, st);
    }
  }
  float l_tot = st.l + __shfl_xor(st.l, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (!col_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  uint16_t* orow = a.out + (static_cast<size_t>(q0 + i0 + ci) * a.hq + g * a.group + h_base + ch) * D;
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) {
    const f32x4_t v = st.acc[sl];
    const uint2 packed = Mfma<Tag>::pack(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    *reinterpret_cast<uint2*>(orow + sl * 16 + kg * 4) = packed;
  }
}

template <typename Tag>
pa_status launch_prefill(const PrefillArgs& a, int head_dim, int64_t units, hipStream_t st) {
  const dim3 g3(static_cast<uint32_t>(units)), b3(kWave);
  if (head_dim == 128)
    prefill_kernel<Tag, 128><<<g3, b3, 0, st>>>(a);
  else
    prefill_kernel<Tag, 64><<<g3, b3, 0, st>>>(a);
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
  a.head_blocks = (a.group + 15) / 16;
  a.max_blocks = max_blocks_per_seq;
  a.cols_heads = std::min(a.group, 16);
  a.qpw = 16 / a.cols_heads;
  a.groups_max = (max_chunk_len + a.qpw - 1) / a.qpw;
  const int64_t units =
      static_cast<int64_t>(a.groups_max) * num_seqs * num_kv_heads * a.head_blocks;
  if (units > 0x7fffffff) return PA_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int slot = timing_start(PA_KERNEL_PREFILL, st);
  const pa_status s = dtype == PA_BF16 ? launch_prefill<BF16T>(a, head_dim, units, st)
                                       : launch_prefill<F16T>(a, head_dim, units, st);
  timing_stop(slot, st);
  return s;
}

}  // extern "C"
