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
#include <mutex>

#include "pa_decode_int8.h"
#include "pa_cache_write.h"
#include "pa_decode_common.h"
namespace pa {
namespace {

// ---- fixed partitions: work items from a plan ----

// Size class of a last partition of `tokens` positions: 0 (the longest) ..
// kClasses - 1 (an empty sequence).  An item's duration is set by its rounds,
// the blocks each wave of its work-group streams (ceil(blocks / waves)), so
// the classes follow rounds: with at most 16 rounds per partition each round
// count has its own class, with more (long partitions on few waves) two or
// more adjacent round counts share one.  Ordering by rounds keeps every item
// that streams more behind none that streams less, which is what keeps the
// end of the list short.
constexpr int kRoundClasses = 16;
constexpr int kClasses = kRoundClasses + 1;
#ifndef PA_FUSED_MERGE
#define PA_FUSED_MERGE 1
#endif
constexpr bool kFusedMerge = PA_FUSED_MERGE != 0;
__device__ __forceinline__ int size_class(int tokens, int part_size, int waves) {
  if (tokens <= 0) return kClasses - 1;
  const int max_rounds = ((part_size + kBlock - 1) / kBlock + waves - 1) / waves;
  const int rounds = ((tokens + kBlock - 1) / kBlock + waves - 1) / waves;
  return (max_rounds - min(rounds, max_rounds)) * kRoundClasses / max_rounds;
}

// Entries of the item list: a private item per (sequence, partition) and a
// prefix item per (group tile, partition of the shared prefix), rounded up to
// a multiple of 32 and padded with end markers.
__host__ __device__ inline int plan_capacity(int num_seqs, int np_max, int num_members = 0) {
  return ((num_seqs + num_members) * np_max + 31) / 32 * 32;
}

// Item records (int4):
//   private item  (s, start, end, slot | nparts << 16): positions [start, end)
//                 of sequence s; its partial goes to slot `slot` of s's rows,
//                 and s has nparts partials in all (nparts <= 1: no merge, the
//                 item writes the output);
//   prefix item   (-2 - j, start, end, p | t << 16): positions [start, end) of
//                 group j's shared prefix, for the members of its tile t (the
//                 listed sequences t * members_per_tile ..), partial slot p
//                 of each;
//   end marker    (-1, 0, 0, 0).
constexpr int kMaxPartitions = 1 << 15;  // slot, nparts and tile fit 15 bits each
constexpr int kMaxMembers = 1 << 24;     // sequences listed in shared-prefix groups

struct PlanArgs {
  const int32_t* lens;
  int4* items;  // [capacity] records above
  int* split;   // [num_seqs] sequences with more than one partition, then -1
  int* meta;    // [0] items, [1] split sequences
  int num_seqs, max_blocks, part_size, np_max;
  int max_len;       // positions a sequence may hold (the call's max_context_len)
  int* arrivals;     // per (sequence, head group): partials stored so far (zeroed here)
  int num_arrivals;
  int max_items;     // items the decode grid serves (see plan_partition)
  int waves;         // waves per decode work-group (size classes count rounds of these)
  // shared prefixes (num_groups == 0: none)
  const int32_t* pfx_seqs;    // [num_members] sequences of every group, group by group
  const int32_t* pfx_start;   // [num_groups + 1]
  const int32_t* pfx_blocks;  // [num_groups] leading table entries the group shares
  int num_groups, num_members;
  int members_per_tile;       // floor(16 / query heads per KV head)
  int* grp_of;                // workspace [num_seqs]: group of each sequence, or -1
  int* nparts_of;             // workspace [num_seqs]: partials of each sequence
  int* grp_tokens;            // workspace [num_groups]: shared positions of each group
  int* grp_leader;            // workspace [num_groups]: a member whose row holds them
  int capacity;               // entries of the item list
  int heads = 0;              // head groups per item (work-groups per list entry)
  int even_doubling = 0;      // the partition is automatic: double it for even batches
};

// A length beyond the call's bound is cut to it, so that no sequence has more
// partitions than its rows of the workspace hold.
__device__ __forceinline__ int plan_len(const PlanArgs& a, int i) {
  return min(max(a.lens[i], 0), a.max_len);
}
__device__ __forceinline__ int ceil_div(int x, int y) { return (x + y - 1) / y; }

// Members of group j, clamped to the member list.
__device__ __forceinline__ void group_range(const PlanArgs& a, int j, int* m0, int* m1) {
  *m0 = min(max(a.pfx_start[j], 0), a.num_members);
  *m1 = min(max(a.pfx_start[j + 1], *m0), a.num_members);
}

// A group of at most kMemberBatch members is taken by one thread, every list
// entry and length loaded before any store (one pair of dependent round trips
// per group); a larger one by the whole work-group, which splits its members
// and reduces the shortest length, the count and the first valid member in
// LDS.  One thread walking a group of 256 members took 74 us of plan (53 us in
// batches of 16): each dependent round trip costs 1-2 us.  Both forms give
// the same results.
constexpr int kMemberBatch = 16;
constexpr int kBigGroups = 64;  // large groups the work-group takes; more: one thread each

__device__ __forceinline__ int wave_reduce(int x, bool take_min) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const int y = __shfl_xor(x, off);
    x = take_min ? min(x, y) : x + y;
  }
  return x;
}

// min (take_min) or sum of x over the work-group; red: kWaves ints of LDS
__device__ __forceinline__ int block_reduce(int x, bool take_min, int* red) {
  x = wave_reduce(x, take_min);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = x;
  __syncthreads();
  int r = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = take_min ? min(r, red[w]) : r + red[w];
  __syncthreads();  // red is written again by the next reduction
  return r;
}

__device__ __forceinline__ void set_group(const PlanArgs& a, int j, int shortest, int valid,
                                          int leader) {
  const int listed = min(max(a.pfx_blocks[j], 0), a.max_len / kBlock);
  a.grp_tokens[j] = valid >= 2 ? min(listed, shortest / kBlock) * kBlock : 0;
  a.grp_leader[j] = leader;
}

// Group membership and each group's shared positions: the listed blocks, cut
// to whole blocks below every member's length, so that every shared position
// is a written slot of every member (no column needs its own mask there).
// Members out of range are ignored; a sequence listed twice keeps one group.
__device__ __forceinline__ void plan_groups(const PlanArgs& a) {
  __shared__ int big[kBigGroups];
  __shared__ int num_big;
  __shared__ int red[kWaves];
  if (threadIdx.x == 0) num_big = 0;
  for (int i = threadIdx.x; i < a.num_seqs; i += kThreads) a.grp_of[i] = -1;
  __syncthreads();
  for (int j = threadIdx.x; j < a.num_groups; j += kThreads) {
    int m0, m1;
    group_range(a, j, &m0, &m1);
    if (m1 - m0 > kMemberBatch) {
      const int k = atomicAdd(&num_big, 1);
      if (k < kBigGroups) {
        big[k] = j;
        continue;
      }
    }
    int shortest = a.max_len, valid = 0, leader = -1;
    for (int mb = m0; mb < m1; mb += kMemberBatch) {
      int seq[kMemberBatch], len[kMemberBatch];
#pragma unroll
      for (int k = 0; k < kMemberBatch; ++k) {
        const int s = mb + k < m1 ? a.pfx_seqs[mb + k] : -1;
        seq[k] = s >= 0 && s < a.num_seqs ? s : -1;
      }
#pragma unroll
      for (int k = 0; k < kMemberBatch; ++k) len[k] = seq[k] >= 0 ? plan_len(a, seq[k]) : 0;
#pragma unroll
      for (int k = 0; k < kMemberBatch; ++k) {
        if (seq[k] < 0) continue;
        a.grp_of[seq[k]] = j;
        shortest = min(shortest, len[k]);
        if (leader < 0) leader = seq[k];
        ++valid;
      }
    }
    set_group(a, j, shortest, valid, leader);
  }
  __syncthreads();
  const int nbig = min(num_big, kBigGroups);
  for (int q = 0; q < nbig; ++q) {  // uniform: every thread takes every large group
    const int j = big[q];
    int m0, m1;
    group_range(a, j, &m0, &m1);
    int shortest = a.max_len, valid = 0, first = a.num_members;
    for (int m = m0 + static_cast<int>(threadIdx.x); m < m1; m += kThreads) {
      const int s = a.pfx_seqs[m];
      if (s < 0 || s >= a.num_seqs) continue;
      a.grp_of[s] = j;
      shortest = min(shortest, plan_len(a, s));
      first = min(first, m);
      ++valid;
    }
    shortest = block_reduce(shortest, true, red);
    valid = block_reduce(valid, false, red);
    first = block_reduce(first, true, red);
    if (threadIdx.x == 0)
      set_group(a, j, shortest, valid, first < a.num_members ? a.pfx_seqs[first] : -1);
  }
  __syncthreads();
}

// Positions of sequence i before its private range (its group's shared ones).
__device__ __forceinline__ int plan_shared(const PlanArgs& a, int i) {
  if (a.num_groups == 0) return 0;
  const int j = a.grp_of[i];
  return j < 0 ? 0 : a.grp_tokens[j];
}

// Counts of one sequence / one group at partition size `part`: cnt[class] for
// the last partition of each range, cnt[kFull] for the full ones, cnt[kSplit]
// for a sequence with more than one partial.
constexpr int kFull = kClasses, kSplit = kClasses + 1;
constexpr int kPlanVals = kClasses + 2;
// two more values in the plan's first scan: items and rounds at twice the
// partition (even_batch)
constexpr int kEvenItems = kPlanVals, kEvenRounds = kPlanVals + 1;
constexpr int kScanVals = kPlanVals + 2;

struct SeqPlan {
  int len, shared, np_pre, np_priv;  // np_priv: private partitions (0: none)
  bool emits;                        // some private item (an empty sequence has one)
};

__device__ __forceinline__ SeqPlan seq_plan(const PlanArgs& a, int i, int part) {
  SeqPlan p;
  p.len = plan_len(a, i);
  p.shared = plan_shared(a, i);
  p.np_pre = ceil_div(p.shared, part);
  p.np_priv = ceil_div(p.len - p.shared, part);
  p.emits = p.np_priv > 0 || p.shared == 0;
  return p;
}

// Tiles of group j: runs of members_per_tile listed members (at most
// kMaxPartitions of them; members past those get no shared pass, so their
// outputs stay unwritten -- the documented limit on a group's size).
__device__ __forceinline__ int group_tiles(const PlanArgs& a, int j) {
  int m0, m1;
  group_range(a, j, &m0, &m1);
  return a.grp_tokens[j] > 0 ? min(ceil_div(m1 - m0, a.members_per_tile), kMaxPartitions - 1)
                             : 0;
}

__device__ __forceinline__ void plan_count(const PlanArgs& a, int part, int i0, int i1, int j0,
                                           int j1, int* cnt) {
#pragma unroll
  for (int c = 0; c < kPlanVals; ++c) cnt[c] = 0;
  for (int i = i0; i < i1; ++i) {
    const SeqPlan p = seq_plan(a, i, part);
    if (!p.emits) continue;
    const int last = p.np_priv > 0 ? p.len - p.shared - (p.np_priv - 1) * part : 0;
    const int cls = size_class(last, part, a.waves);
#pragma unroll
    for (int c = 0; c < kClasses; ++c) cnt[c] += cls == c;
    cnt[kFull] += max(p.np_priv - 1, 0);
    cnt[kSplit] += p.np_pre + p.np_priv > 1;
  }
  for (int j = j0; j < j1; ++j) {
    const int tiles = group_tiles(a, j);
    if (tiles == 0) continue;
    const int tokens = a.grp_tokens[j];
    const int np = ceil_div(tokens, part);
    const int cls = size_class(tokens - (np - 1) * part, part, a.waves);
#pragma unroll
    for (int c = 0; c < kClasses; ++c) cnt[c] += cls == c ? tiles : 0;
    cnt[kFull] += (np - 1) * tiles;
  }
}

// The partition size of a list longer than max_items.  The decode grid is
// sized for max_items items -- the list's full capacity (every sequence at the
// longest length) would dispatch thousands of work-groups that find only an
// end marker -- so such a list takes part_size doubled, up to kDoublings
// times, until it fits, else one partition per sequence.  Larger partitions
// are fewer, longer items over the same blocks.
constexpr int kDoublings = 6;

__device__ __forceinline__ int doubled(const PlanArgs& a, int k) {
  return static_cast<int>(min(static_cast<int64_t>(a.part_size) << k,
                              static_cast<int64_t>(a.max_blocks) * kBlock));
}

__device__ __forceinline__ int plan_partition(const PlanArgs& a, int i0, int i1, int j0, int j1,
                                              int* wave_tot) {
  int cnt[kDoublings + 1];
#pragma unroll
  for (int k = 0; k <= kDoublings; ++k) {
    int c[kPlanVals];
    plan_count(a, doubled(a, k), i0, i1, j0, j1, c);
    int n = c[kFull];
#pragma unroll
    for (int q = 0; q < kClasses; ++q) n += c[q];
    cnt[k] = n;
  }
  int excl[kDoublings + 1], all[kDoublings + 1];
  block_scan<kDoublings + 1>(cnt, excl, all, wave_tot);
  __syncthreads();  // wave_tot is written again by the caller's scan
#pragma unroll
  for (int k = 0; k <= kDoublings; ++k)
    if (all[k] <= a.max_items) return doubled(a, k);
  return a.max_blocks * kBlock;
}

// Items and rounds (blocks per wave, summed over items) of sequences i0..i1
// at partition part2, for the choice below.
__device__ __forceinline__ void even_counts(const PlanArgs& a, int part2, int i0, int i1,
                                            int* items, int* rounds) {
  const int r_full = ceil_div(ceil_div(part2, kBlock), a.waves);
  int n = 0, r = 0;
  for (int i = i0; i < i1; ++i) {
    const int len = plan_len(a, i);
    const int full = len / part2, rest = len - full * part2;
    n += max(1, ceil_div(len, part2));
    r += full * r_full + (rest > 0 ? ceil_div(ceil_div(rest, kBlock), a.waves) : 0);
  }
  *items = n;
  *rounds = r;
}

// An automatic partition is doubled once for a batch of evenly long
// sequences: when at twice the size the list still gives every CU two
// work-groups and its longest item streams at most 1.5x the rounds of the
// mean one.  Fewer, longer items then lose no parallelism and save the
// per-item start-up and merges (Llama-3-8B layer, 64 sequences of
// U{128..4096}: 104.6 -> 98.5 us at 2048; 8 x 32K: 181.6 -> 173.9 us at
// 4096), while a skewed batch, whose longest items would then trail the
// rest, keeps its partition (70B mixed batch: 96.6 us at 1024, 98.1 at 2048).
__device__ __forceinline__ bool even_batch(const PlanArgs& a, int part2, int items2,
                                           int rounds2) {
  const int max_rounds = ceil_div(ceil_div(min(part2, a.max_len), kBlock), a.waves);
  return static_cast<int64_t>(items2) * a.heads >= 512 &&
         2 * static_cast<int64_t>(max_rounds) * items2 <= 3 * static_cast<int64_t>(rounds2);
}

// The item list, largest first (see the file header).  One work-group; each
// thread takes a run of consecutive sequences and a run of consecutive
// groups, so one exclusive scan of its per-class counts places every item
// (sequences before groups within a thread's share of a class).
// The plan reads every length several times (counts, the even-batch test,
// the emission; the group pass): batches of up to kLensLds sequences read
// them from LDS after one pass over global memory.
constexpr int kLensLds = 4096;

__device__ __forceinline__ void plan_body(const PlanArgs& args, int* wave_tot) {
  __shared__ int s_lens[kLensLds];
  PlanArgs a = args;
  if (args.num_seqs <= kLensLds) {
    for (int i = threadIdx.x; i < args.num_seqs; i += kThreads) s_lens[i] = args.lens[i];
    __syncthreads();
    a.lens = s_lens;
  }
  constexpr int kVals = kScanVals;
  const int S = a.num_seqs;
  const int per = ceil_div(S, kThreads);
  const int i0 = min(S, threadIdx.x * per), i1 = min(S, i0 + per);
  const int gper = ceil_div(a.num_groups, kThreads);
  const int j0 = min(a.num_groups, static_cast<int>(threadIdx.x) * gper);
  const int j1 = min(a.num_groups, j0 + gper);
  if (a.num_groups > 0) plan_groups(a);
  int part = a.part_size;
  int cnt[kVals], excl[kVals], all[kVals];
  plan_count(a, part, i0, i1, j0, j1, cnt);
  // uniform: the candidate for an even batch (no shared prefixes; lengths
  // whose block count fits an int)
  const int part2 = static_cast<int>(
      min(static_cast<int64_t>(part) * 2, static_cast<int64_t>(a.max_blocks) * kBlock));
  const bool even_try = a.even_doubling && a.num_groups == 0 && part < a.max_len &&
                        part2 > part &&
                        static_cast<int64_t>(S) * ceil_div(a.max_len, kBlock) < (1 << 30);
  cnt[kEvenItems] = cnt[kEvenRounds] = 0;
  if (even_try) even_counts(a, part2, i0, i1, &cnt[kEvenItems], &cnt[kEvenRounds]);
  block_scan<kVals>(cnt, excl, all, wave_tot);
  int listed = all[kFull];
#pragma unroll
  for (int c = 0; c < kClasses; ++c) listed += all[c];
  if (listed > a.max_items) {  // the same on every thread
    __syncthreads();  // the scan's totals are read before they are rewritten
    part = plan_partition(a, i0, i1, j0, j1, wave_tot);
    plan_count(a, part, i0, i1, j0, j1, cnt);
    cnt[kEvenItems] = cnt[kEvenRounds] = 0;
    block_scan<kVals>(cnt, excl, all, wave_tot);
  } else if (even_try && even_batch(a, part2, all[kEvenItems], all[kEvenRounds])) {
    __syncthreads();
    part = part2;
    plan_count(a, part, i0, i1, j0, j1, cnt);
    cnt[kEvenItems] = cnt[kEvenRounds] = 0;
    block_scan<kVals>(cnt, excl, all, wave_tot);
  }
  // item positions: full partitions from 0, then classes in order
  const int num_full = all[kFull];
  int pos[kClasses];
  int run = num_full;
#pragma unroll
  for (int c = 0; c < kClasses; ++c) {
    pos[c] = run + excl[c];
    run += all[c];
  }
  const int total = min(run, a.capacity);
  // list positions are a permutation of [0, run); those past the capacity
  // (a listing whose group ranges overlap) are dropped, never written
  auto put = [&](int at, int4 item) {
    if (at < a.capacity) a.items[at] = item;
  };
  int full_pos = excl[kFull];
  int split_pos = excl[kSplit];
  for (int i = i0; i < i1; ++i) {
    const SeqPlan p = seq_plan(a, i, part);
    const int nparts = p.np_pre + p.np_priv;
    if (a.num_groups > 0) a.nparts_of[i] = nparts;
    if (!p.emits) continue;
    for (int q = 0; q + 1 < p.np_priv; ++q) {
      const int start = p.shared + q * part;
      put(full_pos++, make_int4(i, start, start + part, (p.np_pre + q) | nparts << 16));
    }
    const int q = max(p.np_priv - 1, 0);
    const int start = p.shared + q * part;
    const int cls = size_class(p.np_priv > 0 ? p.len - start : 0, part, a.waves);
    int at = 0;
#pragma unroll
    for (int c = 0; c < kClasses; ++c)
      if (cls == c) at = pos[c]++;
    put(at, make_int4(i, start, p.len, (p.np_pre + q) | nparts << 16));
    if (nparts > 1) a.split[split_pos++] = i;
  }
  for (int j = j0; j < j1; ++j) {
    const int tiles = group_tiles(a, j);
    if (tiles == 0) continue;
    const int tokens = a.grp_tokens[j];
    const int np = ceil_div(tokens, part);
    const int cls = size_class(tokens - (np - 1) * part, part, a.waves);
    for (int t = 0; t < tiles; ++t) {
      for (int q = 0; q + 1 < np; ++q)
        put(full_pos++, make_int4(-2 - j, q * part, (q + 1) * part, q | t << 16));
      int at = 0;
#pragma unroll
      for (int c = 0; c < kClasses; ++c)
        if (cls == c) at = pos[c]++;
      put(at, make_int4(-2 - j, (np - 1) * part, tokens, (np - 1) | t << 16));
    }
  }
  for (int u = total + threadIdx.x; u < a.capacity; u += kThreads)
    a.items[u] = make_int4(-1, 0, 0, 0);
  for (int i = all[kSplit] + threadIdx.x; i < S; i += kThreads) a.split[i] = -1;
  if (threadIdx.x == 0) {
    a.meta[0] = total;
    a.meta[1] = all[kSplit];
    a.meta[2] = part;
  }
  for (int i = threadIdx.x; i < a.num_arrivals; i += kThreads) a.arrivals[i] = 0;
}

__global__ __launch_bounds__(kThreads) void decode_plan_kernel(PlanArgs a) {
  __shared__ int wave_tot[kWaves * kScanVals];
  plan_body(a, wave_tot);
}

// One decode step in fewer launches: work-group 0 builds the plan while the
// others write the step's new tokens into the cache (both only read their
// inputs, so they can run side by side); the decode kernels follow on the
// stream.
//
// The plan's registers set this kernel's occupancy (2 waves per SIMD), so a
// run of tokens (kNT false: more tokens than sequences) is written kStepBatch
// chunks per thread, all loaded before any is stored, to keep as many loads
// in flight as the plain writer does at full occupancy (a 39K-token step:
// 105 -> ~80 us).  A decode step's tokens, one per sequence, keep one chunk
// per thread.
constexpr int kStepBatch = 4;

template <bool kNT>
__host__ __device__ constexpr int step_batch() {
  return kNT ? 1 : kStepBatch;
}

template <typename W, bool kNT>
__global__ __launch_bounds__(kThreads) void decode_prep_kernel(PlanArgs a, W w) {
  __shared__ int wave_tot[kWaves * kScanVals];
  if (blockIdx.x == 0) {
    plan_body(a, wave_tot);
    return;
  }
  const int64_t writers = static_cast<int64_t>(gridDim.x - 1) * kThreads;
  w.template write_many<kNT, step_batch<kNT>()>(
      static_cast<int64_t>(blockIdx.x - 1) * kThreads + threadIdx.x, writers);
}

// Merge of a split sequence's partials by the last of its work-groups to
// finish (running maximum / log-sum-exp rule, as decode_reduce_kernel): each
// work-group publishes its partial at device scope and counts itself in;
// the one that completes the count reads every partial back and writes the
// output rows, so no second launch is needed.
//
// Partials are written with device-scope (relaxed) atomic stores, which
// write through to the device-coherent level instead of staying in the XCD's
// L2, and every store has completed (s_waitcnt: the hardware acknowledges a
// device-scope store once it has reached that level) before the arrival
// count moves.  The publishing side therefore needs no release fence, whose
// L2 write-back made the kernel twice as slow when every work-group paid it.
// The work-group that completes the count takes an agent-scope acquire
// fence before it reads the partials back (with device-scope loads), so its
// reads cannot be served from lines cached before the count was observed;
// that is one fence per split (sequence, head group), not per work-group.
__device__ __forceinline__ void publish(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float fetch(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Counts this work-group in on (sequence s, head group gh); true for the one
// that completes the count of nparts.  Called by one thread after every
// partial store of the work-group has completed.
__device__ __forceinline__ bool arrive(const DecodeArgs& a, int s, int gh, int nparts) {
  const int heads = a.hkv * a.head_blocks;
  return __hip_atomic_fetch_add(a.arrivals + static_cast<size_t>(s) * heads + gh, 1,
                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nparts - 1;
}

// The merge itself: rows row0 .. row0 + nh - 1, nparts partials each, all
// threads of the work-group.
template <typename Tag, int D, int W>
__device__ __forceinline__ void merge_rows(const DecodeArgs& a, int nparts, size_t row0, int nh) {
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

template <typename Tag, int D, int W>
__device__ __forceinline__ void merge_if_last(const DecodeArgs& a, int s, int gh, int nparts,
                                              size_t row0, int nh) {
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are complete
  __syncthreads();                 // ... and every thread's
  if (threadIdx.x == 0) s_last = arrive(a, s, gh, nparts);
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  merge_rows<Tag, D, W>(a, nparts, row0, nh);
}

// Stores one combined (M, L, A) of row `row`, dimension d: the output when
// the row has one partial, else partial `slot` of the row.
template <typename Tag, int D>
__device__ __forceinline__ void store_result(const DecodeArgs& a, size_t row, int d, int slot,
                                             int nparts, float M, float L, float A) {
  if (nparts <= 1) {
    a.out[row * D + d] = Tag::from_f32(L > 0.f ? A / L : 0.f);
    return;
  }
  const size_t part = row * a.np_max + slot;
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

// The end of an item: the waves' partials are combined through LDS; a
// sequence with one partial is normalised and stored, a split one leaves
// its partial (m, l, acc) in slot `slot` for the merge (in-kernel when
// a.arrivals is set, else by the merge kernel).  vs: INT8 cache only, the V
// scales of head g, applied to each combined accumulator.
template <typename Tag, int D, int W>
__device__ __forceinline__ void finish_item(const DecodeArgs& a, float* comb, int s, int slot,
                                            int nparts, int g, int h0, int nh, int gh,
                                            const float* vs) {
  const size_t row0 = static_cast<size_t>(s) * a.hq_total + g * a.group + h0;
  for (int e = threadIdx.x; e < nh * D; e += W * kWave) {
    const int h = e / D, d = e % D;
    float M, L, A;
    combine_waves<W>(comb, a.nh_max, D, h, d, M, L, A);
    if (vs) A *= vs[d];
    store_result<Tag, D>(a, row0 + h, d, slot, nparts, M, L, A);
  }
  if (nparts > 1 && a.arrivals) merge_if_last<Tag, D, W>(a, s, gh, nparts, row0, nh);
}

// Waves of a decode work-group: 4, or 8 for long partitions (item_waves).
__host__ __device__ constexpr int item_threads(int waves) { return waves * kWave; }

// One private item (sequence it.x, positions [it.y, it.z), partial slot and
// count in it.w) for head group gh (KV head x query head block): the waves
// take the item's blocks round-robin, then finish_item.
template <typename Tag, int D, bool kInt8, int W>
__device__ __forceinline__ void decode_item(const DecodeArgs& a, int4 it, int gh, float* comb) {
  const int s = it.x, start = it.y, end = it.z;
  const int slot = it.w & 0xFFFF, nparts = it.w >> 16;
  const int g = gh / a.head_blocks, h0 = (gh % a.head_blocks) * 16;
  const int nh = min(16, a.group - h0);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
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
  finish_item<Tag, D, W>(a, comb, s, slot, nparts, g, h0, nh, gh,
                         kInt8 ? a.v_scale + static_cast<size_t>(g) * D : nullptr);
}

// One prefix item: positions [it.y, it.z) of the blocks a group of sequences
// shares ("KV Cache and PagedAttention: why your LLM server slows down",
// section "How PagedAttention fixes this": one copy of a shared prompt's
// blocks serves every sample), read once for up to 16 query heads of KV head
// g drawn from several of the group's sequences -- column c of the 16-wide
// products is member c / G, head c % G -- instead of once per sequence.
// Each member's partial goes to slot it.w of its rows and is merged with its
// private partials like any other.  Only for query-head groups G <= 16.
// kInt8: an INT8 cache (the K scale folded into each column's query, the V
// scale applied to each partial, as in decode_item).
template <typename Tag, int D, int W, bool kInt8>
__device__ __forceinline__ void decode_prefix_tile(const DecodeArgs& a, int4 it, int g,
                                                   float* comb) {
  __shared__ int s_mem[16], s_np[16], s_last[16];
  const int j = -2 - it.x, start = it.y, end = it.z;
  const int slot = it.w & 0xFFFF, tile = it.w >> 16;
  const int G = a.group, mpt = a.members_per_tile;
  const int leader = uniform_load(a.grp_leader, j);
  const int m0 = min(max(uniform_load(a.pfx_start, j), 0), a.num_members);
  const int m1 = min(max(uniform_load(a.pfx_start, j + 1), m0), a.num_members);
  const int first = m0 + tile * mpt;
  const int k = min(max(m1 - first, 0), mpt);
  if (threadIdx.x < 16) {
    // a listed sequence out of range, or kept by another group, is left out
    const int t = threadIdx.x;
    const int seq = t < k ? a.pfx_seqs[first + t] : -1;
    const bool ok = seq >= 0 && seq < a.num_seqs && a.grp_of[seq] == j;
    s_mem[t] = ok ? seq : -1;
    s_np[t] = ok ? a.nparts_of[seq] : 0;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int nblk = (end - start + kBlock - 1) / kBlock;
  const int b_first = start / kBlock + wave;
  const int count = nblk > wave ? (nblk - wave + W - 1) / W : 0;
  const int32_t* trow = a.tables + static_cast<size_t>(leader) * a.max_blocks;
  const int ids = load_ids<W>(trow, b_first, count);
  __syncthreads();
  // B operand of the QK products: lane l holds column l % 16 (member m, head
  // hh), dims (j * 4 + l / 16) * 8 .. +7 of k-step j; empty columns read 0
  const int lane = threadIdx.x & (kWave - 1);
  const int n = lane & 15, kg = lane >> 4;
  const int m = n / G, hh = n % G;
  const int seq = m < k ? s_mem[m] : -1;
  uint4 qf[D / 32];
  WaveState<D> st;
  st.reset();
  if constexpr (kInt8) {
    const uint16_t* qrow =
        seq >= 0 ? a.q + (static_cast<size_t>(seq) * a.hq_total + g * G + hh) * D : nullptr;
    const float back = load_q_i8_cols<Tag, D>(a, qrow, g, qf);
    attend_blocks_i8<D, W>(a, trow, ids, b_first, count, end, g, qf, a.scale_log2 * back, st);
  } else {
    if (seq >= 0) {
      const uint4* qrow = reinterpret_cast<const uint4*>(
          a.q + (static_cast<size_t>(seq) * a.hq_total + g * G + hh) * D + kg * 8);
#pragma unroll
      for (int step = 0; step < D / 32; ++step) qf[step] = qrow[step * 4];
    } else {
#pragma unroll
      for (int step = 0; step < D / 32; ++step) qf[step] = make_uint4(0, 0, 0, 0);
    }
    attend_blocks<Tag, D, W>(a, trow, ids, b_first, count, end, g, qf, st);
  }
  stage_partials<D, W>(comb, 16, 16, st);
  __syncthreads();
  for (int e = threadIdx.x; e < 16 * D; e += W * kWave) {
    const int c = e / D, d = e % D;
    const int mc = c / G;
    if (mc >= k || s_mem[mc] < 0) continue;
    float M, L, A;
    combine_waves<W>(comb, 16, D, c, d, M, L, A);
    if constexpr (kInt8) A *= a.v_scale[static_cast<size_t>(g) * D + d];
    const size_t row = static_cast<size_t>(s_mem[mc]) * a.hq_total + g * G + c % G;
    store_result<Tag, D>(a, row, d, slot, s_np[mc], M, L, A);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are complete
  __syncthreads();                 // ... and every thread's
  if (threadIdx.x < 16) {
    const int t = threadIdx.x;
    s_last[t] = t < k && s_mem[t] >= 0 && s_np[t] > 1 && arrive(a, s_mem[t], g, s_np[t]);
  }
  __syncthreads();
  bool fenced = false;
  for (int t = 0; t < k; ++t) {
    if (!s_last[t]) continue;
    if (!fenced) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      fenced = true;
    }
    merge_rows<Tag, D, W>(a, s_np[t], static_cast<size_t>(s_mem[t]) * a.hq_total + g * G, G);
  }
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
  if (it.x == -1) return;
  if (it.x < -1) {
    if (a.pfx_seqs) decode_prefix_tile<Tag, D, W, false>(a, it, blockIdx.x % heads, comb);
    return;
  }
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
  if (it.x < 0) {  // the end of the list, or a prefix item
    if (it.x < -1 && a.pfx_seqs)
      decode_prefix_tile<Tag, D, W, true>(a, it, blockIdx.x % heads, comb);
    return;
  }
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
constexpr int kLongContext = 16384;

int auto_partition(int num_seqs, int hkv, int max_len, int kv_bytes = 2) {
  const int k = kv_bytes == 1 ? 2 : 1;
  if (max_len <= 1024 * k) return PA_PARTITION_NONE;
  const int long_part = 2048 * k;
  if (max_len >= kLongContext &&
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
  out->long_context = max_len >= kLongContext;
  out->max_len = max_len;
  out->auto_part = partition_size == PA_PARTITION_AUTO;
  return true;
}

// Waves per work-group of the items kernels: 8 for the long partitions of a
// long-context batch (>= 16K positions; partitions >= 2048 positions, INT8 >=
// 4096), where each wave still streams many blocks and the 32K context
// decodes ~4 % faster; 4 otherwise (mixed batches of short items lose up to
// 8 % at 8 waves), and 4 whenever 8 waves' partials would not fit the 64 KiB
// of LDS a work-group gets by default (query-head groups of 16 at D = 128).
int item_waves(const Split& sp, bool int8, int nh_rows, int head_dim) {
  const bool long_part = sp.part >= (int8 ? 4096 : 2048);
  const size_t lds = comb_floats(8, nh_rows, head_dim) * sizeof(float);
  return sp.long_context && long_part && lds <= 65536 ? 8 : kItemWaves;
}

// Workspace of the fixed-partition path: [plan: meta (256 B), items, split
// list] [m, l of every partial] [acc of every partial]; the partial areas
// exist only when some sequence is split.

Layout workspace_layout(int num_seqs, int hq, int head_dim, const Split& sp,
                        const SharedPrefix* sh = nullptr) {
  Layout l;
  const int members = sh ? sh->num_members : 0;
  // a member of a group has its shared prefix's partitions besides its own,
  // at most one more than the longest context's
  l.np_slots = sp.np + (sh ? 1 : 0);
  const size_t cap = static_cast<size_t>(plan_capacity(num_seqs, l.np_slots, members));
  l.meta = 0;
  l.items = kAlign;
  l.split = l.items + align_up(cap * sizeof(int4));
  l.grp_of = l.split + align_up(static_cast<size_t>(num_seqs) * sizeof(int));
  l.nparts_of = l.grp_tokens = l.grp_leader = l.ml = l.grp_of;
  if (sh) {
    const size_t seqs = align_up(static_cast<size_t>(num_seqs) * sizeof(int));
    const size_t groups = align_up(static_cast<size_t>(sh->num_groups) * sizeof(int));
    l.nparts_of = l.grp_of + seqs;
    l.grp_tokens = l.nparts_of + seqs;
    l.grp_leader = l.grp_tokens + groups;
    l.ml = l.grp_leader + groups;
  }
  l.acc = l.ml;
  l.total = l.ml;
  l.arrivals = l.total;
  if (l.np_slots > 1) {
    const size_t parts = static_cast<size_t>(num_seqs) * l.np_slots * hq;
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
                 const W* write = nullptr, const SharedPrefix* sh = nullptr) {
  using E = typename Tag::Bits;
  const int group = hq / hkv;
  const int head_blocks = use_mfma ? (group + 15) / 16 : 1;
  const Layout lay = workspace_layout(num_seqs, hq, head_dim, sp, sh);
  const int np_slots = lay.np_slots;
  if (static_cast<int64_t>(np_slots) * num_seqs * hq > 0x7fffffff / 2 ||
      np_slots >= kMaxPartitions)
    return PA_ERR_INVALID_ARG;
  // the matrix-core path's grid: items for two per sequence and at least 2048
  // work-groups, or the list's whole capacity when that is smaller; a longer
  // list takes larger partitions (plan_partition).  The merge kernel of the
  // other paths reads partitions of sp.part, so their plan keeps it.
  const bool fused_merge = use_mfma && np_slots > 1 && kFusedMerge;
  const int cap = plan_capacity(num_seqs, np_slots, sh ? sh->num_members : 0);
  const int heads = hkv * head_blocks;
  const int item_grid =
      fused_merge ? std::min(cap, std::max(2 * num_seqs, (2048 + heads - 1) / heads)) : cap;
  const int64_t grid = use_mfma ? static_cast<int64_t>(item_grid) * heads
                                : static_cast<int64_t>(sp.np) * num_seqs * hq;
  int* meta = reinterpret_cast<int*>(ws + lay.meta);
  int4* items = reinterpret_cast<int4*>(ws + lay.items);
  int* split = reinterpret_cast<int*>(ws + lay.split);
  float* ws_ml = reinterpret_cast<float*>(ws + lay.ml);
  float* ws_acc = reinterpret_cast<float*>(ws + lay.acc);
  // the matrix-core kernels merge split sequences themselves (merge_if_last)
  int* arrivals = fused_merge ? reinterpret_cast<int*>(ws + lay.arrivals) : nullptr;
  // LDS rows per wave: the head group, or 16 columns of a prefix tile
  const int nh_rows = sh ? 16 : std::min(16, group);
  const int waves = use_mfma ? item_waves(sp, k_scale != nullptr, nh_rows, head_dim) : kWaves;
  if (use_mfma || sp.np > 1) {
    PlanArgs pa{lens, items, split, meta, num_seqs, max_blocks, sp.part, np_slots,
                std::min(sp.max_len, max_blocks * kBlock), arrivals,
                fused_merge ? num_seqs * hkv * head_blocks : 0,  // one per (sequence, head group)
                item_grid, waves};
    pa.capacity = cap;
    pa.heads = heads;
    // the fused merge takes any partition; the merge kernel of the other
    // paths reads partitions of sp.part, and shared prefixes keep theirs
    pa.even_doubling = fused_merge && sp.auto_part && !sh;
    if (sh) {
      pa.pfx_seqs = sh->seqs;
      pa.pfx_start = sh->start;
      pa.pfx_blocks = sh->blocks;
      pa.num_groups = sh->num_groups;
      pa.num_members = sh->num_members;
      pa.members_per_tile = 16 / group;
      pa.grp_of = reinterpret_cast<int*>(ws + lay.grp_of);
      pa.nparts_of = reinterpret_cast<int*>(ws + lay.nparts_of);
      pa.grp_tokens = reinterpret_cast<int*>(ws + lay.grp_tokens);
      pa.grp_leader = reinterpret_cast<int*>(ws + lay.grp_leader);
    }
    pa_status ps;
    if (write) {  // the step's cache writes ride along with the plan
      // one token per sequence: stored past the caches (see store_token_chunk)
      const bool nt = write->window == 1;
      const int64_t per_group = static_cast<int64_t>(kThreads) * (nt ? step_batch<true>()
                                                                      : step_batch<false>());
      const dim3 g(static_cast<uint32_t>(1 + (write->threads() + per_group - 1) / per_group));
      ps = nt ? launch_kernel(PA_KERNEL_DECODE_PLAN, decode_prep_kernel<W, true>, g,
                              dim3(kThreads), 0, st, pa, *write)
              : launch_kernel(PA_KERNEL_DECODE_PLAN, decode_prep_kernel<W, false>, g,
                              dim3(kThreads), 0, st, pa, *write);
    } else {
      ps = launch_kernel(PA_KERNEL_DECODE_PLAN, decode_plan_kernel, dim3(1), dim3(kThreads), 0, st,
                         pa);
    }
    if (ps != PA_OK) return ps;
  }
  pa_status status = PA_OK;
  if (use_mfma) {
    if constexpr (sizeof(E) == 2) {
      DecodeArgs a = mfma_args<Tag>(q, k_cache, v_cache, tables, lens, scale_log2, out,
                                    num_seqs, hq, hkv, max_blocks, sp, ws_ml, ws_acc);
      a.k_scale = k_scale;
      a.v_scale = v_scale;
      a.arrivals = arrivals;
      if (sh) {
        a.pfx_seqs = sh->seqs;
        a.pfx_start = sh->start;
        a.grp_of = reinterpret_cast<const int*>(ws + lay.grp_of);
        a.nparts_of = reinterpret_cast<const int*>(ws + lay.nparts_of);
        a.grp_leader = reinterpret_cast<const int*>(ws + lay.grp_leader);
        a.num_members = sh->num_members;
        a.members_per_tile = 16 / group;
      }
      a.np_max = np_slots;
      a.nh_max = nh_rows;
      const size_t lds = comb_floats(waves, a.nh_max, head_dim) * sizeof(float);
      const dim3 g3(static_cast<uint32_t>(grid)), b3(item_threads(waves));
      const int4* it = items;
      constexpr int kK = PA_KERNEL_DECODE;
      if (k_scale) {  // INT8 cache
        if (head_dim == 128)
          status = waves == 8 ? launch_kernel(kK, decode_items_i8_kernel<Tag, 128, 8>, g3, b3, lds, st, a, it)
                              : launch_kernel(kK, decode_items_i8_kernel<Tag, 128, 4>, g3, b3, lds, st, a, it);
        else
          status = waves == 8 ? launch_kernel(kK, decode_items_i8_kernel<Tag, 64, 8>, g3, b3, lds, st, a, it)
                              : launch_kernel(kK, decode_items_i8_kernel<Tag, 64, 4>, g3, b3, lds, st, a, it);
      } else if (head_dim == 128) {
        status = waves == 8 ? launch_kernel(kK, decode_items_kernel<Tag, 128, 8>, g3, b3, lds, st, a, it)
                            : launch_kernel(kK, decode_items_kernel<Tag, 128, 4>, g3, b3, lds, st, a, it);
      } else {
        status = waves == 8 ? launch_kernel(kK, decode_items_kernel<Tag, 64, 8>, g3, b3, lds, st, a, it)
                            : launch_kernel(kK, decode_items_kernel<Tag, 64, 4>, g3, b3, lds, st, a, it);
      }
    }
  } else {
    status = launch_kernel(
        PA_KERNEL_DECODE, decode_generic_kernel<Tag>, dim3(static_cast<uint32_t>(grid)),
        dim3(kThreads), 0, st, static_cast<const E*>(q), static_cast<const E*>(k_cache),
        static_cast<const E*>(v_cache), tables, lens, scale_log2, static_cast<E*>(out), ws_ml,
        ws_acc, num_seqs, hq, hkv, group, head_dim, max_blocks, sp.part, sp.np);
  }
  if (status != PA_OK || sp.np <= 1 || fused_merge) return status;
  const int rows = static_cast<int>(std::min<int64_t>(static_cast<int64_t>(num_seqs) * hq, 2048));
  return launch_kernel(PA_KERNEL_DECODE_REDUCE, decode_reduce_kernel<Tag>, dim3(rows),
                       dim3(kThreads), 0, st, ws_ml, ws_acc, split, meta, lens,
                       static_cast<E*>(out), hq, head_dim, max_blocks, sp.part, sp.np);
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
  // the automatic choice shrinks partitions for fewer KV heads, so sizing with
  // one KV head covers every head count
  if (!pa::resolve_split(partition_size, num_seqs, 1, max_context_len, &sp)) return 0;
  const size_t fixed = pa::workspace_layout(num_seqs, num_q_heads, head_dim, sp).total;
  return fixed;
}

size_t pa_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                        int32_t max_context_len, int32_t partition_size,
                                        int32_t num_groups, int32_t num_members) {
  if (num_groups < 0 || num_members < 0 || num_members > pa::kMaxMembers) return 0;
  if (num_groups == 0)
    return pa_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len,
                                     partition_size);
  pa::Split sp;
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0) return 0;
  // the smallest automatic partition needs the most slots: size for it
  if (!pa::resolve_split(partition_size, num_seqs, 1, max_context_len, &sp)) return 0;
  pa::SharedPrefix sh;
  sh.num_groups = num_groups;
  sh.num_members = num_members;
  return pa::workspace_layout(num_seqs, num_q_heads, head_dim, sp, &sh).total;
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
                      pa_dtype dtype, void* stream, const StepWrite& wr,
                      const SharedPrefix* shared = nullptr) {
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
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return PA_ERR_INVALID_ARG;
  Split sp{kBlock, 1};
  if (!resolve_split(partition_size, num_seqs, num_kv_heads, max_context_len, &sp))
    return PA_ERR_INVALID_ARG;
  // shared prefixes are read once on the matrix-core path with query-head
  // groups of at most 16; elsewhere every sequence reads its own (same results)
  const SharedPrefix* sh =
      shared && shared->num_groups > 0 && use_mfma && num_q_heads / num_kv_heads <= 16
          ? shared
          : nullptr;
  // with shared prefixes the automatic partition doubles: a prefix item
  // serves several sequences, and fewer, longer ones (fewer partials to merge
  // per sequence) measured faster -- 64 prompts x 4 samples of 2048 shared
  // positions: 145 us at 2048 against 161 us at 1024 (MI355X)
  if (sh && partition_size == PA_PARTITION_AUTO && sp.np > 1 &&
      !resolve_split(2 * sp.part, num_seqs, num_kv_heads, max_context_len, &sp))
    return PA_ERR_INVALID_ARG;
  const size_t need = workspace_layout(num_seqs, num_q_heads, head_dim, sp, sh).total;
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return PA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  const float scale_log2 = scale * kLog2e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool fused = wr.key != nullptr && wr.num_tokens > 0 && use_mfma;
  if (wr.key != nullptr && wr.num_tokens > 0 && !fused) {  // write first, then decode
    const pa_status ws_st =
        pa_reshape_and_cache(wr.key, wr.value, const_cast<void*>(k_cache),
                             const_cast<void*>(v_cache), wr.slots, wr.num_tokens, wr.num_blocks,
                             num_kv_heads, head_dim, dtype, stream);
    if (ws_st != PA_OK) return ws_st;
  }
  const int64_t num_slots = static_cast<int64_t>(wr.num_blocks) * kBlock;
  switch (dtype) {
    case PA_BF16: {
      auto w = cache_write_args<uint16_t>(wr.key, wr.value, const_cast<void*>(k_cache),
                                          const_cast<void*>(v_cache), wr.slots, wr.num_tokens,
                                          num_slots, num_kv_heads, head_dim);
      w.window = step_window(wr.num_tokens, num_seqs);
      return launch<BF16T>(q, k_cache, v_cache, block_tables, context_lens, scale_log2, out,
                           num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, sp,
                           ws, use_mfma, st, nullptr, nullptr, fused ? &w : nullptr, sh);
    }
    case PA_F16: {
      auto w = cache_write_args<uint16_t>(wr.key, wr.value, const_cast<void*>(k_cache),
                                          const_cast<void*>(v_cache), wr.slots, wr.num_tokens,
                                          num_slots, num_kv_heads, head_dim);
      w.window = step_window(wr.num_tokens, num_seqs);
      return launch<F16T>(q, k_cache, v_cache, block_tables, context_lens, scale_log2, out,
                          num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, sp,
                          ws, use_mfma, st, nullptr, nullptr, fused ? &w : nullptr, sh);
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
                           pa_dtype dtype, void* stream, const StepWrite& wr,
                           const SharedPrefix* shared = nullptr) {
  if (dtype != PA_BF16 && dtype != PA_F16) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
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
  // shared prefixes as in decode_impl (this path is always the matrix-core one)
  const SharedPrefix* sh =
      shared && shared->num_groups > 0 && num_q_heads / num_kv_heads <= 16 ? shared : nullptr;
  if (sh && partition_size == PA_PARTITION_AUTO && sp.np > 1 &&
      !resolve_split(2 * sp.part, num_seqs, num_kv_heads, max_context_len, &sp, 1))
    return PA_ERR_INVALID_ARG;
  const size_t need = workspace_layout(num_seqs, num_q_heads, head_dim, sp, sh).total;
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
                         ws, true, st, k_scale, v_scale, fused ? &w : nullptr, sh);
  }
  CacheWriteI8Args<F16T> w{static_cast<const uint16_t*>(wr.key),
                           static_cast<const uint16_t*>(wr.value), kc, vc, wr.slots, k_scale,
                           v_scale, wr.num_tokens, num_slots, num_kv_heads, head_dim};
  w.window = step_window(wr.num_tokens, num_seqs);
  return launch<F16T>(q, k_cache, v_cache, block_tables, context_lens, scale_log2, out, num_seqs,
                      num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, sp, ws, true, st,
                      k_scale, v_scale, fused ? &w : nullptr, sh);
}

}  // namespace
}  // namespace pa

// ---- the decode entry point that allocates nothing ----
//
// pa_paged_attention_decode_noalloc runs the same kernels with its workspace
// in `scratch`, a file-scope array of PA_DECODE_SCRATCH_BYTES in device
// memory: each device the library runs on holds its own copy, at its own
// address, until the process ends.  Host code never names the array in a
// launch or a copy: on the host its name is only a stand-in, so the device
// address comes from hipGetSymbolAddress, taken once per device with that
// device current and kept.
static __device__ __align__(256) char scratch[PA_DECODE_SCRATCH_BYTES];

namespace pa {
namespace {

constexpr int kMaxDevices = 64;

// Device address of the current device's `scratch`, or null (no device, or
// the symbol cannot be resolved).
void* scratch_address() {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
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

pa_status pa_paged_attention_decode_noalloc(const void* q, const void* k_cache,
                                            const void* v_cache, const int32_t* block_tables,
                                            const int32_t* context_lens, float scale, void* out,
                                            int32_t num_seqs, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t max_blocks_per_seq, int32_t max_context_len,
                                            int32_t partition_size, pa_dtype dtype, void* stream) {
  // an empty batch (or an argument error) needs no device and no workspace
  void* ws = num_seqs > 0 ? pa::scratch_address() : nullptr;
  if (num_seqs > 0 && ws == nullptr) return PA_ERR_DEVICE;
  return pa::decode_impl(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs,
                         num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                         max_context_len, partition_size, ws,
                         ws ? static_cast<size_t>(PA_DECODE_SCRATCH_BYTES) : 0, dtype, stream,
                         pa::StepWrite{nullptr, nullptr, nullptr, 0, 0});
}

namespace {

// Argument checks of the shared-prefix calls; the groups themselves are
// device data that the plan bounds (members out of range are ignored).
pa_status shared_args(const int32_t* prefix_seqs, const int32_t* prefix_start,
                      const int32_t* prefix_blocks, int32_t num_groups, int32_t num_members,
                      pa::SharedPrefix* out) {
  if (num_groups < 0 || num_members < 0 || num_members > pa::kMaxMembers)
    return PA_ERR_INVALID_ARG;
  if (num_groups > 0 && (!prefix_seqs || !prefix_start || !prefix_blocks))
    return PA_ERR_INVALID_ARG;
  out->seqs = prefix_seqs;
  out->start = prefix_start;
  out->blocks = prefix_blocks;
  out->num_groups = num_members > 0 ? num_groups : 0;
  out->num_members = num_members;
  return PA_OK;
}

}  // namespace

pa_status pa_paged_attention_decode_shared(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
    const int32_t* context_lens, const int32_t* prefix_seqs, const int32_t* prefix_start,
    const int32_t* prefix_blocks, int32_t num_groups, int32_t num_members, float scale, void* out,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t max_blocks_per_seq, int32_t max_context_len, int32_t partition_size, void* workspace,
    size_t workspace_bytes, pa_dtype dtype, void* stream) {
  pa::SharedPrefix sh;
  const pa_status st =
      shared_args(prefix_seqs, prefix_start, prefix_blocks, num_groups, num_members, &sh);
  if (st != PA_OK) return st;
  return pa::decode_impl(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs,
                         num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                         max_context_len, partition_size, workspace, workspace_bytes, dtype,
                         stream, pa::StepWrite{nullptr, nullptr, nullptr, 0, 0}, &sh);
}

pa_status pa_decode_step_shared(
    const void* key, const void* value, const int64_t* slot_mapping, int32_t num_new_tokens,
    int32_t num_blocks, const void* q, void* k_cache, void* v_cache, const int32_t* block_tables,
    const int32_t* context_lens, const int32_t* prefix_seqs, const int32_t* prefix_start,
    const int32_t* prefix_blocks, int32_t num_groups, int32_t num_members, float scale, void* out,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t max_blocks_per_seq, int32_t max_context_len, int32_t partition_size, void* workspace,
    size_t workspace_bytes, pa_dtype dtype, void* stream) {
  using namespace pa;
  pa::SharedPrefix sh;
  const pa_status st =
      shared_args(prefix_seqs, prefix_start, prefix_blocks, num_groups, num_members, &sh);
  if (st != PA_OK) return st;
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
                     StepWrite{key, value, slot_mapping, num_new_tokens, num_blocks}, &sh);
}

pa_status pa_paged_attention_decode_int8_shared(
    const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
    const float* v_scale, const int32_t* block_tables, const int32_t* context_lens,
    const int32_t* prefix_seqs, const int32_t* prefix_start, const int32_t* prefix_blocks,
    int32_t num_groups, int32_t num_members, float scale, void* out, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
    int32_t max_context_len, int32_t partition_size, void* workspace, size_t workspace_bytes,
    pa_dtype dtype, void* stream) {
  pa::SharedPrefix sh;
  const pa_status st =
      shared_args(prefix_seqs, prefix_start, prefix_blocks, num_groups, num_members, &sh);
  if (st != PA_OK) return st;
  return pa::decode_int8_impl(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                              scale, out, num_seqs, num_q_heads, num_kv_heads, head_dim,
                              max_blocks_per_seq, max_context_len, partition_size, workspace,
                              workspace_bytes, dtype, stream,
                              pa::StepWrite{nullptr, nullptr, nullptr, 0, 0}, &sh);
}

pa_status pa_decode_step_int8_shared(
    const void* key, const void* value, const int64_t* slot_mapping, int32_t num_new_tokens,
    int32_t num_blocks, const void* q, void* k_cache, void* v_cache, const float* k_scale,
    const float* v_scale, const int32_t* block_tables, const int32_t* context_lens,
    const int32_t* prefix_seqs, const int32_t* prefix_start, const int32_t* prefix_blocks,
    int32_t num_groups, int32_t num_members, float scale, void* out, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
    int32_t max_context_len, int32_t partition_size, void* workspace, size_t workspace_bytes,
    pa_dtype dtype, void* stream) {
  using namespace pa;
  pa::SharedPrefix sh;
  const pa_status st =
      shared_args(prefix_seqs, prefix_start, prefix_blocks, num_groups, num_members, &sh);
  if (st != PA_OK) return st;
  // the write's own checks, as pa_decode_step_int8 makes them
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
                          StepWrite{key, value, slot_mapping, num_new_tokens, num_blocks}, &sh);
}

}  // extern "C"
