// Matrix-core decode over an INT8 KV cache: block loads, code conversion and
// the query operand.  K and V are kept as 8-bit codes with one fp32 scale per
// (KV head, channel) ("KV Cache for the intermediate", section "KV Cache
// Quantization"); a cached value stands for code * scale.
//
// Per block and wave the codes arrive in the layout of include/pa.h (one
// 16-byte load per lane per 64-dimension slab for K and for V) and become
// exact fp16 matrix-core operands with two integer ops and one packed fp16
// subtraction per pair of codes.  The scales never touch the K/V stream:
//   score_t = sum_d q_d * sK_d * code_t,d : the K scale is folded into the
//             query once per item; q * sK enters the product as an fp16
//             hi + lo pair, pre-scaled by a power of two per head so that it
//             stays in fp16 range (the exponent is taken back out of the score);
//   out_d   = sV_d * sum_t p_t * code_t,d / sum_t p_t : the V scale multiplies
//             the item's merged result once.
#pragma once

#include "pa_decode_common.h"

namespace pa {
namespace {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Four int8 codes (byte i of w is code i) as four exact fp16 values: the
// biased byte c + 128 becomes the low mantissa byte of fp16 1024 + (c + 128),
// then 1152 is subtracted from both halves at once.
__device__ __forceinline__ uint2 codes_to_f16(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  // byte permutes of {0x64646464 : u}: selector bytes 0-3 pick u, 4 picks 0x64
  const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);  // u0, 64, u1, 64
  const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);  // u2, 64, u3, 64
  const f16x2_t bias = {static_cast<_Float16>(1152.f), static_cast<_Float16>(1152.f)};
  const f16x2_t a = __builtin_bit_cast(f16x2_t, lo) - bias;
  const f16x2_t b = __builtin_bit_cast(f16x2_t, hi) - bias;
  return make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
}

// Codes of one block of KV head g: lane l holds, per 64-dimension slab i,
// 16 K codes (token l%16, dims 64i + 16*(l/16) .. +15) and 16 V codes
// (dims 64i + 16*tt + l%16 for tt < 4, tokens 4*(l/16) .. +3).
template <int D>
struct I8Regs {
  uint4 k[D / 64];
  uint4 v[D / 64];
};

// `valid` false: the loads are issued with an empty range, read nothing and
// give zeros (so that a wave's load sequence does not depend on its count).
template <int D>
__device__ __forceinline__ void load_block_i8(const DecodeArgs& a, int g, int phys,
                                              I8Regs<D>& r, bool valid = true) {
  const uint32_t lane = threadIdx.x & (kWave - 1);
  constexpr uint32_t kBytes = D * kBlock;  // one KV head of one block
  const size_t off = (static_cast<size_t>(phys) * a.hkv + g) * kBytes;
  const uint32_t range = valid ? kBytes : 0u;
  const auto rk = buffer_of(reinterpret_cast<const char*>(a.k_cache) + off, range);
  const auto rv = buffer_of(reinterpret_cast<const char*>(a.v_cache) + off, range);
#pragma unroll
  for (int i = 0; i < D / 64; ++i) r.k[i] = stream_load16(rk, lane * 16 + i * 1024);
#pragma unroll
  for (int i = 0; i < D / 64; ++i) r.v[i] = stream_load16(rv, lane * 16 + i * 1024);
}

// Matrix-core operands of the block: kf[m] is the A operand of QK step m
// (k index 8*(l/16) + e <-> dim 64*(m/2) + 16*(l/16) + 8*(m%2) + e), vf[sl]
// the A operand of PV slice sl (dim 16*sl + l%16, tokens 4*(l/16) .. +3).
template <int D>
__device__ __forceinline__ void convert_block_i8(const I8Regs<D>& r, uint4* kf, uint2* vf) {
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    const uint2 k0 = codes_to_f16(r.k[i].x), k1 = codes_to_f16(r.k[i].y);
    const uint2 k2 = codes_to_f16(r.k[i].z), k3 = codes_to_f16(r.k[i].w);
    kf[2 * i] = make_uint4(k0.x, k0.y, k1.x, k1.y);
    kf[2 * i + 1] = make_uint4(k2.x, k2.y, k3.x, k3.y);
    vf[4 * i + 0] = codes_to_f16(r.v[i].x);
    vf[4 * i + 1] = codes_to_f16(r.v[i].y);
    vf[4 * i + 2] = codes_to_f16(r.v[i].z);
    vf[4 * i + 3] = codes_to_f16(r.v[i].w);
  }
}

// B operands of QK for query heads h0 .. h0+nh-1 of KV head g over an INT8
// cache: lane l holds head l%16 and, for step m, q * sK at the dims of kf[m]
// above, times 2^(15 - e) where 2^e bounds the head's largest |q * sK|, as an
// fp16 hi + lo pair.  Returns 2^(e - 15), the factor that takes the
// pre-scaling back out of this lane's scores.  Rows past nh read 0.
template <typename Tag, int D>
__device__ __forceinline__ float load_q_i8(const DecodeArgs& a, int s, int g, int h0, int nh,
                                           uint4* qh) {
  const uint32_t lane = threadIdx.x & (kWave - 1);
  const uint32_t n = lane & 15, kg = lane >> 4;
  const auto rq = buffer_of(a.q + (static_cast<size_t>(s) * a.hq_total + g * a.group + h0) * D,
                            static_cast<uint32_t>(nh) * D * 2);
  const auto rs = buffer_of(a.k_scale + static_cast<size_t>(g) * D, D * 4);
  float x[D / 32][8];
  float amax = 0.f;
#pragma unroll
  for (int m = 0; m < D / 32; ++m) {
    const uint32_t d0 = 64 * (m >> 1) + 16 * kg + 8 * (m & 1);
    const uint4 qv = buffer_load16(rq, (n * D + d0) * 2);
    const uint4 s0 = buffer_load16(rs, d0 * 4);
    const uint4 s1 = buffer_load16(rs, d0 * 4 + 16);
    const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
    const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t bits = static_cast<uint16_t>(qw[e / 2] >> (16 * (e & 1)));
      x[m][e] = Tag::to_f32(bits) * __uint_as_float(sw[e]);
      amax = fmaxf(amax, fabsf(x[m][e]));
    }
  }
  amax = fmaxf(amax, __shfl_xor(amax, 16));
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  int ex;
  (void)frexpf(amax, &ex);  // amax < 2^ex (ex = 0 for amax = 0)
  const float up = ldexpf(1.f, 15 - ex);
#pragma unroll
  for (int m = 0; m < D / 32; ++m) {
    uint32_t hw[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const f16x2_t v = {static_cast<_Float16>(x[m][e] * up),
                         static_cast<_Float16>(x[m][e + 1] * up)};
      hw[e / 2] = __builtin_bit_cast(uint32_t, v);
    }
    qh[m] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
  }
  return ldexpf(1.f, ex - 15);
}

// load_q_i8 for the columns of a prefix tile, whose query rows belong to
// different sequences: qrow is this lane's column's row (every lane of a
// column passes the same one), nullptr for an empty column (reads 0).
template <typename Tag, int D>
__device__ __forceinline__ float load_q_i8_cols(const DecodeArgs& a, const uint16_t* qrow, int g,
                                                uint4* qh) {
  const uint32_t kg = (threadIdx.x & (kWave - 1)) >> 4;
  const float* sk = a.k_scale + static_cast<size_t>(g) * D;
  float x[D / 32][8];
  float amax = 0.f;
#pragma unroll
  for (int m = 0; m < D / 32; ++m) {
    const uint32_t d0 = 64 * (m >> 1) + 16 * kg + 8 * (m & 1);
    const uint4 qv = qrow ? *reinterpret_cast<const uint4*>(qrow + d0) : make_uint4(0, 0, 0, 0);
    const uint4 s0 = *reinterpret_cast<const uint4*>(sk + d0);
    const uint4 s1 = *reinterpret_cast<const uint4*>(sk + d0 + 4);
    const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
    const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t bits = static_cast<uint16_t>(qw[e / 2] >> (16 * (e & 1)));
      x[m][e] = Tag::to_f32(bits) * __uint_as_float(sw[e]);
      amax = fmaxf(amax, fabsf(x[m][e]));
    }
  }
  amax = fmaxf(amax, __shfl_xor(amax, 16));
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  int ex;
  (void)frexpf(amax, &ex);  // amax < 2^ex (ex = 0 for amax = 0)
  const float up = ldexpf(1.f, 15 - ex);
#pragma unroll
  for (int m = 0; m < D / 32; ++m) {
    uint32_t hw[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const f16x2_t v = {static_cast<_Float16>(x[m][e] * up),
                         static_cast<_Float16>(x[m][e + 1] * up)};
      hw[e / 2] = __builtin_bit_cast(uint32_t, v);
    }
    qh[m] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
  }
  return ldexpf(1.f, ex - 15);
}

// attend_blocks over an INT8 cache: sl2 is the per-lane score factor (the
// softmax scale in log2 units times load_q_i8's return value).
template <int D, int W>
__device__ __forceinline__ void attend_blocks_i8(const DecodeArgs& a, const int32_t* trow,
                                                 int ids, int b_first, int count, int len, int g,
                                                 const uint4* qh, float sl2,
                                                 WaveState<D>& st) {
  auto attend = [&](const I8Regs<D>& r, int blk) {
    uint4 kf[D / 32];
    uint2 vf[D / 16];
    convert_block_i8<D>(r, kf, vf);
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < D / 32; ++m) sc = Mfma<F16T>::qk(kf[m], qh[m], sc);
    block_update<F16T, D>(vf, sc, sl2, blk, len, st);
  };
  // Software pipeline over two register sets: the next block's loads are in
  // flight while the current one is converted and multiplied (an INT8 block is
  // half the bytes of a 16-bit one for the same compute).  Every iteration
  // issues the same loads, empty-ranged past the end, so the waits stay exact.
  for (int c0 = 0; c0 < count; c0 += 64) {
    if (c0 > 0) ids = load_ids<W>(trow, b_first + W * c0, count - c0);
    const int n = min(64, count - c0);
    const int blk0 = b_first + W * c0;
    I8Regs<D> ra, rb;
    load_block_i8<D>(a, g, __builtin_amdgcn_readlane(ids, 0), ra);
    for (int j = 0; j < n; j += 2) {
      load_block_i8<D>(a, g, __builtin_amdgcn_readlane(ids, (j + 1) & 63), rb, j + 1 < n);
      __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the compute
      attend(ra, blk0 + W * j);
      if (j + 1 >= n) break;
      load_block_i8<D>(a, g, __builtin_amdgcn_readlane(ids, (j + 2) & 63), ra, j + 2 < n);
      __builtin_amdgcn_sched_barrier(0);
      attend(rb, blk0 + W * (j + 1));
    }
  }
}

}  // namespace
}  // namespace pa
