// Shared helpers of the HIP kernels and their launchers (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "pa.h"

namespace pa {

constexpr int kBlock = PA_BLOCK_SIZE;  // token slots per KV block
constexpr int kWave = 64;

inline int elem_bytes(pa_dtype dt) { return dt == PA_F32 ? 4 : dt == PA_I8 ? 1 : 2; }
inline bool valid_dtype(pa_dtype dt) { return dt == PA_F32 || dt == PA_F16 || dt == PA_BF16; }

// ---- scalar conversions (storage bits <-> fp32) ----
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float f16_to_f32(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}
// round to nearest, ties to even (the hardware conversions round the same way)
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ uint16_t f32_to_f16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// Storage traits: Bits is the element as stored; to_f32/from_f32 convert.
struct F32T {
  using Bits = float;
  static constexpr int kBytes = 4;
  __device__ static float to_f32(float x) { return x; }
  __device__ static float from_f32(float x) { return x; }
};
struct BF16T {
  using Bits = uint16_t;
  static constexpr int kBytes = 2;
  __device__ static float to_f32(uint16_t x) { return bf16_to_f32(x); }
  __device__ static uint16_t from_f32(float x) { return f32_to_bf16(x); }
};
struct F16T {
  using Bits = uint16_t;
  static constexpr int kBytes = 2;
  __device__ static float to_f32(uint16_t x) { return f16_to_f32(x); }
  __device__ static uint16_t from_f32(float x) { return f32_to_f16(x); }
};

// ---- kernel timing hooks (pa_timing.hip) ----
// Returns a slot index when timing is on and capacity remains, else -1.
int timing_start(int kind, hipStream_t stream);
void timing_stop(int slot, hipStream_t stream);

// Launch check: converts the last launch error to a status.
inline pa_status launch_status() {
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_DEVICE;
}

}  // namespace pa
