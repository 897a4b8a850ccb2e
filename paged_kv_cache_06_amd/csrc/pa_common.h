// Shared helpers of the HIP kernels and their launchers (gfx950, wave64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <utility>

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

// ---- cache stores ----
// Stores with the non-temporal hint, for cache data that later kernels read
// back through HBM, not this one: left dirty in the XCDs' L2 caches, a decode
// step's few new tokens slowed the decode kernel that followed by ~4 us on
// MI355X (100.9 against 96.7 us on the 70B-layer batch).
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void stream_store16(void* p, uint4 v) {
  __builtin_nontemporal_store(u32x4_nt{v.x, v.y, v.z, v.w}, static_cast<u32x4_nt*>(p));
}
template <typename T>
__device__ __forceinline__ void stream_store(T* p, T v) {
  __builtin_nontemporal_store(v, p);
}

// ---- kernel timing hooks (pa_timing.hip) ----
// The events of the next launch of kernel kind `kind` while timing is on and
// capacity remains, else two null events (an untimed launch).
struct TimedLaunch {
  hipEvent_t start, stop;
};
TimedLaunch timing_events(int kind);

// Launch check: converts the last launch error to a status.
inline pa_status launch_status() {
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_DEVICE;
}

// Launches kernel<<<grid, block, lds, stream>>>(args...).  While timing is on
// the launch carries two HIP events attached to its dispatch, which record
// the start and the end of the kernel's own execution on its stream (no
// separate marker packets around it).
template <typename... Params, typename... Args>
pa_status launch_kernel(int kind, void (*kernel)(Params...), dim3 grid, dim3 block, size_t lds,
                        hipStream_t stream, Args&&... args) {
  static_assert(sizeof...(Params) == sizeof...(Args), "kernel argument count");
  const TimedLaunch t = timing_events(kind);
  hipExtLaunchKernelGGL(kernel, grid, block, static_cast<uint32_t>(lds), stream, t.start, t.stop,
                        0, static_cast<Params>(std::forward<Args>(args))...);
  return launch_status();
}

}  // namespace pa
