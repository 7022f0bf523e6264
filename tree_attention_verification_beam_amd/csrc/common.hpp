// common.hpp -- device and host helpers shared by the library's HIP sources.
// gfx950 only: 64-wide wavefronts, bf16 MFMA, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "../../include/specverify.h"

namespace spec {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- status word
__device__ inline void raise_status(int32_t* status, int32_t bits) {
  if (status) atomicOr(status, bits);
}

// ---------------------------------------------------------------- cross-workgroup hand-over
// The per-XCD L2 caches are not coherent with each other.  Agent-scope relaxed
// atomic stores and loads reach the device-coherent level directly, so data
// passed between workgroups of one kernel goes through these, and a writer
// waits for its stores to complete (vmcnt) before it signals with an atomic;
// no cache-wide write-back or invalidate is needed.
__device__ inline void store_coherent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t load_coherent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void wait_stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------- reductions
__device__ inline float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ inline double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ inline float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// (value, index) maximum: larger value wins; equal values keep the lower index.
__device__ inline void argmax_merge(float& m, int& a, float m2, int a2) {
  if (m2 > m || (m2 == m && a2 < a)) {
    m = m2;
    a = a2;
  }
}

__device__ inline void wave_argmax(float& m, int& a) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float m2 = __shfl_xor(m, o, kWave);
    int a2 = __shfl_xor(a, o, kWave);
    argmax_merge(m, a, m2, a2);
  }
}

// ---------------------------------------------------------------- host side
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Launch of a kernel whose workgroups meet (every workgroup must be resident;
// the grid is sized from the occupancy query to fit the device at once).  An
// ordinary launch is the default: a cooperative launch costs some 17 us more
// per call on MI355X.  SPEC_COOPERATIVE_LAUNCH=1 in the environment selects the
// cooperative launch, which also guarantees residency when other streams keep
// CUs busy; without it a meeting that cannot complete ends at its wait bound
// and raises SPEC_DEV_SYNC_TIMEOUT.
inline hipError_t launch_meeting_kernel(const void* fn, dim3 grid, dim3 block, void** args,
                                        hipStream_t s) {
  static const bool coop = [] {
    const char* e = getenv("SPEC_COOPERATIVE_LAUNCH");
    return e && e[0] == '1';
  }();
  return coop ? hipLaunchCooperativeKernel(fn, grid, block, args, 0, s)
              : hipLaunchKernel(fn, grid, block, args, 0, s);
}

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

}  // namespace spec
