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
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
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

// Cache-policy operand of buffer loads for data that is read once (the K/V
// tiles of a key range only one workgroup reads, logits rows): non-temporal,
// so such a stream does not displace lines that other loads will reuse.
constexpr int kLoadOnce = 2;

// ---------------------------------------------------------------- reductions
// Cross-lane exchanges without the LDS crossbar: within a 16-lane row, DPP
// quad permutes (partner l ^ 1, l ^ 2) and row mirrors (partner 7 - l within
// each half-row, then 15 - l within the row); across rows, gfx950's
// v_permlane16_swap / v_permlane32_swap (partner l ^ 16, l ^ 32).  Each step
// pairs lanes whose partial results cover disjoint lane sets, so five steps
// leave every lane with the whole wave's combination, and partners compute
// the same value (the combining operations are commutative), so the result is
// identical in every lane.  Every lane of the wave must be active.
template <int STEP>
__device__ inline uint32_t lane_partner(uint32_t v) {
  if constexpr (STEP == 0) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);  // quad 1,0,3,2
  } else if constexpr (STEP == 1) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);  // quad 2,3,0,1
  } else if constexpr (STEP == 2) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);  // half mirror
  } else if constexpr (STEP == 3) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);  // row mirror
  } else if constexpr (STEP == 4) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return ((__lane_id() >> 4) & 1) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (__lane_id() >> 5) ? r[0] : r[1];
  }
}

template <int STEP>
__device__ inline float partner_f32(float v) {
  return __uint_as_float(lane_partner<STEP>(__float_as_uint(v)));
}
template <int STEP>
__device__ inline int partner_i32(int v) {
  return (int)lane_partner<STEP>((uint32_t)v);
}
template <int STEP>
__device__ inline double partner_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint64_t lo = lane_partner<STEP>((uint32_t)b), hi = lane_partner<STEP>((uint32_t)(b >> 32));
  return __longlong_as_double((long long)((hi << 32) | lo));
}

__device__ inline float wave_max_f32(float v) {
  v = fmaxf(v, partner_f32<0>(v));
  v = fmaxf(v, partner_f32<1>(v));
  v = fmaxf(v, partner_f32<2>(v));
  v = fmaxf(v, partner_f32<3>(v));
  v = fmaxf(v, partner_f32<4>(v));
  return fmaxf(v, partner_f32<5>(v));
}

__device__ inline int wave_min_i32(int v) {
  v = min(v, partner_i32<0>(v));
  v = min(v, partner_i32<1>(v));
  v = min(v, partner_i32<2>(v));
  v = min(v, partner_i32<3>(v));
  v = min(v, partner_i32<4>(v));
  return min(v, partner_i32<5>(v));
}

__device__ inline double wave_sum_f64(double v) {
  v += partner_f64<0>(v);
  v += partner_f64<1>(v);
  v += partner_f64<2>(v);
  v += partner_f64<3>(v);
  v += partner_f64<4>(v);
  return v + partner_f64<5>(v);
}

__device__ inline float wave_sum_f32(float v) {
  v += partner_f32<0>(v);
  v += partner_f32<1>(v);
  v += partner_f32<2>(v);
  v += partner_f32<3>(v);
  v += partner_f32<4>(v);
  return v + partner_f32<5>(v);
}

// (value, index) maximum: larger value wins; equal values keep the lower index.
__device__ inline void argmax_merge(float& m, int& a, float m2, int a2) {
  if (m2 > m || (m2 == m && a2 < a)) {
    m = m2;
    a = a2;
  }
}

template <int STEP>
__device__ inline void argmax_step(float& m, int& a) {
  const float m2 = partner_f32<STEP>(m);
  const int a2 = partner_i32<STEP>(a);
  argmax_merge(m, a, m2, a2);
}

__device__ inline void wave_argmax(float& m, int& a) {
  argmax_step<0>(m, a);
  argmax_step<1>(m, a);
  argmax_step<2>(m, a);
  argmax_step<3>(m, a);
  argmax_step<4>(m, a);
  argmax_step<5>(m, a);
}

// ---------------------------------------------------------------- host side
// The caller's status word, or the library's own word on the current device
// when the caller passes none (status.hip).
int32_t* status_or_library(int32_t* status);

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Launch of a kernel whose workgroups meet (every workgroup must be resident;
// the grid is sized from the occupancy query to fit the device at once).  An
// ordinary launch is the default: a cooperative launch costs some 17 us more
// per call on MI355X.  SPEC_COOPERATIVE_LAUNCH=1 in the environment (read at
// each call) selects the cooperative launch, which also guarantees residency
// when other streams keep CUs busy; without it a meeting that cannot complete
// ends at its wait bound and raises SPEC_DEV_SYNC_TIMEOUT.
inline hipError_t launch_meeting_kernel(const void* fn, dim3 grid, dim3 block, void** args,
                                        hipStream_t s) {
  const char* e = getenv("SPEC_COOPERATIVE_LAUNCH");  // read per call
  const bool coop = e && e[0] == '1';
  return coop ? hipLaunchCooperativeKernel(fn, grid, block, args, 0, s)
              : hipLaunchKernel(fn, grid, block, args, 0, s);
}

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

}  // namespace spec
