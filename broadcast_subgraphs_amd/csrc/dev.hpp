// Device primitives shared by the stitched and GEMM-epilogue kernels (gfx950, wave64).
//
//  * 16-byte fragments: the largest element group one vector memory instruction
//    moves ([ComFuse] Stage-Stream Execution Model, compute phase: data streams
//    through elementwise nodes one Fragment at a time).
//  * Reductions at each level of [ComFuse] Fig. 4: thread-local, then within a
//    wavefront by lane exchange, then across the waves of a workgroup through
//    one LDS scratch region that every reduction reuses ([ComFuse] "a single,
//    unified SMEM buffer"), then across workgroups through global memory.
//  * The cross-workgroup join: a counter that the last arriver resets and a
//    generation word it advances ([sass2mlir] "Counter-based mini-joins" and
//    "Grid-barrier synthesis": one release arrive per workgroup, a bounded spin,
//    one trailing acquire, self-cleaning state).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cf {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// Spin cap for cross-workgroup waits.  A wait that exceeds it sets the error
// word and returns, so every wave always exits even if the co-residency
// assumption were violated.  About a second of spinning on MI355X.
constexpr uint32_t kSpinCap = 1u << 20;

// ---------------------------------------------------------------- fragments

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }

__device__ __forceinline__ float4 ld4_stream(const float* p) {
  // single-use stream: non-temporal hint so it does not displace reused lines
  float4 v;
  v.x = __builtin_nontemporal_load(p + 0);
  v.y = __builtin_nontemporal_load(p + 1);
  v.z = __builtin_nontemporal_load(p + 2);
  v.w = __builtin_nontemporal_load(p + 3);
  return v;
}

__device__ __forceinline__ void st4_stream(float* p, float4 v) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  f4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<f4*>(p));
}

__device__ __forceinline__ void st4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }

// fp32 -> bf16 bits, round to nearest even (inputs finite).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ------------------------------------------------------------ reduce ops

struct OpSum {
  __device__ static float id() { return 0.0f; }
  __device__ static float op(float a, float b) { return a + b; }
};
struct OpMax {
  __device__ static float id() { return -INFINITY; }
  __device__ static float op(float a, float b) { return fmaxf(a, b); }
};

// Butterfly over groups of G consecutive lanes (G a power of two, G <= 64):
// every lane of the group ends with the group's reduction.
template <class Op, int G>
__device__ __forceinline__ float group_reduce(float v) {
#pragma unroll
  for (int o = G / 2; o >= 1; o >>= 1) v = Op::op(v, __shfl_xor(v, o, kWave));
  return v;
}

// ------------------------------------------------------ cross-workgroup join
//
// Join state for one group of workgroups: {count, gen}.  A workgroup publishes
// its partials, then calls join_arrive_and_wait().  Preconditions: count == 0
// when the first member arrives (true for a zero-filled workspace and after
// every completed join).  All members of the group must be resident at once.

struct JoinWord {
  uint32_t count;
  uint32_t gen;
};

// Called by ONE thread of the workgroup, after that thread (or its whole wave,
// followed by the wave-wide wait the release implies) stored the partials.
// Returns true if the group completed, false if the spin cap was hit.
__device__ __forceinline__ bool join_arrive_and_wait(JoinWord* j, uint32_t members, uint32_t* err) {
  const uint32_t g0 = __hip_atomic_load(&j->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t old =
      __hip_atomic_fetch_add(&j->count, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  if (old == members - 1) {
    // last arriver: every member's partials happen-before this point
    __hip_atomic_store(&j->count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(&j->gen, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    return true;
  }
  for (uint32_t it = 0; it < kSpinCap; ++it) {
    if (__hip_atomic_load(&j->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != g0) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      return true;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return false;
}

// Coherent (agent-scope) loads of partials written by other workgroups.
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Logical workgroup index that keeps consecutive logical ids on one XCD.
// MI355X hands workgroups to its 8 XCDs round-robin (physical id % 8), so
// logical = (phys % 8) * (G / 8) + phys / 8 places logical ids [x*G/8, (x+1)*G/8)
// on XCD x.  Identity when G is not a multiple of 8.
__device__ __forceinline__ uint32_t xcd_local_id(uint32_t phys, uint32_t G) {
  if ((G & 7u) != 0u) return phys;
  return (phys & 7u) * (G >> 3) + (phys >> 3);
}

}  // namespace cf
