// Device primitives shared by the stitched and GEMM-epilogue kernels (gfx950, wave64).
//
//  * 16-byte fragments: the largest element group one vector memory instruction
//    moves ([ComFuse] Stage-Stream Execution Model, compute phase: data streams
//    through elementwise nodes one Fragment at a time).
//  * Reductions at each level of [ComFuse] Fig. 4: thread-local, then within a
//    wavefront by lane exchange, then across the waves of a workgroup through
//    one LDS scratch region that every reduction reuses ([ComFuse] "a single,
//    unified SMEM buffer"), then across workgroups through global memory.
//  * The cross-workgroup join: an arrival counter the last arriver resets and a
//    generation it advances, packed in one word ([sass2mlir] "Counter-based
//    mini-joins" and "Grid-barrier synthesis": one arrive per workgroup, an
//    atomic-load spin, self-cleaning state, coherent cross-workgroup reads).
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

// ------------------------------------------------- online pair reductions
//
// Softmax statistics as one (max, sum) pair in the base-2 domain: the sum is
// taken relative to the pair's own max, and two pairs merge by rescaling both
// sums to the larger max (the online softmax identity; an empty pair is
// (-inf, 0)).  LayerNorm statistics as (count, mean, M2), merged with Chan's
// pairwise update.  Each merges a row's statistics in ONE reduction instead of
// two chained ones (max then sum; mean then centred second moment), equal in
// exact arithmetic.
struct SmPair {
  float m, l;
};
__device__ __forceinline__ SmPair sm_merge(SmPair a, SmPair b) {
  const float M = fmaxf(a.m, b.m);
  if (M == -INFINITY) return {M, 0.0f};
  return {M, a.l * __builtin_amdgcn_exp2f(a.m - M) + b.l * __builtin_amdgcn_exp2f(b.m - M)};
}
struct MomPair {
  float n, mean, m2;
};
__device__ __forceinline__ MomPair mom_merge(MomPair a, MomPair b) {
  const float n = a.n + b.n;
  if (b.n == 0.0f) return a;
  if (a.n == 0.0f) return b;
  const float d = b.mean - a.mean, f = b.n / n;
  return {n, fmaf(d, f, a.mean), a.m2 + b.m2 + d * d * (a.n * f)};
}
// Butterfly over all 64 lanes of the wave: every lane ends with the wave's
// pair.  Both lanes of an exchange merge (lower lane's pair, upper lane's
// pair), so they compute the same bits even where the merge is not symmetric.
__device__ __forceinline__ SmPair wave_reduce(SmPair p) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const SmPair q = {__shfl_xor(p.m, o, kWave), __shfl_xor(p.l, o, kWave)};
    p = (threadIdx.x & o) ? sm_merge(q, p) : sm_merge(p, q);
  }
  return p;
}
__device__ __forceinline__ MomPair wave_reduce(MomPair p) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const MomPair q = {__shfl_xor(p.n, o, kWave), __shfl_xor(p.mean, o, kWave), __shfl_xor(p.m2, o, kWave)};
    p = (threadIdx.x & o) ? mom_merge(q, p) : mom_merge(p, q);
  }
  return p;
}

// ------------------------------------------------------ cross-workgroup join
//
// One 64-bit join word per group of cooperating workgroups:
//   bits 63..32  generation (completed joins, wraps)
//   bits 31..0   arrivals in the current generation
// A member publishes its partials with device-scope stores and waits for them
// to complete, then arrives with ONE device-scope fetch-add that also returns
// the generation it arrived in.  The member that sees arrivals == members-1 is
// last: it adds 2^32 - members, which advances the generation and returns the
// count to 0 in a single atomic.  Every other member polls the word until the
// generation moves, then reads the partials with device-scope loads.
//
// Device-scope (sc1) accesses are performed at the device's coherence point,
// so no L2 write-back or invalidate fence is needed on either side; measured
// on MI355X a join costs ~5 us this way against 12-28 us with agent-scope
// release/acquire fences.  Preconditions: arrivals == 0 when the first member
// arrives (a zero-filled workspace, and every completed join leaves it so);
// all members resident at once.

// Wait until every store this wave issued has completed at its scope.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev4(float4* p, float4 v) {
  float* f = reinterpret_cast<float*>(p);
  st_dev(f + 0, v.x);
  st_dev(f + 1, v.y);
  st_dev(f + 2, v.z);
  st_dev(f + 3, v.w);
}
__device__ __forceinline__ float4 ld_dev4(const float4* p) {
  const float* f = reinterpret_cast<const float*>(p);
  return make_float4(ld_dev(f + 0), ld_dev(f + 1), ld_dev(f + 2), ld_dev(f + 3));
}

// 8-byte pairs as one device-scope access.
__device__ __forceinline__ void st_dev2(float2* p, float2 v) {
  const uint64_t b = (uint64_t)__float_as_uint(v.x) | ((uint64_t)__float_as_uint(v.y) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ld_dev2(const float2* p) {
  const uint64_t b = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float2*>(p)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32)));
}

// Called by ONE lane after the caller's wave published its partials with
// st_dev*/wait_stores().  Returns false if the spin cap was hit (the error
// word is then set); true once every member has arrived.
__device__ __forceinline__ bool join_arrive_and_wait(uint64_t* j, uint32_t members, uint32_t* err) {
  const uint64_t old = __hip_atomic_fetch_add(j, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t gen0 = (uint32_t)(old >> 32);
  if ((uint32_t)old == members - 1) {
    __hip_atomic_fetch_add(j, (1ull << 32) - members, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
  }
  for (uint32_t it = 0; it < kSpinCap; ++it) {
    const uint64_t w = __hip_atomic_load(j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(w >> 32) != gen0) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return false;
}

// Split form of the join, for a launch join: arrive early (the last arriver
// advances the generation at once), await later with the returned word, so the
// wait overlaps whatever runs between the two.
__device__ __forceinline__ uint64_t join_arrive(uint64_t* j, uint32_t members) {
  const uint64_t old = __hip_atomic_fetch_add(j, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((uint32_t)old == members - 1)
    __hip_atomic_fetch_add(j, (1ull << 32) - members, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return old;
}
__device__ __forceinline__ bool join_await(uint64_t* j, uint64_t old, uint32_t members, uint32_t* err) {
  const uint32_t gen0 = (uint32_t)(old >> 32);
  if ((uint32_t)old == members - 1) return true;
  for (uint32_t it = 0; it < kSpinCap; ++it) {
    const uint64_t w = __hip_atomic_load(j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(w >> 32) != gen0) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return false;
}

// ------------------------------------------------------------ tagged slots
//
// A 64-bit slot {tag:32 | value:32} written with ONE device-scope store: a
// reader that sees the tag it waits for has the value that came with it, so
// publishing a partial needs no separate arrival, fence or reload.  Tags are
// the 1-based index of the row within the launch; a launch join after every
// member has cleared its own slots makes sure no slot a reader polls still
// holds an earlier launch's word (tag 0 never matches).
__device__ __forceinline__ void slot_put(uint64_t* s, uint32_t tag, float v) {
  __hip_atomic_store(s, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void slot_clear(uint64_t* s) {
  __hip_atomic_store(s, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The slot's value once it carries `tag`; capped spin: on giving up the error
// word is set and 0 returned, so the kernel still finishes.
__device__ __forceinline__ float slot_take(uint64_t* s, uint32_t tag, uint32_t* err) {
  for (uint32_t it = 0; it < kSpinCap; ++it) {
    const uint64_t w = __hip_atomic_load(s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(w >> 32) == tag) return __uint_as_float((uint32_t)w);
    __builtin_amdgcn_s_sleep(1);
  }
  __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return 0.0f;
}

// Two slots taken together: both loads of each poll are in flight at once.
__device__ __forceinline__ void slot_take2(uint64_t* s0, uint64_t* s1, uint32_t tag, uint32_t* err, float* v0,
                                           float* v1) {
  bool h0 = false, h1 = false;
  for (uint32_t it = 0; it < kSpinCap; ++it) {
    const uint64_t w0 = __hip_atomic_load(s0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t w1 = __hip_atomic_load(s1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!h0 && (uint32_t)(w0 >> 32) == tag) {
      *v0 = __uint_as_float((uint32_t)w0);
      h0 = true;
    }
    if (!h1 && (uint32_t)(w1 >> 32) == tag) {
      *v1 = __uint_as_float((uint32_t)w1);
      h1 = true;
    }
    if (h0 && h1) return;
    __builtin_amdgcn_s_sleep(1);
  }
  __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!h0) *v0 = 0.0f;
  if (!h1) *v1 = 0.0f;
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
