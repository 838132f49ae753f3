// Hand-off of data between the phases of a step.
//
// The phase functions (phases.h, core_mfma.h) take a policy that says how a
// phase publishes what it writes for the next phase and how it waits for what
// it reads:
//   - HandoffNone: every phase runs in its own kernel, so the kernel boundary
//     makes the previous phase's stores visible; stores are plain, no waits.
//   - HandoffFlags: all phases run in one launch (the single-launch step).
//     MI355X's eight L2 caches (one per XCD) are not coherent with each other,
//     so a store that a workgroup on another XCD reads in the same launch is
//     made with device scope (it writes through its L2), and the producer
//     raises its own arrival flag only once those stores are complete.  A
//     consumer issues its first weight loads, then waits for the flags of the
//     producers it reads (one wave polls them with device-scope loads), then
//     reads their data with device-scope loads too: a line it reads may hold
//     data of a producer it did not wait for, which an ordinary load could
//     leave stale in its L2 for a later reader.  (Where a wait covers every
//     producer of the lines read, ordinary loads are safe: the launch starts
//     with clean caches.)
//     Waiting per producer rather than per phase matters: a few dozen flags
//     in one or two cache lines per consumer, instead of every consumer of a
//     phase polling all of the previous phase's flags, cut a measured
//     hand-off from about 4.4 to 1.9 us.
// A flag holds the number of the step (the epoch) that last raised it, so
// flags never need clearing; the last workgroup of a step advances the epoch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mfma_util.h"
#include "mla_gather_decode.h"

namespace mla {

constexpr int kHandoffSpin = 1 << 20;  // polls before a wait gives up (and reports it)

struct HandoffNone {
  static constexpr bool kWeightsFirst = false;  // keep each phase's own load order
  __device__ __forceinline__ void wait() const {}
  template <class T>
  __device__ __forceinline__ void st(T* p, T v) const { *p = v; }
  __device__ __forceinline__ void st4(float* p, float4 v) const { *reinterpret_cast<float4*>(p) = v; }
  __device__ __forceinline__ float ld(const float* p) const { return *p; }
  __device__ __forceinline__ float4 ld4(const float* p) const { return *reinterpret_cast<const float4*>(p); }
};

// Device-scope (write-through) stores and loads.
template <class T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float* p, float v) {
  st_dev(reinterpret_cast<uint32_t*>(p), __float_as_uint(v));
}
__device__ __forceinline__ void st_dev(int32_t* p, int32_t v) { st_dev(reinterpret_cast<uint32_t*>(p), (uint32_t)v); }
__device__ __forceinline__ unsigned ld_dev(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) { return __uint_as_float(ld_dev(reinterpret_cast<const unsigned*>(p))); }
__device__ __forceinline__ float4 ld_dev4(const float* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float4(__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)), __uint_as_float((uint32_t)b),
                     __uint_as_float((uint32_t)(b >> 32)));
}

// Stores that a later workgroup of the same kernel reads (no waits): the
// o-projection's slab partials, which the last slab of a column tile to
// arrive adds up.
struct HandoffDevStores {
  static constexpr bool kWeightsFirst = false;
  __device__ __forceinline__ void wait() const {}
  template <class T>
  __device__ __forceinline__ void st(T* p, T v) const { st_dev(p, v); }
  __device__ __forceinline__ void st4(float* p, float4 v) const {
    uint64_t* q = reinterpret_cast<uint64_t*>(p);
    st_dev(q, (uint64_t)__float_as_uint(v.x) | ((uint64_t)__float_as_uint(v.y) << 32));
    st_dev(q + 1, (uint64_t)__float_as_uint(v.z) | ((uint64_t)__float_as_uint(v.w) << 32));
  }
  __device__ __forceinline__ float ld(const float* p) const { return *p; }
  __device__ __forceinline__ float4 ld4(const float* p) const { return *reinterpret_cast<const float4*>(p); }
};

// Up to three ranges of arrival flags: flags[lo[r] .. lo[r] + n[r]).
struct FlagSet {
  int lo[3] = {0, 0, 0};
  int n[3] = {0, 0, 0};
  int k = 0;
  __device__ __forceinline__ FlagSet& add(int l, int m) {
    lo[k] = l;
    n[k] = m;
    ++k;
    return *this;
  }
};

// Wait until every flag of `fs` equals e.  Every thread of the workgroup calls
// it; wave 0 polls the flags (concatenated, 1024 at a time: 16 per lane,
// issued together) and moves on once a group is complete.  After kHandoffSpin
// polls it sets MLA_GD_CHECK_WAIT_TIMEOUT in the error word and returns.
__device__ __forceinline__ void wait_flags(const unsigned* flags, const FlagSet& fs, unsigned e, unsigned* err) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int n01 = fs.n[0] + fs.n[1], total = n01 + fs.n[2];
    int g0 = 0;
    for (int it = 0; g0 * 1024 < total; ++it) {
      bool ok = true;
      unsigned v[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int i = g0 * 1024 + lane + 64 * k;
        const int f = i < fs.n[0] ? fs.lo[0] + i : (i < n01 ? fs.lo[1] + i - fs.n[0] : fs.lo[2] + i - n01);
        v[k] = i < total ? ld_dev(flags + f) : e;
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) ok &= (v[k] == e);
      if (__builtin_amdgcn_ballot_w64(!ok) == 0) {
        ++g0;
        continue;
      }
      if (it >= kHandoffSpin) {
        if (lane == 0) atomicOr(err, MLA_GD_CHECK_WAIT_TIMEOUT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

// Raise flag `f` once every thread's stores are complete.
__device__ __forceinline__ void publish_flag(unsigned* f, unsigned e) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  wait_vmcnt<0>();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0) st_dev(f, e);
}

// Policy of the single-launch step: waits for the flags of `fs` to reach
// epoch e; loads what other workgroups of the launch wrote with device scope
// (a waited-for producer may share a cache line with one not waited for).
struct HandoffFlags {
  static constexpr bool kWeightsFirst = true;  // weights out before the wait
  const unsigned* flags;
  unsigned* err;
  unsigned e;
  FlagSet fs;
  __device__ __forceinline__ void wait() const { wait_flags(flags, fs, e, err); }
  __device__ __forceinline__ float ld(const float* p) const { return ld_dev(p); }
  __device__ __forceinline__ float4 ld4(const float* p) const { return ld_dev4(p); }
  template <class T>
  __device__ __forceinline__ void st(T* p, T v) const { st_dev(p, v); }
  __device__ __forceinline__ void st4(float* p, float4 v) const {
    uint64_t* q = reinterpret_cast<uint64_t*>(p);
    st_dev(q, (uint64_t)__float_as_uint(v.x) | ((uint64_t)__float_as_uint(v.y) << 32));
    st_dev(q + 1, (uint64_t)__float_as_uint(v.z) | ((uint64_t)__float_as_uint(v.w) << 32));
  }
};

}  // namespace mla
