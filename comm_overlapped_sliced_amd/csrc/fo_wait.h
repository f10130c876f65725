// Device-side waits on the emulated arrivals, shared by the kernels of libflashovl. Not part of
// the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fo_internal.h"

namespace fo {

// The wait record of the device: err[0] accumulates what went wrong (1: a wait ran past its
// bound, 2: a copy engine reported a failed transfer) until fo_check reads and clears it;
// err[1] is the number of the last call that failed. A call's waits give up at once only when
// that call itself has already failed (a missing arrival costs one bound, not one per
// workgroup); the calls after it wait as usual.
__device__ __forceinline__ void wait_fail(uint32_t* err, uint32_t kind, uint32_t gen) {
  __hip_atomic_fetch_or(err, kind, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __hip_atomic_fetch_max(err + 1, gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ bool wait_failed(const uint32_t* err, uint32_t gen) {
  return __hip_atomic_load(err + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == gen;
}

// Bounded wait of call `gen` until a signal value has dropped to zero (the copy engine
// decrements it from 1 when its transfer has landed; a negative value reports a failed copy).
__device__ __forceinline__ void wait_signal(const int64_t* v, uint64_t limit, uint32_t* err,
                                            uint32_t gen) {
  const uint64_t t0 = wall_clock64();
  for (;;) {
    const int64_t x = __hip_atomic_load(v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (x <= 0) {
      if (x < 0) wait_fail(err, 2u, gen);
      return;
    }
    if (wait_failed(err, gen)) return;
    if (wall_clock64() - t0 > limit) {
      wait_fail(err, 1u, gen);
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Bounded wait of call `gen` until a device word has reached `gen` (or a wait of the call has
// failed). The word is uncached device memory, so every read sees the latest store from any XCD.
__device__ __forceinline__ void wait_gen(const uint32_t* w, uint32_t gen, uint64_t limit,
                                         uint32_t* err) {
  const uint64_t t0 = wall_clock64();
  while (__hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < gen) {
    if (wait_failed(err, gen)) return;
    if (wall_clock64() - t0 > limit) {
      wait_fail(err, 1u, gen);
      return;
    }
    __builtin_amdgcn_s_sleep(8);
  }
}

// Wait for group `grp` of `slice` to have landed. The signal values live in host memory, and
// hundreds of workgroups polling them slow the copy engines down, so only one workgroup per
// (slice, group) and call polls the signal: the first to get there, elected by raising
// lead[slice][group] to the call's number `gen` (numbers only grow, so nothing is re-armed
// between calls). It then raises ready[slice][group] to gen, which the other workgroups poll in
// device memory. A failed or timed-out wait still raises it (the call's error record is set).
__device__ __forceinline__ void wait_group(const int64_t* const* comp_tab, uint32_t* lead,
                                           uint32_t* ready, uint32_t gen, uint64_t spin_limit,
                                           uint32_t* err, int slice, int grp) {
  const int k = slice * kMaxGroups + grp;
  const uint32_t prev =
      __hip_atomic_fetch_max(lead + k, gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (prev < gen) {
    wait_signal(comp_tab[k], spin_limit, err, gen);
    __hip_atomic_store(ready + k, gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    wait_gen(ready + k, gen, spin_limit, err);
  }
}

// The call's copies wait for its start signal. Workgroup 0, the first one dispatched, stores 0
// into it when the kernel starts (everything enqueued before the kernel is then complete), after
// a system-scope release so that the copy engines see that work's writes.
__device__ __forceinline__ void release_start(int64_t* start) {
  if (start != nullptr && blockIdx.x == 0 && threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");
    __hip_atomic_store(start, (int64_t)0, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

}  // namespace fo
