// residency.h -- how a grid launched plainly settles whether all of its
// workgroups run at once.  Used by the two persistent step kernels, whose
// workgroups wait on one another; each kernel has its own fallback for when
// they do not (the workgroups that arrived take the place of the others in
// turn, through the same arithmetic).  HIP's cooperative launch guarantees
// co-residency but costs about 18 us per launch on this runtime; a plain
// launch (after a host check that the grid fits the device) plus this
// decision gives the same guarantee: GO only when every workgroup has taken
// its ticket, i.e. is running.  Internal.
#pragma once

#include "cells.h"

namespace rnnhip {

// Residency decision, taken by thread 0 of every workgroup.  coop[0] counts
// arrivals, coop[1] holds the decision: 1 (GO: every workgroup is running)
// or 2 | count << 8 (ABORT: the workgroups with tickets below count run the
// kernel's fallback).  Both are zeroed by the state setup that precedes the kernel on
// the stream.  `forced` > 0 makes the first arrival record ABORT with that
// count at once (tests of the fallback).
// A workgroup waits this long for the others before it records ABORT: a
// healthy grid arrives within a few microseconds, but the first launch in a
// process has been seen to take longer, and a needless fallback costs far
// more than the wait.
constexpr unsigned long long kArrivalWindow = 100000;  // ticks of the 100 MHz real-time counter: 1 ms

// Split in two so that a workgroup can do its own set-up (say, load its rows
// of R) between taking its ticket and waiting for the decision: the last
// workgroup to arrive records GO itself.
__device__ __forceinline__ int arrive_ticket(int* coop) {
  return __hip_atomic_fetch_add(&coop[0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline int arrive_decide(int* coop, int n_groups, int forced, int ticket) {
  int want = 0;
  if (forced > 0) {
    if (ticket == 0) want = 2 | (min(forced, n_groups) << 8);
  } else if (ticket == n_groups - 1) {
    want = 1;
  }
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    if (want != 0) {
      int expect = 0;
      __hip_atomic_compare_exchange_strong(&coop[1], &expect, want, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      want = 0;
    }
    const int dec = __hip_atomic_load(&coop[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (dec != 0) return dec;
    if (__builtin_amdgcn_s_memrealtime() - t0 > kArrivalWindow)
      want = 2 | (__hip_atomic_load(&coop[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) << 8);
    else
      __builtin_amdgcn_s_sleep(2);
  }
}

}  // namespace rnnhip
