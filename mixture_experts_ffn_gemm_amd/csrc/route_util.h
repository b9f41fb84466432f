// route_util.h -- wavefront helpers of the two routing paths (prefill
// routing in router.hip, decode routing in decode.hip).
#pragma once

#include <hip/hip_runtime.h>

namespace moe {

// Rank of this lane's 64-bit key among the wavefront's 64 keys: the number
// of larger ones (keys distinct, or 0 for absent entries, which rank below
// every real key).  Every lane must be active.  The keys pass through the
// wavefront's own 64-entry LDS area kl and come back as broadcast pairs: one
// pass of 64 compares instead of one wavefront maximum per rank.
__device__ __forceinline__ int wave_key_rank(unsigned long long key, unsigned long long* kl, int lane) {
  kl[lane] = key;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int r = 0;
#pragma unroll
  for (int j = 0; j < 64; j += 2) {
    const ulonglong2 two = *reinterpret_cast<const ulonglong2*>(kl + j);
    r += two.x > key ? 1 : 0;
    r += two.y > key ? 1 : 0;
  }
  return r;
}

}  // namespace moe
