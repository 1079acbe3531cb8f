// The dispatch of one wavefront (Grok-1 Admin & Architecture Guide, section 3, warning under
// the MoE steps: a gather in place of the dense one-hot selection): a stable counting sort of
// at most 64 tokens' expert assignments, shared by the dispatch kernel, the routing kernel of
// small batches and the one-launch layer. Integer work, so the result is bit-exact and
// independent of scheduling.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Batches of at most 64 tokens: the same stable counting sort in one wavefront, lane t = token
// t, without LDS or barriers. emask: the experts of the lane's valid slots; slot_of(e): the
// first slot holding expert e. For each expert in order, a ballot gives its count and each
// token's rank among the earlier tokens; the running sum of the counts is the offset. Lanes
// >= T pass emask 0.
template <typename SlotOf>
__device__ __forceinline__ void dispatch_wave(uint64_t emask, SlotOf slot_of, int T, int E, int k,
                                              int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ perm, int32_t* __restrict__ pos) {
  const int t = threadIdx.x & 63;
  const uint64_t lt_mask = (t == 0) ? 0ull : (~0ull >> (64 - t));
  if (t < T)
    for (int j = 0; j < k; ++j) pos[(size_t)t * k + j] = -1;
  int base = 0;
  for (int e = 0; e < E; ++e) {
    const bool has = (emask >> e) & 1ull;
    const uint64_t m = __ballot(has);
    if (has) {
      const int p = base + __popcll(m & lt_mask);
      perm[p] = t;
      pos[(size_t)t * k + slot_of(e)] = p;
    }
    if (t == 0) counts[e] = __popcll(m), offsets[e] = base;
    base += __popcll(m);
  }
  if (t == 0) offsets[E] = base;
}

}  // namespace moe
