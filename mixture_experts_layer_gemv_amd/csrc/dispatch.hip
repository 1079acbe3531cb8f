// Dispatch: stable counting sort of the (token, slot) assignments by expert. This is the
// gather that replaces the dense one-hot selection (Grok-1 Admin & Architecture Guide,
// section 3, warning under the MoE steps; section 10, first item). Integer work, so the
// result is bit-exact and independent of scheduling.
//
// One workgroup of 1024 threads (16 wavefronts) handles all T tokens:
//   pass 1  counts[e] by LDS integer atomics (the order of integer adds does not matter),
//           then offsets = exclusive prefix sum;
//   pass 2  tokens in chunks of 1024, one per thread. For each expert e a wavefront ballot
//           of "this token has e" gives each token its rank among the earlier tokens of its
//           wavefront; per-wavefront totals, prefix-summed over the 16 wavefronts, and a
//           running base per expert carried across chunks give the global rank. So the
//           tokens of each expert appear in ascending t, which is the stable order.
// A slot counts only if its id is in [0, E) and differs from the token's earlier slots.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxE = 64;
}  // namespace

__device__ __forceinline__ bool slot_valid(const int32_t* ids_t, int j, int E) {
  int e = ids_t[j];
  if (e < 0 || e >= E) return false;
  for (int q = 0; q < j; ++q)
    if (ids_t[q] == e) return false;
  return true;
}

__global__ __launch_bounds__(kThreads) void dispatch_kernel(const int32_t* __restrict__ ids,
                                                            const uint8_t* __restrict__ pad_mask,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ perm,
                                                            int32_t* __restrict__ pos, int T, int E,
                                                            int k) {
  __shared__ int s_count[kMaxE];
  __shared__ int s_base[kMaxE];
  __shared__ int s_wave[kWaves][kMaxE];
  __shared__ int s_chunk[kMaxE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  if (tid < kMaxE) s_count[tid] = 0;
  __syncthreads();
  for (int t = tid; t < T; t += kThreads) {
    if (pad_mask && pad_mask[t] == 0) continue;
    const int32_t* it = ids + (size_t)t * k;
    for (int j = 0; j < k; ++j)
      if (slot_valid(it, j, E)) atomicAdd(&s_count[it[j]], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      counts[e] = s_count[e];
      offsets[e] = run;
      s_base[e] = run;
      run += s_count[e];
    }
    offsets[E] = run;
  }
  __syncthreads();

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = 0; c0 < T; c0 += kThreads) {
    const int t = c0 + tid;
    const bool real = t < T && (pad_mask == nullptr || pad_mask[t] != 0);
    const int32_t* it = ids + (size_t)(t < T ? t : 0) * k;
    uint64_t emask = 0;  // experts of this token's valid slots (at most one slot each)
    if (real)
      for (int j = 0; j < k; ++j)
        if (slot_valid(it, j, E)) emask |= 1ull << it[j];
    // all lanes run every ballot: the loop bounds are uniform
    for (int e = 0; e < E; ++e) {
      uint64_t m = __ballot((emask >> e) & 1ull);
      if (lane == 0) s_wave[wave][e] = __popcll(m);
    }
    __syncthreads();
    if (tid < E) {
      int run = 0;
      for (int w = 0; w < kWaves; ++w) {
        int c = s_wave[w][tid];
        s_wave[w][tid] = run;
        run += c;
      }
      s_chunk[tid] = run;
    }
    __syncthreads();
    if (t < T)
      for (int j = 0; j < k; ++j) pos[(size_t)t * k + j] = -1;
    for (int e = 0; e < E; ++e) {
      const bool has = (emask >> e) & 1ull;
      uint64_t m = __ballot(has);
      if (has) {
        int p = s_base[e] + s_wave[wave][e] + __popcll(m & lt_mask);
        perm[p] = t;
        for (int j = 0; j < k; ++j)
          if (it[j] == e) {
            pos[(size_t)t * k + j] = p;
            break;  // later slots with the same id are repeats and stay -1
          }
      }
    }
    __syncthreads();
    if (tid < E) s_base[tid] += s_chunk[tid];
    __syncthreads();
  }
}

hipError_t launch_dispatch(const int32_t* ids, const uint8_t* pad_mask, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* pos, int T, int E, int k,
                           hipStream_t stream) {
  hipLaunchKernelGGL(dispatch_kernel, dim3(1), dim3(kThreads), 0, stream, ids, pad_mask, counts,
                     offsets, perm, pos, T, E, k);
  return hipGetLastError();
}

}  // namespace moe
