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
#include "dispatch_common.h"
#include "kernels.h"
#include "router_common.h"

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

// The single-workgroup dispatch; every thread of the 1024 must call it.
__device__ __forceinline__ void dispatch_block(const int32_t* __restrict__ ids, const uint8_t* __restrict__ pad_mask,
                                               int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ perm, int32_t* __restrict__ pos, int T,
                                               int E, int k) {
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

__global__ __launch_bounds__(kThreads) void dispatch_kernel(const int32_t* __restrict__ ids,
                                                            const uint8_t* __restrict__ pad_mask,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ perm,
                                                            int32_t* __restrict__ pos, int T, int E,
                                                            int k) {
  if (T <= 64) {
    if (threadIdx.x >= 64) return;
    const int t = threadIdx.x;
    const int32_t* it = ids + (size_t)max(min(t, T - 1), 0) * k;
    uint64_t emask = 0;
    if (t < T && (pad_mask == nullptr || pad_mask[t] != 0))
      for (int j = 0; j < k; ++j)
        if (slot_valid(it, j, E)) emask |= 1ull << it[j];
    auto slot_of = [&](int e) {
      int j = 0;
      while (it[j] != e) ++j;  // e is in emask, so some slot holds it
      return j;
    };
    dispatch_wave(emask, slot_of, T, E, k, counts, offsets, perm, pos);
    return;
  }
  dispatch_block(ids, pad_mask, counts, offsets, perm, pos, T, E, k);
}

// ------------------------------------------------------------------------------------
// Routing of small batches, second half (the first is router_partial_kernel): thread
// (t, e) = (tid / 8, tid % 8) adds token t's group sums for expert e in group order, lane
// t < T of wavefront 0 takes the softmax and the top k (router_common.h); with kDispatch the
// same wavefront then dispatches the experts it holds. E == 8, T <= kRouterSplitMaxT (64).
template <bool kDispatch>
__global__ __launch_bounds__(kThreads) void route_finish_kernel(
    const float* __restrict__ partial, const float* __restrict__ router_bias, const uint8_t* __restrict__ pad_mask,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ pos, int T, int G, int k) {
  constexpr int E = 8;
  __shared__ float s_logit[kRouterSplitMaxT * E];
  const int tid = threadIdx.x;
  if (tid < T * E) {
    const float* src = partial + (size_t)(tid / E) * G * E + (tid % E);
    float logit = 0.0f;
    constexpr int kBatch = 64;  // up to 64 loads in flight, then the adds in group order
    for (int g0 = 0; g0 < G; g0 += kBatch) {
      float v[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q)
        if (g0 + q < G) v[q] = src[(size_t)(g0 + q) * E];
#pragma unroll
      for (int q = 0; q < kBatch; ++q)
        if (g0 + q < G) logit += v[q];
    }
    s_logit[tid] = logit;
  }
  __syncthreads();
  if (tid >= 64) return;  // wavefront 0: lane t finishes token t (T <= 64)
  uint64_t emask = 0;
  uint32_t slots = 0;
  if (tid < T) {
    float p[E];
#pragma unroll
    for (int e = 0; e < E; ++e) p[e] = s_logit[tid * E + e];
    const bool real = pad_mask == nullptr || pad_mask[tid] != 0;
    emask = finish_token<E>(p, E, k, router_bias, real, topk_ids + (size_t)tid * k, topk_w + (size_t)tid * k,
                            &slots);
  }
  if constexpr (kDispatch)
    dispatch_wave(emask, [&](int e) { return (int)((slots >> (4 * e)) & 15u); }, T, E, k, counts, offsets, perm,
                  pos);
}

hipError_t launch_route_finish(const float* partial, const float* router_bias, const uint8_t* pad_mask,
                               int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                               int32_t* pos, int T, int d, int E, int k, hipStream_t stream) {
  if (E != 8 || T <= 0 || T > kRouterSplitMaxT) return hipErrorInvalidValue;
  const int G = d / 128;
  if (counts != nullptr)
    hipLaunchKernelGGL(route_finish_kernel<true>, dim3(1), dim3(kThreads), 0, stream, partial, router_bias,
                       pad_mask, topk_ids, topk_w, counts, offsets, perm, pos, T, G, k);
  else
    hipLaunchKernelGGL(route_finish_kernel<false>, dim3(1), dim3(kThreads), 0, stream, partial, router_bias,
                       pad_mask, topk_ids, topk_w, counts, offsets, perm, pos, T, G, k);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// Large batches: the same counting sort over chunks of 1024 tokens in parallel. chunk
// counts per expert (one workgroup per chunk), then one workgroup scans them into each
// chunk's base position per expert, then each chunk ranks and scatters its tokens as pass 2
// above does with a running base. A token's position is the same in both schemes, so the
// arrays are identical.

__global__ __launch_bounds__(kThreads) void dispatch_count_kernel(const int32_t* __restrict__ ids,
                                                                  const uint8_t* __restrict__ pad_mask,
                                                                  int32_t* __restrict__ chunk_counts, int T,
                                                                  int E, int k) {
  __shared__ int s_count[kMaxE];
  const int tid = threadIdx.x;
  if (tid < kMaxE) s_count[tid] = 0;
  __syncthreads();
  const int t = blockIdx.x * kThreads + tid;
  if (t < T && (pad_mask == nullptr || pad_mask[t] != 0)) {
    const int32_t* it = ids + (size_t)t * k;
    for (int j = 0; j < k; ++j)
      if (slot_valid(it, j, E)) atomicAdd(&s_count[it[j]], 1);
  }
  __syncthreads();
  if (tid < E) chunk_counts[(size_t)blockIdx.x * E + tid] = s_count[tid];
}

// counts, offsets, and chunk_base[c][e] = offsets[e] + sum over earlier chunks of their counts
__global__ __launch_bounds__(kMaxE) void dispatch_scan_kernel(const int32_t* __restrict__ chunk_counts,
                                                              int32_t* __restrict__ chunk_base,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets, int nchunks,
                                                              int E) {
  __shared__ int s_total[kMaxE];
  const int e = threadIdx.x;
  int total = 0;
  if (e < E)
    for (int c = 0; c < nchunks; ++c) total += chunk_counts[(size_t)c * E + e];
  s_total[e] = total;
  __syncthreads();
  if (e < E) {
    int base = 0;
    for (int q = 0; q < e; ++q) base += s_total[q];
    counts[e] = total;
    offsets[e] = base;
    if (e == E - 1) offsets[E] = base + total;
    for (int c = 0; c < nchunks; ++c) {
      chunk_base[(size_t)c * E + e] = base;
      base += chunk_counts[(size_t)c * E + e];
    }
  }
}

__global__ __launch_bounds__(kThreads) void dispatch_scatter_kernel(const int32_t* __restrict__ ids,
                                                                    const uint8_t* __restrict__ pad_mask,
                                                                    const int32_t* __restrict__ chunk_base,
                                                                    int32_t* __restrict__ perm,
                                                                    int32_t* __restrict__ pos, int T, int E,
                                                                    int k) {
  __shared__ int s_wave[kWaves][kMaxE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int t = blockIdx.x * kThreads + tid;
  const bool real = t < T && (pad_mask == nullptr || pad_mask[t] != 0);
  const int32_t* it = ids + (size_t)(t < T ? t : 0) * k;
  uint64_t emask = 0;
  if (real)
    for (int j = 0; j < k; ++j)
      if (slot_valid(it, j, E)) emask |= 1ull << it[j];
  for (int e = 0; e < E; ++e) {
    uint64_t m = __ballot((emask >> e) & 1ull);
    if (lane == 0) s_wave[wave][e] = __popcll(m);
  }
  __syncthreads();
  if (tid < E) {
    int run = chunk_base[(size_t)blockIdx.x * E + tid];
    for (int w = 0; w < kWaves; ++w) {
      int c = s_wave[w][tid];
      s_wave[w][tid] = run;
      run += c;
    }
  }
  __syncthreads();
  if (t < T)
    for (int j = 0; j < k; ++j) pos[(size_t)t * k + j] = -1;
  for (int e = 0; e < E; ++e) {
    const bool has = (emask >> e) & 1ull;
    uint64_t m = __ballot(has);
    if (has) {
      int p = s_wave[wave][e] + __popcll(m & lt_mask);
      perm[p] = t;
      for (int j = 0; j < k; ++j)
        if (it[j] == e) {
          pos[(size_t)t * k + j] = p;
          break;  // later slots with the same id are repeats and stay -1
        }
    }
  }
}

int dispatch_chunks(int T) { return T >= kDispatchChunkedMinT ? (T + kThreads - 1) / kThreads : 0; }

hipError_t launch_dispatch(const int32_t* ids, const uint8_t* pad_mask, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* pos, int T, int E, int k,
                           int32_t* chunk_scratch, hipStream_t stream) {
  const int nchunks = dispatch_chunks(T);
  if (nchunks == 0 || chunk_scratch == nullptr) {
    hipLaunchKernelGGL(dispatch_kernel, dim3(1), dim3(kThreads), 0, stream, ids, pad_mask, counts,
                       offsets, perm, pos, T, E, k);
    return hipGetLastError();
  }
  int32_t* chunk_counts = chunk_scratch;
  int32_t* chunk_base = chunk_scratch + (size_t)nchunks * E;
  hipLaunchKernelGGL(dispatch_count_kernel, dim3(nchunks), dim3(kThreads), 0, stream, ids, pad_mask, chunk_counts,
                     T, E, k);
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(kMaxE), 0, stream, chunk_counts, chunk_base, counts,
                     offsets, nchunks, E);
  hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(nchunks), dim3(kThreads), 0, stream, ids, pad_mask, chunk_base,
                     perm, pos, T, E, k);
  return hipGetLastError();
}

}  // namespace moe
