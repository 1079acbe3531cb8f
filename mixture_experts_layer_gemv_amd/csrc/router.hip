// Router: fp32 logits, softmax and top-k selection (Grok-1 Admin & Architecture Guide,
// section 3 "Mixture of Experts", steps 1-2; routing and softmax in fp32, section 9).
// The logit order every kernel follows is set out in router_common.h.
//
//   router_partial_kernel  small batches (T <= 64), E = 8: one workgroup per 128-feature group
//                          and 16 tokens writes the group sums, so the router weights are read
//                          by d / 128 workgroups at once; route_finish_kernel (dispatch.hip)
//                          adds them, in moe_forward together with the dispatch.
//   router_topk_kernel     one workgroup of 256 threads per token (any E <= 64).
//   router_topk_multi_kernel  from 1024 tokens, E = 8: one workgroup per 8 tokens, so each
//                          router_w load serves 8 tokens.
// In the last two, thread i holds the runs of features 8 i + 2048 s .. + 7 (s = 0, 1, ...): the
// 16 threads of a wavefront segment hold one group, so each group's butterfly stays inside a
// segment; lane 0 of the segment puts the group sum in LDS and the threads of (token, expert)
// add the groups of each pass in group order.
//
// kNorm (the decoder layer's MoE block, Guide section 3 "Transformer stack": RMSNorm before the
// MoE block): x is the layer input h, and the router and the experts (through x_norm) see
// x = bf16(h * (1 / sqrt(mean(h^2) + eps)) * norm_pre). The sum of squares: per run of 8
// features an fma chain from 0, the thread's runs added in order, a butterfly over each
// wavefront, the 4 wavefronts in index order.
#include "kernels.h"
#include "router_common.h"

namespace moe {

namespace {
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kPass = kThreads * 8;  // features per pass of a workgroup (16 groups)
constexpr int kTPW = 8;                 // tokens per workgroup of the large-batch kernel
constexpr int kRouterMultiMinT = 1024;  // batches from this size take it (E == 8)
}  // namespace

// Sum over the workgroup of one value per thread, in a fixed order (butterfly in each
// wavefront, then the wavefronts in index order); every thread gets the result.
__device__ __forceinline__ float block_sum(float v, float* s_red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  float r = s_red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r += s_red[w];
  __syncthreads();
  return r;
}

__device__ __forceinline__ float sum_squares8(const u32x4& hv) {
  const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w};
  float ss = 0.0f;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const float v = bf16_feature(hw, r);
    ss = __builtin_fmaf(v, v, ss);
  }
  return ss;
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float v) {
  uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// 8 bf16 features of h times rnorm times their 8 norm weights, rounded to bf16 (RNE)
__device__ __forceinline__ u32x4 normalize8(const u32x4& hv, float rnorm, const f32x4& n0, const f32x4& n1) {
  const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w};
  const float ns[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float v0 = __uint_as_float(hw[q] << 16), v1 = __uint_as_float(hw[q] & 0xFFFF0000u);
    o[q] = bf16_rne_bits(v0 * rnorm * ns[2 * q]) | (bf16_rne_bits(v1 * rnorm * ns[2 * q + 1]) << 16);
  }
  return u32x4{o[0], o[1], o[2], o[3]};
}

// ------------------------------------------------------------------------------------
// grid (d / 128, ceil(T / 16)), block 256: segment s (16 lanes) takes token 16 blockIdx.y + s,
// lane b the run of features 128 g + 8 b .. + 7 of group g = blockIdx.x.
// partial[t][g][e] = group g's sum for token t (fp32, [T][d / 128][8]).
__global__ __launch_bounds__(kThreads) void router_partial_kernel(const uint16_t* __restrict__ x,
                                                                  const float* __restrict__ router_w,
                                                                  float* __restrict__ partial, int T, int d) {
  const int g = blockIdx.x, G = gridDim.x;
  const int seg = threadIdx.x >> 4, b = threadIdx.x & 15;
  const int t = blockIdx.y * 16 + seg;
  const int i0 = kRouterGroup * g + 8 * b;
  f32x4 w[16];
  load_rows8(router_w, i0, w);
  const u32x4 xv = *reinterpret_cast<const u32x4*>(x + (size_t)min(t, T - 1) * d + i0);
  float S[8];
  run_sums8(xv, w, S);
#pragma unroll
  for (int e = 0; e < 8; ++e) S[e] = group_sum16(S[e]);
  if (b == 0 && t < T) {
    f32x4* dst = reinterpret_cast<f32x4*>(partial + ((size_t)t * G + g) * 8);
    dst[0] = f32x4{S[0], S[1], S[2], S[3]};
    dst[1] = f32x4{S[4], S[5], S[6], S[7]};
  }
}

// ------------------------------------------------------------------------------------
// One workgroup per token.
template <int EMAX, bool kNorm>
__global__ __launch_bounds__(kThreads) void router_topk_kernel(const uint16_t* __restrict__ x,
                                                               const float* __restrict__ router_w,
                                                               const float* __restrict__ router_bias,
                                                               const uint8_t* __restrict__ pad_mask,
                                                               int32_t* __restrict__ topk_ids,
                                                               float* __restrict__ topk_w, int d, int E,
                                                               int k, const float* __restrict__ norm_pre,
                                                               float eps, uint16_t* __restrict__ x_norm) {
  __shared__ float s_red[kWaves];
  __shared__ float s_grp[2][16][EMAX];
  __shared__ float s_logit[EMAX];
  const int t = blockIdx.x, tid = threadIdx.x, seg = tid >> 4, b = tid & 15;
  const uint16_t* xt = x + (size_t)t * d;
  const int G = d / kRouterGroup, passes = (G + 15) / 16;

  float logit = 0.0f;  // thread e < E: expert e's running sum over the groups
  // this thread's run sums of pass s into the group sums, added in group order
  auto add_groups = [&](int s, float (&S)[EMAX]) {
    const bool live = 16 * s + seg < G;
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      if (e < E) {
        const float v = group_sum16(S[e]);
        if (b == 0 && live) s_grp[s & 1][seg][e] = v;
      }
    __syncthreads();
    if (tid < E)
      for (int q = 0; q < 16 && 16 * s + q < G; ++q) logit += s_grp[s & 1][q][tid];
  };

  // Up to 3 passes (d <= 6144), E == 8: every pass's loads go out before the first FMA (one
  // memory round trip instead of one per pass).
  constexpr int kPrefetch = 3;
  const bool prefetched = EMAX == 8 && E == 8 && d <= kPrefetch * kPass;
  float rnorm = 1.0f;
  if (prefetched) {
    u32x4 xv[kPrefetch];
    f32x4 w[kPrefetch][16];
    f32x4 np[kPrefetch][2];
#pragma unroll
    for (int s = 0; s < kPrefetch; ++s) {
      const int i0 = tid * 8 + s * kPass;
      if (i0 < d) {
        xv[s] = *reinterpret_cast<const u32x4*>(xt + i0);
        load_rows8(router_w, i0, w[s]);
        if constexpr (kNorm) {
          np[s][0] = *reinterpret_cast<const f32x4*>(norm_pre + i0);
          np[s][1] = *reinterpret_cast<const f32x4*>(norm_pre + i0 + 4);
        }
      }
    }
    if constexpr (kNorm) {
      float ss = 0.0f;
#pragma unroll
      for (int s = 0; s < kPrefetch; ++s)
        if (tid * 8 + s * kPass < d) ss += sum_squares8(xv[s]);
      rnorm = 1.0f / sqrtf(block_sum(ss, s_red) / (float)d + eps);
#pragma unroll
      for (int s = 0; s < kPrefetch; ++s) {
        const int i0 = tid * 8 + s * kPass;
        if (i0 < d) {
          xv[s] = normalize8(xv[s], rnorm, np[s][0], np[s][1]);
          *reinterpret_cast<u32x4*>(x_norm + (size_t)t * d + i0) = xv[s];
        }
      }
    }
#pragma unroll
    for (int s = 0; s < kPrefetch; ++s) {
      if (s < passes) {
        float S[EMAX];
        if (tid * 8 + s * kPass < d) {
          run_sums8(xv[s], w[s], reinterpret_cast<float(&)[8]>(S));
        } else {
#pragma unroll
          for (int e = 0; e < EMAX; ++e) S[e] = 0.0f;
        }
        add_groups(s, S);
      }
    }
  } else {
    if constexpr (kNorm) {
      float ss = 0.0f;
      for (int i0 = tid * 8; i0 < d; i0 += kPass) ss += sum_squares8(*reinterpret_cast<const u32x4*>(xt + i0));
      rnorm = 1.0f / sqrtf(block_sum(ss, s_red) / (float)d + eps);
    }
    for (int s = 0; s < passes; ++s) {
      const int i0 = tid * 8 + s * kPass;
      float S[EMAX];
      if (i0 < d) {
        u32x4 xv = *reinterpret_cast<const u32x4*>(xt + i0);
        if constexpr (kNorm) {
          const f32x4* np4 = reinterpret_cast<const f32x4*>(norm_pre + i0);
          xv = normalize8(xv, rnorm, np4[0], np4[1]);
          *reinterpret_cast<u32x4*>(x_norm + (size_t)t * d + i0) = xv;
        }
        if (EMAX == 8 && E == 8) {
          f32x4 w[16];
          load_rows8(router_w, i0, w);
          run_sums8(xv, w, reinterpret_cast<float(&)[8]>(S));
        } else {
          run_sums<EMAX>(xv, router_w + (size_t)i0 * E, E, S);
        }
      } else {
#pragma unroll
        for (int e = 0; e < EMAX; ++e) S[e] = 0.0f;
      }
      add_groups(s, S);
    }
  }
  if (tid < E) s_logit[tid] = logit;
  __syncthreads();
  if (tid != 0) return;
  float p[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) p[e] = e < E ? s_logit[e] : 0.0f;
  const bool real = pad_mask == nullptr || pad_mask[t] != 0;
  finish_token<EMAX>(p, E, k, router_bias, real, topk_ids + (size_t)t * k, topk_w + (size_t)t * k);
}

// ------------------------------------------------------------------------------------
// Large batches, E == 8: one workgroup per TPW tokens. Thread (j, e) = (tid / 8, tid % 8)
// keeps token j's running logit for expert e; lane j < TPW of wavefront 0 finishes token j.
template <int TPW, bool kNorm>
__global__ __launch_bounds__(kThreads) void router_topk_multi_kernel(const uint16_t* __restrict__ x,
                                                                     const float* __restrict__ router_w,
                                                                     const float* __restrict__ router_bias,
                                                                     const uint8_t* __restrict__ pad_mask,
                                                                     int32_t* __restrict__ topk_ids,
                                                                     float* __restrict__ topk_w, int T, int d,
                                                                     int k, const float* __restrict__ norm_pre,
                                                                     float eps, uint16_t* __restrict__ x_norm) {
  constexpr int E = 8;
  static_assert(TPW * E <= kThreads, "one thread per (token, expert)");
  __shared__ float s_ss[kWaves][TPW];
  __shared__ float s_grp[2][16][TPW * E];
  __shared__ float s_logit[TPW * E];
  const int t0 = blockIdx.x * TPW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, seg = tid >> 4, b = tid & 15;
  const int ntok = min(TPW, T - t0);
  const int G = d / kRouterGroup, passes = (G + 15) / 16;

  float rnorm[TPW];
  if constexpr (kNorm) {
    // per token, the order of block_sum: thread partials, butterfly, wavefronts in order
    float ss[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) ss[j] = 0.0f;
    for (int i0 = tid * 8; i0 < d; i0 += kPass) {
#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        const int t = t0 + min(j, ntok - 1);
        ss[j] += sum_squares8(*reinterpret_cast<const u32x4*>(x + (size_t)t * d + i0));
      }
    }
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      float v = ss[j];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
      if (lane == 0) s_ss[wave][j] = v;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      float r = s_ss[0][j];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) r += s_ss[w][j];
      rnorm[j] = 1.0f / sqrtf(r / (float)d + eps);
    }
  }

  float logit = 0.0f;
  for (int s = 0; s < passes; ++s) {
    const int i0 = tid * 8 + s * kPass;
    const bool live = i0 < d;  // uniform over each 16-lane segment
    f32x4 w[16];
    f32x4 n0, n1;
    if (live) {
      load_rows8(router_w, i0, w);
      if constexpr (kNorm) {
        n0 = *reinterpret_cast<const f32x4*>(norm_pre + i0);
        n1 = *reinterpret_cast<const f32x4*>(norm_pre + i0 + 4);
      }
    }
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      float S[E];
      if (live) {
        const int t = t0 + min(j, ntok - 1);  // past the batch end: a live row, result unused
        u32x4 xv = *reinterpret_cast<const u32x4*>(x + (size_t)t * d + i0);
        if constexpr (kNorm) {
          xv = normalize8(xv, rnorm[j], n0, n1);
          if (j < ntok) *reinterpret_cast<u32x4*>(x_norm + (size_t)t * d + i0) = xv;
        }
        run_sums8(xv, w, S);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) S[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float v = group_sum16(S[e]);
        if (b == 0 && live) s_grp[s & 1][seg][j * E + e] = v;
      }
    }
    __syncthreads();
    if (tid < TPW * E)
      for (int q = 0; q < 16 && 16 * s + q < G; ++q) logit += s_grp[s & 1][q][tid];
  }
  if (tid < TPW * E) s_logit[tid] = logit;
  __syncthreads();
  if (wave != 0 || lane >= ntok) return;
  const int t = t0 + lane;
  float p[E];
#pragma unroll
  for (int e = 0; e < E; ++e) p[e] = s_logit[lane * E + e];
  const bool real = pad_mask == nullptr || pad_mask[t] != 0;
  finish_token<E>(p, E, k, router_bias, real, topk_ids + (size_t)t * k, topk_w + (size_t)t * k);
}

// ------------------------------------------------------------------------------------
// The pre-norm alone, one workgroup per token: x_norm exactly as router_topk_kernel<., true>
// writes it (the same threads, runs and sums of squares). Small batches of the MoE block run
// it before router_partial_kernel.
__global__ __launch_bounds__(kThreads) void rmsnorm_kernel(const uint16_t* __restrict__ h,
                                                           const float* __restrict__ norm_pre, float eps,
                                                           uint16_t* __restrict__ x_norm, int d) {
  __shared__ float s_red[kWaves];
  const int t = blockIdx.x, tid = threadIdx.x;
  const uint16_t* ht = h + (size_t)t * d;
  constexpr int kPrefetch = 3;
  if (d <= kPrefetch * kPass) {
    u32x4 hv[kPrefetch];
    float ss = 0.0f;
#pragma unroll
    for (int s = 0; s < kPrefetch; ++s)
      if (tid * 8 + s * kPass < d) hv[s] = *reinterpret_cast<const u32x4*>(ht + tid * 8 + s * kPass);
#pragma unroll
    for (int s = 0; s < kPrefetch; ++s)
      if (tid * 8 + s * kPass < d) ss += sum_squares8(hv[s]);
    const float rnorm = 1.0f / sqrtf(block_sum(ss, s_red) / (float)d + eps);
#pragma unroll
    for (int s = 0; s < kPrefetch; ++s) {
      const int i0 = tid * 8 + s * kPass;
      if (i0 < d) {
        const f32x4* np4 = reinterpret_cast<const f32x4*>(norm_pre + i0);
        *reinterpret_cast<u32x4*>(x_norm + (size_t)t * d + i0) = normalize8(hv[s], rnorm, np4[0], np4[1]);
      }
    }
    return;
  }
  float ss = 0.0f;
  for (int i0 = tid * 8; i0 < d; i0 += kPass) ss += sum_squares8(*reinterpret_cast<const u32x4*>(ht + i0));
  const float rnorm = 1.0f / sqrtf(block_sum(ss, s_red) / (float)d + eps);
  for (int i0 = tid * 8; i0 < d; i0 += kPass) {
    const f32x4* np4 = reinterpret_cast<const f32x4*>(norm_pre + i0);
    *reinterpret_cast<u32x4*>(x_norm + (size_t)t * d + i0) =
        normalize8(*reinterpret_cast<const u32x4*>(ht + i0), rnorm, np4[0], np4[1]);
  }
}

hipError_t launch_rmsnorm(const uint16_t* h, const float* norm_pre, float eps, uint16_t* x_norm, int T, int d,
                          hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(kThreads), 0, stream, h, norm_pre, eps, x_norm, d);
  return hipGetLastError();
}

size_t router_partial_floats(int T, int d, int E) {
  return (E == 8 && T > 0 && T <= kRouterSplitMaxT) ? (size_t)T * (d / kRouterGroup) * 8 : 0;
}

hipError_t launch_router_partial(const uint16_t* x, const float* router_w, float* partial, int T, int d,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(router_partial_kernel, dim3(d / kRouterGroup, (T + 15) / 16), dim3(kThreads), 0, stream, x,
                     router_w, partial, T, d);
  return hipGetLastError();
}

hipError_t launch_router(const uint16_t* x, const float* router_w, const float* router_bias,
                         const uint8_t* pad_mask, int32_t* topk_ids, float* topk_w, float* partial, int T, int d,
                         int E, int k, hipStream_t stream) {
  if (partial != nullptr && router_partial_floats(T, d, E) > 0) {
    hipError_t err = launch_router_partial(x, router_w, partial, T, d, stream);
    if (err != hipSuccess) return err;
    return launch_route_finish(partial, router_bias, pad_mask, topk_ids, topk_w, nullptr, nullptr, nullptr,
                               nullptr, T, d, E, k, stream);
  }
  if (E == 8 && T >= kRouterMultiMinT) {
    hipLaunchKernelGGL((router_topk_multi_kernel<kTPW, false>), dim3((T + kTPW - 1) / kTPW), dim3(kThreads), 0,
                       stream, x, router_w, router_bias, pad_mask, topk_ids, topk_w, T, d, k,
                       (const float*)nullptr, 0.0f, (uint16_t*)nullptr);
    return hipGetLastError();
  }
  dim3 grid(T), block(kThreads);
  if (E <= 8)
    hipLaunchKernelGGL((router_topk_kernel<8, false>), grid, block, 0, stream, x, router_w, router_bias, pad_mask,
                       topk_ids, topk_w, d, E, k, (const float*)nullptr, 0.0f, (uint16_t*)nullptr);
  else
    hipLaunchKernelGGL((router_topk_kernel<64, false>), grid, block, 0, stream, x, router_w, router_bias,
                       pad_mask, topk_ids, topk_w, d, E, k, (const float*)nullptr, 0.0f, (uint16_t*)nullptr);
  return hipGetLastError();
}

hipError_t launch_prenorm_router(const uint16_t* h, const float* norm_pre, float eps, uint16_t* x_norm,
                                 const float* router_w, const float* router_bias, const uint8_t* pad_mask,
                                 int32_t* topk_ids, float* topk_w, int T, int d, int E, int k,
                                 hipStream_t stream) {
  if (E == 8 && T >= kRouterMultiMinT) {
    hipLaunchKernelGGL((router_topk_multi_kernel<kTPW, true>), dim3((T + kTPW - 1) / kTPW), dim3(kThreads), 0,
                       stream, h, router_w, router_bias, pad_mask, topk_ids, topk_w, T, d, k, norm_pre, eps,
                       x_norm);
    return hipGetLastError();
  }
  dim3 grid(T), block(kThreads);
  if (E <= 8)
    hipLaunchKernelGGL((router_topk_kernel<8, true>), grid, block, 0, stream, h, router_w, router_bias, pad_mask,
                       topk_ids, topk_w, d, E, k, norm_pre, eps, x_norm);
  else
    hipLaunchKernelGGL((router_topk_kernel<64, true>), grid, block, 0, stream, h, router_w, router_bias,
                       pad_mask, topk_ids, topk_w, d, E, k, norm_pre, eps, x_norm);
  return hipGetLastError();
}

}  // namespace moe
