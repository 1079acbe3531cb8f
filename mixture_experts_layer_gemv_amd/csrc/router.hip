// Router: fp32 logits, softmax and top-k selection (Grok-1 Admin & Architecture Guide,
// section 3 "Mixture of Experts", steps 1-2; routing and softmax in fp32, section 9).
//
// One workgroup of 256 threads per token (small batches; large batches with E = 8 take
// router_topk_multi_kernel, 8 tokens per workgroup, same arithmetic). Thread i takes the 8
// input features 8 i + 2048 s .. + 7 (s = 0, 1, ...): one 16-byte load of x and the 8
// matching rows of router_w (8 E contiguous floats), all issued before use. Partial logits are reduced by
// a butterfly over each wavefront (the xor pairing makes every lane add the same two
// values, so all lanes agree bit for bit) and then over the 4 wavefronts in a fixed order
// through LDS, so the logits are identical run to run. Every lane of wavefront 0 then
// computes the softmax (max-subtracted, denominator summed in expert order) and picks
// the k largest probabilities, ties to the lower index; lane j < k writes slot j.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
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

__device__ __forceinline__ uint32_t bf16_rne_bits(float v) {
  uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// kNorm: x is the layer input h; the router (and the experts, through x_norm) see
// x = bf16(h * (1 / sqrt(mean(h^2) + eps)) * norm_pre), the pre-norm of the decoder layer's
// MoE block (Guide section 3 "Transformer stack": RMSNorm before the MoE block).
template <int EMAX, bool kNorm>
__global__ __launch_bounds__(kThreads) void router_topk_kernel(const uint16_t* __restrict__ x,
                                                               const float* __restrict__ router_w,
                                                               const float* __restrict__ router_bias,
                                                               const uint8_t* __restrict__ pad_mask,
                                                               int32_t* __restrict__ topk_ids,
                                                               float* __restrict__ topk_w, int d, int E,
                                                               int k, const float* __restrict__ norm_pre,
                                                               float eps, uint16_t* __restrict__ x_norm) {
  __shared__ float s_part[kWaves][EMAX];
  __shared__ float s_red[kWaves];
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  float acc[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) acc[e] = 0.0f;

  const uint16_t* xt = x + (size_t)t * d;
  float rnorm = 1.0f;
  if constexpr (kNorm) {
    float ss = 0.0f;
    for (int i0 = tid * 8; i0 < d; i0 += kThreads * 8) {
      u32x4 xv = *reinterpret_cast<const u32x4*>(xt + i0);
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float v = __uint_as_float((r & 1) ? (xw[r >> 1] & 0xFFFF0000u) : (xw[r >> 1] << 16));
        ss += v * v;
      }
    }
    rnorm = 1.0f / sqrtf(block_sum(ss, s_red) / (float)d + eps);
  }
  // acc += the 8 features of x chunk xv against their 8 router_w rows (E == 8)
  auto accumulate8 = [&](const u32x4& xv, const f32x4 (&w)[16]) {
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float xf = __uint_as_float((r & 1) ? (xw[r >> 1] & 0xFFFF0000u) : (xw[r >> 1] << 16));
      const f32x4 lo = w[2 * r], hi = w[2 * r + 1];
      acc[0] += xf * lo.x, acc[1] += xf * lo.y, acc[2] += xf * lo.z, acc[3] += xf * lo.w;
      acc[4] += xf * hi.x, acc[5] += xf * hi.y, acc[6] += xf * hi.z, acc[7] += xf * hi.w;
    }
  };
  // Up to 3 chunks per thread (d <= 6144), E == 8: every chunk's loads go out before the first
  // FMA (one memory round trip instead of one per chunk); the sums keep the chunk order.
  constexpr int kPrefetch = 3;
  const bool prefetched = !kNorm && EMAX == 8 && E == 8 && d <= kPrefetch * kThreads * 8;
  if (prefetched) {
    u32x4 xv[kPrefetch];
    f32x4 w[kPrefetch][16];
#pragma unroll
    for (int s = 0; s < kPrefetch; ++s) {
      const int i0 = tid * 8 + s * kThreads * 8;
      if (i0 < d) {
        xv[s] = *reinterpret_cast<const u32x4*>(xt + i0);
        const f32x4* rw = reinterpret_cast<const f32x4*>(router_w + (size_t)i0 * 8);
#pragma unroll
        for (int q = 0; q < 16; ++q) w[s][q] = rw[q];
      }
    }
#pragma unroll
    for (int s = 0; s < kPrefetch; ++s)
      if (tid * 8 + s * kThreads * 8 < d) accumulate8(xv[s], w[s]);
  }
  for (int i0 = tid * 8; !prefetched && i0 < d; i0 += kThreads * 8) {
    u32x4 xv = *reinterpret_cast<const u32x4*>(xt + i0);
    uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
    if constexpr (kNorm) {
      const f32x4* np4 = reinterpret_cast<const f32x4*>(norm_pre + i0);
      const f32x4 n0 = np4[0], n1 = np4[1];
      const float ns[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float v0 = __uint_as_float(xw[q] << 16), v1 = __uint_as_float(xw[q] & 0xFFFF0000u);
        xw[q] = bf16_rne_bits(v0 * rnorm * ns[2 * q]) | (bf16_rne_bits(v1 * rnorm * ns[2 * q + 1]) << 16);
      }
      u32x4 o = {xw[0], xw[1], xw[2], xw[3]};
      *reinterpret_cast<u32x4*>(x_norm + (size_t)t * d + i0) = o;
    }
    if (EMAX == 8 && E == 8) {
      // 8 rows x 8 experts = 256 contiguous bytes
      const f32x4* rw = reinterpret_cast<const f32x4*>(router_w + (size_t)i0 * 8);
      f32x4 w[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) w[q] = rw[q];
      accumulate8(u32x4{xw[0], xw[1], xw[2], xw[3]}, w);
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float xf = __uint_as_float((r & 1) ? (xw[r >> 1] & 0xFFFF0000u) : (xw[r >> 1] << 16));
        const float* row = router_w + (size_t)(i0 + r) * E;
#pragma unroll
        for (int e = 0; e < EMAX; ++e)
          if (e < E) acc[e] += xf * row[e];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    if (e < E) {
      float v = acc[e];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
      if (lane == 0) s_part[wave][e] = v;
    }
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int e = 0; e < EMAX; ++e)
    if (e < E) {
      float v = s_part[0][e];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) v += s_part[w][e];
      acc[e] = v;
    }

  const bool real = pad_mask == nullptr || pad_mask[t] != 0;
  if (!real) {
    if (lane < k) {
      topk_ids[(size_t)t * k + lane] = -1;
      topk_w[(size_t)t * k + lane] = 0.0f;
    }
    return;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < EMAX; ++e)
    if (e < E) {
      if (router_bias) acc[e] += router_bias[e];
      mx = fmaxf(mx, acc[e]);
    }
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < EMAX; ++e)
    if (e < E) {
      acc[e] = expf(acc[e] - mx);
      s += acc[e];
    }
#pragma unroll
  for (int e = 0; e < EMAX; ++e)
    if (e < E) acc[e] = acc[e] / s;

  // k rounds of "largest not yet taken" (strict >, so the lower index wins ties).
  uint64_t taken = 0;
  for (int j = 0; j < k; ++j) {
    int best = -1;
    float bp = 0.0f;
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      if (e < E && !((taken >> e) & 1ull) && (best < 0 || acc[e] > bp)) {
        best = e;
        bp = acc[e];
      }
    }
    taken |= 1ull << best;
    if (lane == j) {
      topk_ids[(size_t)t * k + j] = best;
      topk_w[(size_t)t * k + j] = bp;
    }
  }
}

// Large batches, E == 8: one workgroup per TPW tokens, so that each router_w load (the 8
// rows x 8 experts of a thread's features) serves TPW tokens instead of one. Each token's
// sums are formed in exactly the order of router_topk_kernel (thread partials over the
// feature chunks in order, butterfly per wavefront, wavefronts in index order), so a token
// gets bit-identical logits whatever kernel and batch size route it. Lane j < TPW of
// wavefront 0 finishes token j.
template <int TPW>
__global__ __launch_bounds__(kThreads) void router_topk_multi_kernel(const uint16_t* __restrict__ x,
                                                                     const float* __restrict__ router_w,
                                                                     const float* __restrict__ router_bias,
                                                                     const uint8_t* __restrict__ pad_mask,
                                                                     int32_t* __restrict__ topk_ids,
                                                                     float* __restrict__ topk_w, int T, int d,
                                                                     int k) {
  constexpr int E = 8;
  __shared__ float s_part[kWaves][TPW][E];
  const int t0 = blockIdx.x * TPW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntok = min(TPW, T - t0);

  float acc[TPW][E];
#pragma unroll
  for (int j = 0; j < TPW; ++j)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[j][e] = 0.0f;

  for (int i0 = tid * 8; i0 < d; i0 += kThreads * 8) {
    const f32x4* rw = reinterpret_cast<const f32x4*>(router_w + (size_t)i0 * 8);
    f32x4 w[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) w[q] = rw[q];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int t = t0 + min(j, ntok - 1);  // past the batch end: a live row, result unused
      const u32x4 xv = *reinterpret_cast<const u32x4*>(x + (size_t)t * d + i0);
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float xf = __uint_as_float((r & 1) ? (xw[r >> 1] & 0xFFFF0000u) : (xw[r >> 1] << 16));
        const f32x4 lo = w[2 * r], hi = w[2 * r + 1];
        acc[j][0] += xf * lo.x, acc[j][1] += xf * lo.y, acc[j][2] += xf * lo.z, acc[j][3] += xf * lo.w;
        acc[j][4] += xf * hi.x, acc[j][5] += xf * hi.y, acc[j][6] += xf * hi.z, acc[j][7] += xf * hi.w;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < TPW; ++j)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float v = acc[j][e];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
      if (lane == 0) s_part[wave][j][e] = v;
    }
  __syncthreads();
  if (wave != 0 || lane >= ntok) return;

  const int t = t0 + lane;
  const bool real = pad_mask == nullptr || pad_mask[t] != 0;
  if (!real) {
    for (int j = 0; j < k; ++j) {
      topk_ids[(size_t)t * k + j] = -1;
      topk_w[(size_t)t * k + j] = 0.0f;
    }
    return;
  }
  float p[E];
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    float v = s_part[0][lane][e];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += s_part[w][lane][e];
    if (router_bias) v += router_bias[e];
    p[e] = v;
    mx = fmaxf(mx, v);
  }
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    p[e] = expf(p[e] - mx);
    s += p[e];
  }
#pragma unroll
  for (int e = 0; e < E; ++e) p[e] = p[e] / s;
  // k rounds of "largest not yet taken" (strict >, so the lower index wins ties)
  uint32_t taken = 0;
  for (int j = 0; j < k; ++j) {
    int best = -1;
    float bp = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (!((taken >> e) & 1u) && (best < 0 || p[e] > bp)) {
        best = e;
        bp = p[e];
      }
    taken |= 1u << best;
    topk_ids[(size_t)t * k + j] = best;
    topk_w[(size_t)t * k + j] = bp;
  }
}

hipError_t launch_router(const uint16_t* x, const float* router_w, const float* router_bias,
                         const uint8_t* pad_mask, int32_t* topk_ids, float* topk_w, int T, int d,
                         int E, int k, hipStream_t stream) {
  constexpr int kTPW = 8;  // tokens per workgroup of the large-batch kernel
  if (E == 8 && T >= 1024) {
    hipLaunchKernelGGL(router_topk_multi_kernel<kTPW>, dim3((T + kTPW - 1) / kTPW), dim3(kThreads), 0, stream, x,
                       router_w, router_bias, pad_mask, topk_ids, topk_w, T, d, k);
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
