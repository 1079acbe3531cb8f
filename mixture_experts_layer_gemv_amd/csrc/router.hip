// Router: fp32 logits, softmax and top-k selection (Grok-1 Admin & Architecture Guide,
// section 3 "Mixture of Experts", steps 1-2; routing and softmax in fp32, section 9).
//
// One wavefront per token. Lane l accumulates the logits of all E experts over the
// input features i = 8 l + 512 s + r (a 16-byte bf16 load of x and the matching rows of
// router_w per step), then a butterfly reduction over the 64 lanes gives every lane the
// same fp32 logits (the xor-pairing makes each lane add the same two values, so the
// result is identical in all lanes and run to run). Every lane then computes the softmax
// (max-subtracted, denominator summed in expert order) and picks the k largest
// probabilities, ties to the lower index; lane j < k writes slot j.
#include "device_common.h"
#include "kernels.h"

namespace moe {

template <int EMAX>
__global__ __launch_bounds__(256) void router_topk_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ router_w,
                                                          const float* __restrict__ router_bias,
                                                          const uint8_t* __restrict__ pad_mask,
                                                          int32_t* __restrict__ topk_ids,
                                                          float* __restrict__ topk_w, int T, int d,
                                                          int E, int k) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wavefront exits together

  float acc[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) acc[e] = 0.0f;

  const uint16_t* xt = x + (size_t)t * d;
  for (int i0 = lane * 8; i0 < d; i0 += 512) {
    u32x4 xv = *reinterpret_cast<const u32x4*>(xt + i0);
    uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float xf = __uint_as_float((r & 1) ? (xw[r >> 1] & 0xFFFF0000u) : (xw[r >> 1] << 16));
      const float* row = router_w + (size_t)(i0 + r) * E;
#pragma unroll
      for (int e = 0; e < EMAX; ++e)
        if (e < E) acc[e] += xf * row[e];
    }
  }
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    if (e < E) {
      float v = acc[e];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
      acc[e] = v;
    }
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

hipError_t launch_router(const uint16_t* x, const float* router_w, const float* router_bias,
                         const uint8_t* pad_mask, int32_t* topk_ids, float* topk_w, int T, int d,
                         int E, int k, hipStream_t stream) {
  dim3 grid((T + 3) / 4), block(256);
  if (E <= 8)
    hipLaunchKernelGGL(router_topk_kernel<8>, grid, block, 0, stream, x, router_w, router_bias,
                       pad_mask, topk_ids, topk_w, T, d, E, k);
  else
    hipLaunchKernelGGL(router_topk_kernel<64>, grid, block, 0, stream, x, router_w, router_bias,
                       pad_mask, topk_ids, topk_w, T, d, E, k);
  return hipGetLastError();
}

}  // namespace moe
