// Arithmetic shared by the router kernels (Grok-1 Admin & Architecture Guide, section 3
// "Mixture of Experts", steps 1-2; fp32 routing, section 9). Every kernel forms a token's
// logits in one fixed order, so a token gets the same bits whichever kernel, batch size or
// launch routes it:
//   - the features are cut into groups of 128 (d is a multiple of 256) and each group into
//     16 runs of 8 adjacent features;
//   - a run's sum S[e] is a chain of fused multiply-adds over its 8 features in order,
//     starting from 0;
//   - a group's sum is a butterfly over its 16 runs (xor 8, 4, 2, 1 across the 16 lanes that
//     hold them; the xor pairing makes every lane add the same two values);
//   - the logit is the group sums added in group order, starting from 0.
// finish_token then adds the bias and takes the softmax and the top k.
#pragma once

#include "device_common.h"

namespace moe {

constexpr int kRouterGroup = 128;  // features per group

__device__ __forceinline__ float bf16_feature(const uint32_t (&xw)[4], int r) {
  return __uint_as_float((r & 1) ? (xw[r >> 1] & 0xFFFF0000u) : (xw[r >> 1] << 16));
}

// E == 8: the 8 router_w rows (8 floats each) of the run starting at feature i0.
__device__ __forceinline__ void load_rows8(const float* __restrict__ router_w, int i0, f32x4 (&w)[16]) {
  const f32x4* rw = reinterpret_cast<const f32x4*>(router_w + (size_t)i0 * 8);
#pragma unroll
  for (int q = 0; q < 16; ++q) w[q] = rw[q];
}

// E == 8: S[e] over one run; xv holds its 8 bf16 features, w its 8 router_w rows (16 f32x4,
// row r = w[2 r], w[2 r + 1]).
__device__ __forceinline__ void run_sums8(const u32x4& xv, const f32x4 (&w)[16], float (&S)[8]) {
  const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) S[e] = 0.0f;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const float xf = bf16_feature(xw, r);
    const f32x4 lo = w[2 * r], hi = w[2 * r + 1];
    S[0] = __builtin_fmaf(xf, lo.x, S[0]), S[1] = __builtin_fmaf(xf, lo.y, S[1]);
    S[2] = __builtin_fmaf(xf, lo.z, S[2]), S[3] = __builtin_fmaf(xf, lo.w, S[3]);
    S[4] = __builtin_fmaf(xf, hi.x, S[4]), S[5] = __builtin_fmaf(xf, hi.y, S[5]);
    S[6] = __builtin_fmaf(xf, hi.z, S[6]), S[7] = __builtin_fmaf(xf, hi.w, S[7]);
  }
}

// Any E <= EMAX: the same chain with router_w rows of E floats (rows = the run's first row).
template <int EMAX>
__device__ __forceinline__ void run_sums(const u32x4& xv, const float* __restrict__ rows, int E, float (&S)[EMAX]) {
  const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
  for (int e = 0; e < EMAX; ++e) S[e] = 0.0f;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const float xf = bf16_feature(xw, r);
    const float* row = rows + (size_t)r * E;
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      if (e < E) S[e] = __builtin_fmaf(xf, row[e], S[e]);
  }
}

// Group sum: butterfly over the 16 lanes of a segment (lanes 16 s .. 16 s + 15 of a
// wavefront). Every lane of the wavefront must call it.
__device__ __forceinline__ float group_sum16(float v) {
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// p: the token's E logits. Adds the bias, takes the softmax (max-subtracted, denominator
// summed in expert order) and writes the k largest probabilities, ties to the lower index
// (k rounds of "largest not yet taken", strict >). Padded tokens: ids -1, weights 0.
// Returns the experts taken as a bit mask (0 for a padded token); for E <= 8, *slots gets the
// slot of each taken expert e in bits 4 e .. 4 e + 3.
template <int EMAX>
__device__ __forceinline__ uint64_t finish_token(float (&p)[EMAX], int E, int k, const float* __restrict__ bias,
                                                 bool real, int32_t* __restrict__ ids_t, float* __restrict__ w_t,
                                                 uint32_t* slots = nullptr) {
  if (!real) {
    for (int j = 0; j < k; ++j) ids_t[j] = -1, w_t[j] = 0.0f;
    return 0;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < EMAX; ++e)
    if (e < E) {
      if (bias) p[e] += bias[e];
      mx = fmaxf(mx, p[e]);
    }
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < EMAX; ++e)
    if (e < E) {
      p[e] = expf(p[e] - mx);
      s += p[e];
    }
#pragma unroll
  for (int e = 0; e < EMAX; ++e)
    if (e < E) p[e] = p[e] / s;
  uint64_t taken = 0;
  for (int j = 0; j < k; ++j) {
    int best = -1;
    float bp = 0.0f;
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      if (e < E && !((taken >> e) & 1ull) && (best < 0 || p[e] > bp)) {
        best = e;
        bp = p[e];
      }
    taken |= 1ull << best;
    ids_t[j] = best;
    w_t[j] = bp;
    if (slots) *slots |= (uint32_t)j << (4 * best);
  }
  return taken;
}

}  // namespace moe
