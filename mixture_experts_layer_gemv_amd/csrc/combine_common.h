// The combine of one token's columns (Grok-1 Admin & Architecture Guide, section 3, MoE step 4:
// the expert outputs weighted by the routing gate), shared by the combine kernels and the
// one-launch layer so that every path adds in the same order:
//   out[t][c .. c + 3] = sum over slots j (in order) of w[t][j] * y_(t,j),
//   y_(t,j) = sum over parts s (in order) of Y[s][pos[t][j]][c .. c + 3];
// slots with pos < 0 contribute nothing.
#pragma once

#include "device_common.h"

namespace moe {

__device__ __forceinline__ f32x4 gather_combine(const float* __restrict__ Y, int splits, size_t part_stride,
                                                const int32_t* __restrict__ pos,
                                                const float* __restrict__ topk_w, int t, int c, int d, int k) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int p = pos[(size_t)t * k + j];
    if (p < 0) continue;
    const float wj = topk_w[(size_t)t * k + j];
    const float* src = Y + (size_t)p * d + c;
    f32x4 y = *reinterpret_cast<const f32x4*>(src);
    for (int s = 1; s < splits; ++s) y += *reinterpret_cast<const f32x4*>(src + (size_t)s * part_stride);
    acc += wj * y;
  }
  return acc;
}

}  // namespace moe
