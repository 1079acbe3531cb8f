// Combine (Grok-1 Admin & Architecture Guide, section 3, MoE step 4: expert outputs are
// combined with the selection scaled by the routing gate), as a gather:
//   out[t][c] = sum over slots j (in order) of w[t][j] * y_(t,j)[c],
//   y_(t,j)[c] = sum over parts s (in order) of Y[s][pos[t][j]][c],
// fp32, a fixed order per element, so the result is deterministic. Padded tokens (and
// slots with pos < 0) contribute nothing; padded rows are +0.0.
// grid (T, ceil(d / 1024)), block 256: each thread writes 4 adjacent columns.
#include "device_common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ Y, int splits,
                                                      size_t part_stride,
                                                      const int32_t* __restrict__ pos,
                                                      const float* __restrict__ topk_w,
                                                      const uint8_t* __restrict__ pad_mask,
                                                      float* __restrict__ out, int d, int k) {
  const int t = blockIdx.x;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (c >= d) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (pad_mask == nullptr || pad_mask[t] != 0) {
    for (int j = 0; j < k; ++j) {
      const int p = pos[(size_t)t * k + j];
      if (p < 0) continue;
      const float wj = topk_w[(size_t)t * k + j];
      const float* src = Y + (size_t)p * d + c;
      f32x4 y = *reinterpret_cast<const f32x4*>(src);
      for (int s = 1; s < splits; ++s) y += *reinterpret_cast<const f32x4*>(src + (size_t)s * part_stride);
      acc += wj * y;
    }
  }
  *reinterpret_cast<f32x4*>(out + (size_t)t * d + c) = acc;
}

hipError_t launch_combine(const float* Y, int splits, size_t part_stride, const int32_t* pos,
                          const float* topk_w, const uint8_t* pad_mask, float* out, int T, int d,
                          int k, hipStream_t stream) {
  dim3 grid(T, (d + 1023) / 1024);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, stream, Y, splits, part_stride, pos,
                     topk_w, pad_mask, out, d, k);
  return hipGetLastError();
}

}  // namespace moe
