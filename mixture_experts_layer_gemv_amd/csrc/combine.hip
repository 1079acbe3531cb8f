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

// Combine followed by the post-norm and the residual add of the decoder layer's MoE block
// (Guide section 3 "Transformer stack": RMSNorm after the MoE block, h += h_dense):
//   m[t] = combine as above, h_out[t] = h[t] + m[t] * (1 / sqrt(mean(m[t]^2) + eps)) * norm_post.
// One workgroup of 256 threads per token: the first pass writes m into h_out and sums
// m^2 (fixed order), the second rescales in place and adds h. Padded rows: m = 0, h_out = h.
__global__ __launch_bounds__(256) void combine_postnorm_kernel(
    const float* __restrict__ Y, int splits, size_t part_stride, const int32_t* __restrict__ pos,
    const float* __restrict__ topk_w, const uint8_t* __restrict__ pad_mask, const uint16_t* __restrict__ h,
    const float* __restrict__ norm_post, float eps, float* __restrict__ out, int d, int k) {
  __shared__ float s_red[4];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool real = pad_mask == nullptr || pad_mask[t] != 0;
  float* row = out + (size_t)t * d;
  float ss = 0.0f;
  for (int c = tid * 4; c < d; c += 1024) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (real) {
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
    ss += acc.x * acc.x + acc.y * acc.y + acc.z * acc.z + acc.w * acc.w;
    *reinterpret_cast<f32x4*>(row + c) = acc;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  if (lane == 0) s_red[wave] = ss;
  __syncthreads();
  const float total = s_red[0] + s_red[1] + s_red[2] + s_red[3];
  const float r = 1.0f / sqrtf(total / (float)d + eps);
  for (int c = tid * 4; c < d; c += 1024) {
    const f32x4 m4 = *reinterpret_cast<const f32x4*>(row + c);  // this thread's own writes
    const f32x4 n4 = *reinterpret_cast<const f32x4*>(norm_post + c);
    const uint2 hb = *reinterpret_cast<const uint2*>(h + (size_t)t * d + c);
    f32x4 o;
    o.x = bf16_bits_to_float(hb.x & 0xFFFFu) + m4.x * r * n4.x;
    o.y = bf16_bits_to_float(hb.x >> 16) + m4.y * r * n4.y;
    o.z = bf16_bits_to_float(hb.y & 0xFFFFu) + m4.z * r * n4.z;
    o.w = bf16_bits_to_float(hb.y >> 16) + m4.w * r * n4.w;
    *reinterpret_cast<f32x4*>(row + c) = o;
  }
}

hipError_t launch_combine_postnorm(const float* Y, int splits, size_t part_stride, const int32_t* pos,
                                   const float* topk_w, const uint8_t* pad_mask, const uint16_t* h,
                                   const float* norm_post, float eps, float* out, int T, int d, int k,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(combine_postnorm_kernel, dim3(T), dim3(256), 0, stream, Y, splits, part_stride, pos, topk_w,
                     pad_mask, h, norm_post, eps, out, d, k);
  return hipGetLastError();
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
