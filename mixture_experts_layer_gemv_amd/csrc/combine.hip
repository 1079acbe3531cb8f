// Combine (Grok-1 Admin & Architecture Guide, section 3, MoE step 4: expert outputs are
// combined with the selection scaled by the routing gate), as a gather:
//   out[t][c] = sum over slots j (in order) of w[t][j] * y_(t,j)[c],
//   y_(t,j)[c] = sum over parts s (in order) of Y[s][pos[t][j]][c],
// fp32, a fixed order per element, so the result is deterministic. Padded tokens (and
// slots with pos < 0) contribute nothing; padded rows are +0.0.
// grid (T, ceil(d / (4 * block))), block 64 (T <= 160) or 256: each thread writes 4 adjacent
// columns.
#include "combine_common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ Y, int splits,
                                                      const int* __restrict__ splits_dev, size_t part_stride,
                                                      const int32_t* __restrict__ pos,
                                                      const float* __restrict__ topk_w,
                                                      const uint8_t* __restrict__ pad_mask,
                                                      float* __restrict__ out, int d, int k) {
  const int t = blockIdx.x;
  const int c = (blockIdx.y * blockDim.x + threadIdx.x) * 4;
  if (c >= d) return;
  if (splits_dev) splits = *splits_dev;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (pad_mask == nullptr || pad_mask[t] != 0) acc = gather_combine(Y, splits, part_stride, pos, topk_w, t, c, d, k);
  *reinterpret_cast<f32x4*>(out + (size_t)t * d + c) = acc;
}

// Combine followed by the post-norm and the residual add of the decoder layer's MoE block
// (Guide section 3 "Transformer stack": RMSNorm after the MoE block, h += h_dense):
//   m[t] = combine as above, h_out[t] = h[t] + m[t] * (1 / sqrt(mean(m[t]^2) + eps)) * norm_post.
// Padded rows: m = 0, h_out = h.
//
// The sum of m[t]^2 has one fixed order, whichever path computes it: per 1024-column chunk
// (thread i holds columns 4 i .. 4 i + 3 of the chunk), the thread's four squares in column
// order, a butterfly over each wavefront, the 4 wavefronts in index order; then the chunk
// sums in chunk order. Small batches take two launches over (T, chunks) workgroups
// (combine with chunk sums, then norm and residual), so that every CU streams part of the
// expert outputs; large batches take one workgroup per token, which rereads its own row
// from cache instead of from HBM. Both give the same bits.

// chunk sum of the 4 squares held by each thread of the workgroup (256 threads), in the fixed
// order above; s_red has 4 floats. Every thread gets the result; all threads must call.
__device__ __forceinline__ float chunk_sumsq(const f32x4& m, float* s_red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float v = m.x * m.x + m.y * m.y + m.z * m.z + m.w * m.w;
#pragma unroll
  for (int b = 32; b >= 1; b >>= 1) v += __shfl_xor(v, b, 64);
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  return s_red[0] + s_red[1] + s_red[2] + s_red[3];
}

__device__ __forceinline__ f32x4 residual_postnorm(const f32x4& m, float r, const float* __restrict__ norm_post,
                                                   const uint16_t* __restrict__ h, int t, int c, int d) {
  const f32x4 n4 = *reinterpret_cast<const f32x4*>(norm_post + c);
  const uint2 hb = *reinterpret_cast<const uint2*>(h + (size_t)t * d + c);
  f32x4 o;
  o.x = bf16_bits_to_float(hb.x & 0xFFFFu) + m.x * r * n4.x;
  o.y = bf16_bits_to_float(hb.x >> 16) + m.y * r * n4.y;
  o.z = bf16_bits_to_float(hb.y & 0xFFFFu) + m.z * r * n4.z;
  o.w = bf16_bits_to_float(hb.y >> 16) + m.w * r * n4.w;
  return o;
}

// Large batches: one workgroup per token. The first pass writes m into h_out and forms the
// chunk sums (the LDS slot alternates between chunks, so one barrier per chunk suffices); the
// second rescales in place (each thread rereads only its own writes) and adds h.
__global__ __launch_bounds__(256) void combine_postnorm_kernel(
    const float* __restrict__ Y, int splits, const int* __restrict__ splits_dev, size_t part_stride,
    const int32_t* __restrict__ pos,
    const float* __restrict__ topk_w, const uint8_t* __restrict__ pad_mask, const uint16_t* __restrict__ h,
    const float* __restrict__ norm_post, float eps, float* __restrict__ out, int d, int k) {
  __shared__ float s_red[2][4];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (splits_dev) splits = *splits_dev;
  const bool real = pad_mask == nullptr || pad_mask[t] != 0;
  float* row = out + (size_t)t * d;
  const int nchunks = (d + 1023) / 1024;
  float total = 0.0f;
  for (int i = 0; i < nchunks; ++i) {
    const int c = i * 1024 + tid * 4;
    f32x4 m = {0.f, 0.f, 0.f, 0.f};
    if (c < d) {
      if (real) m = gather_combine(Y, splits, part_stride, pos, topk_w, t, c, d, k);
      *reinterpret_cast<f32x4*>(row + c) = m;
    }
    total += chunk_sumsq(m, s_red[i & 1]);
  }
  const float r = 1.0f / sqrtf(total / (float)d + eps);
  for (int c = tid * 4; c < d; c += 1024) {
    const f32x4 m = *reinterpret_cast<const f32x4*>(row + c);  // this thread's own writes
    *reinterpret_cast<f32x4*>(row + c) = residual_postnorm(m, r, norm_post, h, t, c, d);
  }
}

// Small batches, first launch: grid (T, chunks); m of the chunk into h_out, its chunk sum
// into sumsq[t][chunk].
__global__ __launch_bounds__(256) void combine_sumsq_kernel(const float* __restrict__ Y, int splits,
                                                            const int* __restrict__ splits_dev, size_t part_stride,
                                                            const int32_t* __restrict__ pos,
                                                            const float* __restrict__ topk_w,
                                                            const uint8_t* __restrict__ pad_mask,
                                                            float* __restrict__ out, float* __restrict__ sumsq,
                                                            int d, int k) {
  __shared__ float s_red[4];
  const int t = blockIdx.x, i = blockIdx.y;
  if (splits_dev) splits = *splits_dev;
  const int c = i * 1024 + threadIdx.x * 4;
  f32x4 m = {0.f, 0.f, 0.f, 0.f};
  if (c < d) {
    if (pad_mask == nullptr || pad_mask[t] != 0) m = gather_combine(Y, splits, part_stride, pos, topk_w, t, c, d, k);
    *reinterpret_cast<f32x4*>(out + (size_t)t * d + c) = m;
  }
  const float v = chunk_sumsq(m, s_red);
  if (threadIdx.x == 0) sumsq[(size_t)t * gridDim.y + i] = v;
}

// Small batches, second launch: grid (T, chunks); the token's chunk sums in chunk order, then
// h_out = h + m * r * norm_post for the chunk.
__global__ __launch_bounds__(256) void postnorm_residual_kernel(const float* __restrict__ sumsq,
                                                                const uint16_t* __restrict__ h,
                                                                const float* __restrict__ norm_post, float eps,
                                                                float* __restrict__ out, int d) {
  const int t = blockIdx.x, nchunks = gridDim.y;
  const int c = blockIdx.y * 1024 + threadIdx.x * 4;
  if (c >= d) return;
  float total = 0.0f;
  for (int i = 0; i < nchunks; ++i) total += sumsq[(size_t)t * nchunks + i];
  const float r = 1.0f / sqrtf(total / (float)d + eps);
  float* p = out + (size_t)t * d + c;
  *reinterpret_cast<f32x4*>(p) = residual_postnorm(*reinterpret_cast<const f32x4*>(p), r, norm_post, h, t, c, d);
}

int combine_postnorm_scratch_floats(int T, int d) {
  return T < kCombineRowMinT ? T * ((d + 1023) / 1024) : 0;
}

hipError_t launch_combine_postnorm(const float* Y, int splits, const int* splits_dev, size_t part_stride,
                                   const int32_t* pos,
                                   const float* topk_w, const uint8_t* pad_mask, const uint16_t* h,
                                   const float* norm_post, float eps, float* out, float* sumsq, int T, int d,
                                   int k, hipStream_t stream) {
  if (T < kCombineRowMinT && sumsq != nullptr) {
    const dim3 grid(T, (d + 1023) / 1024);
    hipLaunchKernelGGL(combine_sumsq_kernel, grid, dim3(256), 0, stream, Y, splits, splits_dev, part_stride, pos,
                       topk_w, pad_mask, out, sumsq, d, k);
    hipLaunchKernelGGL(postnorm_residual_kernel, grid, dim3(256), 0, stream, sumsq, h, norm_post, eps, out, d);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(combine_postnorm_kernel, dim3(T), dim3(256), 0, stream, Y, splits, splits_dev, part_stride,
                     pos, topk_w, pad_mask, h, norm_post, eps, out, d, k);
  return hipGetLastError();
}

hipError_t launch_combine(const float* Y, int splits, const int* splits_dev, size_t part_stride,
                          const int32_t* pos, const float* topk_w, const uint8_t* pad_mask, float* out,
                          int T, int d, int k, hipStream_t stream) {
  // small batches: 256 columns per workgroup, so that more CUs share the gather
  const int threads = T <= kDecodeMaxT ? 64 : 256;
  dim3 grid(T, (d + 4 * threads - 1) / (4 * threads));
  hipLaunchKernelGGL(combine_kernel, grid, dim3(threads), 0, stream, Y, splits, splits_dev, part_stride, pos,
                     topk_w, pad_mask, out, d, k);
  return hipGetLastError();
}

}  // namespace moe
