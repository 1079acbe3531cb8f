// Host-side launchers of the MoE layer's gfx950 kernels (internal to libmoe).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// T at or below which the expert FFN takes the weight-streaming (decode) kernels.
constexpr int kDecodeMaxT = 64;

hipError_t launch_router(const uint16_t* x, const float* router_w, const float* router_bias,
                         const uint8_t* pad_mask, int32_t* topk_ids, float* topk_w, int T, int d,
                         int E, int k, hipStream_t stream);

hipError_t launch_prenorm_router(const uint16_t* h, const float* norm_pre, float eps, uint16_t* x_norm,
                                 const float* router_w, const float* router_bias, const uint8_t* pad_mask,
                                 int32_t* topk_ids, float* topk_w, int T, int d, int E, int k,
                                 hipStream_t stream);

// T at or above which the dispatch runs over 1024-token chunks in parallel (three launches)
constexpr int kDispatchChunkedMinT = 4096;
// chunks of the parallel dispatch for T (0 below the threshold); its scratch holds
// 2 * chunks * E int32
int dispatch_chunks(int T);
// chunk_scratch NULL: the single-workgroup dispatch at any T
hipError_t launch_dispatch(const int32_t* ids, const uint8_t* pad_mask, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* pos, int T, int E, int k,
                           int32_t* chunk_scratch, hipStream_t stream);

// parts > 1: the contraction over d is split in `parts`; P (fp32, 2 * parts * T * k * f
// elements) holds the partial sums, completed into H by a second launch.
hipError_t launch_gate_up_decode(const uint16_t* x, const int32_t* perm, const int32_t* offsets,
                                 const int8_t* w_gate, const int8_t* w_up, const uint16_t* scales,
                                 _Float16* H, float* P, int parts, int T, int k, int d, int f, int E,
                                 hipStream_t stream);

hipError_t launch_down_decode(const _Float16* H, const int32_t* offsets, const int8_t* w_down,
                              const uint16_t* scales, float* Y, int splits, int rows_cap, int T,
                              int d, int f, int E, hipStream_t stream);

hipError_t launch_gate_up_prefill(const uint16_t* x, const int32_t* perm, const int32_t* offsets,
                                  const int8_t* w_gate, const int8_t* w_up, const uint16_t* scales,
                                  _Float16* H, int rows_cap, int d, int f, int E, hipStream_t stream);

hipError_t launch_down_prefill(const _Float16* H, const int32_t* offsets, const int8_t* w_down,
                               const uint16_t* scales, float* Y, int splits, int rows_cap, int d,
                               int f, int E, hipStream_t stream);

hipError_t launch_onehot_expand(const int32_t* ids, const float* w, const uint8_t* pad_mask,
                                int32_t* ids_all, float* gates, int T, int E, int k, hipStream_t stream);

hipError_t launch_combine(const float* Y, int splits, size_t part_stride, const int32_t* pos,
                          const float* topk_w, const uint8_t* pad_mask, float* out, int T, int d,
                          int k, hipStream_t stream);

hipError_t launch_combine_postnorm(const float* Y, int splits, size_t part_stride, const int32_t* pos,
                                   const float* topk_w, const uint8_t* pad_mask, const uint16_t* h,
                                   const float* norm_post, float eps, float* out, int T, int d, int k,
                                   hipStream_t stream);

}  // namespace moe
