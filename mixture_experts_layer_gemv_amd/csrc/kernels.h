// Host-side launchers of the MoE layer's gfx950 kernels (internal to libmoe).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// T at or below which the expert FFN takes the weight-streaming (decode) kernels: they read
// each touched expert's weights once per pass of up to 16 (T <= 16), 32 (T <= 64) or 48 rows.
constexpr int kDecodeMaxT = 160;

// T at or below which routing with E == 8 can run in two launches: router_partial_kernel
// (group sums, fp32 [T][d / 128][8]) and route_finish_kernel (sums, softmax, top-k, and
// optionally the dispatch).
constexpr int kRouterSplitMaxT = 64;
// floats of the group-sum scratch for (T, d, E); 0 where the two-launch routing does not apply
size_t router_partial_floats(int T, int d, int E);
hipError_t launch_router_partial(const uint16_t* x, const float* router_w, float* partial, int T, int d,
                                 hipStream_t stream);
// counts == NULL: routing only; otherwise the dispatch follows in the same launch
// (counts, offsets, perm and pos as for launch_dispatch).
hipError_t launch_route_finish(const float* partial, const float* router_bias, const uint8_t* pad_mask,
                               int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                               int32_t* pos, int T, int d, int E, int k, hipStream_t stream);
// partial NULL (or a batch the two-launch routing does not take): one launch
hipError_t launch_router(const uint16_t* x, const float* router_w, const float* router_bias,
                         const uint8_t* pad_mask, int32_t* topk_ids, float* topk_w, float* partial, int T,
                         int d, int E, int k, hipStream_t stream);

// x_norm = bf16(h * rnorm * norm_pre), bit-identical to what launch_prenorm_router writes
hipError_t launch_rmsnorm(const uint16_t* h, const float* norm_pre, float eps, uint16_t* x_norm, int T, int d,
                          hipStream_t stream);

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

// The whole layer in one launch for small batches (routing, dispatch, gate/up, down and
// combine as work items of one kernel; same bits as the launch-per-stage sequence). It
// applies where layer_decode_fits says so. ctl: kLayerCtlWords int32 of device memory that
// must be zero at launch and is zero again when the kernel ends (launch_layer_ctl_clear
// zeroes one); rp, P and Y as for launch_router_partial, launch_gate_up_decode and
// launch_down_decode with the parts of gate_up_parts / down_splits.
constexpr int kLayerCtlWords = 4096;
bool layer_decode_fits(int T, int d, int f, int E, int k);
hipError_t launch_layer_ctl_clear(int* ctl, hipStream_t stream);
hipError_t launch_layer_decode(const uint16_t* x, const float* router_w, const float* router_bias,
                               const uint8_t* pad_mask, const int8_t* w_gate, const int8_t* w_up,
                               const int8_t* w_down, const uint16_t* scales, float* rp, int32_t* ids,
                               float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos,
                               _Float16* H, float* P, float* Y, float* out, int* ctl, int T, int d, int f, int E,
                               int k, hipStream_t stream);

// Row height (128 or 256) of the tiled kernels' m-tiles for rows_cap = T * k assignments.
int prefill_bm(int rows_cap, int E);

hipError_t launch_gate_up_prefill(const uint16_t* x, const int32_t* perm, const int32_t* offsets,
                                  const int8_t* w_gate, const int8_t* w_up, const uint16_t* scales,
                                  _Float16* H, int rows_cap, int d, int f, int E, hipStream_t stream);

// splits_used NULL: exactly `splits` parts. Otherwise (splits == 2) the kernel keeps one or
// two parts, whichever fills the chip's rounds of workgroups better net of the second
// partial's traffic, and writes the count to *splits_used for launch_combine.
hipError_t launch_down_prefill(const _Float16* H, const int32_t* offsets, const int8_t* w_down,
                               const uint16_t* scales, float* Y, int splits, int rows_cap, int d,
                               int f, int E, int* splits_used, hipStream_t stream);

hipError_t launch_onehot_expand(const int32_t* ids, const float* w, const uint8_t* pad_mask,
                                int32_t* ids_all, float* gates, int T, int E, int k, hipStream_t stream);

// splits_dev non-NULL: the number of partials is read there (written by the down kernel)
hipError_t launch_combine(const float* Y, int splits, const int* splits_dev, size_t part_stride,
                          const int32_t* pos, const float* topk_w, const uint8_t* pad_mask, float* out,
                          int T, int d, int k, hipStream_t stream);

// T at or above which the post-norm combine runs one workgroup per token (one launch);
// below it, two launches over (T, d / 1024) workgroups with sumsq (fp32, T * ceil(d / 1024)
// elements) as scratch. sumsq NULL: one workgroup per token at any T.
constexpr int kCombineRowMinT = 1024;
int combine_postnorm_scratch_floats(int T, int d);
hipError_t launch_combine_postnorm(const float* Y, int splits, const int* splits_dev, size_t part_stride,
                                   const int32_t* pos,
                                   const float* topk_w, const uint8_t* pad_mask, const uint16_t* h,
                                   const float* norm_post, float eps, float* out, float* sumsq, int T, int d,
                                   int k, hipStream_t stream);

}  // namespace moe
