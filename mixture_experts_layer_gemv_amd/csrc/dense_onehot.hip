// The dense one-hot-gated formulation of the layer, as the sources describe their own
// implementation (Grok-1 Admin & Architecture Guide, section 3, MoE step 4 and the warning
// under it: every expert runs on every token, and the outputs are combined with one-hot
// selection masks scaled by the routing gate). Kept as a baseline next to the gather path.
//
// This kernel turns the top-k routing into that form: for every real token t and every
// expert e, slot e of the token points at expert e and carries the gate
//   gate[t][e] = sum over j of [ids[t][j] == e] * w[t][j]
// (0 for the experts the router did not select). Dispatch, the expert kernels and the
// combine then run unchanged with k = E, so out[t] = sum over e (in order) of
// gate[t][e] * y_e(t).
#include "device_common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void onehot_expand_kernel(const int32_t* __restrict__ ids,
                                                            const float* __restrict__ w,
                                                            const uint8_t* __restrict__ pad_mask,
                                                            int32_t* __restrict__ ids_all,
                                                            float* __restrict__ gates, int T, int E, int k) {
  const long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  if (i >= (long long)T * E) return;
  const int t = (int)(i / E), e = (int)(i % E);
  const bool real = pad_mask == nullptr || pad_mask[t] != 0;
  float g = 0.0f;
  for (int j = 0; j < k; ++j)
    if (ids[(size_t)t * k + j] == e) g += w[(size_t)t * k + j];
  ids_all[i] = real ? e : -1;
  gates[i] = real ? g : 0.0f;
}

hipError_t launch_onehot_expand(const int32_t* ids, const float* w, const uint8_t* pad_mask,
                                int32_t* ids_all, float* gates, int T, int E, int k, hipStream_t stream) {
  const long long n = (long long)T * E;
  hipLaunchKernelGGL(onehot_expand_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, ids, w,
                     pad_mask, ids_all, gates, T, E, k);
  return hipGetLastError();
}

}  // namespace moe
