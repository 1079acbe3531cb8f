// Expert FFN for small batches (T <= 64): the layer streams the int8 weights of the
// experts it touches once from HBM, so these kernels are built for bytes in flight,
// not for reuse. (Grok-1 Admin & Architecture Guide, section 3, MoE step 3: the gated
// GeLU expert gelu(linear(x)) * linear_v(x) -> linear_1; "Quantized weights": int8
// weights dequantised as q * s, one scale per output channel.)
//
// Work split: one wavefront owns a 128-column slab of one matrix of one touched expert
// and runs down the whole contraction (or one of `splits` parts of it for the down
// projection). For gate/up a workgroup holds two wavefronts, one per matrix, on the same
// slab; they meet in LDS for the GeGLU epilogue. Lane l takes the 8 adjacent columns
// n0 + 8 (l % 16) .. + 7 and, per 32-deep step, the rows k0 + 8 (l / 16) .. + 7: eight
// 8-byte loads, so each row segment a wavefront touches is one full 128-byte line. Byte
// j of those eight rows is exactly the B operand of one 16x16x32 MFMA (column j of the
// lane's 8 columns); the matching A operand (8 bf16/fp16 activations of the same
// k-group) is one 16-byte load. The k order inside an MFMA is the same permutation for A
// and B, so it does not change D. The int8 -> bf16 / fp16 conversion is exact (one
// sign-extending byte convert plus half a pack per element); scales are applied in fp32
// after the contraction. Loads run kStages steps ahead of the MFMAs (register ring).
//
// Rows: an expert's segment of the dispatch has M rows (M <= T). A pass covers MT
// 16-row MFMA tiles (MT = 1 when T <= 16, else 2);
// longer segments take further passes over the weights.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int kSlab = 128;   // columns per wavefront
constexpr int kStep = 32;    // contraction rows per MFMA step
constexpr int kStages = 4;   // steps of loads in flight per wavefront
// Cache policy of the weight loads: non-temporal (each weight byte is read once).
constexpr int kWeightLoadPolicy = 2;
// Buffer resource word 3 for raw byte buffers on gfx9-family parts.
constexpr int kBufferFlags = 0x00020000;
}  // namespace

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

template <int J, typename V>
__device__ __forceinline__ V col_operand(const uint32_t (&w)[8][2]) {
  uint32_t s[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) s[r] = w[r][J >> 2];
  if constexpr (__is_same(V, bf16x8))
    return rows_to_bf16<J & 3>(s);
  else
    return rows_to_f16<J & 3>(s);
}

// acc[mt][j] += A rows (tile mt) x column j of the lane's 8, over `steps` 32-deep steps.
// wr: buffer resource of this expert's matrix; voff: byte offset of this lane's first
// weight (row 8 kg, column n0); row r of step s is at voff + (32 s + r) * ld, with the
// uniform part in the scalar offset, so all eight row loads share one address register.
// a[mt]: this lane's first activation of tile mt (row cl of the tile, k 8 kg). Rows past
// the segment end point at a live row: MFMA rows are independent, so their results are
// simply not stored. steps must be a multiple of kStages; the steady-state loop has no
// branches, so the loads of the next kStages - 1 steps stay in flight across the MFMAs.
template <typename Frag, int MT>
__device__ __forceinline__ void stream_slab(__amdgpu_buffer_rsrc_t wr, uint32_t voff, uint32_t ld, int steps,
                                            const uint16_t* const (&a)[MT], f32x4 (&acc)[MT][8]) {
  uint32_t b[kStages][8][2];
  u32x4 av[kStages][MT];
  auto load = [&](int s, int step) {
    const uint32_t base = (uint32_t)step * kStep * ld;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      auto v = __builtin_amdgcn_raw_buffer_load_b64(wr, voff, base + r * ld, kWeightLoadPolicy);
      b[s][r][0] = v[0];
      b[s][r][1] = v[1];
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) av[s][mt] = load16(a[mt] + step * kStep);
  };
  auto compute = [&](int s) {
    Frag af[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) af[mt] = __builtin_bit_cast(Frag, av[s][mt]);
#define MOE_DEC_COL(J)                                                          \
  {                                                                             \
    Frag bfr = col_operand<J, Frag>(b[s]);                                      \
    _Pragma("unroll") for (int mt = 0; mt < MT; ++mt)                           \
        acc[mt][J] = Mfma<Frag>::run(af[mt], bfr, acc[mt][J]);                  \
  }
    MOE_DEC_COL(0) MOE_DEC_COL(1) MOE_DEC_COL(2) MOE_DEC_COL(3)
    MOE_DEC_COL(4) MOE_DEC_COL(5) MOE_DEC_COL(6) MOE_DEC_COL(7)
#undef MOE_DEC_COL
  };

#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) load(s, s);
  int st = 0;
  for (; st < steps - kStages; st += kStages) {
#pragma unroll
    for (int s = 0; s < kStages; ++s) {
      load((s + kStages - 1) % kStages, st + s + kStages - 1);
      compute(s);
    }
  }
  load(kStages - 1, st + kStages - 1);  // the last step
#pragma unroll
  for (int s = 0; s < kStages; ++s) compute(s);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t weight_rsrc(const int8_t* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(base), (short)0, (int)bytes, kBufferFlags);
}

__device__ __forceinline__ void load_scales8(const uint16_t* p, float (&s)[8]) {
  u32x4 v = load16(p);
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) s[j] = bf16_bits_to_float((w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
}

// ------------------------------------------------------------------------------------
// gate/up + GeGLU: H[row0 + m][n] = fp16(gelu_tanh(s_g[n] * G[m][n]) * (s_u[n] * U[m][n]))
// grid (f / 128, E), block 128: wavefront 0 = gate, wavefront 1 = up.
template <int MT>
__global__ __launch_bounds__(128) void gate_up_decode_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const int8_t* __restrict__ w_gate,
    const int8_t* __restrict__ w_up, const uint16_t* __restrict__ scales, _Float16* __restrict__ H,
    int d, int f) {
  __shared__ float s_up[MT * 16][kSlab + 4];  // s_u * U of the pass, [row][slab column]
  const int e = blockIdx.y;
  const int row0 = offsets[e];
  const int M = offsets[e + 1] - row0;
  if (M <= 0) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wavefront
  const int lane = threadIdx.x & 63, kg = lane >> 4, cl = lane & 15;
  const int nl = 8 * cl;  // first of the lane's 8 columns within the slab
  const int n0 = blockIdx.x * kSlab + nl;
  const __amdgpu_buffer_rsrc_t wr = weight_rsrc((wave == 0 ? w_gate : w_up) + (size_t)e * d * f, (size_t)d * f);
  const uint32_t voff = (uint32_t)(8 * kg) * (uint32_t)f + (uint32_t)n0;
  float s8[8];
  load_scales8(scales + (size_t)e * (2 * (size_t)f + d) + (wave == 0 ? 0 : f) + n0, s8);

  for (int pb = 0; pb < M; pb += 16 * MT) {
    const uint16_t* a[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = min(pb + 16 * mt + cl, M - 1);
      a[mt] = x + (size_t)perm[row0 + m] * d + 8 * kg;
    }
    f32x4 acc[MT][8];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    stream_slab<bf16x8, MT>(wr, voff, (uint32_t)f, d / kStep, a, acc);

    // lane holds rows 16 mt + 4 kg + i of the pass, columns nl .. nl + 7 of the slab
    if (wave == 1) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) s_up[16 * mt + 4 * kg + i][nl + j] = acc[mt][j][i] * s8[j];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = pb + 16 * mt + 4 * kg + i;
          if (m < M) {
            const float* urow = s_up[16 * mt + 4 * kg + i] + nl;
            uint32_t packed[4];
#pragma unroll
            for (int j = 0; j < 8; j += 2)
              packed[j >> 1] = pack_f16_rne(gelu_tanh(acc[mt][j][i] * s8[j]) * urow[j],
                                            gelu_tanh(acc[mt][j + 1][i] * s8[j + 1]) * urow[j + 1]);
            u32x4 v = {packed[0], packed[1], packed[2], packed[3]};
            *reinterpret_cast<u32x4*>(H + (size_t)(row0 + m) * f + n0) = v;
          }
        }
    }
    __syncthreads();  // s_up is rewritten by the next pass
  }
}

// ------------------------------------------------------------------------------------
// down: Y[s][row0 + m][n] = s_d[n] * sum over k in part s of H[row0 + m][k] * q_d[k][n]
// grid (d / 128, splits, E), block 64.
template <int MT>
__global__ __launch_bounds__(64) void down_decode_kernel(
    const _Float16* __restrict__ H, const int32_t* __restrict__ offsets,
    const int8_t* __restrict__ w_down, const uint16_t* __restrict__ scales, float* __restrict__ Y,
    int d, int f, int rows_cap) {
  const int e = blockIdx.z, part = blockIdx.y;
  const int row0 = offsets[e];
  const int M = offsets[e + 1] - row0;
  if (M <= 0) return;
  const int kspan = f / gridDim.y, kbeg = part * kspan;
  const int lane = threadIdx.x, kg = lane >> 4, cl = lane & 15;
  const int n0 = blockIdx.x * kSlab + 8 * cl;
  const __amdgpu_buffer_rsrc_t wr = weight_rsrc(w_down + (size_t)e * f * d, (size_t)f * d);
  const uint32_t voff = (uint32_t)(kbeg + 8 * kg) * (uint32_t)d + (uint32_t)n0;
  float sd[8];
  load_scales8(scales + (size_t)e * (2 * (size_t)f + d) + 2 * (size_t)f + n0, sd);
  float* Yp = Y + (size_t)part * rows_cap * d;

  for (int pb = 0; pb < M; pb += 16 * MT) {
    const uint16_t* a[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = min(pb + 16 * mt + cl, M - 1);
      a[mt] = reinterpret_cast<const uint16_t*>(H) + (size_t)(row0 + m) * f + kbeg + 8 * kg;
    }
    f32x4 acc[MT][8];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    stream_slab<f16x8, MT>(wr, voff, (uint32_t)d, kspan / kStep, a, acc);

#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = pb + 16 * mt + 4 * kg + i;
        if (m < M) {
          float* dst = Yp + (size_t)(row0 + m) * d + n0;
          f32x4 lo = {acc[mt][0][i] * sd[0], acc[mt][1][i] * sd[1], acc[mt][2][i] * sd[2], acc[mt][3][i] * sd[3]};
          f32x4 hi = {acc[mt][4][i] * sd[4], acc[mt][5][i] * sd[5], acc[mt][6][i] * sd[6], acc[mt][7][i] * sd[7]};
          reinterpret_cast<f32x4*>(dst)[0] = lo;
          reinterpret_cast<f32x4*>(dst)[1] = hi;
        }
      }
  }
}

hipError_t launch_gate_up_decode(const uint16_t* x, const int32_t* perm, const int32_t* offsets,
                                 const int8_t* w_gate, const int8_t* w_up, const uint16_t* scales,
                                 _Float16* H, int T, int d, int f, int E, hipStream_t stream) {
  dim3 grid(f / kSlab, E), block(128);
  if (T <= 16)
    hipLaunchKernelGGL(gate_up_decode_kernel<1>, grid, block, 0, stream, x, perm, offsets, w_gate, w_up,
                       scales, H, d, f);
  else
    hipLaunchKernelGGL(gate_up_decode_kernel<2>, grid, block, 0, stream, x, perm, offsets, w_gate, w_up,
                       scales, H, d, f);
  return hipGetLastError();
}

hipError_t launch_down_decode(const _Float16* H, const int32_t* offsets, const int8_t* w_down,
                              const uint16_t* scales, float* Y, int splits, int rows_cap, int T,
                              int d, int f, int E, hipStream_t stream) {
  dim3 grid(d / kSlab, splits, E), block(64);
  if (T <= 16)
    hipLaunchKernelGGL(down_decode_kernel<1>, grid, block, 0, stream, H, offsets, w_down, scales, Y, d,
                       f, rows_cap);
  else
    hipLaunchKernelGGL(down_decode_kernel<2>, grid, block, 0, stream, H, offsets, w_down, scales, Y, d,
                       f, rows_cap);
  return hipGetLastError();
}

}  // namespace moe
