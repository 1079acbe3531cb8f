// Expert FFN for small batches (T <= 160, expert matrices above 2^23 weights): the
// layer streams the int8 weights of the experts it touches once from HBM, so these
// kernels are built for bytes in flight, not for reuse. (Grok-1 Admin & Architecture
// Guide, section 3, MoE step 3: the gated GeLU expert gelu(linear(x)) * linear_v(x) ->
// linear_1; "Quantized weights": int8 weights dequantised as q * s, one scale per output
// channel.)
//
// Work split: one wavefront owns a 256-column slab of one matrix of one touched expert
// and runs down the whole contraction, or one of `splits` parts of it when the slabs
// alone are too few to fill the chip (narrow f, e.g. one GPU's share of a tensor-parallel
// split). For gate/up a workgroup holds two wavefronts, one per matrix, on the same slab;
// they meet in LDS for the GeGLU epilogue, or, when the contraction is split, write fp32
// partial sums that geglu_finish_kernel adds in part order before the same epilogue; at
// T <= 4 one wavefront streams both matrices (gate_up_fused_decode_kernel). The inner loop
// (lane layout, MFMA operands, load ring) is stream_slab in stream_common.h.
//
// Rows: an expert's segment of the dispatch has M rows (M <= T). A pass covers MT
// 16-row MFMA tiles (MT = 1 when T <= 16 (gate/up with the whole contraction: T <= 8), 2
// when T <= 64, else 3, the most the registers hold); longer segments take further passes
// over the weights.
#include "kernels.h"
#include "stream_common.h"

namespace moe {

// The same stream over two matrices at once (gate and up of one slab): both rings share
// the activation loads; accg / accu take the two products.
template <typename Frag, int MT, int kStages>
__device__ __forceinline__ void stream_slab2(__amdgpu_buffer_rsrc_t wg, __amdgpu_buffer_rsrc_t wu, uint32_t voff,
                                             uint32_t ld, int steps, const uint16_t* const (&a)[MT],
                                             f32x4 (&accg)[MT][kNcol], f32x4 (&accu)[MT][kNcol]) {
  constexpr int NW = kNcol / 4;
  uint32_t bg[kStages][8][NW], bu[kStages][8][NW];
  u32x4 av[kStages][MT];
  auto load = [&](int s, int step) {
    const uint32_t base = (uint32_t)step * kStep * ld;
#pragma unroll
    for (int r = 0; r < 8; ++r) load_row<NW>(bg[s][r], wg, voff, base + r * ld);
#pragma unroll
    for (int r = 0; r < 8; ++r) load_row<NW>(bu[s][r], wu, voff, base + r * ld);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) av[s][mt] = load16(a[mt] + step * kStep);
  };
  auto compute = [&](int s) {
    Frag af[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) af[mt] = __builtin_bit_cast(Frag, av[s][mt]);
#define MOE_DEC_COL2(J)                                                         \
  if constexpr ((J) < kNcol) {                                                  \
    Frag bfg = col_operand<(J), Frag, NW>(bg[s]);                               \
    Frag bfu = col_operand<(J), Frag, NW>(bu[s]);                               \
    _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) {                         \
      accg[mt][(J)] = Mfma<Frag>::run(af[mt], bfg, accg[mt][(J)]);              \
      accu[mt][(J)] = Mfma<Frag>::run(af[mt], bfu, accu[mt][(J)]);              \
    }                                                                           \
  }
    MOE_DEC_COL2(0) MOE_DEC_COL2(1) MOE_DEC_COL2(2) MOE_DEC_COL2(3)
    MOE_DEC_COL2(4) MOE_DEC_COL2(5) MOE_DEC_COL2(6) MOE_DEC_COL2(7)
    MOE_DEC_COL2(8) MOE_DEC_COL2(9) MOE_DEC_COL2(10) MOE_DEC_COL2(11)
    MOE_DEC_COL2(12) MOE_DEC_COL2(13) MOE_DEC_COL2(14) MOE_DEC_COL2(15)
#undef MOE_DEC_COL2
  };

#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < steps) load(s, s);
  int st = 0;
  for (; st + 2 * kStages - 1 <= steps; st += kStages) {
#pragma unroll
    for (int s = 0; s < kStages; ++s) {
      load((s + kStages - 1) % kStages, st + s + kStages - 1);
      compute(s);
    }
  }
#pragma unroll
  for (int s = 0; s < 2 * kStages - 1; ++s) {
    if (st + s < steps) {
      if (st + s + kStages - 1 < steps) load((s + kStages - 1) % kStages, st + s + kStages - 1);
      compute(s % kStages);
    }
  }
}

// Rows of the largest expert segment (E <= 64 reads of offsets, the same for every workgroup).
__device__ __forceinline__ int max_segment(const int32_t* __restrict__ offsets, int E) {
  int m = 0;
  for (int e = 0; e < E; ++e) m = max(m, offsets[e + 1] - offsets[e]);
  return m;
}

// kOnly: 0 = always run; 1 = run only if no expert segment exceeds 32 rows; 2 = only if one
// does (the 32- and 48-row kernels launched back to back, one of them leaving at once).
template <int kOnly>
__device__ __forceinline__ bool skip_by_segment(const int32_t* __restrict__ offsets, int E) {
  if constexpr (kOnly == 0) return false;
  const int m = max_segment(offsets, E);
  return kOnly == 1 ? m > 32 : m <= 32;
}

// ------------------------------------------------------------------------------------
// gate/up + GeGLU: H[row0 + m][n] = fp16(gelu_tanh(s_g[n] * G[m][n]) * (s_u[n] * U[m][n]))
// grid (f / kSlab, parts, E), block 128: wavefront 0 = gate, wavefront 1 = up.
// kPartial (parts > 1): part p of the contraction writes its unscaled sums to
// P[(2 p + matrix) * rows_cap + row][n] (fp32) instead; geglu_finish_kernel completes H.
template <int MT, int kStages, bool kPartial, int kOnly = 0>
__global__ __launch_bounds__(128) void gate_up_decode_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const int8_t* __restrict__ w_gate,
    const int8_t* __restrict__ w_up, const uint16_t* __restrict__ scales, _Float16* __restrict__ H,
    float* __restrict__ P, int d, int f, int rows_cap) {
  __shared__ float s_up[kPartial ? 1 : MT * 16][kSlab + 4];  // s_u * U of the pass, [row][slab column]
  if (skip_by_segment<kOnly>(offsets, gridDim.z)) return;
  const int e = blockIdx.z, part = blockIdx.y;
  const int row0 = offsets[e];
  const int M = offsets[e + 1] - row0;
  if (M <= 0) return;
  const int kspan = d / gridDim.y, kbeg = part * kspan;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wavefront
  const int lane = threadIdx.x & 63, kg = lane >> 4, cl = lane & 15;
  const int nl = kNcol * cl;  // first of the lane's columns within the slab
  const int n0 = blockIdx.x * kSlab + nl;
  const __amdgpu_buffer_rsrc_t wr = weight_rsrc((wave == 0 ? w_gate : w_up) + (size_t)e * d * f, (size_t)d * f);
  const uint32_t voff = (uint32_t)(kbeg + 8 * kg) * (uint32_t)f + (uint32_t)n0;
  float s8[kNcol];
  if constexpr (!kPartial)
    load_scales<kNcol>(scales + (size_t)e * (2 * (size_t)f + d) + (wave == 0 ? 0 : f) + n0, s8);

  for (int pb = 0; pb < M; pb += 16 * MT) {
    const uint16_t* a[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = min(pb + 16 * mt + cl, M - 1);
      a[mt] = x + (size_t)perm[row0 + m] * d + kbeg + 8 * kg;
    }
    f32x4 acc[MT][kNcol];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < kNcol; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    stream_slab<bf16x8, MT, kStages>(wr, voff, (uint32_t)f, kspan / kStep, a, acc);

    if constexpr (kPartial) {
      // lane holds rows 16 mt + 4 kg + i of the pass, columns n0 .. n0 + kNcol - 1
      float* Pp = P + (size_t)(2 * part + wave) * rows_cap * f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = pb + 16 * mt + 4 * kg + i;
          if (m < M) {
            float* dst = Pp + (size_t)(row0 + m) * f + n0;
#pragma unroll
            for (int q = 0; q < kNcol / 4; ++q)
              reinterpret_cast<f32x4*>(dst)[q] =
                  f32x4{acc[mt][4 * q][i], acc[mt][4 * q + 1][i], acc[mt][4 * q + 2][i], acc[mt][4 * q + 3][i]};
          }
        }
    } else {
      // lane holds rows 16 mt + 4 kg + i of the pass, columns nl .. nl + kNcol - 1 of the slab
      if (wave == 1) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < kNcol; ++j) s_up[16 * mt + 4 * kg + i][nl + j] = acc[mt][j][i] * s8[j];
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
#pragma unroll
              for (int q = 0; q < kNcol / 8; ++q) {
                uint32_t packed[4];
#pragma unroll
                for (int j = 8 * q; j < 8 * q + 8; j += 2)
                  packed[(j >> 1) & 3] = pack_f16_rne(gelu_tanh(acc[mt][j][i] * s8[j]) * urow[j],
                                                      gelu_tanh(acc[mt][j + 1][i] * s8[j + 1]) * urow[j + 1]);
                u32x4 v = {packed[0], packed[1], packed[2], packed[3]};
                *reinterpret_cast<u32x4*>(H + (size_t)(row0 + m) * f + n0 + 8 * q) = v;
              }
            }
          }
      }
      __syncthreads();  // s_up is rewritten by the next pass
    }
  }
}

// gate/up + GeGLU for T <= 4 (whole contraction): one wavefront per slab streams both
// matrices with a 2-step ring each, sharing the activation loads, and applies the GeGLU in
// registers (no LDS exchange). Same MFMA sequence per output as gate_up_decode_kernel, so the
// same bits. With 2-5 touched experts the two-wavefront form runs 1.3-1.5 rounds of
// wavefronts where this one runs under one (T = 3: 565 -> 487 us per forward at the Grok
// shape); from T = 5 the deeper single-matrix rings win.
// grid (f / kSlab, 1, E), block 64.
template <int MT, int kStages>
__global__ __launch_bounds__(64) void gate_up_fused_decode_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets,
    const int8_t* __restrict__ w_gate, const int8_t* __restrict__ w_up, const uint16_t* __restrict__ scales,
    _Float16* __restrict__ H, int d, int f) {
  const int e = blockIdx.z;
  const int row0 = offsets[e];
  const int M = offsets[e + 1] - row0;
  if (M <= 0) return;
  const int lane = threadIdx.x, kg = lane >> 4, cl = lane & 15;
  const int n0 = blockIdx.x * kSlab + kNcol * cl;
  const __amdgpu_buffer_rsrc_t wg = weight_rsrc(w_gate + (size_t)e * d * f, (size_t)d * f);
  const __amdgpu_buffer_rsrc_t wu = weight_rsrc(w_up + (size_t)e * d * f, (size_t)d * f);
  const uint32_t voff = (uint32_t)(8 * kg) * (uint32_t)f + (uint32_t)n0;
  for (int pb = 0; pb < M; pb += 16 * MT) {
    const uint16_t* a[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = min(pb + 16 * mt + cl, M - 1);
      a[mt] = x + (size_t)perm[row0 + m] * d + 8 * kg;
    }
    f32x4 accg[MT][kNcol], accu[MT][kNcol];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < kNcol; ++j) accg[mt][j] = accu[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    stream_slab2<bf16x8, MT, kStages>(wg, wu, voff, (uint32_t)f, d / kStep, a, accg, accu);
    float sg[kNcol], su[kNcol];
    load_scales<kNcol>(scales + (size_t)e * (2 * (size_t)f + d) + n0, sg);
    load_scales<kNcol>(scales + (size_t)e * (2 * (size_t)f + d) + f + n0, su);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = pb + 16 * mt + 4 * kg + i;
        if (m < M) {
#pragma unroll
          for (int q = 0; q < kNcol / 8; ++q) {
            uint32_t packed[4];
#pragma unroll
            for (int j = 8 * q; j < 8 * q + 8; j += 2)
              packed[(j >> 1) & 3] = pack_f16_rne(gelu_tanh(accg[mt][j][i] * sg[j]) * (accu[mt][j][i] * su[j]),
                                                  gelu_tanh(accg[mt][j + 1][i] * sg[j + 1]) * (accu[mt][j + 1][i] * su[j + 1]));
            u32x4 v = {packed[0], packed[1], packed[2], packed[3]};
            *reinterpret_cast<u32x4*>(H + (size_t)(row0 + m) * f + n0 + 8 * q) = v;
          }
        }
      }
  }
}

// ------------------------------------------------------------------------------------
// The GeGLU epilogue of a split gate/up contraction: for row r < offsets[E] (expert e),
// g = s_g * (sum over parts p in order of P[2p][r]), u likewise from P[2p + 1]; H[r] =
// fp16(gelu_tanh(g) * u). grid (rows_cap, ceil(f / 2048)), block 256, 8 columns per thread.
__global__ __launch_bounds__(256) void geglu_finish_kernel(const float* __restrict__ P,
                                                           const int32_t* __restrict__ offsets,
                                                           const uint16_t* __restrict__ scales,
                                                           _Float16* __restrict__ H, int parts, int d, int f,
                                                           int E, int rows_cap) {
  const int r = blockIdx.x;
  if (r >= offsets[E]) return;
  int e = 0;
  while (e + 1 < E && offsets[e + 1] <= r) ++e;
  const uint16_t* sc = scales + (size_t)e * (2 * (size_t)f + d);
  const size_t plane = (size_t)rows_cap * f;
  const int n = 2048 * blockIdx.y + 8 * threadIdx.x;
  if (n < f) *reinterpret_cast<u32x4*>(H + (size_t)r * f + n) = geglu_from_parts(P, plane, parts, r, f, n, sc);
}

// ------------------------------------------------------------------------------------
// down: Y[s][row0 + m][n] = s_d[n] * sum over k in part s of H[row0 + m][k] * q_d[k][n]
// grid (d / kSlab, splits, E), block 64.
template <int MT, int kStages, int kOnly = 0>
__global__ __launch_bounds__(64) void down_decode_kernel(
    const _Float16* __restrict__ H, const int32_t* __restrict__ offsets,
    const int8_t* __restrict__ w_down, const uint16_t* __restrict__ scales, float* __restrict__ Y,
    int d, int f, int rows_cap) {
  if (skip_by_segment<kOnly>(offsets, gridDim.z)) return;
  const int e = blockIdx.z, part = blockIdx.y;
  const int row0 = offsets[e];
  const int M = offsets[e + 1] - row0;
  if (M <= 0) return;
  const int kspan = f / gridDim.y, kbeg = part * kspan;
  const int lane = threadIdx.x, kg = lane >> 4, cl = lane & 15;
  const int n0 = blockIdx.x * kSlab + kNcol * cl;
  const __amdgpu_buffer_rsrc_t wr = weight_rsrc(w_down + (size_t)e * f * d, (size_t)f * d);
  const uint32_t voff = (uint32_t)(kbeg + 8 * kg) * (uint32_t)d + (uint32_t)n0;
  float sd[kNcol];
  load_scales<kNcol>(scales + (size_t)e * (2 * (size_t)f + d) + 2 * (size_t)f + n0, sd);
  float* Yp = Y + (size_t)part * rows_cap * d;

  for (int pb = 0; pb < M; pb += 16 * MT) {
    const uint16_t* a[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = min(pb + 16 * mt + cl, M - 1);
      a[mt] = reinterpret_cast<const uint16_t*>(H) + (size_t)(row0 + m) * f + kbeg + 8 * kg;
    }
    f32x4 acc[MT][kNcol];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < kNcol; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    stream_slab<f16x8, MT, kStages>(wr, voff, (uint32_t)d, kspan / kStep, a, acc);

#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = pb + 16 * mt + 4 * kg + i;
        if (m < M) {
          float* dst = Yp + (size_t)(row0 + m) * d + n0;
#pragma unroll
          for (int q = 0; q < kNcol / 4; ++q) {
            f32x4 v = {acc[mt][4 * q][i] * sd[4 * q], acc[mt][4 * q + 1][i] * sd[4 * q + 1],
                       acc[mt][4 * q + 2][i] * sd[4 * q + 2], acc[mt][4 * q + 3][i] * sd[4 * q + 3]};
            reinterpret_cast<f32x4*>(dst)[q] = v;
          }
        }
      }
  }
}

hipError_t launch_gate_up_decode(const uint16_t* x, const int32_t* perm, const int32_t* offsets,
                                 const int8_t* w_gate, const int8_t* w_up, const uint16_t* scales,
                                 _Float16* H, float* P, int parts, int T, int k, int d, int f, int E,
                                 hipStream_t stream) {
  dim3 grid(f / kSlab, parts, E), block(128);
  const int rows_cap = T * k;
  // ring depths measured best at the Grok-1 shape (T = 8 and T = 64)
  if (parts > 1) {
    if (T <= 16)
      hipLaunchKernelGGL((gate_up_decode_kernel<1, 4, true>), grid, block, 0, stream, x, perm, offsets, w_gate,
                         w_up, scales, H, P, d, f, rows_cap);
    else if (T <= 64)
      hipLaunchKernelGGL((gate_up_decode_kernel<2, 3, true>), grid, block, 0, stream, x, perm, offsets, w_gate,
                         w_up, scales, H, P, d, f, rows_cap);
    else
      hipLaunchKernelGGL((gate_up_decode_kernel<3, 3, true>), grid, block, 0, stream, x, perm, offsets, w_gate,
                         w_up, scales, H, P, d, f, rows_cap);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(geglu_finish_kernel, dim3(rows_cap, (f + 2047) / 2048), dim3(256), 0, stream, P, offsets,
                       scales, H, parts, d, f, E, rows_cap);
  } else if (T <= 4) {
    hipLaunchKernelGGL((gate_up_fused_decode_kernel<1, 2>), dim3(f / kSlab, 1, E), dim3(64), 0, stream, x, perm,
                       offsets, w_gate, w_up, scales, H, d, f);
  } else if (T <= 8) {  // 9-16 tokens: the 32-row passes below were as fast or faster (T = 16: -1.8%)
    hipLaunchKernelGGL((gate_up_decode_kernel<1, 4, false>), grid, block, 0, stream, x, perm, offsets, w_gate,
                       w_up, scales, H, P, d, f, rows_cap);
  } else if (T <= 64) {
    hipLaunchKernelGGL((gate_up_decode_kernel<2, 3, false>), grid, block, 0, stream, x, perm, offsets, w_gate,
                       w_up, scales, H, P, d, f, rows_cap);
  } else if (T <= 96) {
    // 65-96 tokens: the 32-row passes stream 2% faster while no expert exceeds 32 rows, which
    // only the device knows; both kernels are launched and one of them leaves at once
    hipLaunchKernelGGL((gate_up_decode_kernel<2, 3, false, 1>), grid, block, 0, stream, x, perm, offsets, w_gate,
                       w_up, scales, H, P, d, f, rows_cap);
    hipLaunchKernelGGL((gate_up_decode_kernel<3, 3, false, 2>), grid, block, 0, stream, x, perm, offsets, w_gate,
                       w_up, scales, H, P, d, f, rows_cap);
  } else {
    hipLaunchKernelGGL((gate_up_decode_kernel<3, 3, false>), grid, block, 0, stream, x, perm, offsets, w_gate,
                       w_up, scales, H, P, d, f, rows_cap);
  }
  return hipGetLastError();
}

hipError_t launch_down_decode(const _Float16* H, const int32_t* offsets, const int8_t* w_down,
                              const uint16_t* scales, float* Y, int splits, int rows_cap, int T,
                              int d, int f, int E, hipStream_t stream) {
  dim3 grid(d / kSlab, splits, E), block(64);
  if (T <= 16)
    hipLaunchKernelGGL((down_decode_kernel<1, 4>), grid, block, 0, stream, H, offsets, w_down, scales, Y, d,
                       f, rows_cap);
  else if (T <= 64)
    hipLaunchKernelGGL((down_decode_kernel<2, 4>), grid, block, 0, stream, H, offsets, w_down, scales, Y, d,
                       f, rows_cap);
  else if (T <= 96) {  // as for gate/up: 32-row passes unless an expert exceeds 32 rows
    hipLaunchKernelGGL((down_decode_kernel<2, 4, 1>), grid, block, 0, stream, H, offsets, w_down, scales, Y, d,
                       f, rows_cap);
    hipLaunchKernelGGL((down_decode_kernel<3, 3, 2>), grid, block, 0, stream, H, offsets, w_down, scales, Y, d,
                       f, rows_cap);
  } else
    hipLaunchKernelGGL((down_decode_kernel<3, 3>), grid, block, 0, stream, H, offsets, w_down, scales, Y, d,
                       f, rows_cap);
  return hipGetLastError();
}

}  // namespace moe
