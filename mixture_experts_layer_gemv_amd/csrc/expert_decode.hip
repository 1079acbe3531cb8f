// Expert FFN for small batches (T <= 64): the layer streams the int8 weights of the
// experts it touches once from HBM, so these kernels are built for bytes in flight,
// not for reuse. (Grok-1 Admin & Architecture Guide, section 3, MoE step 3: the gated
// GeLU expert gelu(linear(x)) * linear_v(x) -> linear_1; "Quantized weights": int8
// weights dequantised as q * s, one scale per output channel.)
//
// Work split: one wavefront per workgroup owns a 128-column slab of one expert's
// matrix (gate and up together for the first kernel) and runs down the whole
// contraction (or one of `splits` parts of it for the down projection). Lane l takes the
// 8 adjacent columns n0 + 8 (l % 16) .. + 7 and, per 32-deep step, the rows
// k0 + 8 (l / 16) .. + 7: eight 8-byte loads per matrix, so each row segment a
// wavefront touches is one full 128-byte line. Byte j of those eight rows is exactly
// the B operand of one 16x16x32 MFMA (column j of the lane's 8 columns); the matching A
// operand (8 bf16/fp16 activations of the same k-group) is one 16-byte load. The k
// order inside an MFMA is the same permutation for A and B, so it does not change D.
// The int8 -> bf16 / fp16 conversion is exact (one sign-extending byte convert plus
// half a pack per element); scales are applied in fp32 after the contraction.
// Loads for step s + 1 are issued before the MFMAs of step s (two register stages).
//
// Rows: an expert's segment of the dispatch has M rows (M <= T); a pass covers 32 of
// them as two 16-row MFMA tiles (the second is skipped when the pass has <= 16 rows),
// and segments longer than 32 rows take further passes over the weights.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int kSlab = 128;  // columns per wavefront
constexpr int kStep = 32;   // contraction rows per MFMA step
}  // namespace

// A operand: 8 consecutive activations (16 bytes) of one row; zero for rows past M.
__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ void load_rows8(uint32_t (&w)[8][2], const int8_t* p, size_t ld) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    u32x2 v = *reinterpret_cast<const u32x2*>(p + (size_t)r * ld);
    w[r][0] = v.x;
    w[r][1] = v.y;
  }
}

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

// ------------------------------------------------------------------------------------
// gate/up + GeGLU: H[row0 + m][n] = fp16(gelu_tanh(s_g[n] * G[m][n]) * (s_u[n] * U[m][n]))
// grid (f / 128, E), block 64.
__global__ __launch_bounds__(64) void gate_up_decode_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const int8_t* __restrict__ w_gate,
    const int8_t* __restrict__ w_up, const uint16_t* __restrict__ scales, _Float16* __restrict__ H,
    int d, int f) {
  const int e = blockIdx.y;
  const int row0 = offsets[e];
  const int M = offsets[e + 1] - row0;
  if (M <= 0) return;
  const int lane = threadIdx.x, kg = lane >> 4, cl = lane & 15;
  const int n0 = blockIdx.x * kSlab + 8 * cl;
  const size_t ld = (size_t)f;
  const int8_t* pg = w_gate + (size_t)e * d * f + (size_t)(8 * kg) * ld + n0;
  const int8_t* pu = w_up + (size_t)e * d * f + (size_t)(8 * kg) * ld + n0;
  const uint16_t* sc = scales + (size_t)e * (2 * (size_t)f + d);

  for (int pb = 0; pb < M; pb += 32) {
    const bool two = (M - pb) > 16;
    // A rows of this lane: m = pb + cl (tile 0) and pb + 16 + cl (tile 1).
    const uint16_t* xa[2];
    bool va[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      int m = pb + 16 * mt + cl;
      va[mt] = m < M;
      int tok = va[mt] ? perm[row0 + m] : 0;
      xa[mt] = x + (size_t)tok * d + 8 * kg;
    }
    f32x4 accg[2][8], accu[2][8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int j = 0; j < 8; ++j) accg[mt][j] = accu[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint32_t bg[2][8][2], bu[2][8][2];
    u32x4 av[2][2];
    auto load_stage = [&](int s, int kk) {
      load_rows8(bg[s], pg + (size_t)kk * ld, ld);
      load_rows8(bu[s], pu + (size_t)kk * ld, ld);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) av[s][mt] = va[mt] ? load16(xa[mt] + kk) : zero_u32x4();
    };
    auto compute_stage = [&](int s) {
      bf16x8 a0 = __builtin_bit_cast(bf16x8, av[s][0]);
      bf16x8 a1 = __builtin_bit_cast(bf16x8, av[s][1]);
#define MOE_GU_COL(J)                                                   \
  {                                                                     \
    bf16x8 b = col_operand<J, bf16x8>(bg[s]);                           \
    accg[0][J] = Mfma<bf16x8>::run(a0, b, accg[0][J]);                  \
    if (two) accg[1][J] = Mfma<bf16x8>::run(a1, b, accg[1][J]);         \
    bf16x8 c = col_operand<J, bf16x8>(bu[s]);                           \
    accu[0][J] = Mfma<bf16x8>::run(a0, c, accu[0][J]);                  \
    if (two) accu[1][J] = Mfma<bf16x8>::run(a1, c, accu[1][J]);         \
  }
      MOE_GU_COL(0) MOE_GU_COL(1) MOE_GU_COL(2) MOE_GU_COL(3)
      MOE_GU_COL(4) MOE_GU_COL(5) MOE_GU_COL(6) MOE_GU_COL(7)
#undef MOE_GU_COL
    };

    load_stage(0, 0);
    for (int kk = 0; kk < d; kk += 2 * kStep) {
      load_stage(1, kk + kStep);
      compute_stage(0);
      if (kk + 2 * kStep < d) load_stage(0, kk + 2 * kStep);
      compute_stage(1);
    }

    // Epilogue: lane holds rows 4 kg + i of each tile, columns n0 .. n0 + 7.
    float sg[8], su[8];
    {
      u32x4 g4 = load16(sc + n0), u4 = load16(sc + f + n0);
      uint32_t gw[4] = {g4.x, g4.y, g4.z, g4.w}, uw[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        sg[j] = bf16_bits_to_float((gw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
        su[j] = bf16_bits_to_float((uw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
      }
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = pb + 16 * mt + 4 * kg + i;
        if (m < M) {
          uint32_t packed[4];
#pragma unroll
          for (int j = 0; j < 8; j += 2) {
            float h0 = gelu_tanh(accg[mt][j][i] * sg[j]) * (accu[mt][j][i] * su[j]);
            float h1 = gelu_tanh(accg[mt][j + 1][i] * sg[j + 1]) * (accu[mt][j + 1][i] * su[j + 1]);
            packed[j >> 1] = pack_f16_rne(h0, h1);
          }
          u32x4 v = {packed[0], packed[1], packed[2], packed[3]};
          *reinterpret_cast<u32x4*>(H + (size_t)(row0 + m) * f + n0) = v;
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// down: Y[s][row0 + m][n] = s_d[n] * sum over k in part s of H[row0 + m][k] * q_d[k][n]
// grid (d / 128, splits, E), block 64.
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
  const size_t ld = (size_t)d;
  const int8_t* pd = w_down + (size_t)e * f * d + (size_t)(kbeg + 8 * kg) * ld + n0;
  const uint16_t* sc = scales + (size_t)e * (2 * (size_t)f + d) + 2 * (size_t)f;
  float* Yp = Y + (size_t)part * rows_cap * d;

  for (int pb = 0; pb < M; pb += 32) {
    const bool two = (M - pb) > 16;
    const _Float16* ha[2];
    bool va[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      int m = pb + 16 * mt + cl;
      va[mt] = m < M;
      ha[mt] = H + (size_t)(row0 + (va[mt] ? m : 0)) * f + kbeg + 8 * kg;
    }
    f32x4 acc[2][8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint32_t bd[2][8][2];
    u32x4 av[2][2];
    auto load_stage = [&](int s, int kk) {
      load_rows8(bd[s], pd + (size_t)kk * ld, ld);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) av[s][mt] = va[mt] ? load16(ha[mt] + kk) : zero_u32x4();
    };
    auto compute_stage = [&](int s) {
      f16x8 a0 = __builtin_bit_cast(f16x8, av[s][0]);
      f16x8 a1 = __builtin_bit_cast(f16x8, av[s][1]);
#define MOE_DN_COL(J)                                                 \
  {                                                                   \
    f16x8 b = col_operand<J, f16x8>(bd[s]);                           \
    acc[0][J] = Mfma<f16x8>::run(a0, b, acc[0][J]);                   \
    if (two) acc[1][J] = Mfma<f16x8>::run(a1, b, acc[1][J]);          \
  }
      MOE_DN_COL(0) MOE_DN_COL(1) MOE_DN_COL(2) MOE_DN_COL(3)
      MOE_DN_COL(4) MOE_DN_COL(5) MOE_DN_COL(6) MOE_DN_COL(7)
#undef MOE_DN_COL
    };

    load_stage(0, 0);
    for (int kk = 0; kk < kspan; kk += 2 * kStep) {
      load_stage(1, kk + kStep);
      compute_stage(0);
      if (kk + 2 * kStep < kspan) load_stage(0, kk + 2 * kStep);
      compute_stage(1);
    }

    float sd[8];
    {
      u32x4 d4 = load16(sc + n0);
      uint32_t dw[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) sd[j] = bf16_bits_to_float((dw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
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
}

hipError_t launch_gate_up_decode(const uint16_t* x, const int32_t* perm, const int32_t* offsets,
                                 const int8_t* w_gate, const int8_t* w_up, const uint16_t* scales,
                                 _Float16* H, int d, int f, int E, hipStream_t stream) {
  hipLaunchKernelGGL(gate_up_decode_kernel, dim3(f / kSlab, E), dim3(64), 0, stream, x, perm,
                     offsets, w_gate, w_up, scales, H, d, f);
  return hipGetLastError();
}

hipError_t launch_down_decode(const _Float16* H, const int32_t* offsets, const int8_t* w_down,
                              const uint16_t* scales, float* Y, int splits, int rows_cap, int d,
                              int f, int E, hipStream_t stream) {
  hipLaunchKernelGGL(down_decode_kernel, dim3(d / kSlab, splits, E), dim3(64), 0, stream, H,
                     offsets, w_down, scales, Y, d, f, rows_cap);
  return hipGetLastError();
}

}  // namespace moe
