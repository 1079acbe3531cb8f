// Weight streaming for small batches: the inner loop shared by the decode expert kernels
// and the one-launch layer (Grok-1 Admin & Architecture Guide, section 3, MoE step 3, and
// "Quantized weights": int8 weights dequantised as q * s, one scale per output channel).
//
// A wavefront owns a 256-column slab of one expert matrix and runs down the contraction
// (or one part of it). Lane l takes the 16 adjacent columns n0 + 16 (l % 16) .. + 15 and, per
// 32-deep step, the rows k0 + 8 (l / 16) .. + 7: eight 16-byte loads, so each row segment a
// wavefront instruction touches is 256 contiguous bytes. Byte j of those eight rows is exactly
// the B operand of one 16x16x32 MFMA (column j of the lane's 16 columns); the matching A
// operand (8 bf16/fp16 activations of the same k-group) is one 16-byte load. The k order inside
// an MFMA is the same permutation for A and B, so it does not change D. The int8 -> bf16 /
// fp16 conversion is exact (one sign-extending byte convert plus half a pack per element);
// scales are applied in fp32 after the contraction. Loads run kStages - 1 steps ahead of the
// MFMAs (a register ring); the first kStages - 1 steps of weights can be issued before the
// rows are known (stream_slab_rows), since they depend only on the slab.
#pragma once

#include "device_common.h"

namespace moe {

constexpr int kStep = 32;  // contraction rows per MFMA step
// Cache policy of the weight loads: non-temporal (each weight byte is read once).
constexpr int kWeightLoadPolicy = 2;
// Buffer resource word 3 for raw byte buffers on gfx9-family parts.
constexpr int kBufferFlags = 0x00020000;

// kNcol adjacent columns per lane (16-byte loads, so a wavefront instruction reads 256-byte
// row segments and a wavefront owns a 256-column slab).
constexpr int kNcol = 16;
constexpr int kSlab = 16 * kNcol;  // columns per wavefront

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

template <int J, typename V, int NW>
__device__ __forceinline__ V col_operand(const uint32_t (&w)[8][NW]) {
  uint32_t s[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) s[r] = w[r][J >> 2];
  if constexpr (__is_same(V, bf16x8))
    return rows_to_bf16<J & 3>(s);
  else
    return rows_to_f16<J & 3>(s);
}

template <int NW>
__device__ __forceinline__ void load_row(uint32_t (&dst)[NW], __amdgpu_buffer_rsrc_t wr, uint32_t voff, uint32_t soff) {
  if constexpr (NW == 2) {
    auto v = __builtin_amdgcn_raw_buffer_load_b64(wr, voff, soff, kWeightLoadPolicy);
    dst[0] = v[0], dst[1] = v[1];
  } else {
    auto v = __builtin_amdgcn_raw_buffer_load_b128(wr, voff, soff, kWeightLoadPolicy);
    dst[0] = v[0], dst[1] = v[1], dst[2] = v[2], dst[3] = v[3];
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t weight_rsrc(const int8_t* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(base), (short)0, (int)bytes, kBufferFlags);
}

template <int N>
__device__ __forceinline__ void load_scales(const uint16_t* p, float (&s)[N]) {
#pragma unroll
  for (int q = 0; q < N / 8; ++q) {
    u32x4 v = load16(p + 8 * q);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) s[8 * q + j] = bf16_bits_to_float((w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
  }
}

// acc[mt][j] += A rows (tile mt) x column j of the lane's kNcol, over `steps` 32-deep steps.
// wr: buffer resource of this expert's matrix; voff: byte offset of this lane's first weight
// (row 8 kg, column n0); row r of step s is at voff + (32 s + r) * ld, with the uniform part in
// the scalar offset, so all eight row loads share one address register.
// rows(a) is called once the first kStages - 1 steps of weights are in flight (they depend
// only on the slab): it fills a[mt], this lane's first activation of tile mt (row cl of the
// tile, k 8 kg), or returns false to leave without computing. Rows past the segment end point
// at a live row: MFMA rows are independent, so their results are simply not stored. The
// steady-state loop has no branches, so the loads of the next kStages - 1 steps stay in
// flight across the MFMAs; a short unrolled tail finishes.
template <typename Frag, int MT, int kStages, typename Rows>
__device__ __forceinline__ bool stream_slab_rows(__amdgpu_buffer_rsrc_t wr, uint32_t voff, uint32_t ld, int steps,
                                                 Rows&& rows, f32x4 (&acc)[MT][kNcol]) {
  constexpr int NW = kNcol / 4;
  uint32_t b[kStages][8][NW];
  u32x4 av[kStages][MT];
  const uint16_t* a[MT];
  auto load_w = [&](int s, int step) {
    const uint32_t base = (uint32_t)step * kStep * ld;
#pragma unroll
    for (int r = 0; r < 8; ++r) load_row<NW>(b[s][r], wr, voff, base + r * ld);
  };
  auto load_a = [&](int s, int step) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) av[s][mt] = load16(a[mt] + step * kStep);
  };
  auto compute = [&](int s) {
    Frag af[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) af[mt] = __builtin_bit_cast(Frag, av[s][mt]);
#define MOE_DEC_COL(J)                                                          \
  if constexpr ((J) < kNcol) {                                                  \
    Frag bfr = col_operand<(J), Frag, NW>(b[s]);                                \
    _Pragma("unroll") for (int mt = 0; mt < MT; ++mt)                           \
        acc[mt][(J)] = Mfma<Frag>::run(af[mt], bfr, acc[mt][(J)]);              \
  }
    MOE_DEC_COL(0) MOE_DEC_COL(1) MOE_DEC_COL(2) MOE_DEC_COL(3)
    MOE_DEC_COL(4) MOE_DEC_COL(5) MOE_DEC_COL(6) MOE_DEC_COL(7)
    MOE_DEC_COL(8) MOE_DEC_COL(9) MOE_DEC_COL(10) MOE_DEC_COL(11)
    MOE_DEC_COL(12) MOE_DEC_COL(13) MOE_DEC_COL(14) MOE_DEC_COL(15)
#undef MOE_DEC_COL
  };

#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < steps) load_w(s, s);
  if (!rows(a)) return false;
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < steps) load_a(s, s);
  int st = 0;
  for (; st + 2 * kStages - 1 <= steps; st += kStages) {
#pragma unroll
    for (int s = 0; s < kStages; ++s) {
      load_w((s + kStages - 1) % kStages, st + s + kStages - 1);
      load_a((s + kStages - 1) % kStages, st + s + kStages - 1);
      compute(s);
    }
  }
#pragma unroll
  for (int s = 0; s < 2 * kStages - 1; ++s) {
    if (st + s < steps) {
      if (st + s + kStages - 1 < steps) {
        load_w((s + kStages - 1) % kStages, st + s + kStages - 1);
        load_a((s + kStages - 1) % kStages, st + s + kStages - 1);
      }
      compute(s % kStages);
    }
  }
  return true;
}

// The stream with the rows known up front.
template <typename Frag, int MT, int kStages>
__device__ __forceinline__ void stream_slab(__amdgpu_buffer_rsrc_t wr, uint32_t voff, uint32_t ld, int steps,
                                            const uint16_t* const (&a)[MT], f32x4 (&acc)[MT][kNcol]) {
  stream_slab_rows<Frag, MT, kStages>(
      wr, voff, ld, steps,
      [&](const uint16_t* (&dst)[MT]) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) dst[mt] = a[mt];
        return true;
      },
      acc);
}

// H[r][n .. n + 7] of a gate/up contraction split in `parts`: g = s_g * (sum over parts p in
// order, from 0, of P[2p][r]), u likewise from P[2p + 1]; h = fp16(gelu_tanh(g) * u). P holds
// 2 * parts planes of `plane` floats ([rows][f] each); sc: the expert's gate scales (up at + f).
__device__ __forceinline__ u32x4 geglu_from_parts(const float* __restrict__ P, size_t plane, int parts, int r, int f,
                                                  int n, const uint16_t* __restrict__ sc) {
  f32x4 g[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  f32x4 u[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (int p = 0; p < parts; ++p) {
    const f32x4* gp = reinterpret_cast<const f32x4*>(P + (2 * p) * plane + (size_t)r * f + n);
    const f32x4* up = reinterpret_cast<const f32x4*>(P + (2 * p + 1) * plane + (size_t)r * f + n);
    g[0] += gp[0], g[1] += gp[1];
    u[0] += up[0], u[1] += up[1];
  }
  float sg[8], su[8];
  load_scales<8>(sc + n, sg);
  load_scales<8>(sc + f + n, su);
  uint32_t packed[4];
#pragma unroll
  for (int j = 0; j < 8; j += 2)
    packed[j >> 1] = pack_f16_rne(gelu_tanh(g[j >> 2][j & 3] * sg[j]) * (u[j >> 2][j & 3] * su[j]),
                                  gelu_tanh(g[j >> 2][(j & 3) + 1] * sg[j + 1]) * (u[j >> 2][(j & 3) + 1] * su[j + 1]));
  return u32x4{packed[0], packed[1], packed[2], packed[3]};
}

}  // namespace moe
