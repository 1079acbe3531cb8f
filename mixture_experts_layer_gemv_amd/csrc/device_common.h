// Device helpers shared by the gfx950 kernels of the MoE layer: vector types, bf16/fp16
// bit conversions, the int8 -> bf16/fp16 operand builders and MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

// Two fp32 values whose low 16 bits are zero (small integers, bf16 values) packed as a
// bf16 pair by taking their high halves: low half <- a, high half <- b. Exact for such inputs.
__device__ __forceinline__ uint32_t pack_bf16_hi(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// Signed byte j (0..3) of w as fp32 (exact). hipcc emits one v_cvt_f32_i32 with a
// sign-extended byte select for this.
template <int J>
__device__ __forceinline__ float sbyte(uint32_t w) {
  return (float)(int8_t)(w >> (8 * J));
}

// Column j of eight int8 rows (byte j of each row's dword) as an 8-element bf16 operand:
// element r <- row r. Every int8 value is exact in bf16.
template <int J>
__device__ __forceinline__ bf16x8 rows_to_bf16(const uint32_t (&w)[8]) {
  u32x4 v;
  v.x = pack_bf16_hi(sbyte<J>(w[0]), sbyte<J>(w[1]));
  v.y = pack_bf16_hi(sbyte<J>(w[2]), sbyte<J>(w[3]));
  v.z = pack_bf16_hi(sbyte<J>(w[4]), sbyte<J>(w[5]));
  v.w = pack_bf16_hi(sbyte<J>(w[6]), sbyte<J>(w[7]));
  return __builtin_bit_cast(bf16x8, v);
}

// The same as fp16 (int8 values are exact in fp16; the round-toward-zero pack is exact).
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// Two fp32 values rounded to nearest-even fp16 and packed (low half <- a).
__device__ __forceinline__ uint32_t pack_f16_rne(float a, float b) {
  _Float16 ha = (_Float16)a, hb = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

template <int J>
__device__ __forceinline__ f16x8 rows_to_f16(const uint32_t (&w)[8]) {
  u32x4 v;
  v.x = pack_f16(sbyte<J>(w[0]), sbyte<J>(w[1]));
  v.y = pack_f16(sbyte<J>(w[2]), sbyte<J>(w[3]));
  v.z = pack_f16(sbyte<J>(w[4]), sbyte<J>(w[5]));
  v.w = pack_f16(sbyte<J>(w[6]), sbyte<J>(w[7]));
  return __builtin_bit_cast(f16x8, v);
}

template <typename T>
struct Mfma;

// D(16x16 fp32) += A(16x32) * B(32x16). Lane l supplies A row (l % 16) and B column
// (l % 16), each with the 8 k-values of k-group (l / 16); D comes back as rows
// 4 * (l / 16) + i, i = 0..3, of column l % 16. A and B use the same k-group mapping,
// so any permutation of k applied to both leaves D unchanged.
template <>
struct Mfma<bf16x8> {
  static __device__ __forceinline__ f32x4 run(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Mfma<f16x8> {
  static __device__ __forceinline__ f32x4 run(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// tanh-form GeLU, 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))), written as
// v * sigmoid(2 sqrt(2/pi) (v + 0.044715 v^3)) (the same function: 0.5 (1 + tanh z) =
// 1 / (1 + exp(-2 z))), with the hardware reciprocal (1 ulp). Saturates cleanly:
// exp -> inf gives -0, exp -> 0 gives v.
// No multiply-add contraction here: the compiler would otherwise choose per call site whether to
// fuse, and the kernels that compute the same H element (decode, tiled, narrow tiles, split
// contractions) must round it identically.
__device__ __forceinline__ float gelu_tanh(float v) {
#pragma clang fp contract(off)
  const float c2 = 2.0f * 0.7978845608028654f;
  float z = c2 * (v + 0.044715f * v * v * v);
  return v * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

__device__ __forceinline__ u32x4 zero_u32x4() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return z;
}

}  // namespace moe
