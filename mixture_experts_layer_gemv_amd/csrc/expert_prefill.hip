// Expert FFN for large batches (T > 64): grouped W8A16 GEMMs on the MFMA units.
// (Grok-1 Admin & Architecture Guide, section 3, MoE step 3, the gated GeLU expert
// gelu(linear(x)) * linear_v(x) -> linear_1; "Quantized weights": int8 weights
// dequantised as q * s with one scale per output channel, compute in bf16.)
//
// One workgroup (256 threads, 4 wavefronts in a 2 x 2 arrangement) computes a
// 128-row x 256-column tile of one expert: for the gate/up kernel 128 columns of gate
// and the same 128 of up (so the GeGLU is applied in registers), for the down kernel
// 256 columns of the down projection. The contraction runs in 64-deep slices:
//   * the next slice's activations (16 B per load) and int8 weights (one dword of 4
//     columns from each of 8 rows per thread and half-tile) are loaded into registers
//     while the MFMAs of the current slice run;
//   * the weights are converted int8 -> bf16 (gate/up) or fp16 (down) once per
//     workgroup, on the way into LDS, and stored transposed ([column][k]), so every
//     MFMA operand is one 16-byte LDS read; column 4 c + q of a 64-column group goes to
//     LDS row 16 q + c, which keeps those reads conflict-free and gives each lane 4
//     adjacent output columns in the epilogue;
//   * each wavefront owns 64 rows x 128 columns: 4 x 8 MFMA tiles of 16x16x32.
// Rows are gathered through the dispatch permutation (gate/up) or read in segment order
// (down). Tiles are assigned on the device: blockIdx.x enumerates the m-tiles of all
// expert segments in expert order (read from offsets), surplus slots exit at once.
// Scales, GeLU and the fp16 rounding of h are applied in fp32 after the contraction.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int BM = 128;        // rows per workgroup tile
constexpr int BK = 64;         // contraction depth per slice
constexpr int HALF = 128;      // columns per weight half-tile
constexpr int LDS_LD = BK + 8; // 16-bit elements per LDS row (16-byte pad)
constexpr int kThreads = 256;
}  // namespace

// (expert, m-tile) of m-slot `slot`, or false when the slot is surplus.
__device__ __forceinline__ bool find_tile(const int32_t* offsets, int E, int slot, int& e, int& row0,
                                          int& rows) {
  int s = slot;
  for (int ee = 0; ee < E; ++ee) {
    int M = offsets[ee + 1] - offsets[ee];
    int nt = (M + BM - 1) / BM;
    if (s < nt) {
      e = ee;
      row0 = offsets[ee] + s * BM;
      rows = min(BM, M - s * BM);
      return true;
    }
    s -= nt;
  }
  return false;
}

template <bool kGateUp>
struct PrefillTraits;

template <>
struct PrefillTraits<true> {
  using Frag = bf16x8;
  static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_bf16_hi(a, b); }
};
template <>
struct PrefillTraits<false> {
  using Frag = f16x8;
  static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_f16(a, b); }
};

// Writes the 4 columns x 8 rows held by a thread (dword per row) into LDS, transposed and
// converted: column q of the thread's 4 goes to LDS row `row_base + 16 q`.
template <bool kGateUp, int Q>
__device__ __forceinline__ void store_col(uint16_t* sB, int row_base, int koff, const uint32_t (&w)[8]) {
  using P = PrefillTraits<kGateUp>;
  u32x4 v;
  v.x = P::pack(sbyte<Q>(w[0]), sbyte<Q>(w[1]));
  v.y = P::pack(sbyte<Q>(w[2]), sbyte<Q>(w[3]));
  v.z = P::pack(sbyte<Q>(w[4]), sbyte<Q>(w[5]));
  v.w = P::pack(sbyte<Q>(w[6]), sbyte<Q>(w[7]));
  *reinterpret_cast<u32x4*>(sB + (size_t)(row_base + 16 * Q) * LDS_LD + koff) = v;
}

// kGateUp: A = x rows gathered by perm (bf16), B halves = gate / up at columns n0..n0+127,
//          output H fp16 = gelu_tanh(s_g g) * (s_u u).
// !kGateUp: A = H rows (fp16), B halves = down columns n0..n0+127 and n0+128..n0+255,
//          output Y fp32 (part blockIdx.z of the contraction) = s_d y.
template <bool kGateUp>
__global__ __launch_bounds__(kThreads, 2) void expert_prefill_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const int8_t* __restrict__ B0,
    const int8_t* __restrict__ B1, const uint16_t* __restrict__ scales, void* __restrict__ out,
    int d, int f, int E, int rows_cap) {
  using Frag = typename PrefillTraits<kGateUp>::Frag;
  __shared__ __attribute__((aligned(16))) uint16_t sA[BM * LDS_LD];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2 * HALF * LDS_LD];

  int e, row0, rows;
  if (!find_tile(offsets, E, blockIdx.x, e, row0, rows)) return;

  const int K = kGateUp ? d : f;             // contraction length
  const int N = kGateUp ? f : d;             // output columns (per matrix)
  const int kspan = K / gridDim.z, kbeg = blockIdx.z * kspan;
  const int n0 = blockIdx.y * (kGateUp ? HALF : 2 * HALF);
  const size_t ldb = (size_t)N;
  const size_t ebase = (size_t)e * d * f;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- per-thread global load descriptors
  // A: rows tid / 8 + 32 i (i = 0..3), 16-byte chunk tid % 8 of the slice
  const uint16_t* arow[4];
  bool avalid[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int m = tid / 8 + 32 * i;
    avalid[i] = m < rows;
    int r = row0 + (avalid[i] ? m : 0);
    size_t src_row = kGateUp ? (size_t)perm[r] : (size_t)r;
    arow[i] = A + src_row * K + kbeg + 8 * (tid % 8);
  }
  // B: columns 4 cg .. 4 cg + 3 of each half, rows 8 kg .. 8 kg + 7 of the slice
  const int cg = tid % 32, kg = tid / 32;
  const int8_t* bsrc[2];
  bsrc[0] = B0 + ebase + (size_t)(kbeg + 8 * kg) * ldb + n0 + 4 * cg;
  bsrc[1] = (kGateUp ? B1 + ebase + n0 : B0 + ebase + n0 + HALF) + (size_t)(kbeg + 8 * kg) * ldb + 4 * cg;
  // LDS row of column 4 c + q (c = cg % 16) of 64-column group cg / 16, half h:
  //   h * 128 + (cg / 16) * 64 + 16 q + cg % 16
  const int brow = (cg / 16) * 64 + (cg % 16);

  u32x4 ra[4];
  uint32_t rb[2][8];
  auto gload = [&](int kk) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = avalid[i] ? *reinterpret_cast<const u32x4*>(arow[i] + kk) : zero_u32x4();
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 8; ++r) rb[h][r] = *reinterpret_cast<const uint32_t*>(bsrc[h] + (size_t)(kk + r) * ldb);
  };
  auto lds_store = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(sA + (size_t)(tid / 8 + 32 * i) * LDS_LD + 8 * (tid % 8)) = ra[i];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      store_col<kGateUp, 0>(sB, h * HALF + brow, 8 * kg, rb[h]);
      store_col<kGateUp, 1>(sB, h * HALF + brow, 8 * kg, rb[h]);
      store_col<kGateUp, 2>(sB, h * HALF + brow, 8 * kg, rb[h]);
      store_col<kGateUp, 3>(sB, h * HALF + brow, 8 * kg, rb[h]);
    }
  };

  // ---- wavefront tile: rows wm * 64 + 16 mt + (lane % 16); B tiles nt = 4 grp + q
  //   gate/up: grp 0 = gate, grp 1 = up, both at columns wn * 64 .. + 63 of the half
  //   down:    grp 0/1 = columns wn * 128 + grp * 64 .. + 63
  int bro[2];
#pragma unroll
  for (int g = 0; g < 2; ++g)
    bro[g] = kGateUp ? g * HALF + wn * 64 : wn * HALF + g * 64;
  const int kq = 8 * (lane >> 4), lr = lane & 15;

  f32x4 acc[4][8];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  for (int kk = 0; kk < kspan; kk += BK) {
    __syncthreads();  // previous slice's LDS reads are done
    lds_store();
    __syncthreads();
    if (kk + BK < kspan) gload(kk + BK);
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      Frag af[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        af[mt] = __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(
                                              sA + (size_t)(wm * 64 + 16 * mt + lr) * LDS_LD + ks + kq));
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int row = bro[nt >> 2] + 16 * (nt & 3) + lr;
        Frag bfr = __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(sB + (size_t)row * LDS_LD + ks + kq));
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt][nt] = Mfma<Frag>::run(af[mt], bfr, acc[mt][nt]);
      }
    }
  }

  // ---- epilogue: lane holds rows wm*64 + 16 mt + 4 (lane/16) + i and, per group,
  //      the 4 adjacent columns 4 (lane % 16) + q, q = 0..3
  const uint16_t* sc = scales + (size_t)e * (2 * (size_t)f + d);
  const int rq = 4 * (lane >> 4);
  if constexpr (kGateUp) {
    const int n = n0 + wn * 64 + 4 * lr;
    float sg[4], su[4];
    u32x2 g2 = *reinterpret_cast<const u32x2*>(sc + n), u2 = *reinterpret_cast<const u32x2*>(sc + f + n);
    sg[0] = bf16_bits_to_float(g2.x & 0xFFFFu), sg[1] = bf16_bits_to_float(g2.x >> 16);
    sg[2] = bf16_bits_to_float(g2.y & 0xFFFFu), sg[3] = bf16_bits_to_float(g2.y >> 16);
    su[0] = bf16_bits_to_float(u2.x & 0xFFFFu), su[1] = bf16_bits_to_float(u2.x >> 16);
    su[2] = bf16_bits_to_float(u2.y & 0xFFFFu), su[3] = bf16_bits_to_float(u2.y >> 16);
    _Float16* H = reinterpret_cast<_Float16*>(out);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = wm * 64 + 16 * mt + rq + i;
        if (m < rows) {
          float h[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) h[q] = gelu_tanh(acc[mt][q][i] * sg[q]) * (acc[mt][4 + q][i] * su[q]);
          u32x2 v = {pack_f16_rne(h[0], h[1]), pack_f16_rne(h[2], h[3])};
          *reinterpret_cast<u32x2*>(H + (size_t)(row0 + m) * f + n) = v;
        }
      }
  } else {
    float* Y = reinterpret_cast<float*>(out) + (size_t)blockIdx.z * rows_cap * d;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int n = n0 + wn * HALF + g * 64 + 4 * lr;
      u32x2 s2 = *reinterpret_cast<const u32x2*>(sc + 2 * (size_t)f + n);
      float sd[4] = {bf16_bits_to_float(s2.x & 0xFFFFu), bf16_bits_to_float(s2.x >> 16),
                     bf16_bits_to_float(s2.y & 0xFFFFu), bf16_bits_to_float(s2.y >> 16)};
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = wm * 64 + 16 * mt + rq + i;
          if (m < rows) {
            f32x4 v = {acc[mt][4 * g + 0][i] * sd[0], acc[mt][4 * g + 1][i] * sd[1],
                       acc[mt][4 * g + 2][i] * sd[2], acc[mt][4 * g + 3][i] * sd[3]};
            *reinterpret_cast<f32x4*>(Y + (size_t)(row0 + m) * d + n) = v;
          }
        }
    }
  }
}

int prefill_mslots(int rows_cap, int E) { return (rows_cap + BM - 1) / BM + E; }

hipError_t launch_gate_up_prefill(const uint16_t* x, const int32_t* perm, const int32_t* offsets,
                                  const int8_t* w_gate, const int8_t* w_up, const uint16_t* scales,
                                  _Float16* H, int rows_cap, int d, int f, int E, hipStream_t stream) {
  dim3 grid(prefill_mslots(rows_cap, E), f / HALF, 1);
  hipLaunchKernelGGL(expert_prefill_kernel<true>, grid, dim3(kThreads), 0, stream, x, perm, offsets,
                     w_gate, w_up, scales, (void*)H, d, f, E, rows_cap);
  return hipGetLastError();
}

hipError_t launch_down_prefill(const _Float16* H, const int32_t* offsets, const int8_t* w_down,
                               const uint16_t* scales, float* Y, int splits, int rows_cap, int d,
                               int f, int E, hipStream_t stream) {
  dim3 grid(prefill_mslots(rows_cap, E), d / (2 * HALF), splits);
  hipLaunchKernelGGL(expert_prefill_kernel<false>, grid, dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint16_t*>(H), (const int32_t*)nullptr, offsets, w_down,
                     (const int8_t*)nullptr, scales, (void*)Y, d, f, E, rows_cap);
  return hipGetLastError();
}

}  // namespace moe
