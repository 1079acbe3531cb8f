// Expert FFN for large batches (T > 160), and for expert matrices of at most 2^23 weights at
// any batch size: grouped W8A16 GEMMs on the MFMA units.
// (Grok-1 Admin & Architecture Guide, section 3, MoE step 3, the gated GeLU expert
// gelu(linear(x)) * linear_v(x) -> linear_1; "Quantized weights": int8 weights
// dequantised as q * s with one scale per output channel, compute in bf16.)
//
// Two kernels, one per tile height:
//   * 256-row tiles (experts averaging more than 96 rows, e.g. prefill): expert_wide_kernel,
//     four wavefronts of 128 x 128 (described where it is defined);
//   * 128-row tiles (mid-size batches) and tiles of at most 64 rows: expert_prefill_kernel,
//     eight wavefronts of 64 x 128, described here.
// Both compute every output element with the same 32x32x16 MFMA sequence in k order, so a row
// gets the same bits whichever tile height its batch takes.
//
// expert_prefill_kernel: one workgroup (512 threads, 8 wavefronts in a 4 x 2 arrangement, two
// per SIMD) computes a 256-row x 256-column tile of one expert: for the gate/up kernel 128
// columns of gate and the same 128 of up (so the GeGLU is applied in registers), for the down
// kernel 256 columns of the down projection. Each wavefront owns 64 rows x 128 columns as
// 2 x 4 tiles of the 32x32x16 MFMA (128 fp32 accumulators per lane); the second
// wavefront on each SIMD covers the other's waits. The contraction runs in 64-deep slices:
//   * the next slice's activations (16 B per load) and int8 weights (one dword of 4
//     columns from each of 8 rows per thread and half-tile, through buffer loads whose
//     row offset is a scalar) are loaded into registers two slices ahead and written into
//     the other of two LDS buffers interleaved with the current slice's MFMAs (one
//     barrier per slice);
//   * the weights are converted int8 -> bf16 (gate/up) or fp16 (down) once per
//     workgroup, on the way into LDS, and stored transposed ([column][k]), so every MFMA
//     operand is one 16-byte LDS read; column 2 c + q of a 64-column group goes to LDS
//     row 32 q + c, which gives each lane 2 adjacent output columns in the epilogue.
// With 128-row tiles wavefronts 4-7 only move slices; a tile of at most 64 rows gives its
// 32x32 MFMA tiles to wavefronts 0-3, one per SIMD, so that all 4 SIMDs multiply, and moves
// only 64 activation rows per slice.
// Rows are gathered through the dispatch permutation (gate/up) or read in segment order
// (down). Tiles are assigned on the device: m-slots enumerate the m-tiles of all expert
// segments in expert order (read from offsets), surplus slots exit at once; the order of
// (m-slot, n-tile) over workgroups is XCD-aware (tile_of).
// Scales, GeLU and the fp16 rounding of h are applied in fp32 after the contraction.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int BM = 256;         // rows per workgroup tile (LDS is sized for it; a launch may use 128)
constexpr int BK = 64;          // contraction depth per slice
constexpr int HALF = 128;       // columns per weight half-tile
constexpr int LDS_LD = BK + 8;  // 16-bit elements per LDS row (16-byte pad)
constexpr int kThreads = 512;
constexpr int A_ELEMS = BM * LDS_LD;
constexpr int B_ELEMS = 2 * HALF * LDS_LD;
constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;  // 36864 x 2 B = 72 KiB per buffer
constexpr int kBufferFlags = 0x00020000;
}  // namespace

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename T>
struct Mfma32;
// D(32x32 fp32) += A(32x16) * B(16x32). Lane l supplies A row (l % 32) and B column
// (l % 32) with the 8 k-values of k-group (l / 32); D element i of lane l is row
// 8 (i / 4) + 4 (l / 32) + (i % 4), column l % 32.
template <>
struct Mfma32<bf16x8> {
  static __device__ __forceinline__ f32x16 run(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Mfma32<f16x8> {
  static __device__ __forceinline__ f32x16 run(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// (expert, first row, rows) of m-slot `slot` with bm-row tiles, or false when the slot is surplus.
__device__ __forceinline__ bool find_tile(const int32_t* offsets, int E, int slot, int bm, int& e, int& row0,
                                          int& rows) {
  int s = slot;
  for (int ee = 0; ee < E; ++ee) {
    const int M = offsets[ee + 1] - offsets[ee];
    const int nt = (M + bm - 1) / bm;
    if (s < nt) {
      e = ee;
      row0 = offsets[ee] + s * bm;
      rows = min(bm, M - s * bm);
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

// Column JJ (0..3) of the thread's 4 columns over its 8 rows, converted, as one 16-byte
// LDS write at row `row` (k offset koff).
template <bool kGateUp, int JJ>
__device__ __forceinline__ void store_col(uint16_t* sB, int row, int koff, const uint32_t (&w)[8]) {
  using P = PrefillTraits<kGateUp>;
  u32x4 v;
  v.x = P::pack(sbyte<JJ>(w[0]), sbyte<JJ>(w[1]));
  v.y = P::pack(sbyte<JJ>(w[2]), sbyte<JJ>(w[3]));
  v.z = P::pack(sbyte<JJ>(w[4]), sbyte<JJ>(w[5]));
  v.w = P::pack(sbyte<JJ>(w[6]), sbyte<JJ>(w[7]));
  *reinterpret_cast<u32x4*>(sB + (size_t)row * LDS_LD + koff) = v;
}

// kGateUp: A = x rows gathered by perm (bf16), B halves = gate / up at columns n0..n0+127,
//          output H fp16 = gelu_tanh(s_g g) * (s_u u).
// !kGateUp: A = H rows (fp16), B halves = down columns n0..n0+127 and n0+128..n0+255,
//          output Y fp32 (part blockIdx.z of the contraction) = s_d y.
// Workgroup -> tile order. Workgroups go to the 8 XCDs round-robin by linear id, so XCD
// x runs ids x, x + 8, ... in order. The XCDs form an xm x xn grid: XCD x owns the m-slots
// congruent to x / xn (mod xm) and the x % xn-th contiguous block of n-tiles, and walks
// its n-tiles in groups of `ngroup`, m-slot by m-slot inside a group. So each weight tile
// is streamed from HBM by xm XCDs only (xm = 1 for gate/up), the activation tiles are
// re-read from the last-level cache, and the 32 workgroups an XCD holds at once share a
// few activation and weight tiles in its L2.
struct TileOrder {
  int nslots, ntiles, xm, xn, ngroup;
  int ncu;  // compute units: one workgroup of this kernel fits a CU (144 KiB of LDS)
};

__device__ __forceinline__ void tile_of(int w, const TileOrder& o, int& mslot, int& ntile) {
  const int xcd = w & 7, l = w >> 3;
  const int xi = xcd / o.xn, xj = xcd - xi * o.xn;
  const int ms = o.nslots / o.xm;            // m-slots per XCD
  const int nblk = o.ntiles / o.xn;          // n-tiles per XCD
  const int per_group = ms * o.ngroup;
  const int g = l / per_group, rem = l - g * per_group;
  mslot = xi + o.xm * (rem / o.ngroup);
  ntile = xj * nblk + g * o.ngroup + rem % o.ngroup;
}

// Parts of the down contraction when the kernel may choose 1, 2 or 4 (at most maxp): the live
// workgroups run in rounds of ncu (one per CU), so p parts take ceil(p r) / p full-length
// rounds for r = live tiles / ncu; more parts fill a ragged last round better, but each extra
// one costs an fp32 partial, 8 bytes per output element (written, then read by the combine)
// at about 5 TB/s against 2 f FLOPs at about 1 PFLOP/s, i.e. about 800 / f of the kernel's time.
// Four parts only while one part cannot fill a round (r <= 1): beyond that the model overrates
// quarter-length workgroups (measured at 1024 tokens: 4 parts 0.6% slower than the 2 it kept).
__device__ __forceinline__ int down_parts(const int32_t* offsets, int E, int bm, int ntiles, int ncu, int f,
                                          int maxp) {
  int live = 0;
  for (int e = 0; e < E; ++e) live += (offsets[e + 1] - offsets[e] + bm - 1) / bm;
  if (live == 0) return 1;
  const float r1 = (float)(live * ntiles) / (float)ncu;
  int best = 1;
  float bt = ceilf(r1) / r1;
  for (int p = 2; p <= maxp && (p == 2 || r1 <= 1.0f); p *= 2) {
    const float rp = (float)p * r1;
    const float t = ceilf(rp) / rp + (float)(p - 1) * 800.0f / (float)f;
    if (t < bt) best = p, bt = t;
  }
  return best;
}

// kBM: rows per tile, 256 or 128.
template <bool kGateUp, int kBM>
__global__ __launch_bounds__(kThreads) void expert_prefill_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const int8_t* __restrict__ B0,
    const int8_t* __restrict__ B1, const uint16_t* __restrict__ scales, void* __restrict__ out,
    int d, int f, int E, int rows_cap, TileOrder order, int* __restrict__ splits_used) {
  using Frag = typename PrefillTraits<kGateUp>::Frag;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE_ELEMS];

  int parts = gridDim.z;
  if (!kGateUp && splits_used != nullptr) {  // launched with 2 or 4 parts: keep 1, 2 or 4
    parts = down_parts(offsets, E, kBM, order.ntiles, order.ncu, f, (int)gridDim.z);
    if (blockIdx.x == 0 && blockIdx.z == 0 && threadIdx.x == 0) *splits_used = parts;
    if ((int)blockIdx.z >= parts) return;
  }
  int mslot, ntile;
  tile_of(blockIdx.x, order, mslot, ntile);
  int e, row0, rows;
  if (!find_tile(offsets, E, mslot, kBM, e, row0, rows)) return;

  const int K = kGateUp ? d : f;  // contraction length
  const int N = kGateUp ? f : d;  // columns of each weight matrix
  const int kspan = K / parts, kbeg = blockIdx.z * kspan;
  const int n0 = ntile * (kGateUp ? HALF : 2 * HALF);
  const uint32_t ldb = (uint32_t)N;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // 4 x 2 wavefronts, 64 rows x 128 columns each

  // ---- global -> register loads of one slice
  // A: rows tid / 8 + 64 i (i < kBM / 64), 16-byte chunk tid % 8 of the slice
  constexpr int kArows = kBM / 64;
  const uint16_t* arow[kArows];
#pragma unroll
  for (int i = 0; i < kArows; ++i) {
    const int m = min(tid / 8 + 64 * i, rows - 1);  // rows past the tile end repeat a live row
    const size_t src_row = kGateUp ? (size_t)perm[row0 + m] : (size_t)(row0 + m);
    arow[i] = A + src_row * K + kbeg + 8 * (tid % 8);
  }
  // B: half hb = tid / 256, columns 4 cg .. 4 cg + 3 of it, rows 8 kg .. 8 kg + 7 of the slice
  const int cg = tid % 32, kg = (tid / 32) % 8;
  const int hb = __builtin_amdgcn_readfirstlane(tid / 256);  // uniform per wavefront
  const size_t ebytes = (size_t)d * f;
  const int8_t* hbase0 = B0 + (size_t)e * ebytes;
  const int8_t* hbase1 = kGateUp ? B1 + (size_t)e * ebytes : hbase0;
  const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(hb == 0 ? hbase0 : hbase1), (short)0, (int)ebytes, kBufferFlags);
  const uint32_t bvoff = (uint32_t)(8 * kg) * ldb + (uint32_t)(n0 + 4 * cg) + (kGateUp ? 0u : (uint32_t)(HALF * hb));
  // LDS row of the thread's column jj: half h, group cg / 16, column 4 (cg % 16) + jj
  //   -> h * 128 + (cg / 16) * 64 + 32 (jj % 2) + 2 (cg % 16) + jj / 2
  const int brow = (cg / 16) * 64 + 2 * (cg % 16);

  // two register stages: the loads of slices i + 1 and i + 2 are in flight while slice i
  // is multiplied out of LDS
  u32x4 ra[2][kArows];
  uint32_t rb[2][8];
  auto gload = [&](auto stage, int kk) {
    constexpr int rs = decltype(stage)::value;
#pragma unroll
    for (int i = 0; i < kArows; ++i) ra[rs][i] = *reinterpret_cast<const u32x4*>(arow[i] + kk);
    const uint32_t sbase = (uint32_t)(kbeg + kk) * ldb;
#pragma unroll
    for (int r = 0; r < 8; ++r) rb[rs][r] = __builtin_amdgcn_raw_buffer_load_b32(br, bvoff, sbase + r * ldb, 0);
  };
  auto lds_store = [&](auto stage, uint16_t* st) {
    constexpr int rs = decltype(stage)::value;
    uint16_t* sA = st;
    uint16_t* sB = st + A_ELEMS;
#pragma unroll
    for (int i = 0; i < kArows; ++i)
      *reinterpret_cast<u32x4*>(sA + (size_t)(tid / 8 + 64 * i) * LDS_LD + 8 * (tid % 8)) = ra[rs][i];
    store_col<kGateUp, 0>(sB, hb * HALF + brow + 0, 8 * kg, rb[rs]);
    store_col<kGateUp, 1>(sB, hb * HALF + brow + 32, 8 * kg, rb[rs]);
    store_col<kGateUp, 2>(sB, hb * HALF + brow + 1, 8 * kg, rb[rs]);
    store_col<kGateUp, 3>(sB, hb * HALF + brow + 33, 8 * kg, rb[rs]);
  };
  const std::integral_constant<int, 0> R0{};
  const std::integral_constant<int, 1> R1{};

  // ---- wavefront tile: rows wm * 64 + 32 mt + (lane % 32); B tiles nt: LDS rows
  //   gate/up: (nt / 2) * 128 + wn * 64 + 32 (nt % 2) + (lane % 32)   (nt 0,1 gate; 2,3 up)
  //   down:    wn * 128 + (nt / 2) * 64 + 32 (nt % 2) + (lane % 32)
  int bro[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
    bro[nt] = (kGateUp ? (nt >> 1) * HALF + wn * 64 : wn * HALF + (nt >> 1) * 64) + 32 * (nt & 1) + (lane & 31);
  const int kq = 8 * (lane >> 5);
  const int arl = wm * 64 + (lane & 31);

  f32x16 acc[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.0f;

  const int nslices = kspan / BK;
  Frag af[2][2], bfr[2][4];
  auto read_frags = [&](const uint16_t* st, int buf, int ks) {
    const uint16_t* sA = st;
    const uint16_t* sB = st + A_ELEMS;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      af[buf][mt] = __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(sA + (size_t)(arl + 32 * mt) * LDS_LD + ks + kq));
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      bfr[buf][nt] = __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(sB + (size_t)bro[nt] * LDS_LD + ks + kq));
  };
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) acc[mt][nt] = Mfma32<Frag>::run(af[buf][mt], bfr[buf][nt], acc[mt][nt]);
  };
  // One slice: 4 sub-steps of 16 k; the fragments of sub-step kk + 1 are read before the
  // MFMAs of sub-step kk.
  auto slice = [&](const uint16_t* cur) {
    read_frags(cur, 0, 0);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      if (kk + 1 < BK / 16) read_frags(cur, (kk + 1) & 1, (kk + 1) * 16);
      mfmas(kk & 1);
    }
  };

  // Instruction order of one slice plus the next slice's LDS store: every MFMA is followed
  // by one fragment read, two conversion instructions and one LDS write, so that the store
  // of the next slice runs in the shadow of this slice's MFMAs instead of after them (the
  // two wavefronts of a SIMD reach the store phase together, between the same barriers).
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
    }
  };

  // slices it (even) and it + 1 (odd) per trip; nslices is even (the launchers reject a
  // contraction part that is not a multiple of 128). The loads and
  // stores are unconditional (past the end they re-read the last slice into a buffer that
  // is not read again): a conditional load would make the compiler's wait counts at the
  // stores assume the path without it, i.e. wait for the loads just issued.
  uint16_t* L0 = lds;
  uint16_t* L1 = lds + STAGE_ELEMS;
  const int klast = (nslices - 1) * BK;
  gload(R0, 0);
  gload(R1, min(BK, klast));
  lds_store(R0, L0);
  __syncthreads();
  if constexpr (kBM == 128) {
    if (rows <= 64) {  // uniform per workgroup
      // Tiles of at most 64 rows: the same 32x32 MFMA tiles as below (so the same sums, bit
      // for bit), taken by wavefronts 0-3, one per SIMD, instead of the two of row group 0;
      // wavefronts 4-7 only move slices. Wavefront c (0-3) takes both 32-row tiles and
      //   gate/up: the gate and up tiles at LDS rows (c / 2) * 64 + 32 (c % 2) (+ 128 for
      //            up), i.e. column 2 (lane % 32) + c % 2 of 64-column group c / 2;
      //   down:    LDS rows (c / 2) * 128 + (c % 2) * 64 + 32 q (q = 0, 1), i.e. columns
      //            2 (lane % 32) + q of that group.
      // Each weight tile is read by one wavefront (by two when 8 wavefronts took 32 rows
      // each: 1.5x the LDS reads, measured 4% slower), and only the first 64 activation rows
      // are moved after the first slice.
      const int c = wave & 3;
      int nbro[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        nbro[j] = (kGateUp ? j * HALF + (c >> 1) * 64 + 32 * (c & 1) : (c >> 1) * HALF + (c & 1) * 64 + 32 * j) +
                  (lane & 31);
      const int narl = lane & 31;
      f32x16 accn[2][2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 16; ++i) accn[mt][j][i] = 0.0f;
      Frag na[2][2], nb[2][2];
      auto read_n = [&](const uint16_t* st, int buf, int ks) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          na[buf][mt] =
              __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(st + (size_t)(narl + 32 * mt) * LDS_LD + ks + kq));
#pragma unroll
        for (int j = 0; j < 2; ++j)
          nb[buf][j] =
              __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(st + A_ELEMS + (size_t)nbro[j] * LDS_LD + ks + kq));
      };
      auto slice_n = [&](const uint16_t* cur) {
        read_n(cur, 0, 0);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
          if (kk + 1 < BK / 16) read_n(cur, (kk + 1) & 1, (kk + 1) * 16);
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) accn[mt][j] = Mfma32<Frag>::run(na[kk & 1][mt], nb[kk & 1][j], accn[mt][j]);
        }
      };
      auto gload_n = [&](auto stage, int kk) {
        constexpr int rs = decltype(stage)::value;
        ra[rs][0] = *reinterpret_cast<const u32x4*>(arow[0] + kk);
        const uint32_t sbase = (uint32_t)(kbeg + kk) * ldb;
#pragma unroll
        for (int r = 0; r < 8; ++r) rb[rs][r] = __builtin_amdgcn_raw_buffer_load_b32(br, bvoff, sbase + r * ldb, 0);
      };
      auto store_n = [&](auto stage, uint16_t* st) {
        constexpr int rs = decltype(stage)::value;
        uint16_t* sB = st + A_ELEMS;
        *reinterpret_cast<u32x4*>(st + (size_t)(tid / 8) * LDS_LD + 8 * (tid % 8)) = ra[rs][0];
        store_col<kGateUp, 0>(sB, hb * HALF + brow + 0, 8 * kg, rb[rs]);
        store_col<kGateUp, 1>(sB, hb * HALF + brow + 32, 8 * kg, rb[rs]);
        store_col<kGateUp, 2>(sB, hb * HALF + brow + 1, 8 * kg, rb[rs]);
        store_col<kGateUp, 3>(sB, hb * HALF + brow + 33, 8 * kg, rb[rs]);
      };
      if (__builtin_amdgcn_readfirstlane(wave < 4 ? 1 : 0)) {  // uniform per wavefront
        for (int it = 0; it < nslices; it += 2) {
          gload_n(R0, min((it + 2) * BK, klast));
          slice_n(L0);
          store_n(R1, L1);
          __syncthreads();
          gload_n(R1, min((it + 3) * BK, klast));
          slice_n(L1);
          store_n(R0, L0);
          __syncthreads();
        }
      } else {
        for (int it = 0; it < nslices; it += 2) {
          gload_n(R0, min((it + 2) * BK, klast));
          store_n(R1, L1);
          __syncthreads();
          gload_n(R1, min((it + 3) * BK, klast));
          store_n(R0, L0);
          __syncthreads();
        }
        return;
      }
      const uint16_t* sc = scales + (size_t)e * (2 * (size_t)f + d);
      const int rq = 4 * (lane >> 5);
      if constexpr (kGateUp) {
        const int n = n0 + (c >> 1) * 64 + 2 * (lane & 31) + (c & 1);
        const float sg = bf16_bits_to_float(sc[n]), su = bf16_bits_to_float(sc[f + n]);
        _Float16* H = reinterpret_cast<_Float16*>(out);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int m = 32 * mt + 8 * (i >> 2) + rq + (i & 3);
            if (m < rows)
              H[(size_t)(row0 + m) * f + n] = (_Float16)(gelu_tanh(accn[mt][0][i] * sg) * (accn[mt][1][i] * su));
          }
      } else {
        float* Y = reinterpret_cast<float*>(out) + (size_t)blockIdx.z * rows_cap * d;
        const int n = n0 + (c >> 1) * HALF + (c & 1) * 64 + 2 * (lane & 31);
        const uint32_t s2 = *reinterpret_cast<const uint32_t*>(sc + 2 * (size_t)f + n);
        const float sd0 = bf16_bits_to_float(s2 & 0xFFFFu), sd1 = bf16_bits_to_float(s2 >> 16);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int m = 32 * mt + 8 * (i >> 2) + rq + (i & 3);
            if (m < rows) {
              u32x2 v = {__float_as_uint(accn[mt][0][i] * sd0), __float_as_uint(accn[mt][1][i] * sd1)};
              *reinterpret_cast<u32x2*>(Y + (size_t)(row0 + m) * d + n) = v;
            }
          }
      }
      return;
    }
  }
  if (__builtin_amdgcn_readfirstlane(wm * 64 < rows ? 1 : 0)) {  // uniform per wavefront
    for (int it = 0; it < nslices; it += 2) {
      gload(R0, min((it + 2) * BK, klast));
      slice(L0);
      lds_store(R1, L1);
      interleave();
      __syncthreads();
      gload(R1, min((it + 3) * BK, klast));
      slice(L1);
      lds_store(R0, L0);
      interleave();
      __syncthreads();
    }
  } else {
    // every row of this wavefront's 64 is past the tile end (the last tile of a segment):
    // it only moves the slices, with the same barriers, and leaves the MFMA pipe of its SIMD
    // to the other wavefront there (waves w and w + 4 share a SIMD: wm 0 / 2 and 1 / 3)
    for (int it = 0; it < nslices; it += 2) {
      gload(R0, min((it + 2) * BK, klast));
      lds_store(R1, L1);
      __syncthreads();
      gload(R1, min((it + 3) * BK, klast));
      lds_store(R0, L0);
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds, per tile (mt, nt), rows wm*64 + 32 mt + 8 (i/4) + 4 (lane/32)
  //      + i % 4 (i = 0..15) of column 2 (lane % 32) + (nt % 2) of its 64-column group
  const uint16_t* sc = scales + (size_t)e * (2 * (size_t)f + d);
  const int c2 = 2 * (lane & 31);
  const int rq = 4 * (lane >> 5);
  if constexpr (kGateUp) {
    const int n = n0 + wn * 64 + c2;
    const uint32_t g2 = *reinterpret_cast<const uint32_t*>(sc + n);
    const uint32_t u2 = *reinterpret_cast<const uint32_t*>(sc + f + n);
    const float sg0 = bf16_bits_to_float(g2 & 0xFFFFu), sg1 = bf16_bits_to_float(g2 >> 16);
    const float su0 = bf16_bits_to_float(u2 & 0xFFFFu), su1 = bf16_bits_to_float(u2 >> 16);
    _Float16* H = reinterpret_cast<_Float16*>(out);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = wm * 64 + 32 * mt + 8 * (i >> 2) + rq + (i & 3);
        if (m < rows) {
          const float h0 = gelu_tanh(acc[mt][0][i] * sg0) * (acc[mt][2][i] * su0);
          const float h1 = gelu_tanh(acc[mt][1][i] * sg1) * (acc[mt][3][i] * su1);
          *reinterpret_cast<uint32_t*>(H + (size_t)(row0 + m) * f + n) = pack_f16_rne(h0, h1);
        }
      }
  } else {
    float* Y = reinterpret_cast<float*>(out) + (size_t)blockIdx.z * rows_cap * d;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int n = n0 + wn * HALF + g * 64 + c2;
      const uint32_t s2 = *reinterpret_cast<const uint32_t*>(sc + 2 * (size_t)f + n);
      const float sd0 = bf16_bits_to_float(s2 & 0xFFFFu), sd1 = bf16_bits_to_float(s2 >> 16);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = wm * 64 + 32 * mt + 8 * (i >> 2) + rq + (i & 3);
          if (m < rows) {
            u32x2 v = {__float_as_uint(acc[mt][2 * g][i] * sd0), __float_as_uint(acc[mt][2 * g + 1][i] * sd1)};
            *reinterpret_cast<u32x2*>(Y + (size_t)(row0 + m) * d + n) = v;
          }
        }
    }
  }
}

// ---------------------------------------------------------------------------------------
// expert_wide_kernel, for 256-row tiles: four wavefronts, one per SIMD, each 128 rows x 128
// columns.
//
// A wavefront multiplies 4 x 4 tiles of the 32x32x16 MFMA (256 fp32 accumulators per lane,
// held in the accumulation registers), so each fragment read from LDS feeds four MFMAs
// instead of two (half the LDS bytes per FLOP of a 64-row wavefront tile). One workgroup
// (256 threads) holds a 256 x 256 tile: for gate/up 128 columns of gate and the same 128 of
// up, for down 256 columns. The contraction runs in 64-deep slices through two LDS stages:
//   * while slice i is multiplied, the weights of slice i + 3 (four register sets: they
//     stream from HBM and have the longest latency) and the activations of slice i + 2 (two
//     sets) are loaded into registers, the loads spread over the slice (back-to-back 1 KB
//     loads stall the in-order wavefront on the memory pipeline), and slice i + 1 is
//     converted and written into the other LDS stage in the shadow of slice i's first 48
//     MFMAs;
//   * one barrier per slice, after the first MFMA of its last 16-deep step: the fragments
//     of the next slice's first step are read while that step's other MFMAs run, so no
//     MFMA waits on a read issued after the barrier;
//   * the order of MFMAs, LDS reads, conversions, LDS writes and global loads inside a slice
//     is fixed in the source (scheduling fences between MFMA slots).
// Weights: each thread loads 8 columns x 8 rows of one matrix (eight 8-byte buffer loads),
// converts them exactly (int8 -> bf16 for gate/up, fp16 for down) and writes each column's
// 8 values as one 16-byte LDS row segment ([column][k] layout). Column 8 g + 2 a + q
// (g < 16, a < 4, q < 2) of a 128-column half goes to LDS row 64 q + 16 a + g: a write
// instruction then covers 16 consecutive LDS rows (no bank conflicts), and the two columns
// 8 g + 2 a and 8 g + 2 a + 1 land in the same lane of two MFMA tiles, so the epilogue
// stores adjacent pairs. Every output element sees the same MFMA sequence as in the
// 8-wavefront kernel (32x32x16 steps in k order), so both give the same bits.
namespace {
constexpr int WBM = 256, WBK = 64, WLD = WBK + 8;
constexpr int kWideThreads = 256;
constexpr int W_A_ELEMS = WBM * WLD;
constexpr int W_STAGE = W_A_ELEMS + 256 * WLD;  // 73728 B per stage, two stages
}  // namespace

// body(integral_constant<int, I>) for I = B .. E - 1, each index a compile-time constant
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& body) {
  if constexpr (B < E) {
    body(std::integral_constant<int, B>{});
    static_for<B + 1, E>(body);
  }
}

// Column jj (0..7) of the thread's 8 weight columns over its 8 rows (byte jj % 4 of word
// jj / 4 of each row's 8 bytes), converted and packed: element r <- row r.
template <bool kGateUp, int JJ, int P>
__device__ __forceinline__ uint32_t wide_quarter(const u32x2 (&w)[8]) {
  using T = PrefillTraits<kGateUp>;
  constexpr int W = JJ / 4, BY = JJ % 4;
  return T::pack(sbyte<BY>(w[2 * P][W]), sbyte<BY>(w[2 * P + 1][W]));
}

template <bool kGateUp, int JJ>
__device__ __forceinline__ u32x4 wide_col(const u32x2 (&w)[8]) {
  using P = PrefillTraits<kGateUp>;
  constexpr int W = JJ / 4, BY = JJ % 4;
  u32x4 v;
  v.x = P::pack(sbyte<BY>(w[0][W]), sbyte<BY>(w[1][W]));
  v.y = P::pack(sbyte<BY>(w[2][W]), sbyte<BY>(w[3][W]));
  v.z = P::pack(sbyte<BY>(w[4][W]), sbyte<BY>(w[5][W]));
  v.w = P::pack(sbyte<BY>(w[6][W]), sbyte<BY>(w[7][W]));
  return v;
}

template <bool kGateUp>
__global__ __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void expert_wide_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets,
    const int8_t* __restrict__ B0, const int8_t* __restrict__ B1, const uint16_t* __restrict__ scales,
    void* __restrict__ out, int d, int f, int E, int rows_cap, TileOrder order, int* __restrict__ splits_used) {
  using Frag = typename PrefillTraits<kGateUp>::Frag;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * W_STAGE];

  int parts = gridDim.z;
  if (!kGateUp && splits_used != nullptr) {  // launched with 2 or 4 parts: keep 1, 2 or 4
    parts = down_parts(offsets, E, WBM, order.ntiles, order.ncu, f, (int)gridDim.z);
    if (blockIdx.x == 0 && blockIdx.z == 0 && threadIdx.x == 0) *splits_used = parts;
    if ((int)blockIdx.z >= parts) return;
  }
  int mslot, ntile;
  tile_of(blockIdx.x, order, mslot, ntile);
  int e, row0, rows;
  if (!find_tile(offsets, E, mslot, WBM, e, row0, rows)) return;

  const int K = kGateUp ? d : f;  // contraction length
  const int N = kGateUp ? f : d;  // columns of each weight matrix
  const int kspan = K / parts, kbeg = blockIdx.z * kspan;
  const int n0 = ntile * (kGateUp ? HALF : 2 * HALF);
  const uint32_t ldb = (uint32_t)N;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // 2 x 2 wavefronts of 128 x 128

  // ---- A: rows tid / 8 + 32 i (i < 8), 16-byte chunk tid % 8 of the slice
  const uint16_t* arow[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = min(tid / 8 + 32 * i, rows - 1);  // rows past the tile end repeat a live row
    const size_t src_row = kGateUp ? (size_t)perm[row0 + m] : (size_t)(row0 + m);
    arow[i] = A + src_row * K + kbeg + 8 * (tid % 8);
  }
  // ---- B: half hb = wave / 2 (gate / up, or columns 0-127 / 128-255 of down), column group
  //      g (columns 8 g .. 8 g + 7 of the half), rows 8 kg .. 8 kg + 7 of the slice
  const int hb = wave >> 1;
  const int g = lane & 15, kg = (lane >> 4) + 4 * (wave & 1);
  const size_t ebytes = (size_t)d * f;
  const int8_t* bmat = (kGateUp && hb == 1 ? B1 : B0) + (size_t)e * ebytes;
  const __amdgpu_buffer_rsrc_t br =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(bmat), (short)0, (int)ebytes, kBufferFlags);
  const uint32_t bvoff = (uint32_t)(8 * kg) * ldb + (uint32_t)(n0 + 8 * g) + (kGateUp ? 0u : (uint32_t)(HALF * hb));

  // activations: two register sets (slice it + 2 is loaded while slice it + 1 is written to
  // LDS); weights: four (slice it + 3 is loaded, two slices before its conversion, since the
  // weights stream from HBM and their loads have the longest latency)
  u32x4 ra[2][8];
  u32x2 rb[4][8];
  auto gload_a = [&](auto set, int i, int kk) {
    constexpr int rs = decltype(set)::value;
    ra[rs][i] = *reinterpret_cast<const u32x4*>(arow[i] + kk);
  };
  auto gload_b = [&](auto set, int r, int kk) {
    constexpr int rs = decltype(set)::value;
    const uint32_t sbase = (uint32_t)(kbeg + kk) * ldb;
    rb[rs][r] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(br, bvoff, sbase + r * ldb, 0));
  };
  // LDS addresses (16-bit element offsets within a stage)
  const int a_st = (tid / 8) * WLD + 8 * (tid % 8);                   // + 32 i rows
  const int b_st = W_A_ELEMS + (hb * HALF + g) * WLD + 8 * kg;        // + (64 q + 16 a) rows
  auto store_a = [&](auto set, uint16_t* st, int i) {
    constexpr int rs = decltype(set)::value;
    *reinterpret_cast<u32x4*>(st + a_st + 32 * i * WLD) = ra[rs][i];
  };
  auto store_b = [&](uint16_t* st, int jj, u32x4 v) {
    const int q = jj & 1, a = jj >> 1;
    *reinterpret_cast<u32x4*>(st + b_st + (64 * q + 16 * a) * WLD) = v;
  };
  // a whole slice (A rows of register set sa, B columns of set sb) into an LDS stage
  auto store_slice = [&](auto sa, auto sb, uint16_t* st) {
    constexpr int rb_set = decltype(sb)::value;
#pragma unroll
    for (int i = 0; i < 8; ++i) store_a(sa, st, i);
    static_for<0, 8>([&](auto J) { store_b(st, J.value, wide_col<kGateUp, J.value>(rb[rb_set])); });
  };

  // ---- fragments: A tiles mt at LDS rows wm*128 + 32 mt + lane % 32; B tiles j at LDS rows
  //   gate/up: (j / 2) * 128 + (j % 2) * 64 + 32 wn + lane % 32 (gate q=0, q=1, up q=0, q=1)
  //   down:    128 wn + 32 j + lane % 32
  const int kq = 8 * (lane >> 5);
  const int afo = (wm * 128 + (lane & 31)) * WLD + kq;
  int bfo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    bfo[j] = W_A_ELEMS + ((kGateUp ? (j >> 1) * 128 + (j & 1) * 64 + 32 * wn : 128 * wn + 32 * j) + (lane & 31)) * WLD + kq;
  Frag fa[2][4], fb[2][4];
  auto read_frag = [&](auto buf, const uint16_t* st, int ks, int j) {
    constexpr int fbuf = decltype(buf)::value;
    // order: B0, A0, A1, A2, A3, B1, B2, B3 (the first MFMAs of a step use A0..A3 with B0)
    if (j == 0) fb[fbuf][0] = __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(st + bfo[0] + ks));
    else if (j <= 4) fa[fbuf][j - 1] = __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(st + afo + (32 * (j - 1)) * WLD + ks));
    else fb[fbuf][j - 4] = __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(st + bfo[j - 4] + ks));
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.0f;

  const int nslices = kspan / WBK;  // even (checked by the launchers)
  const int klast = (nslices - 1) * WBK;
  uint16_t* S0 = lds;
  uint16_t* S1 = lds + W_STAGE;
  const std::integral_constant<int, 0> C0{};
  const std::integral_constant<int, 1> C1{};
  const std::integral_constant<int, 2> C2{};
  const std::integral_constant<int, 3> C3{};

  // prologue: activations of slices 0, 1 and weights of slices 0, 1, 2 into their register
  // sets (slice j: activation set j % 2, weight set j % 4), slice 0 into stage 0, first fragments
#pragma unroll
  for (int r = 0; r < 8; ++r) gload_b(C0, r, 0);
#pragma unroll
  for (int i = 0; i < 8; ++i) gload_a(C0, i, 0);
#pragma unroll
  for (int r = 0; r < 8; ++r) gload_b(C1, r, min(WBK, klast));
#pragma unroll
  for (int r = 0; r < 8; ++r) gload_b(C2, r, min(2 * WBK, klast));
#pragma unroll
  for (int i = 0; i < 8; ++i) gload_a(C1, i, min(WBK, klast));
  store_slice(C0, C0, S0);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 8; ++j) read_frag(C0, S0, 0, j);

  // One slice it (q4 = it % 4; LDS stage and activation set q4 % 2): 64 MFMA slots (4 steps x
  // 16, nt-major), with the other work placed in them:
  //   steps 0-2, every other slot: one fragment read of the next step (this stage)
  //   slots 0-7: the 8 weight loads of slice it + 3 (weight set (q4 + 3) % 4)
  //   slots 16, 18, .. 30: the 8 activation loads of slice it + 2 (activation set q4 % 2)
  //   slots 8-39: one quarter column of slice it + 1's weights (set (q4 + 1) % 4) converted per
  //     slot; each column written to the other stage in the slot after its last quarter; the
  //     activation rows of slice it + 1 written in between
  //   after the first MFMA of step 3: wait for this wavefront's LDS work, barrier; then every
  //     other slot reads a fragment of the next slice's first step (the other stage)
  auto run_slice = [&](auto q4_sel, int it) {
    constexpr int q4 = decltype(q4_sel)::value;
    const std::integral_constant<int, q4 & 1> LDA{};          // activations of slice it + 2
    const std::integral_constant<int, 1 - (q4 & 1)> STA{};    // activations of slice it + 1
    const std::integral_constant<int, (q4 + 3) & 3> LDB{};    // weights of slice it + 3
    constexpr int stb = (q4 + 1) & 3;                         // weights of slice it + 1
    uint16_t* cur = (q4 & 1) ? S1 : S0;
    uint16_t* nxt = (q4 & 1) ? S0 : S1;
    const int kload_a = min((it + 2) * WBK, klast);
    const int kload_b = min((it + 3) * WBK, klast);
    u32x4 col;  // the weight column being converted
    static_for<0, 64>([&](auto S) {
      constexpr int s = decltype(S)::value;
      constexpr int kk = s >> 4, m = s & 15;
      constexpr int nt = m >> 2, mt = m & 3;
      constexpr int fbuf = kk & 1;
      // the MFMA of this slot
      acc[mt][nt] = Mfma32<Frag>::run(fa[fbuf][mt], fb[fbuf][nt], acc[mt][nt]);
      if constexpr (s == 48) {
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
      }
      // fragment reads: steps 0-2 read step kk + 1 of this slice, step 3 step 0 of the next
      if constexpr ((m & 1) == 0) {
        constexpr int j = m >> 1;
        if constexpr (kk == 3)
          read_frag(C0, nxt, 0, j);
        else
          read_frag(std::integral_constant<int, 1 - fbuf>{}, cur, 16 * (kk + 1), j);
      }
      if constexpr (s < 8) gload_b(LDB, s, kload_b);
      if constexpr (s >= 16 && s < 32 && (s & 1) == 0) gload_a(LDA, (s - 16) >> 1, kload_a);
      // the column's write comes before the next column's first quarter reuses `col`
      if constexpr (s >= 12 && s <= 40 && (s & 3) == 0) store_b(nxt, (s - 12) >> 2, col);
      if constexpr (s >= 8 && s < 40) {
        constexpr int q = s - 8, jj = q >> 2, p = q & 3;
        const uint32_t v = wide_quarter<kGateUp, jj, p>(rb[stb]);
        if constexpr (p == 0) col.x = v;
        if constexpr (p == 1) col.y = v;
        if constexpr (p == 2) col.z = v;
        if constexpr (p == 3) col.w = v;
        if constexpr (p == 1) store_a(STA, nxt, jj);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // the same loads, writes and barriers without MFMAs (wavefronts whose rows are all past the
  // end of the tile)
  auto move_slice = [&](auto q4_sel, int it) {
    constexpr int q4 = decltype(q4_sel)::value;
    const std::integral_constant<int, q4 & 1> LDA{};
    const std::integral_constant<int, 1 - (q4 & 1)> STA{};
    const std::integral_constant<int, (q4 + 3) & 3> LDB{};
    const std::integral_constant<int, (q4 + 1) & 3> STB{};
    uint16_t* nxt = (q4 & 1) ? S0 : S1;
    const int kload_a = min((it + 2) * WBK, klast);
    const int kload_b = min((it + 3) * WBK, klast);
#pragma unroll
    for (int r = 0; r < 8; ++r) gload_b(LDB, r, kload_b);
#pragma unroll
    for (int i = 0; i < 8; ++i) gload_a(LDA, i, kload_a);
    store_slice(STA, STB, nxt);
    __syncthreads();
  };

  if (__builtin_amdgcn_readfirstlane(wm * 128 < rows ? 1 : 0)) {  // uniform per wavefront
    int it = 0;
    for (; it + 4 <= nslices; it += 4) {
      run_slice(C0, it);
      run_slice(C1, it + 1);
      run_slice(C2, it + 2);
      run_slice(C3, it + 3);
    }
    if (it < nslices) {  // two slices left
      run_slice(C0, it);
      run_slice(C1, it + 1);
    }
  } else {
    // every row of this wavefront's 128 is past the tile end (the last tile of a segment): it
    // only moves slices, with the same barriers, and issues no MFMAs
    int it = 0;
    for (; it + 4 <= nslices; it += 4) {
      move_slice(C0, it);
      move_slice(C1, it + 1);
      move_slice(C2, it + 2);
      move_slice(C3, it + 3);
    }
    if (it < nslices) {
      move_slice(C0, it);
      move_slice(C1, it + 1);
    }
    return;
  }

  // ---- epilogue: lane holds, per tile (mt, j), rows wm*128 + 32 mt + 8 (i/4) + 4 (lane/32) + i % 4
  //      (i = 0..15). Columns: a = 2 p + (lane % 32) / 16, g = lane % 16; tile pair (p, p + 2)
  //      holds half-columns 8 g + 2 a and 8 g + 2 a + 1 (down: p = 0, 1 of half wn; gate/up:
  //      p = wn, gate tiles 0, 1 and up tiles 2, 3)
  const uint16_t* sc = scales + (size_t)e * (2 * (size_t)f + d);
  const int rq = 4 * (lane >> 5);
  if constexpr (kGateUp) {
    const int a = 2 * wn + ((lane & 31) >> 4);
    const int n = n0 + 8 * g + 2 * a;
    const uint32_t g2 = *reinterpret_cast<const uint32_t*>(sc + n);
    const uint32_t u2 = *reinterpret_cast<const uint32_t*>(sc + f + n);
    const float sg0 = bf16_bits_to_float(g2 & 0xFFFFu), sg1 = bf16_bits_to_float(g2 >> 16);
    const float su0 = bf16_bits_to_float(u2 & 0xFFFFu), su1 = bf16_bits_to_float(u2 >> 16);
    _Float16* hb = reinterpret_cast<_Float16*>(out) + (size_t)(row0 + wm * 128 + rq) * f + n;
    // check(false): all 128 rows of the wavefront are live (every tile but the last of a segment),
    // so the stores need no per-row test (measured 0.7-0.8% faster than testing every row)
    auto store_h = [&](auto check) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int mo = 32 * mt + 8 * (i >> 2) + (i & 3);
          if (!decltype(check)::value || wm * 128 + mo + rq < rows) {
            const float h0 = gelu_tanh(acc[mt][0][i] * sg0) * (acc[mt][2][i] * su0);
            const float h1 = gelu_tanh(acc[mt][1][i] * sg1) * (acc[mt][3][i] * su1);
            *reinterpret_cast<uint32_t*>(hb + (size_t)mo * f) = pack_f16_rne(h0, h1);
          }
        }
    };
    if (__builtin_amdgcn_readfirstlane(wm * 128 + 128 <= rows ? 1 : 0))
      store_h(std::false_type{});
    else
      store_h(std::true_type{});
  } else {
    // Lane (g, h = lane % 32 / 16) holds columns 8 g + 2 h + {0, 1} (tiles 0, 2) and 8 g + 4 + 2 h + {0, 1}
    // (tiles 1, 3) of its half. One swap between the two 16-lane rows of each 32-lane group gives lane
    // h = 0 columns 8 g .. 8 g + 3 and lane h = 1 columns 8 g + 4 .. 8 g + 7, so each row is written as
    // 16-byte pieces that together cover 512 contiguous bytes (measured 1.5-2% faster than 8-byte
    // pieces at every second 16 bytes).
    float* Y = reinterpret_cast<float*>(out) + (size_t)blockIdx.z * rows_cap * d;
    const int h = (lane & 31) >> 4;
    const int nb = n0 + wn * HALF + 8 * g;
    const uint32_t s20 = *reinterpret_cast<const uint32_t*>(sc + 2 * (size_t)f + nb + 2 * h);
    const uint32_t s21 = *reinterpret_cast<const uint32_t*>(sc + 2 * (size_t)f + nb + 4 + 2 * h);
    const float sd00 = bf16_bits_to_float(s20 & 0xFFFFu), sd01 = bf16_bits_to_float(s20 >> 16);
    const float sd10 = bf16_bits_to_float(s21 & 0xFFFFu), sd11 = bf16_bits_to_float(s21 >> 16);
    float* ybase = Y + (size_t)row0 * d + nb + 4 * h;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = wm * 128 + 32 * mt + 8 * (i >> 2) + rq + (i & 3);
        const uint32_t y00 = __float_as_uint(acc[mt][0][i] * sd00), y01 = __float_as_uint(acc[mt][2][i] * sd01);
        const uint32_t y10 = __float_as_uint(acc[mt][1][i] * sd10), y11 = __float_as_uint(acc[mt][3][i] * sd11);
        // odd rows of the first operand <-> even rows of the second: lane h = 0 receives the
        // h = 1 lane's columns 8 g + 2, 3 and hands over its own 8 g + 4, 5 (and likewise)
        const auto r0 = __builtin_amdgcn_permlane16_swap(y00, y10, false, false);
        const auto r1 = __builtin_amdgcn_permlane16_swap(y01, y11, false, false);
        if (m < rows) {  // m is the same for the two lanes of a swap (one 32-lane group)
          const u32x4 v = {r0[0], r1[0], r0[1], r1[1]};
          *reinterpret_cast<u32x4*>(ybase + (size_t)m * d) = v;
        }
      }
  }
}

// m-slots: enough for every expert segment's m-tiles (sum of ceil(M_e / bm) <= rows / bm
// + E), rounded up to a multiple of the 8 XCDs.
int prefill_mslots(int rows_cap, int E, int bm) { return ((rows_cap + bm - 1) / bm + E + 7) / 8 * 8; }

// Tile height: 128 rows while the experts average at most 96 rows (few reach a second
// 128-row tile), else 256.
int prefill_bm(int rows_cap, int E) { return rows_cap <= 96 * E ? 128 : 256; }

// xn = n-tile blocks across XCDs (the rest of the 8 split the m-slots), as preferred by
// the caller when the tile counts allow it; ngroup = n-tiles swept together.
TileOrder make_order(int nslots, int ntiles, int xn_pref) {
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
    ncu = 256;
  TileOrder o{nslots, ntiles, 8, 1, 1, ncu};
  for (int xn = xn_pref; xn >= 1; xn /= 2)
    if (ntiles % xn == 0) {
      o.xn = xn;
      o.xm = 8 / xn;
      break;
    }
  const int nblk = ntiles / o.xn;
  for (int g : {8, 4, 3, 2, 1})
    if (nblk % g == 0) {
      o.ngroup = g;
      break;
    }
  return o;
}

hipError_t launch_gate_up_prefill(const uint16_t* x, const int32_t* perm, const int32_t* offsets,
                                  const int8_t* w_gate, const int8_t* w_up, const uint16_t* scales,
                                  _Float16* H, int rows_cap, int d, int f, int E, hipStream_t stream) {
  // the main loop takes two 64-deep slices per trip: an odd slice count would multiply the
  // re-read last slice twice
  if (d % (2 * BK) != 0 || f % HALF != 0) return hipErrorInvalidValue;
  const int bm = prefill_bm(rows_cap, E);
  const int nslots = prefill_mslots(rows_cap, E, bm), ntiles = f / HALF;
  // the activations fit the last-level cache: every XCD takes its own weight columns
  const TileOrder order = make_order(nslots, ntiles, 8);
  dim3 grid(nslots * ntiles, 1, 1);
  if (bm == 256)
    hipLaunchKernelGGL(expert_wide_kernel<true>, grid, dim3(kWideThreads), 0, stream, x, perm, offsets, w_gate, w_up,
                       scales, (void*)H, d, f, E, rows_cap, order, (int*)nullptr);
  else
    hipLaunchKernelGGL((expert_prefill_kernel<true, 128>), grid, dim3(kThreads), 0, stream, x, perm, offsets, w_gate,
                       w_up, scales, (void*)H, d, f, E, rows_cap, order, (int*)nullptr);
  return hipGetLastError();
}

hipError_t launch_down_prefill(const _Float16* H, const int32_t* offsets, const int8_t* w_down,
                               const uint16_t* scales, float* Y, int splits, int rows_cap, int d,
                               int f, int E, int* splits_used, hipStream_t stream) {
  if (splits_used != nullptr && splits != 2 && splits != 4) return hipErrorInvalidValue;
  // every part, and every part the kernel may keep (1 or 2 of 2; 1, 2 or 4 of 4), is a whole
  // number of 128-deep trips of the main loop, and the columns are whole 256-column tiles
  if (splits < 1 || f % (splits * 2 * BK) != 0 || d % (2 * HALF) != 0) return hipErrorInvalidValue;
  const int bm = prefill_bm(rows_cap, E);
  const int nslots = prefill_mslots(rows_cap, E, bm), ntiles = d / (2 * HALF);
  // every XCD takes its own weight columns, as for gate/up (measured against 2 x 4 and 4 x 2
  // XCD grids: equal at 8192 tokens, 2.6% faster on a skewed 4096-token batch)
  const TileOrder order = make_order(nslots, ntiles, 8);
  dim3 grid(nslots * ntiles, 1, splits);
  if (bm == 256)
    hipLaunchKernelGGL(expert_wide_kernel<false>, grid, dim3(kWideThreads), 0, stream,
                       reinterpret_cast<const uint16_t*>(H), (const int32_t*)nullptr, offsets, w_down,
                       (const int8_t*)nullptr, scales, (void*)Y, d, f, E, rows_cap, order, splits_used);
  else
    hipLaunchKernelGGL((expert_prefill_kernel<false, 128>), grid, dim3(kThreads), 0, stream,
                       reinterpret_cast<const uint16_t*>(H), (const int32_t*)nullptr, offsets, w_down,
                       (const int8_t*)nullptr, scales, (void*)Y, d, f, E, rows_cap, order, splits_used);
  return hipGetLastError();
}

}  // namespace moe
