// The whole MoE layer in one launch for small batches (T <= 64, E = 8, expert matrices
// streamed from HBM): routing, dispatch, gate/up + GeGLU, down and combine
// (Grok-1 Admin & Architecture Guide, section 3 "Mixture of Experts", steps 1-4; fp32
// routing, section 9; "Quantized weights").
//
// At these sizes the layer is a weight stream of a few hundred MB to a few GB plus four small
// launches of about 4.5 us each (the two routing launches, the split-contraction finish, the
// combine). Here every stage is a set of work items of one kernel:
//   R  routing: group sums of 3 feature groups x 8 tokens; the last R item adds the groups,
//      takes the softmax and top-k and dispatches (the same arithmetic, in the same order,
//      as router_partial_kernel + route_finish_kernel);
//   G  gate/up: (slab, part, expert) exactly as gate_up_decode_kernel; with a split
//      contraction the last part of a slab to finish applies the GeGLU to the slab (the
//      arithmetic of geglu_finish_kernel);
//   D  down: (slab, pair of parts, expert), one part per wavefront, as down_decode_kernel;
//   C  combine: (slab, 8 tokens), the arithmetic of combine_kernel.
// so the output has the same bits as the launch-per-stage sequence.
//
// Measured on MI355X it is slower than that sequence (one GPU's tensor-parallel share at T = 8:
// 172 us against 115 us; the Grok-1 shape at T = 8: 765 us against 690 us), so the library takes
// it only on request (MOE_ONE_LAUNCH=1). A per-workgroup timeline shows why: the routing items
// share the memory system with the first weight loads and finish after 16 us instead of 9, and
// with one wavefront per SIMD (the load rings need about 300 registers) a down item that waits
// for its expert's H holds two SIMDs idle (median wait 39 us); the small stages' own latency
// (dependent loads of data just written) remains inside the kernel.
//
// Scheduling. Workgroups take items in order from a counter, so an item is only ever taken
// after every item before it was taken by a running workgroup, and items wait only on items
// before them (R < G < D < C): every wait ends, whatever the number of resident workgroups.
// A G or D item issues its first weight loads (which depend only on its slab) before waiting,
// so the routing and the G -> D hand-over overlap the weight stream. Each wait is bounded (about
// a second of wall clock): an ordering fault then costs a wrong result, never a hung device;
// an item whose wait gave up reads nothing that its wait guards and publishes nothing.
//
// Memory ordering without cache flushes. The per-XCD L2 caches are not coherent with each
// other, and a device-scope release or acquire fence writes back or invalidates a whole L2,
// about a microsecond each: one per item would cost more than the launches saved. So the
// arrays that pass between items are written with device-scope stores (written through the
// L2, as the compiler's own device-scope atomic stores are): rp, P, H and Y. A stage publishes
// by waiting for its stores to complete (s_waitcnt) and then adding to a counter with a
// device-scope atomic; a reader polls the counter the same way and only then loads the data
// with ordinary loads. Those loads cannot hit a stale line: the caches are invalidated when a
// kernel starts, and within the launch no item reads a line of rp, P, H or Y before the
// counter guarding it is complete (each line belongs to one row, and a row's readers all wait
// for every writer of that row). The routing arrays are written by one workgroup and published
// with a single device-scope fence. The counters live in a control block of kLayerCtlWords
// int32 that must be zero at launch; the last workgroup to finish returns it to zero, so a
// block stays usable by every later launch on the same stream.
#include "combine_common.h"
#include "dispatch_common.h"
#include "kernels.h"
#include "launch_policy.h"
#include "router_common.h"
#include "stream_common.h"

namespace moe {

namespace {
constexpr int kThreads = 128;       // two wavefronts per workgroup
constexpr int kRouteTokens = 8;     // tokens per R item (one per 16-lane segment)
constexpr int kRouteGroups = 3;     // 128-feature groups per R item
constexpr int kCombineTokens = 8;   // tokens per C item
constexpr int kE = 8;

// control block words
constexpr int kNext = 0;         // item counter
constexpr int kDrain = 1;        // finished workgroups
constexpr int kRouteTicket = 2;  // finished R items
constexpr int kRouted = 3;       // 1 once the routing and dispatch are written
constexpr int kHDone = 4;        // [E]: gate/up slabs of expert e whose H columns are written
constexpr int kDDone = 68;       // [d / 256]: down parts (all experts) done for column slab c
constexpr int kGTicket = 580;    // [E][f / 256]: finished parts of gate/up slab (e, n)

// wall-clock ticks (100 MHz) after which a wait gives up
constexpr uint64_t kSpinLimit = 100000000ull;
// cache policy of the stores that pass data between items: device scope (sc1), written
// through the L2
constexpr int kDeviceScope = 16;
}  // namespace

static_assert(kGTicket + 8 * 256 <= kLayerCtlWords, "control block");

struct LayerArgs {
  const uint16_t* x;
  const float* router_w;
  const float* router_bias;
  const uint8_t* pad_mask;
  const int8_t* w_gate;
  const int8_t* w_up;
  const int8_t* w_down;
  const uint16_t* scales;
  float* rp;  // group sums [T][d / 128][8]
  int32_t* ids;
  float* topk_w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* pos;
  _Float16* H;
  float* P;  // split gate/up sums, 2 * parts planes of T * k * f
  float* Y;  // down parts, splits planes of T * k * d
  float* out;
  int* ctl;
  int T, d, f, k, parts, splits;
  int nR, nG, nD, nC;
};

__device__ __forceinline__ int load_device(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16 bytes at byte offset off of buffer r, written through to device scope.
__device__ __forceinline__ void store16_device(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kDeviceScope);
}
__device__ __forceinline__ void store16_device(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  store16_device(r, off, __builtin_bit_cast(u32x4, v));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t data_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
}

// Publishes this workgroup's device-scope stores: waits until every wavefront's stores have
// completed, then adds v to *p; returns the previous value to every thread. All threads must
// call.
__device__ __forceinline__ int publish_add(int* p, int v, int* s_word) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) *s_word = __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int old = *s_word;
  __syncthreads();  // s_word is rewritten by the next call
  return old;
}

// Waits until *p >= target (polled by thread 0); false if the wait gave up. All threads must
// call; the loads that follow it are issued after the counter was seen complete.
__device__ __forceinline__ bool wait_at_least(const int* p, int target, int* s_word) {
  if (threadIdx.x == 0) {
    int ok = 1;
    if (load_device(p) < target) {
      const uint64_t t0 = wall_clock64();
      while (load_device(p) < target) {
        __builtin_amdgcn_s_sleep(8);
        if (wall_clock64() - t0 > kSpinLimit) {
          ok = 0;
          break;
        }
      }
    }
    *s_word = ok;
  }
  __syncthreads();
  const bool ok = *s_word != 0;
  __syncthreads();
  return ok;
}

// ------------------------------------------------------------------------------------
// R: segment s (16 lanes) takes token 8 tb + s, lane b the run 128 g + 8 b .. + 7 of each of
// the item's groups g; the group sums go to rp[t][g][e].
__device__ __forceinline__ void route_groups(const LayerArgs& A, int r) {
  const int G = A.d / kRouterGroup;
  const int nchunks = (G + kRouteGroups - 1) / kRouteGroups;
  const int chunk = r % nchunks, tb = r / nchunks;
  const int seg = threadIdx.x >> 4, b = threadIdx.x & 15;
  const int t = tb * kRouteTokens + seg;
  const uint16_t* xt = A.x + (size_t)min(t, A.T - 1) * A.d;
  const __amdgpu_buffer_rsrc_t rp = data_rsrc(A.rp, (size_t)A.T * G * 8 * sizeof(float));
  f32x4 w[kRouteGroups][16];
  u32x4 xv[kRouteGroups];
#pragma unroll
  for (int q = 0; q < kRouteGroups; ++q) {
    const int g = chunk * kRouteGroups + q;
    if (g < G) {
      const int i0 = kRouterGroup * g + 8 * b;
      load_rows8(A.router_w, i0, w[q]);
      xv[q] = *reinterpret_cast<const u32x4*>(xt + i0);
    }
  }
#pragma unroll
  for (int q = 0; q < kRouteGroups; ++q) {
    const int g = chunk * kRouteGroups + q;
    if (g < G) {  // uniform over the workgroup
      float S[8];
      run_sums8(xv[q], w[q], S);
#pragma unroll
      for (int e = 0; e < 8; ++e) S[e] = group_sum16(S[e]);
      if (b == 0 && t < A.T) {
        const uint32_t off = (uint32_t)(((size_t)t * G + g) * 8 * sizeof(float));
        store16_device(rp, off, f32x4{S[0], S[1], S[2], S[3]});
        store16_device(rp, off + 16, f32x4{S[4], S[5], S[6], S[7]});
      }
    }
  }
}

// The last R item: logits (group sums in group order), softmax and top-k, dispatch.
__device__ __forceinline__ void route_finish(const LayerArgs& A, float* s_logit) {
  const int G = A.d / kRouterGroup;
  for (int i = threadIdx.x; i < A.T * kE; i += kThreads) {
    const float* src = A.rp + (size_t)(i / kE) * G * kE + (i % kE);
    float logit = 0.0f;
    constexpr int kBatch = 16;  // loads in flight, then the adds in group order
    for (int g0 = 0; g0 < G; g0 += kBatch) {
      float v[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q)
        if (g0 + q < G) v[q] = src[(size_t)(g0 + q) * kE];
#pragma unroll
      for (int q = 0; q < kBatch; ++q)
        if (g0 + q < G) logit += v[q];
    }
    s_logit[i] = logit;
  }
  __syncthreads();
  if (threadIdx.x < 64) {  // wavefront 0: lane t finishes token t
    const int t = threadIdx.x;
    uint64_t emask = 0;
    uint32_t slots = 0;
    if (t < A.T) {
      float p[kE];
#pragma unroll
      for (int e = 0; e < kE; ++e) p[e] = s_logit[t * kE + e];
      const bool real = A.pad_mask == nullptr || A.pad_mask[t] != 0;
      emask = finish_token<kE>(p, kE, A.k, A.router_bias, real, A.ids + (size_t)t * A.k, A.topk_w + (size_t)t * A.k,
                               &slots);
    }
    dispatch_wave(emask, [&](int e) { return (int)((slots >> (4 * e)) & 15u); }, A.T, kE, A.k, A.counts, A.offsets,
                  A.perm, A.pos);
  }
}

// ------------------------------------------------------------------------------------
// G: wavefront 0 streams the gate slab, wavefront 1 the up slab, over part `part` of d.
template <int MT, int kStages, bool kPartial>
__device__ __forceinline__ void gate_up_item(const LayerArgs& A, int g, float (*s_up)[kSlab + 4], int* s_word) {
  const int nslab = A.f / kSlab;
  const int slab = g % nslab, part = (g / nslab) % A.parts, e = g / (nslab * A.parts);
  const int d = A.d, f = A.f;
  const int kspan = d / A.parts, kbeg = part * kspan, steps = kspan / kStep;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, kg = lane >> 4, cl = lane & 15;
  const int nl = kNcol * cl;
  const int n0 = slab * kSlab + nl;
  const __amdgpu_buffer_rsrc_t wr = weight_rsrc((wave == 0 ? A.w_gate : A.w_up) + (size_t)e * d * f, (size_t)d * f);
  const uint32_t voff = (uint32_t)(kbeg + 8 * kg) * (uint32_t)f + (uint32_t)n0;
  const int rows_cap = A.T * A.k;
  const uint16_t* sc = A.scales + (size_t)e * (2 * (size_t)f + d);
  const __amdgpu_buffer_rsrc_t hr = data_rsrc(A.H, (size_t)rows_cap * f * sizeof(_Float16));
  int row0 = 0, M = 0;

  auto rows_of = [&](int pb, const uint16_t* (&a)[MT]) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = min(pb + 16 * mt + cl, M - 1);
      a[mt] = A.x + (size_t)A.perm[row0 + m] * d + kbeg + 8 * kg;
    }
  };
  f32x4 acc[MT][kNcol];
  auto clear = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < kNcol; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  // the pass's sums: P (split contraction) or, through LDS, H
  auto finish_pass = [&](int pb) __attribute__((always_inline)) {
    if constexpr (kPartial) {
      // lane holds rows 16 mt + 4 kg + i of the pass, columns n0 .. n0 + kNcol - 1
      const __amdgpu_buffer_rsrc_t pr =
          data_rsrc(A.P + (size_t)(2 * part + wave) * rows_cap * f, (size_t)rows_cap * f * sizeof(float));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = pb + 16 * mt + 4 * kg + i;
          if (m < M) {
            const uint32_t off = (uint32_t)(((size_t)(row0 + m) * f + n0) * sizeof(float));
#pragma unroll
            for (int q = 0; q < kNcol / 4; ++q)
              store16_device(pr, off + 16 * q,
                             f32x4{acc[mt][4 * q][i], acc[mt][4 * q + 1][i], acc[mt][4 * q + 2][i],
                                   acc[mt][4 * q + 3][i]});
          }
        }
    } else {
      float s8[kNcol];
      load_scales<kNcol>(sc + (wave == 0 ? 0 : f) + n0, s8);
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
                store16_device(hr, (uint32_t)(((size_t)(row0 + m) * f + n0 + 8 * q) * sizeof(_Float16)), v);
              }
            }
          }
      }
      __syncthreads();  // s_up is rewritten by the next pass
    }
  };

  // first pass: its weights go out before the wait for the routing
  clear();
  const bool live = stream_slab_rows<bf16x8, MT, kStages>(
      wr, voff, (uint32_t)f, steps,
      [&](const uint16_t* (&a)[MT]) __attribute__((always_inline)) {
        if (!wait_at_least(A.ctl + kRouted, 1, s_word)) return false;
        row0 = A.offsets[e];
        M = A.offsets[e + 1] - row0;
        if (M <= 0) return false;
        rows_of(0, a);
        return true;
      },
      acc);
  if (!live) return;
  finish_pass(0);
  for (int pb = 16 * MT; pb < M; pb += 16 * MT) {
    const uint16_t* a[MT];
    rows_of(pb, a);
    clear();
    stream_slab<bf16x8, MT, kStages>(wr, voff, (uint32_t)f, steps, a, acc);
    finish_pass(pb);
  }

  if constexpr (kPartial) {
    // the last part of this slab to finish completes its H columns
    if (publish_add(A.ctl + kGTicket + e * nslab + slab, 1, s_word) != A.parts - 1) return;
    const size_t plane = (size_t)rows_cap * f;
    constexpr int kUnits = kSlab / 8;  // 8-column units per row of the slab
    for (int u = threadIdx.x; u < M * kUnits; u += kThreads) {
      const int r = row0 + u / kUnits, n = slab * kSlab + 8 * (u % kUnits);
      store16_device(hr, (uint32_t)(((size_t)r * f + n) * sizeof(_Float16)),
                     geglu_from_parts(A.P, plane, A.parts, r, f, n, sc));
    }
  }
  publish_add(A.ctl + kHDone + e, 1, s_word);
}

// ------------------------------------------------------------------------------------
// D: wavefront w streams part 2 sp + w of the contraction over f for column slab c.
template <int MT, int kStages>
__device__ __forceinline__ void down_item(const LayerArgs& A, int q, int* s_word) {
  const int nslab = A.d / kSlab, pairs = A.splits / 2;
  const int c = q % nslab, sp = (q / nslab) % pairs, e = q / (nslab * pairs);
  const int d = A.d, f = A.f;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part = 2 * sp + wave;
  const int kspan = f / A.splits, kbeg = part * kspan, steps = kspan / kStep;
  const int lane = threadIdx.x & 63, kg = lane >> 4, cl = lane & 15;
  const int n0 = c * kSlab + kNcol * cl;
  const __amdgpu_buffer_rsrc_t wr = weight_rsrc(A.w_down + (size_t)e * f * d, (size_t)f * d);
  const uint32_t voff = (uint32_t)(kbeg + 8 * kg) * (uint32_t)d + (uint32_t)n0;
  const int rows_cap = A.T * A.k;
  const __amdgpu_buffer_rsrc_t yr = data_rsrc(A.Y + (size_t)part * rows_cap * d, (size_t)rows_cap * d * sizeof(float));
  int row0 = 0, M = 0;
  bool gave_up = false;

  auto rows_of = [&](int pb, const uint16_t* (&a)[MT]) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = min(pb + 16 * mt + cl, M - 1);
      a[mt] = reinterpret_cast<const uint16_t*>(A.H) + (size_t)(row0 + m) * f + kbeg + 8 * kg;
    }
  };
  f32x4 acc[MT][kNcol];
  auto clear = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < kNcol; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto finish_pass = [&](int pb) __attribute__((always_inline)) {
    float sd[kNcol];
    load_scales<kNcol>(A.scales + (size_t)e * (2 * (size_t)f + d) + 2 * (size_t)f + n0, sd);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = pb + 16 * mt + 4 * kg + i;
        if (m < M) {
          const uint32_t off = (uint32_t)(((size_t)(row0 + m) * d + n0) * sizeof(float));
#pragma unroll
          for (int qq = 0; qq < kNcol / 4; ++qq) {
            f32x4 v = {acc[mt][4 * qq][i] * sd[4 * qq], acc[mt][4 * qq + 1][i] * sd[4 * qq + 1],
                       acc[mt][4 * qq + 2][i] * sd[4 * qq + 2], acc[mt][4 * qq + 3][i] * sd[4 * qq + 3]};
            store16_device(yr, off + 16 * qq, v);
          }
        }
      }
  };

  // first pass: its weights go out before the waits for the routing and for the expert's H
  clear();
  const bool live = stream_slab_rows<f16x8, MT, kStages>(
      wr, voff, (uint32_t)d, steps,
      [&](const uint16_t* (&a)[MT]) __attribute__((always_inline)) {
        if (!wait_at_least(A.ctl + kRouted, 1, s_word)) return gave_up = true, false;
        row0 = A.offsets[e];
        M = A.offsets[e + 1] - row0;
        if (M <= 0) return false;
        if (!wait_at_least(A.ctl + kHDone + e, A.f / kSlab, s_word)) return gave_up = true, false;
        rows_of(0, a);
        return true;
      },
      acc);
  if (gave_up) return;
  if (live) {
    finish_pass(0);
    for (int pb = 16 * MT; pb < M; pb += 16 * MT) {
      const uint16_t* a[MT];
      rows_of(pb, a);
      clear();
      stream_slab<f16x8, MT, kStages>(wr, voff, (uint32_t)d, steps, a, acc);
      finish_pass(pb);
    }
  }
  publish_add(A.ctl + kDDone + c, 2, s_word);
}

// ------------------------------------------------------------------------------------
// C: thread i takes token 8 tb + i / 16 and columns 256 c + 4 (i % 16) + 64 j, j = 0..3.
__device__ __forceinline__ void combine_item(const LayerArgs& A, int q, int* s_word) {
  const int nslab = A.d / kSlab;
  const int c = q % nslab, tb = q / nslab;
  if (!wait_at_least(A.ctl + kDDone + c, kE * A.splits, s_word)) return;
  const int t = tb * kCombineTokens + (threadIdx.x >> 4);
  if (t >= A.T) return;
  const bool real = A.pad_mask == nullptr || A.pad_mask[t] != 0;
  const size_t part_stride = (size_t)A.T * A.k * A.d;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = c * kSlab + 4 * (threadIdx.x & 15) + 64 * j;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (real) acc = gather_combine(A.Y, A.splits, part_stride, A.pos, A.topk_w, t, col, A.d, A.k);
    *reinterpret_cast<f32x4*>(A.out + (size_t)t * A.d + col) = acc;
  }
}

// ------------------------------------------------------------------------------------
template <int MTG, int kStG, bool kPartial, int MTD, int kStD>
__global__ __launch_bounds__(kThreads) void layer_decode_kernel(LayerArgs A) {
  __shared__ float s_up[kPartial ? 1 : MTG * 16][kSlab + 4];
  __shared__ float s_logit[kRouterSplitMaxT * kE];
  __shared__ int s_word;
  if (threadIdx.x == 0) s_word = __hip_atomic_fetch_add(A.ctl + kNext, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  int item = s_word;
  __syncthreads();
  if (item < A.nR) {
    route_groups(A, item);
    if (publish_add(A.ctl + kRouteTicket, 1, &s_word) == A.nR - 1) {
      route_finish(A, &s_logit[0]);
      __syncthreads();
      if (threadIdx.x == 0) {
        // the routing arrays (ordinary stores of wavefront 0) to device scope, then the flag
        __threadfence();
        __hip_atomic_store(A.ctl + kRouted, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  } else if ((item -= A.nR) < A.nG) {
    gate_up_item<MTG, kStG, kPartial>(A, item, s_up, &s_word);
  } else if ((item -= A.nG) < A.nD) {
    down_item<MTD, kStD>(A, item, &s_word);
  } else {
    combine_item(A, item - A.nD, &s_word);
  }

  // the last workgroup out returns the control block to zero
  __syncthreads();
  if (threadIdx.x == 0)
    s_word = __hip_atomic_fetch_add(A.ctl + kDrain, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_word == A.nR + A.nG + A.nD + A.nC - 1)
    for (int i = threadIdx.x; i < kLayerCtlWords; i += kThreads) A.ctl[i] = 0;
}

__global__ __launch_bounds__(256) void layer_ctl_clear_kernel(int* __restrict__ ctl) {
  for (int i = threadIdx.x; i < kLayerCtlWords; i += 256) ctl[i] = 0;
}

// ------------------------------------------------------------------------------------
bool layer_decode_fits(int T, int d, int f, int E, int k) {
  if (E != kE || T <= 0 || T > kRouterSplitMaxT || k > kE || !streaming_experts(T, d, f)) return false;
  if (d % kSlab != 0 || f % kSlab != 0 || d / kSlab > kGTicket - kDDone || (f / kSlab) * kE > kLayerCtlWords - kGTicket)
    return false;
  const int parts = gate_up_parts(T, d, f, E, k), splits = down_splits(T, d, f, E, k);
  if (splits < 2 || splits % 2 != 0) return false;
  if (parts == 1 && T <= 4) return false;  // there one wavefront streams both matrices (fused kernel)
  return (d / parts) % kStep == 0 && (f / splits) % kStep == 0;
}

hipError_t launch_layer_ctl_clear(int* ctl, hipStream_t stream) {
  hipLaunchKernelGGL(layer_ctl_clear_kernel, dim3(1), dim3(256), 0, stream, ctl);
  return hipGetLastError();
}

hipError_t launch_layer_decode(const uint16_t* x, const float* router_w, const float* router_bias,
                               const uint8_t* pad_mask, const int8_t* w_gate, const int8_t* w_up,
                               const int8_t* w_down, const uint16_t* scales, float* rp, int32_t* ids,
                               float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos,
                               _Float16* H, float* P, float* Y, float* out, int* ctl, int T, int d, int f, int E,
                               int k, hipStream_t stream) {
  if (!layer_decode_fits(T, d, f, E, k)) return hipErrorInvalidValue;
  LayerArgs A{x, router_w, router_bias, pad_mask, w_gate, w_up, w_down, scales, rp, ids, topk_w, counts, offsets,
              perm, pos, H, P, Y, out, ctl, T, d, f, k, 0, 0, 0, 0, 0, 0};
  A.parts = gate_up_parts(T, d, f, E, k);
  A.splits = down_splits(T, d, f, E, k);
  const int G = d / kRouterGroup;
  A.nR = ((G + kRouteGroups - 1) / kRouteGroups) * ((T + kRouteTokens - 1) / kRouteTokens);
  A.nG = (f / kSlab) * A.parts * E;
  A.nD = (d / kSlab) * (A.splits / 2) * E;
  A.nC = (d / kSlab) * ((T + kCombineTokens - 1) / kCombineTokens);
  const dim3 grid(A.nR + A.nG + A.nD + A.nC), block(kThreads);
  // the row tiles and load rings of the stand-alone kernels at the same T
  if (T <= 16) {
    if (A.parts > 1)
      hipLaunchKernelGGL((layer_decode_kernel<1, 4, true, 1, 4>), grid, block, 0, stream, A);
    else if (T <= 8)
      hipLaunchKernelGGL((layer_decode_kernel<1, 4, false, 1, 4>), grid, block, 0, stream, A);
    else
      hipLaunchKernelGGL((layer_decode_kernel<2, 3, false, 1, 4>), grid, block, 0, stream, A);
  } else {
    if (A.parts > 1)
      hipLaunchKernelGGL((layer_decode_kernel<2, 3, true, 2, 4>), grid, block, 0, stream, A);
    else
      hipLaunchKernelGGL((layer_decode_kernel<2, 3, false, 2, 4>), grid, block, 0, stream, A);
  }
  return hipGetLastError();
}

}  // namespace moe
