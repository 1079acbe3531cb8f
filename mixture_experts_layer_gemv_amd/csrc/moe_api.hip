// C ABI of the MoE layer (declared in include/moe.h): argument checks, workspace
// management and the launch sequence router -> dispatch -> gate/up -> down -> combine,
// all enqueued on the caller's stream with no host synchronisation.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "kernels.h"
#include "launch_policy.h"

namespace {

using moe::down_splits;
using moe::gate_up_parts;

thread_local std::string g_error;

int fail(int code, const std::string& msg) {
  g_error = msg;
  return code;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr long long kMaxAssignments = 1ll << 24;

int check_shape(int T, int d, int f, int E, int k) {
  if (T < 0) return fail(MOE_ERR_INVALID, "T must be >= 0");
  if (d <= 0 || f <= 0 || E <= 0 || k <= 0) return fail(MOE_ERR_INVALID, "d, f, E and k must be > 0");
  if (k > E) return fail(MOE_ERR_INVALID, "k must be <= E");
  if (E > 64) return fail(MOE_ERR_UNSUPPORTED, "E > 64 is not supported");
  if (d % 256 != 0 || f % 256 != 0) return fail(MOE_ERR_UNSUPPORTED, "d and f must be multiples of 256");
  if ((long long)T * k > kMaxAssignments) return fail(MOE_ERR_UNSUPPORTED, "T * k exceeds 2^24 assignments");
  // one expert's weight matrix is addressed with 32-bit byte offsets (buffer loads)
  if ((long long)d * f >= (1ll << 31)) return fail(MOE_ERR_UNSUPPORTED, "d * f must be below 2^31 bytes per matrix");
  return MOE_OK;
}

int check_ptr(const void* p, const char* name, uintptr_t align = 16) {
  if (p == nullptr) return fail(MOE_ERR_INVALID, std::string(name) + " is NULL");
  if (!aligned(p, align)) return fail(MOE_ERR_INVALID, std::string(name) + " is not 16-byte aligned");
  return MOE_OK;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(MOE_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

#define MOE_TRY(expr)           \
  do {                          \
    int _rc = (expr);           \
    if (_rc != MOE_OK) return _rc; \
  } while (0)

#define MOE_HIP(expr, where)                     \
  do {                                           \
    hipError_t _e = (expr);                      \
    if (_e != hipSuccess) return hip_fail(_e, where); \
  } while (0)

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Layout {
  size_t ids, w, counts, offsets, perm, pos, h, y, gp, dchunk, rp, sused, ctl, total;
  int splits, gparts;
  bool one_launch;  // the layer fits the one-launch kernel (moe::layer_decode_fits)
};

Layout make_layout(int T, int d, int f, int E, int k) {
  Layout L{};
  size_t at = 0;
  auto take = [&](size_t bytes) {
    size_t o = at;
    at += round_up(bytes, 256);
    return o;
  };
  const size_t tk = (size_t)T * k;
  L.ids = take(tk * 4);
  L.w = take(tk * 4);
  L.counts = take((size_t)E * 4);
  L.offsets = take((size_t)(E + 1) * 4);
  L.perm = take(tk * 4);
  L.pos = take(tk * 4);
  L.h = take(tk * f * 2);
  L.splits = down_splits(T, d, f, E, k);
  L.y = take((size_t)L.splits * tk * d * 4);
  L.gparts = gate_up_parts(T, d, f, E, k);
  L.gp = L.gparts > 1 ? take((size_t)2 * L.gparts * tk * f * 4) : 0;
  const int nchunks = moe::dispatch_chunks(T);
  L.dchunk = nchunks > 0 ? take((size_t)2 * nchunks * E * 4) : 0;
  const size_t rp_floats = moe::router_partial_floats(T, d, E);
  L.rp = rp_floats > 0 ? take(rp_floats * 4) : 0;
  // large batches: the number of down parts the prefill kernel kept (of the 2 or 4 launched)
  L.sused = (T > moe::kDecodeMaxT && L.splits >= 2) ? take(4) : 0;
  // the one-launch layer's control block, used when the caller brings the workspace
  L.one_launch = moe::layer_decode_fits(T, d, f, E, k);
  L.ctl = L.one_launch ? take((size_t)moe::kLayerCtlWords * 4) : 0;
  L.total = at;
  return L;
}

// Workspace of the dense one-hot formulation: the top-k routing, then the all-expert
// routing (k' = E) with its one-hot gates, and the regular layout for k' = E after it.
struct DenseLayout {
  size_t ids, w, inner, total;
  Layout L;
};

DenseLayout make_dense_layout(int T, int d, int f, int E, int k) {
  DenseLayout D{};
  size_t at = 0;
  const size_t tk = (size_t)T * k;
  D.ids = at;
  at += round_up(tk * 4, 256);
  D.w = at;
  at += round_up(tk * 4, 256);
  D.inner = at;
  D.L = make_layout(T, d, f, E, E);
  D.total = at + D.L.total;
  return D;
}

// The MoE block's workspace starts with x_norm (bf16 [T][d]) and the post-norm combine's
// chunk sums, followed by the layer's layout.
size_t block_sumsq_bytes(int T, int d) {
  return round_up((size_t)moe::combine_postnorm_scratch_floats(T, d) * 4, 256);
}
size_t block_prefix_bytes(int T, int d) { return round_up((size_t)T * d * 2, 256) + block_sumsq_bytes(T, d); }

// Scratch of moe_forward_noalloc: a fixed array in device memory (one copy per device, held
// until the process ends). Host code never passes `scratch` itself to a kernel (on the host the
// name stands for a host-side shadow, not the device address): its device address is looked up
// once per device with hipGetSymbolAddress and kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mutex;
std::vector<void*> g_scratch;

int scratch_address(char** out) {
  int dev = 0;
  MOE_HIP(hipGetDevice(&dev), "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if ((int)g_scratch.size() <= dev) g_scratch.resize(dev + 1, nullptr);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    MOE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch[dev] = p;
  }
  *out = static_cast<char*>(g_scratch[dev]);
  return MOE_OK;
}

// Control blocks of the one-launch layer (kLayerCtlWords int32, zero between launches) for the
// library's own workspace and for moe_forward_noalloc's scratch, one per device each, looked up
// like scratch above. The first use on a device zeroes the block on the call's stream; every
// launch leaves it zero.
static __device__ __align__(256) int layer_ctl_library[moe::kLayerCtlWords];
static __device__ __align__(256) int layer_ctl_noalloc[moe::kLayerCtlWords];
struct CtlBlock {
  void* ptr = nullptr;
  bool cleared = false;
};
std::vector<CtlBlock> g_ctl_library, g_ctl_noalloc;

int library_ctl(bool noalloc, hipStream_t s, int** out) {
  int dev = 0;
  MOE_HIP(hipGetDevice(&dev), "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  std::vector<CtlBlock>& v = noalloc ? g_ctl_noalloc : g_ctl_library;
  if ((int)v.size() <= dev) v.resize(dev + 1);
  CtlBlock& b = v[dev];
  if (b.ptr == nullptr) {
    void* p = nullptr;
    if (noalloc)
      MOE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(layer_ctl_noalloc)), "hipGetSymbolAddress(layer_ctl_noalloc)");
    else
      MOE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(layer_ctl_library)), "hipGetSymbolAddress(layer_ctl_library)");
    if (p == nullptr) return fail(MOE_ERR_HIP, "hipGetSymbolAddress of a control block returned NULL");
    b.ptr = p;
  }
  if (!b.cleared) {
    MOE_HIP(moe::launch_layer_ctl_clear(static_cast<int*>(b.ptr), s), "control block clear");
    b.cleared = true;
  }
  *out = static_cast<int*>(b.ptr);
  return MOE_OK;
}

// MOE_ONE_LAUNCH=1 in the environment runs small batches as the one-launch layer
// (layer_decode.hip) instead of one launch per stage: the same bits, but slower on MI355X, so
// it is off by default and kept for comparison.
bool one_launch_enabled() {
  const char* v = std::getenv("MOE_ONE_LAUNCH");
  return v && v[0] == '1';
}

struct DeviceWorkspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::vector<DeviceWorkspace> g_ws;

int library_workspace(size_t need, char** out) {
  int dev = 0;
  MOE_HIP(hipGetDevice(&dev), "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  if ((int)g_ws.size() <= dev) g_ws.resize(dev + 1);
  DeviceWorkspace& ws = g_ws[dev];
  if (ws.bytes < need) {
    const char* hook = std::getenv("MOE_TEST_FAIL_ALLOC");
    if (hook && hook[0] == '1') return fail(MOE_ERR_NOMEM, "workspace allocation refused (MOE_TEST_FAIL_ALLOC=1)");
    if (ws.ptr) {
      MOE_HIP(hipDeviceSynchronize(), "hipDeviceSynchronize");
      MOE_HIP(hipFree(ws.ptr), "hipFree");
      ws.ptr = nullptr;
      ws.bytes = 0;
    }
    size_t bytes = round_up(need, (size_t)1 << 20);
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, bytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(MOE_ERR_NOMEM, std::string("workspace hipMalloc of ") + std::to_string(bytes) +
                                     " bytes failed: " + hipGetErrorString(e));
    }
    ws.ptr = p;
    ws.bytes = bytes;
  }
  *out = static_cast<char*>(ws.ptr);
  return MOE_OK;
}

int check_layer_args(const void* x, const float* router_w, const int8_t* w_gate, const int8_t* w_up,
                     const int8_t* w_down, const void* scales, float* out, int T, int d, int f, int E,
                     int k) {
  MOE_TRY(check_shape(T, d, f, E, k));
  MOE_TRY(check_ptr(x, "x"));
  MOE_TRY(check_ptr(router_w, "router_w"));
  MOE_TRY(check_ptr(w_gate, "w_gate"));
  MOE_TRY(check_ptr(w_up, "w_up"));
  MOE_TRY(check_ptr(w_down, "w_down"));
  MOE_TRY(check_ptr(scales, "scales"));
  MOE_TRY(check_ptr(out, "out"));
  return MOE_OK;
}

// splits_used: where the prefill down kernel reports the parts it kept (NULL: exactly `splits`)
int run_experts(const uint16_t* x, const int32_t* perm, const int32_t* offsets, const int8_t* w_gate,
                const int8_t* w_up, const int8_t* w_down, const uint16_t* scales, _Float16* h,
                float* y, int splits, int* splits_used, float* gp, int gparts, int T, int d, int f, int E, int k,
                hipStream_t s) {
  const int rows_cap = T * k;
  if (moe::streaming_experts(T, d, f)) {
    MOE_HIP(moe::launch_gate_up_decode(x, perm, offsets, w_gate, w_up, scales, h, gp, gparts, T, k, d, f, E, s),
            "gate_up");
    MOE_HIP(moe::launch_down_decode(h, offsets, w_down, scales, y, splits, rows_cap, T, d, f, E, s), "down");
  } else {
    MOE_HIP(moe::launch_gate_up_prefill(x, perm, offsets, w_gate, w_up, scales, h, rows_cap, d, f, E, s),
            "gate_up");
    // up to kDecodeMaxT tokens the parts are the host's (no count kept on the device)
    MOE_HIP(moe::launch_down_prefill(h, offsets, w_down, scales, y, splits, rows_cap, d, f, E,
                                     T <= moe::kDecodeMaxT ? nullptr : splits_used, s),
            "down");
  }
  return MOE_OK;
}

}  // namespace

// A captured forward (declared opaque in include/moe.h).
struct moe_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  void* own_ws = nullptr;  // the graph's own workspace when the caller passed none
};

namespace {
void destroy_graph(moe_graph* g) {
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  if (g->own_ws) {
    (void)hipDeviceSynchronize();  // a replay may still be running
    (void)hipFree(g->own_ws);
  }
  delete g;
}
}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_last_error(void) { return g_error.c_str(); }

size_t moe_workspace_bytes(int T, int d, int f, int E, int k) {
  if (check_shape(T, d, f, E, k) != MOE_OK || T == 0) return 0;
  return make_layout(T, d, f, E, k).total;
}

int moe_down_splits(int T, int d, int f, int E, int k) {
  if (check_shape(T, d, f, E, k) != MOE_OK) return 0;
  return down_splits(T, d, f, E, k);
}

int moe_gate_up_parts(int T, int d, int f, int E, int k) {
  if (check_shape(T, d, f, E, k) != MOE_OK) return 0;
  return gate_up_parts(T, d, f, E, k);
}

int moe_expert_kernels(int T, int d, int f, int E, int k) {
  if (check_shape(T, d, f, E, k) != MOE_OK) return -1;
  return moe::streaming_experts(T, d, f) ? 0 : moe::prefill_bm(T * k, E);
}

int moe_one_launch(int T, int d, int f, int E, int k) {
  if (check_shape(T, d, f, E, k) != MOE_OK) return -1;
  return T > 0 && moe::layer_decode_fits(T, d, f, E, k) && one_launch_enabled() ? 1 : 0;
}

void moe_release_workspace(void) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int cur = 0;
  (void)hipGetDevice(&cur);
  for (size_t dev = 0; dev < g_ws.size(); ++dev) {
    if (!g_ws[dev].ptr) continue;
    (void)hipSetDevice((int)dev);
    (void)hipDeviceSynchronize();
    (void)hipFree(g_ws[dev].ptr);
    g_ws[dev] = DeviceWorkspace{};
  }
  (void)hipSetDevice(cur);
}

}  // extern "C"

namespace {
// The forward on workspace ws (L.total bytes or more). ctl: a control block of the one-launch
// layer known to be zero (NULL: the one in ws, zeroed by this call first).
int forward_impl(const void* x, const float* router_w, const int8_t* w_gate, const int8_t* w_up,
                 const int8_t* w_down, const void* scales, const uint8_t* pad_mask, float* out, int T, int d, int f,
                 int E, int k, hipStream_t s, const float* router_bias, const Layout& L, char* ws, int* ctl,
                 const moe_debug_out* dbg) {
  auto* ids = reinterpret_cast<int32_t*>(ws + L.ids);
  auto* w = reinterpret_cast<float*>(ws + L.w);
  auto* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  auto* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  auto* perm = reinterpret_cast<int32_t*>(ws + L.perm);
  auto* pos = reinterpret_cast<int32_t*>(ws + L.pos);
  auto* h = reinterpret_cast<_Float16*>(ws + L.h);
  auto* y = reinterpret_cast<float*>(ws + L.y);
  auto* gp = reinterpret_cast<float*>(ws + L.gp);
  const auto* xb = static_cast<const uint16_t*>(x);
  const auto* sc = static_cast<const uint16_t*>(scales);

  const bool one_launch = L.one_launch && one_launch_enabled();
  if (one_launch) {
    if (ctl == nullptr) {
      ctl = reinterpret_cast<int*>(ws + L.ctl);
      MOE_HIP(moe::launch_layer_ctl_clear(ctl, s), "control block clear");
    }
    MOE_HIP(moe::launch_layer_decode(xb, router_w, router_bias, pad_mask, w_gate, w_up, w_down, sc,
                                     reinterpret_cast<float*>(ws + L.rp), ids, w, counts, offsets, perm, pos, h, gp,
                                     y, out, ctl, T, d, f, E, k, s),
            "one-launch layer");
  } else if (L.rp) {
    // small batches: group sums in parallel, then one launch adds them and dispatches
    auto* rp = reinterpret_cast<float*>(ws + L.rp);
    MOE_HIP(moe::launch_router_partial(xb, router_w, rp, T, d, s), "router");
    MOE_HIP(moe::launch_route_finish(rp, router_bias, pad_mask, ids, w, counts, offsets, perm, pos, T, d, E, k, s),
            "route+dispatch");
  } else {
    MOE_HIP(moe::launch_router(xb, router_w, router_bias, pad_mask, ids, w, nullptr, T, d, E, k, s), "router");
    auto* dch = L.dchunk ? reinterpret_cast<int32_t*>(ws + L.dchunk) : nullptr;
    MOE_HIP(moe::launch_dispatch(ids, pad_mask, counts, offsets, perm, pos, T, E, k, dch, s), "dispatch");
  }
  if (!one_launch) {
    auto* su = L.sused ? reinterpret_cast<int*>(ws + L.sused) : nullptr;
    MOE_TRY(run_experts(xb, perm, offsets, w_gate, w_up, w_down, sc, h, y, L.splits, su, gp, L.gparts, T, d, f, E,
                        k, s));
    MOE_HIP(moe::launch_combine(y, L.splits, su, (size_t)T * k * d, pos, w, pad_mask, out, T, d, k, s), "combine");
  }

  if (dbg) {
    const size_t tk = (size_t)T * k;
    struct Copy {
      void* dst;
      const void* src;
      size_t bytes;
    } copies[] = {{dbg->topk_ids, ids, tk * 4}, {dbg->topk_w, w, tk * 4},  {dbg->counts, counts, (size_t)E * 4},
                  {dbg->offsets, offsets, (size_t)(E + 1) * 4}, {dbg->perm, perm, tk * 4}, {dbg->pos, pos, tk * 4}};
    for (const Copy& c : copies)
      if (c.dst) MOE_HIP(hipMemcpyAsync(c.dst, c.src, c.bytes, hipMemcpyDeviceToDevice, s), "debug copy");
  }
  return MOE_OK;
}
}  // namespace

extern "C" {

int moe_forward_ex(const void* x, const float* router_w, const int8_t* w_gate, const int8_t* w_up,
                   const int8_t* w_down, const void* scales, const uint8_t* pad_mask, float* out,
                   int T, int d, int f, int E, int k, void* stream, const float* router_bias,
                   void* workspace, size_t workspace_bytes, const moe_debug_out* dbg) {
  MOE_TRY(check_layer_args(x, router_w, w_gate, w_up, w_down, scales, out, T, d, f, E, k));
  if (router_bias && !aligned(router_bias, 4)) return fail(MOE_ERR_INVALID, "router_bias is not 4-byte aligned");
  if (T == 0) return MOE_OK;
  const Layout L = make_layout(T, d, f, E, k);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = nullptr;
  int* ctl = nullptr;
  if (workspace) {
    if (!aligned(workspace, 256)) return fail(MOE_ERR_INVALID, "workspace is not 256-byte aligned");
    if (workspace_bytes < L.total)
      return fail(MOE_ERR_INVALID, "workspace too small: need " + std::to_string(L.total) + " bytes");
    ws = static_cast<char*>(workspace);
  } else {
    MOE_TRY(library_workspace(L.total, &ws));
    if (L.one_launch && one_launch_enabled()) MOE_TRY(library_ctl(false, s, &ctl));
  }
  return forward_impl(x, router_w, w_gate, w_up, w_down, scales, pad_mask, out, T, d, f, E, k, s, router_bias, L, ws,
                      ctl, dbg);
}

int moe_forward_noalloc(const void* x, const float* router_w, const int8_t* w_gate, const int8_t* w_up,
                        const int8_t* w_down, const void* scales, const uint8_t* pad_mask, float* out, int T, int d,
                        int f, int E, int k, void* stream, const float* router_bias) {
  MOE_TRY(check_layer_args(x, router_w, w_gate, w_up, w_down, scales, out, T, d, f, E, k));
  if (router_bias && !aligned(router_bias, 4)) return fail(MOE_ERR_INVALID, "router_bias is not 4-byte aligned");
  if (T == 0) return MOE_OK;
  const size_t need = make_layout(T, d, f, E, k).total;
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_UNSUPPORTED, "moe_forward_noalloc: this shape needs " + std::to_string(need) +
                                         " bytes of scratch, above its fixed " +
                                         std::to_string((size_t)MOE_NOALLOC_SCRATCH_BYTES) +
                                         " bytes (use moe_forward_ex with a workspace)");
  char* ws = nullptr;
  MOE_TRY(scratch_address(&ws));
  const Layout L = make_layout(T, d, f, E, k);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int* ctl = nullptr;
  if (L.one_launch && one_launch_enabled()) MOE_TRY(library_ctl(true, s, &ctl));
  return forward_impl(x, router_w, w_gate, w_up, w_down, scales, pad_mask, out, T, d, f, E, k, s, router_bias, L, ws,
                      ctl, nullptr);
}

size_t moe_workspace_bytes_dense(int T, int d, int f, int E, int k) {
  if (check_shape(T, d, f, E, k) != MOE_OK || T == 0) return 0;
  if ((long long)T * E > kMaxAssignments) return 0;
  return make_dense_layout(T, d, f, E, k).total;
}

int moe_forward_dense(const void* x, const float* router_w, const int8_t* w_gate, const int8_t* w_up,
                      const int8_t* w_down, const void* scales, const uint8_t* pad_mask, float* out, int T,
                      int d, int f, int E, int k, void* stream, const float* router_bias, void* workspace,
                      size_t workspace_bytes) {
  MOE_TRY(check_layer_args(x, router_w, w_gate, w_up, w_down, scales, out, T, d, f, E, k));
  if (router_bias && !aligned(router_bias, 4)) return fail(MOE_ERR_INVALID, "router_bias is not 4-byte aligned");
  if ((long long)T * E > kMaxAssignments) return fail(MOE_ERR_UNSUPPORTED, "T * E exceeds 2^24 assignments");
  if (T == 0) return MOE_OK;
  const DenseLayout D = make_dense_layout(T, d, f, E, k);
  char* ws = nullptr;
  if (workspace) {
    if (!aligned(workspace, 256)) return fail(MOE_ERR_INVALID, "workspace is not 256-byte aligned");
    if (workspace_bytes < D.total)
      return fail(MOE_ERR_INVALID, "workspace too small: need " + std::to_string(D.total) + " bytes");
    ws = static_cast<char*>(workspace);
  } else {
    MOE_TRY(library_workspace(D.total, &ws));
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto* ids = reinterpret_cast<int32_t*>(ws + D.ids);
  auto* w = reinterpret_cast<float*>(ws + D.w);
  char* in = ws + D.inner;
  const Layout& L = D.L;
  auto* ids_all = reinterpret_cast<int32_t*>(in + L.ids);
  auto* gates = reinterpret_cast<float*>(in + L.w);
  auto* counts = reinterpret_cast<int32_t*>(in + L.counts);
  auto* offsets = reinterpret_cast<int32_t*>(in + L.offsets);
  auto* perm = reinterpret_cast<int32_t*>(in + L.perm);
  auto* pos = reinterpret_cast<int32_t*>(in + L.pos);
  auto* h = reinterpret_cast<_Float16*>(in + L.h);
  auto* y = reinterpret_cast<float*>(in + L.y);
  auto* gp = reinterpret_cast<float*>(in + L.gp);
  const auto* xb = static_cast<const uint16_t*>(x);
  const auto* sc = static_cast<const uint16_t*>(scales);
  auto* rp = L.rp ? reinterpret_cast<float*>(in + L.rp) : nullptr;
  MOE_HIP(moe::launch_router(xb, router_w, router_bias, pad_mask, ids, w, rp, T, d, E, k, s), "router");
  MOE_HIP(moe::launch_onehot_expand(ids, w, pad_mask, ids_all, gates, T, E, k, s), "onehot_expand");
  auto* dch = L.dchunk ? reinterpret_cast<int32_t*>(in + L.dchunk) : nullptr;
  MOE_HIP(moe::launch_dispatch(ids_all, pad_mask, counts, offsets, perm, pos, T, E, E, dch, s), "dispatch");
  auto* su = L.sused ? reinterpret_cast<int*>(in + L.sused) : nullptr;
  MOE_TRY(run_experts(xb, perm, offsets, w_gate, w_up, w_down, sc, h, y, L.splits, su, gp, L.gparts, T, d, f, E, E,
                      s));
  MOE_HIP(moe::launch_combine(y, L.splits, su, (size_t)T * E * d, pos, gates, pad_mask, out, T, d, E, s), "combine");
  return MOE_OK;
}

size_t moe_workspace_bytes_block(int T, int d, int f, int E, int k) {
  if (check_shape(T, d, f, E, k) != MOE_OK || T == 0) return 0;
  return block_prefix_bytes(T, d) + make_layout(T, d, f, E, k).total;
}

int moe_block_forward(const void* h, const float* norm_pre, const float* norm_post, float eps,
                      const float* router_w, const int8_t* w_gate, const int8_t* w_up, const int8_t* w_down,
                      const void* scales, const uint8_t* pad_mask, float* h_out, int T, int d, int f, int E,
                      int k, void* stream, const float* router_bias, void* workspace, size_t workspace_bytes,
                      void* x_norm_out) {
  MOE_TRY(check_layer_args(h, router_w, w_gate, w_up, w_down, scales, h_out, T, d, f, E, k));
  MOE_TRY(check_ptr(norm_pre, "norm_pre"));
  MOE_TRY(check_ptr(norm_post, "norm_post"));
  if (!(eps >= 0.0f)) return fail(MOE_ERR_INVALID, "eps must be >= 0");
  if (router_bias && !aligned(router_bias, 4)) return fail(MOE_ERR_INVALID, "router_bias is not 4-byte aligned");
  if (T == 0) return MOE_OK;
  const size_t xbytes = round_up((size_t)T * d * 2, 256);
  const size_t prefix = block_prefix_bytes(T, d);
  const Layout L = make_layout(T, d, f, E, k);
  const size_t need = prefix + L.total;
  char* ws = nullptr;
  if (workspace) {
    if (!aligned(workspace, 256)) return fail(MOE_ERR_INVALID, "workspace is not 256-byte aligned");
    if (workspace_bytes < need) return fail(MOE_ERR_INVALID, "workspace too small: need " + std::to_string(need) + " bytes");
    ws = static_cast<char*>(workspace);
  } else {
    MOE_TRY(library_workspace(need, &ws));
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto* xn = reinterpret_cast<uint16_t*>(ws);
  auto* sumsq = block_sumsq_bytes(T, d) ? reinterpret_cast<float*>(ws + xbytes) : nullptr;
  char* in = ws + prefix;
  auto* ids = reinterpret_cast<int32_t*>(in + L.ids);
  auto* w = reinterpret_cast<float*>(in + L.w);
  auto* counts = reinterpret_cast<int32_t*>(in + L.counts);
  auto* offsets = reinterpret_cast<int32_t*>(in + L.offsets);
  auto* perm = reinterpret_cast<int32_t*>(in + L.perm);
  auto* pos = reinterpret_cast<int32_t*>(in + L.pos);
  auto* hh = reinterpret_cast<_Float16*>(in + L.h);
  auto* y = reinterpret_cast<float*>(in + L.y);
  auto* gp = reinterpret_cast<float*>(in + L.gp);
  const auto* hb = static_cast<const uint16_t*>(h);
  const auto* sc = static_cast<const uint16_t*>(scales);
  if (L.rp) {
    // small batches: the norm, then the group sums in parallel, then routing + dispatch
    auto* rp = reinterpret_cast<float*>(in + L.rp);
    MOE_HIP(moe::launch_rmsnorm(hb, norm_pre, eps, xn, T, d, s), "rmsnorm");
    MOE_HIP(moe::launch_router_partial(xn, router_w, rp, T, d, s), "router");
    MOE_HIP(moe::launch_route_finish(rp, router_bias, pad_mask, ids, w, counts, offsets, perm, pos, T, d, E, k, s),
            "route+dispatch");
  } else {
    MOE_HIP(moe::launch_prenorm_router(hb, norm_pre, eps, xn, router_w, router_bias, pad_mask, ids, w, T, d, E, k,
                                       s),
            "prenorm_router");
    auto* dch = L.dchunk ? reinterpret_cast<int32_t*>(in + L.dchunk) : nullptr;
    MOE_HIP(moe::launch_dispatch(ids, pad_mask, counts, offsets, perm, pos, T, E, k, dch, s), "dispatch");
  }
  auto* su = L.sused ? reinterpret_cast<int*>(in + L.sused) : nullptr;
  MOE_TRY(run_experts(xn, perm, offsets, w_gate, w_up, w_down, sc, hh, y, L.splits, su, gp, L.gparts, T, d, f, E, k,
                      s));
  MOE_HIP(moe::launch_combine_postnorm(y, L.splits, su, (size_t)T * k * d, pos, w, pad_mask, hb, norm_post, eps, h_out,
                                       sumsq, T, d, k, s),
          "combine_postnorm");
  if (x_norm_out)
    MOE_HIP(hipMemcpyAsync(x_norm_out, xn, (size_t)T * d * 2, hipMemcpyDeviceToDevice, s), "x_norm copy");
  return MOE_OK;
}

int moe_forward(const void* x, const float* router_w, const int8_t* w_gate, const int8_t* w_up,
                const int8_t* w_down, const void* scales, const uint8_t* pad_mask, float* out, int T,
                int d, int f, int E, int k, void* stream) {
  return moe_forward_ex(x, router_w, w_gate, w_up, w_down, scales, pad_mask, out, T, d, f, E, k, stream,
                        nullptr, nullptr, 0, nullptr);
}

int moe_route(const void* x, const float* router_w, const float* router_bias, const uint8_t* pad_mask,
              int32_t* topk_ids, float* topk_w, int T, int d, int E, int k, void* stream) {
  MOE_TRY(check_shape(T, d, 256, E, k));
  MOE_TRY(check_ptr(x, "x"));
  MOE_TRY(check_ptr(router_w, "router_w"));
  MOE_TRY(check_ptr(topk_ids, "topk_ids", 4));
  MOE_TRY(check_ptr(topk_w, "topk_w", 4));
  if (T == 0) return MOE_OK;
  // small batches with E = 8: the group sums in the library workspace
  char* rp = nullptr;
  const size_t rp_floats = moe::router_partial_floats(T, d, E);
  if (rp_floats > 0) MOE_TRY(library_workspace(rp_floats * 4, &rp));
  MOE_HIP(moe::launch_router(static_cast<const uint16_t*>(x), router_w, router_bias, pad_mask, topk_ids,
                             topk_w, reinterpret_cast<float*>(rp), T, d, E, k, static_cast<hipStream_t>(stream)),
          "router");
  return MOE_OK;
}

int moe_dispatch(const int32_t* topk_ids, const uint8_t* pad_mask, int32_t* counts, int32_t* offsets,
                 int32_t* perm, int32_t* pos, int T, int E, int k, void* stream) {
  MOE_TRY(check_shape(T, 256, 256, E, k));
  MOE_TRY(check_ptr(topk_ids, "topk_ids", 4));
  MOE_TRY(check_ptr(counts, "counts", 4));
  MOE_TRY(check_ptr(offsets, "offsets", 4));
  MOE_TRY(check_ptr(pos, "pos", 4));
  if (T > 0) MOE_TRY(check_ptr(perm, "perm", 4));
  // large batches: the chunked dispatch, its per-chunk counts in the library workspace
  char* dch = nullptr;
  const int nchunks = moe::dispatch_chunks(T);
  if (nchunks > 0) MOE_TRY(library_workspace((size_t)2 * nchunks * E * 4, &dch));
  MOE_HIP(moe::launch_dispatch(topk_ids, pad_mask, counts, offsets, perm, pos, T, E, k,
                               reinterpret_cast<int32_t*>(dch), static_cast<hipStream_t>(stream)),
          "dispatch");
  return MOE_OK;
}

int moe_gate_up(const void* x, const int32_t* perm, const int32_t* offsets, const int8_t* w_gate,
                const int8_t* w_up, const void* scales, void* h, int T, int d, int f, int E, int k,
                void* stream) {
  MOE_TRY(check_shape(T, d, f, E, k));
  MOE_TRY(check_ptr(x, "x"));
  MOE_TRY(check_ptr(perm, "perm", 4));
  MOE_TRY(check_ptr(offsets, "offsets", 4));
  MOE_TRY(check_ptr(w_gate, "w_gate"));
  MOE_TRY(check_ptr(w_up, "w_up"));
  MOE_TRY(check_ptr(scales, "scales"));
  MOE_TRY(check_ptr(h, "h"));
  if (T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const auto* xb = static_cast<const uint16_t*>(x);
  const auto* sc = static_cast<const uint16_t*>(scales);
  auto* hh = static_cast<_Float16*>(h);
  if (moe::streaming_experts(T, d, f)) {
    // the same split of the contraction as moe_forward; its partial sums live in the
    // library workspace
    const int parts = gate_up_parts(T, d, f, E, k);
    char* gp = nullptr;
    if (parts > 1) MOE_TRY(library_workspace((size_t)2 * parts * T * k * f * 4, &gp));
    MOE_HIP(moe::launch_gate_up_decode(xb, perm, offsets, w_gate, w_up, sc, hh, reinterpret_cast<float*>(gp), parts,
                                       T, k, d, f, E, s),
            "gate_up");
  } else
    MOE_HIP(moe::launch_gate_up_prefill(xb, perm, offsets, w_gate, w_up, sc, hh, T * k, d, f, E, s), "gate_up");
  return MOE_OK;
}

int moe_down(const void* h, const int32_t* offsets, const int8_t* w_down, const void* scales, float* y,
             int splits, int T, int d, int f, int E, int k, void* stream) {
  MOE_TRY(check_shape(T, d, f, E, k));
  MOE_TRY(check_ptr(h, "h"));
  MOE_TRY(check_ptr(offsets, "offsets", 4));
  MOE_TRY(check_ptr(w_down, "w_down"));
  MOE_TRY(check_ptr(scales, "scales"));
  MOE_TRY(check_ptr(y, "y"));
  if (splits < 1 || (f / 128) % splits != 0) return fail(MOE_ERR_INVALID, "splits must divide f / 128");
  if (T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const auto* hh = static_cast<const _Float16*>(h);
  const auto* sc = static_cast<const uint16_t*>(scales);
  if (moe::streaming_experts(T, d, f))
    MOE_HIP(moe::launch_down_decode(hh, offsets, w_down, sc, y, splits, T * k, T, d, f, E, s), "down");
  else
    MOE_HIP(moe::launch_down_prefill(hh, offsets, w_down, sc, y, splits, T * k, d, f, E, nullptr, s), "down");
  return MOE_OK;
}

int moe_combine(const float* y, int splits, const int32_t* pos, const float* topk_w, const uint8_t* pad_mask,
                float* out, int T, int d, int k, void* stream) {
  MOE_TRY(check_shape(T, d, 256, k, k));
  MOE_TRY(check_ptr(y, "y"));
  MOE_TRY(check_ptr(pos, "pos", 4));
  MOE_TRY(check_ptr(topk_w, "topk_w", 4));
  MOE_TRY(check_ptr(out, "out"));
  if (splits < 1) return fail(MOE_ERR_INVALID, "splits must be >= 1");
  if (T == 0) return MOE_OK;
  MOE_HIP(moe::launch_combine(y, splits, nullptr, (size_t)T * k * d, pos, topk_w, pad_mask, out, T, d, k,
                              static_cast<hipStream_t>(stream)),
          "combine");
  return MOE_OK;
}

// ---------------------------------------------------------------------------------------
// Single-launch forward: the five launches captured once into a HIP graph and replayed.


int moe_graph_create(moe_graph** out_graph, const void* x, const float* router_w, const int8_t* w_gate,
                     const int8_t* w_up, const int8_t* w_down, const void* scales, const uint8_t* pad_mask,
                     float* out, int T, int d, int f, int E, int k, const float* router_bias, void* workspace,
                     size_t workspace_bytes) {
  if (!out_graph) return fail(MOE_ERR_INVALID, "out_graph is NULL");
  *out_graph = nullptr;
  MOE_TRY(check_layer_args(x, router_w, w_gate, w_up, w_down, scales, out, T, d, f, E, k));
  if (T == 0) return fail(MOE_ERR_INVALID, "T must be > 0 for a graph");
  // The workspace must exist before the capture (nothing may allocate inside it) and must
  // live as long as the graph: without a caller workspace the graph allocates its own (the
  // library workspace could be reallocated by a later, larger call).
  if (router_bias && !aligned(router_bias, 4)) return fail(MOE_ERR_INVALID, "router_bias is not 4-byte aligned");
  char* ws = static_cast<char*>(workspace);
  const Layout L = make_layout(T, d, f, E, k);
  const size_t need = L.total;
  if (ws && !aligned(ws, 256)) return fail(MOE_ERR_INVALID, "workspace is not 256-byte aligned");
  if (ws && workspace_bytes < need)
    return fail(MOE_ERR_INVALID, "workspace too small: need " + std::to_string(need) + " bytes");
  int* ctl = nullptr;  // a caller's workspace: the graph zeroes its control block on every replay
  auto* g = new moe_graph();
  if (!ws) {
    const char* hook = std::getenv("MOE_TEST_FAIL_ALLOC");
    hipError_t ea = (hook && hook[0] == '1') ? hipErrorOutOfMemory : hipMalloc(&g->own_ws, round_up(need, 256));
    if (ea != hipSuccess) {
      (void)hipGetLastError();
      g->own_ws = nullptr;
      destroy_graph(g);
      return fail(MOE_ERR_NOMEM, std::string("graph workspace hipMalloc of ") + std::to_string(need) +
                                     " bytes failed: " + hipGetErrorString(ea));
    }
    ws = static_cast<char*>(g->own_ws);
    if (L.one_launch && one_launch_enabled()) {
      // zeroed once here; every replay leaves it zero
      ctl = reinterpret_cast<int*>(ws + L.ctl);
      hipError_t ez = hipMemset(ctl, 0, (size_t)moe::kLayerCtlWords * 4);
      if (ez != hipSuccess) {
        destroy_graph(g);
        return hip_fail(ez, "hipMemset(control block)");
      }
    }
  }
  hipStream_t cs = nullptr;
  hipError_t ec = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (ec != hipSuccess) {
    destroy_graph(g);
    return hip_fail(ec, "hipStreamCreate");
  }
  int rc = MOE_OK;
  hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    rc = hip_fail(e, "hipStreamBeginCapture");
  } else {
    rc = forward_impl(x, router_w, w_gate, w_up, w_down, scales, pad_mask, out, T, d, f, E, k, cs, router_bias, L,
                      ws, ctl, nullptr);
    hipError_t e2 = hipStreamEndCapture(cs, &g->graph);
    if (rc == MOE_OK && e2 != hipSuccess) rc = hip_fail(e2, "hipStreamEndCapture");
  }
  if (rc == MOE_OK) {
    e = hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0);
    if (e != hipSuccess) rc = hip_fail(e, "hipGraphInstantiate");
  }
  (void)hipStreamDestroy(cs);
  if (rc != MOE_OK) {
    destroy_graph(g);
    return rc;
  }
  *out_graph = g;
  return MOE_OK;
}

int moe_graph_launch(moe_graph* g, void* stream) {
  if (!g || !g->exec) return fail(MOE_ERR_INVALID, "graph is NULL");
  MOE_HIP(hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream)), "hipGraphLaunch");
  return MOE_OK;
}

void moe_graph_destroy(moe_graph* g) {
  if (!g) return;
  destroy_graph(g);
}

}  // extern "C"
