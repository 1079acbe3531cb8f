/*
 * moe.h — C ABI of the MI355X (gfx950) forward pass of Grok-1's top-2-of-8
 * Mixture-of-Experts feed-forward layer (MoELayer + Router).
 *
 * The operation (Grok-1 Admin & Architecture Guide, section 3 "The Model",
 * subsection "Mixture of Experts (MoELayer + Router)", steps 1-4; subsection
 * "Quantized weights"; section 9 for fp32 routing):
 *
 *   l[t,e]  = sum_i x[t,i] * router_w[i,e] (+ router_bias[e])         fp32
 *   p[t,:]  = softmax(l[t,:])                                          fp32
 *   ids[t]  = the k experts of largest p (ties -> lower index), slot 0 largest
 *   w[t,j]  = p[t, ids[t,j]]                                (not renormalised)
 *   for each selected expert e = ids[t,j]:
 *     g = x[t] (q_gate[e] * s_gate[e]),  u = x[t] (q_up[e] * s_up[e])
 *     h = gelu_tanh(g) * u
 *     y = h (q_down[e] * s_down[e])
 *   out[t]  = sum_j w[t,j] * y_(t,j);   padded tokens: ids -1, w 0, out row +0.0
 *
 * The expert FFN is the gated GeLU MLP gelu(linear(x)) * linear_v(x) -> linear_1 of
 * step 3; the weights are int8 with one bf16 scale per output channel, dequantised as
 * q * s (section 3 "Quantized weights"). GeLU is the tanh form. The layer is
 * token-wise, so a [B, S, d] activation is passed flattened as T = B * S rows; the
 * caller applies the pre-norm and the residual add around it (grok-field-guide source
 * map, fourth stop: moe(rms_norm(h), padding_mask) added to h).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE memory owned by the caller, row-major, and must
 *     stay valid until the work enqueued on `stream` completes. Pointers to vector data
 *     must be 16-byte aligned (x, router_w, weights, scales, out, h, y). The library never frees
 *     or retains a caller pointer beyond the call.
 *   - `stream` is a hipStream_t (NULL = the default stream). All work is enqueued
 *     asynchronously; no entry point synchronises the host with the device, except the
 *     first call on a device that needs the library workspace (hipMalloc).
 *   - dtypes: x bf16 [T][d]; router_w fp32 [d][E]; router_bias fp32 [E];
 *     w_gate, w_up int8 [E][d][f]; w_down int8 [E][f][d];
 *     scales bf16 [E][2f + d] = per expert gate[f] | up[f] | down[d];
 *     pad_mask uint8 [T] (1 = real token, 0 = padded) or NULL = all real;
 *     out fp32 [T][d].
 *   - Every argument is checked before anything is enqueued. On error nothing is
 *     enqueued, outputs are untouched and a message is available from
 *     moe_last_error() (per thread). Errors:
 *       MOE_ERR_INVALID      a required pointer is NULL or misaligned; T < 0;
 *                            d, f, E or k <= 0; k > E; a workspace that is too small
 *       MOE_ERR_UNSUPPORTED  E > 64; d or f not a multiple of 256; T * k above 2^24
 *                            assignments; d * f of 2^31 bytes or more (one expert's
 *                            matrix is addressed with 32-bit byte offsets)
 *       MOE_ERR_HIP          a HIP launch or copy failed (message holds HIP's string)
 *       MOE_ERR_NOMEM        the library workspace could not be allocated
 *     T == 0 is a successful no-op. Device faults surface at the caller's next sync.
 *   - The library workspace is one buffer per device, grown on demand and shared by
 *     all calls on that device: calls that overlap in time on one device (different
 *     streams, different threads) race unless each passes its own workspace through
 *     moe_forward_ex.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden symbol visibility; these declarations are its exports. */
#pragma GCC visibility push(default)

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_HIP = 3,
  MOE_ERR_NOMEM = 4
} moe_status;

/* Optional device outputs of the routing and dispatch steps (NULL member = not wanted).
   topk_ids int32 [T][k]; topk_w fp32 [T][k]; counts int32 [E]; offsets int32 [E+1];
   perm int32 [T*k] (first offsets[E] entries valid); pos int32 [T][k]. */
typedef struct {
  int32_t* topk_ids;
  float* topk_w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* pos;
} moe_debug_out;

/* The layer forward pass (steps 1-4 above), without router bias. */
int moe_forward(const void* x, const float* router_w, const int8_t* w_gate, const int8_t* w_up,
                const int8_t* w_down, const void* scales, const uint8_t* pad_mask, float* out,
                int T, int d, int f, int E, int k, void* stream);

/* Same as moe_forward, plus:
   router_bias  fp32 [E] added to the logits before the softmax, or NULL;
   workspace    caller-owned device buffer of at least moe_workspace_bytes(T, d, f, E, k)
                bytes (256-byte aligned), or NULL to use the library workspace (on the
                one-launch path, see moe_one_launch, it also holds that kernel's control
                block, which the call zeroes with a small kernel first; any prior contents
                are fine);
   dbg          optional copies of the routing and dispatch arrays, or NULL. */
int moe_forward_ex(const void* x, const float* router_w, const int8_t* w_gate, const int8_t* w_up,
                   const int8_t* w_down, const void* scales, const uint8_t* pad_mask, float* out,
                   int T, int d, int f, int E, int k, void* stream, const float* router_bias,
                   void* workspace, size_t workspace_bytes, const moe_debug_out* dbg);

/* Step 1-2 alone: router logits, softmax and top-k (Guide section 3, MoE steps 1-2).
   Writes topk_ids int32 [T][k] and topk_w fp32 [T][k]; padded tokens get -1 and 0. A token's
   logits are summed in one fixed order whatever the batch size, so its ids and weights are
   the same bits in any batch and in moe_forward. At T <= 64 with E = 8 the per-group partial
   sums live in the library workspace, which this call may allocate (MOE_ERR_NOMEM if it
   cannot) and which overlapping calls share. */
int moe_route(const void* x, const float* router_w, const float* router_bias,
              const uint8_t* pad_mask, int32_t* topk_ids, float* topk_w, int T, int d, int E,
              int k, void* stream);

/* Dispatch: a stable counting sort of the (token, slot) assignments by expert, the
   gather that replaces the one-hot selection of the dense formulation (Guide section 3,
   warning under the MoE steps; section 10, first item). counts[e] = assignments of real
   tokens to e; offsets = exclusive prefix sum [E+1]; perm[offsets[e] + r] = the r-th
   smallest token routed to e; pos[t][j] = index of (t, j) in perm. pos is -1 for padded
   tokens and for slots whose id is out of [0, E) or repeats an earlier slot of the same
   token (such slots are not counted). Integer work; bit-exact. From T = 4096 on the sort
   runs over 1024-token chunks in parallel (same result), with its per-chunk counts in the
   library workspace, which this call may then allocate. */
int moe_dispatch(const int32_t* topk_ids, const uint8_t* pad_mask, int32_t* counts,
                 int32_t* offsets, int32_t* perm, int32_t* pos, int T, int E, int k, void* stream);

/* Step 3, first half, for every expert segment of the dispatch: rows r of expert e's
   segment take x[perm[r]]; g, u = that row times the dequantised gate / up matrices
   (fp32 accumulation, per-output-channel scales applied in fp32); h = gelu_tanh(g) * u,
   stored as fp16 in h [T*k][f] at row r. Rows at or beyond offsets[E] are not written.
   At T <= 160 with narrow f (too few 256-column slabs to fill the chip; expert matrices above
   2^23 weights, which take the streaming kernels there) the contraction over
   d is split as in moe_forward; the partial sums then live in the library workspace, which
   this call may allocate (MOE_ERR_NOMEM if it cannot) and which overlapping calls share. */
int moe_gate_up(const void* x, const int32_t* perm, const int32_t* offsets, const int8_t* w_gate,
                const int8_t* w_up, const void* scales, void* h, int T, int d, int f, int E, int k,
                void* stream);
/* The parts moe_forward and moe_gate_up split gate/up's contraction over d into for a shape: 1,
   or more (a second launch then adds the parts' partial sums and applies the GeGLU); 0 for a
   shape the library rejects. Host only. */
int moe_gate_up_parts(int T, int d, int f, int E, int k);

/* Step 3, second half: y = h (q_down[e] * s_down[e]) for the rows of every expert segment,
   with the contraction over f cut into `splits` equal parts: y fp32 [splits][T*k][d] holds
   one partial sum per part (their sum, in part order, is the result). splits must divide
   f / 128. moe_down_splits() gives the count moe_forward launches with for a shape; at
   T > 160 moe_forward's own down launch may then keep fewer of those 2 or 4 parts (1 or 2;
   1, 2 or 4), which its combine learns on the device (this entry point always writes exactly
   `splits`). */
int moe_down(const void* h, const int32_t* offsets, const int8_t* w_down, const void* scales,
             float* y, int splits, int T, int d, int f, int E, int k, void* stream);
int moe_down_splits(int T, int d, int f, int E, int k);

/* Which expert kernels moe_forward, moe_gate_up and moe_down run for a shape: 0 = the
   weight-streaming kernels (T <= 160 and more than 2^23 weights per expert matrix), else the
   row height of the tiled MFMA kernels' tiles, 128 (at most 96 assignments per expert on
   average) or 256. -1 for a shape the library rejects (moe_last_error() says why). Host only:
   no device call, no allocation. */
int moe_expert_kernels(int T, int d, int f, int E, int k);

/* The one-launch layer, an alternative to the launch-per-stage sequence for small batches
   (T <= 64, E = 8, expert matrices above 2^23 weights; not T <= 4 when the gate/up
   contraction is whole): routing, dispatch, both expert matrices and the combine run as work
   items of one kernel, with the same arithmetic in the same order, so the result is the same
   bits. It is slower on MI355X than one launch per stage (waiting items hold whole SIMDs), so
   moe_forward, moe_forward_ex, moe_forward_noalloc and moe_graph_create take it only when the
   environment variable MOE_ONE_LAUNCH is "1" at the call. Returns 1 if they would take it for
   this shape now, 0 if not, -1 for a shape the library rejects. Host only. */
int moe_one_launch(int T, int d, int f, int E, int k);

/* Step 4: out[t] = sum over j of topk_w[t][j] * (sum over parts s of y[s][pos[t][j]]),
   parts in order, slots in order, fp32; +0.0 rows for padded tokens. */
int moe_combine(const float* y, int splits, const int32_t* pos, const float* topk_w,
                const uint8_t* pad_mask, float* out, int T, int d, int k, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
   loops, harnesses that forbid hipMalloc): moe_forward_ex without workspace or dbg arguments,
   whose scratch (the routing, dispatch, H and Y arrays) is a fixed array of
   MOE_NOALLOC_SCRATCH_BYTES in device memory that the library defines, one per device, held
   until the process ends. The call allocates and frees nothing (no hipMalloc or hipFree, no
   allocating library routine); its first call on a device looks up that device's copy of the
   array. Shapes whose workspace (moe_workspace_bytes) exceeds MOE_NOALLOC_SCRATCH_BYTES are
   rejected with MOE_ERR_UNSUPPORTED before anything is enqueued: 64 MiB hold the Grok-1 shape
   (d = 6144, f = 32768) up to 204 tokens. Every call on a device shares that device's
   array: calls that overlap in time on one device (other streams, other threads) race.
   Results equal moe_forward_ex's bit for bit; errors as moe_forward_ex. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_forward_noalloc(const void* x, const float* router_w, const int8_t* w_gate, const int8_t* w_up,
                        const int8_t* w_down, const void* scales, const uint8_t* pad_mask, float* out,
                        int T, int d, int f, int E, int k, void* stream, const float* router_bias);

/* The dense one-hot-gated formulation the sources describe for their own implementation
   (Guide section 3, MoE step 4 and the warning under it): every one of the E experts runs
   on every real token and out[t] = sum over e (in order) of gate[t][e] * y_e(t), where
   gate[t][e] is the routing weight of e if the router selected it and 0 otherwise. Same
   arguments, layouts, errors and result (up to the order of the fp32 additions) as
   moe_forward_ex without dbg; E / k times the expert work. A baseline for the gather path,
   not a faster one. T * E must not exceed 2^24. Workspace: moe_workspace_bytes_dense. */
int moe_forward_dense(const void* x, const float* router_w, const int8_t* w_gate, const int8_t* w_up,
                      const int8_t* w_down, const void* scales, const uint8_t* pad_mask, float* out,
                      int T, int d, int f, int E, int k, void* stream, const float* router_bias,
                      void* workspace, size_t workspace_bytes);
size_t moe_workspace_bytes_dense(int T, int d, int f, int E, int k);

/* The MoE block of a decoder layer with its neighbours fused (Guide section 3 "Transformer
   stack": pre- and post-norm RMSNorm around the MoE block and the residual h += h_dense;
   grok-field-guide source map, fourth stop):
     x     = bf16(h * (1 / sqrt(mean(h^2) + eps)) * norm_pre)   (fused into the router kernel)
     m     = the layer above on x (same routing, experts and combine)
     h_out = h + m * (1 / sqrt(mean(m^2) + eps)) * norm_post    (fused into the combine kernel)
   h bf16 [T][d]; norm_pre, norm_post fp32 [d] (16-byte aligned); eps >= 0; h_out fp32 [T][d].
   Padded tokens: m = 0, so h_out = h. x_norm_out: optional bf16 [T][d] copy of x (NULL = not
   wanted). The sources give neither eps nor the norm scales' form; these are the readings.
   Workspace: moe_workspace_bytes_block. Errors as moe_forward_ex. */
int moe_block_forward(const void* h, const float* norm_pre, const float* norm_post, float eps,
                      const float* router_w, const int8_t* w_gate, const int8_t* w_up,
                      const int8_t* w_down, const void* scales, const uint8_t* pad_mask, float* h_out,
                      int T, int d, int f, int E, int k, void* stream, const float* router_bias,
                      void* workspace, size_t workspace_bytes, void* x_norm_out);
size_t moe_workspace_bytes_block(int T, int d, int f, int E, int k);

/* Single-launch forward (for decode loops with fixed buffers): the router, dispatch,
   expert and combine launches of one moe_forward_ex call are captured once into a HIP
   graph; each moe_graph_launch replays all of them with one hipGraphLaunch on `stream`.
   The graph holds the pointers and shapes given here: every replay reads the inputs'
   current contents at those addresses and writes out. A caller workspace must stay alive
   as long as the graph and must not be used by overlapping calls; with workspace NULL the
   graph allocates its own (moe_graph_create may return MOE_ERR_NOMEM) and
   moe_graph_destroy frees it after waiting for the device. moe_graph_launch allocates
   nothing; replays of one graph must not overlap. T must be > 0. */
typedef struct moe_graph moe_graph;
int moe_graph_create(moe_graph** graph, const void* x, const float* router_w, const int8_t* w_gate,
                     const int8_t* w_up, const int8_t* w_down, const void* scales,
                     const uint8_t* pad_mask, float* out, int T, int d, int f, int E, int k,
                     const float* router_bias, void* workspace, size_t workspace_bytes);
int moe_graph_launch(moe_graph* graph, void* stream);
void moe_graph_destroy(moe_graph* graph);

/* Bytes of device workspace moe_forward needs for a shape (0 for T == 0). */
size_t moe_workspace_bytes(int T, int d, int f, int E, int k);

/* Frees the library workspace of every device (waits for the device first). */
void moe_release_workspace(void);

/* Message of the last failed call on this thread ("" if none). */
const char* moe_last_error(void);

/* ABI version of this header. */
int moe_abi_version(void);
#define MOE_ABI_VERSION 1

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
