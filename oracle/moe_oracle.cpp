/*
 * CPU oracle for the forward pass of the top-2-of-8 Mixture-of-Experts feed-forward
 * layer of Grok-1 (MoELayer + Router).
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this library. It shares no code, header, table or helper with the GPU
 * library; the two meet only through the seeded inputs of the `synth` package.
 *
 * What it follows (page titles and sections of the sources):
 *   [G3-MoE]   Grok-1 Admin & Architecture Guide, section 3 "The Model", subsection
 *              "Mixture of Experts (MoELayer + Router)", steps 1-4 and the warning under them
 *   [G3-Q]     same guide, section 3, subsection "Quantized weights"
 *   [G9]       same guide, section 9 "Code Quality & Conventions" (routing and softmax in fp32)
 *   [G3-cfg]   same guide, section 3 "Configuration objects" (emb_size, num_experts,
 *              num_selected_experts, fprop dtype) and the ffn_size note under the MoE steps
 *   [FG4]      grok-field-guide source-code map, fourth stop (DecoderLayer): the MoE block is
 *              called as moe(rms_norm(h), padding_mask) and its result added to h outside it;
 *              the page notes that its code leaves out an extra RMSNorm of the source
 *   [G3-stack] same guide, section 3 "Transformer stack and language model head": pre- and
 *              post-norm RMSNorm around the FFN/MoE block, residual h += h_dense
 *
 * Arithmetic: fp32 throughout (routing, softmax, expert FFN, combine), every operation
 * rounded on its own (built with -ffp-contract=off), sums taken in index order.
 * Readings where the sources are silent (each one also listed in the design notes):
 *   - GELU is the tanh form 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)))  [G3-MoE step 3
 *     names only "gelu"; the tanh form is the default gelu of the JAX release the guide names]
 *   - routing weights are the softmax probabilities of the selected experts, not renormalised
 *   - top-k ties go to the lower expert index; slot 0 holds the largest probability
 *   - softmax subtracts the max logit first (same value in exact arithmetic)
 *   - dequantisation w = q * s uses one scale per output channel; q * s is exact in fp32
 *   - the padding mask is 1 for a real token and 0 for a padded one; padded tokens get no
 *     expert, no routing weight and an output row of +0.0
 *   - an optional per-expert router bias is added to the logits before the softmax
 *
 * Layouts (row-major): x bf16 [T][d]; router_w fp32 [d][E]; w_gate, w_up int8 [E][d][f];
 * w_down int8 [E][f][d]; scales bf16 [E][2f+d] = gate[f] | up[f] | down[d];
 * pad_mask uint8 [T] or NULL (all real); out fp32 [T][d].
 */
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

float bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

int thread_count(int requested) {
  if (requested > 0) return requested;
  unsigned h = std::thread::hardware_concurrency();
  return h ? (int)h : 1;
}

// Run body(lo, hi) over [0, n) split into contiguous chunks, one per thread.
template <class F>
void parallel_chunks(int n, int nthreads, F body) {
  nthreads = std::max(1, std::min(nthreads, n));
  if (nthreads == 1) {
    body(0, n);
    return;
  }
  std::vector<std::thread> pool;
  int per = (n + nthreads - 1) / nthreads;
  for (int w = 0; w < nthreads; ++w) {
    int lo = w * per, hi = std::min(n, lo + per);
    if (lo >= hi) break;
    pool.emplace_back([=] { body(lo, hi); });
  }
  for (auto& th : pool) th.join();
}

bool is_real(const uint8_t* pad_mask, int t) { return pad_mask == nullptr || pad_mask[t] != 0; }

}  // namespace

extern "C" {

/* GeLU, tanh form (Hendrycks & Gimpel 2016, eq. for the tanh approximation), fp32.
   [G3-MoE step 3: the expert is a gated GeLU MLP, gelu(linear(x)) * linear_v(x) -> linear_1] */
float oracle_gelu_tanh(float v) {
  const float c = 0.7978845608028654f;  // sqrt(2 / pi)
  float inner = c * (v + 0.044715f * (v * v * v));
  return 0.5f * v * (1.0f + std::tanh(inner));
}

/* Router [G3-MoE steps 1-2, G9]: fp32 logits l[e] = sum_i x[t,i] W_r[i,e] (+ bias[e]),
   softmax over the E experts, then the k most probable experts (ties -> lower index).
   Outputs (NULL = not wanted): logits, probs [T][E]; ids int32 [T][k] (-1 for padded tokens);
   w fp32 [T][k] (the selected probabilities, 0 for padded tokens);
   gap_sel [T] = p_(k) - p_(k+1) (distance of the selection boundary, +inf when k == E);
   gap_order [T] = min over j < k of p_(j) - p_(j+1) (+inf when k == 1); both +inf for pad.
   Returns 0, or -1 on bad sizes. */
int oracle_route(const uint16_t* x, const float* router_w, const float* router_bias,
                 const uint8_t* pad_mask, int T, int d, int E, int k, float* logits, float* probs,
                 int32_t* ids, float* w, float* gap_sel, float* gap_order) {
  if (T < 0 || d <= 0 || E <= 0 || k <= 0 || k > E) return -1;
  std::vector<float> l(E), p(E);
  std::vector<int> order(E);
  for (int t = 0; t < T; ++t) {
    const uint16_t* xt = x + (size_t)t * d;
    for (int e = 0; e < E; ++e) {
      float acc = 0.0f;
      for (int i = 0; i < d; ++i) acc += bf16_value(xt[i]) * router_w[(size_t)i * E + e];
      if (router_bias) acc += router_bias[e];
      l[e] = acc;
    }
    float m = l[0];
    for (int e = 1; e < E; ++e) m = std::max(m, l[e]);
    float s = 0.0f;
    for (int e = 0; e < E; ++e) {
      p[e] = std::exp(l[e] - m);
      s += p[e];
    }
    for (int e = 0; e < E; ++e) p[e] = p[e] / s;
    if (logits)
      for (int e = 0; e < E; ++e) logits[(size_t)t * E + e] = l[e];
    if (probs)
      for (int e = 0; e < E; ++e) probs[(size_t)t * E + e] = p[e];

    for (int e = 0; e < E; ++e) order[e] = e;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return p[a] > p[b]; });
    bool real = is_real(pad_mask, t);
    for (int j = 0; j < k; ++j) {
      if (ids) ids[(size_t)t * k + j] = real ? order[j] : -1;
      if (w) w[(size_t)t * k + j] = real ? p[order[j]] : 0.0f;
    }
    if (gap_sel) gap_sel[t] = (!real || k == E) ? INFINITY : p[order[k - 1]] - p[order[k]];
    if (gap_order) {
      float g = INFINITY;
      if (real)
        for (int j = 0; j + 1 < k; ++j) g = std::min(g, p[order[j]] - p[order[j + 1]]);
      gap_order[t] = g;
    }
  }
  return 0;
}

/* Dispatch: a stable counting sort of the (token, slot) assignments by expert.
   counts[e] = number of real (t, j) with ids[t,j] == e; offsets = exclusive prefix sum [E+1];
   perm[offsets[e] + r] = the r-th smallest token routed to e; pos[t,j] = index of (t, j) in
   perm, -1 for padded tokens. This replaces the one-hot selection of the dense formulation by
   a gather [G3-MoE, warning under the steps; section 10 "Potential Improvements", first item].
   Returns 0, or -1 when an id is out of range. */
int oracle_dispatch(const int32_t* ids, const uint8_t* pad_mask, int T, int E, int k,
                    int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos) {
  if (T < 0 || E <= 0 || k <= 0) return -1;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int t = 0; t < T; ++t) {
    if (!is_real(pad_mask, t)) continue;
    for (int j = 0; j < k; ++j) {
      int e = ids[(size_t)t * k + j];
      if (e < 0 || e >= E) return -1;
      counts[e] += 1;
    }
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  std::vector<int32_t> next(offsets, offsets + E);
  for (int t = 0; t < T; ++t) {
    for (int j = 0; j < k; ++j) {
      if (!is_real(pad_mask, t)) {
        pos[(size_t)t * k + j] = -1;
        continue;
      }
      int e = ids[(size_t)t * k + j];
      int slot = next[e]++;
      perm[slot] = t;
      pos[(size_t)t * k + j] = slot;
    }
  }
  return 0;
}

/* Gate and up projections of expert e with the GeLU gate, for n activation rows
   [G3-MoE step 3; G3-Q dequantisation w = q * s, one scale per output channel]:
     g[r,c] = sum_i x[r,i] * (q_gate[e,i,c] * s_gate[e,c])    (fp32, i ascending)
     u[r,c] = sum_i x[r,i] * (q_up[e,i,c]   * s_up[e,c])
     h[r,c] = gelu_tanh(g[r,c]) * u[r,c]
   x_rows bf16 [n][d]; h fp32 [n][f] (optionally g, u fp32 [n][f]). */
int oracle_expert_hidden(const uint16_t* x_rows, int n, const int8_t* w_gate, const int8_t* w_up,
                         const uint16_t* scales, int d, int f, int E, int e, float* h, float* g_out,
                         float* u_out, int nthreads) {
  if (n < 0 || d <= 0 || f <= 0 || e < 0 || e >= E) return -1;
  const int8_t* qg = w_gate + (size_t)e * d * f;
  const int8_t* qu = w_up + (size_t)e * d * f;
  const uint16_t* sg = scales + (size_t)e * (2 * (size_t)f + d);
  const uint16_t* su = sg + f;
  const int RB = 16;  // rows per block: each weight row is read once per block
  parallel_chunks(f, thread_count(nthreads), [&](int c0, int c1) {
    int w = c1 - c0;
    std::vector<float> G((size_t)RB * w), U((size_t)RB * w), sgv(w), suv(w);
    for (int c = 0; c < w; ++c) sgv[c] = bf16_value(sg[c0 + c]), suv[c] = bf16_value(su[c0 + c]);
    for (int r0 = 0; r0 < n; r0 += RB) {
      int nb = std::min(RB, n - r0);
      std::fill(G.begin(), G.end(), 0.0f);
      std::fill(U.begin(), U.end(), 0.0f);
      for (int i = 0; i < d; ++i) {
        const int8_t* qgi = qg + (size_t)i * f + c0;
        const int8_t* qui = qu + (size_t)i * f + c0;
        for (int r = 0; r < nb; ++r) {
          float xv = bf16_value(x_rows[(size_t)(r0 + r) * d + i]);
          float* Gr = &G[(size_t)r * w];
          float* Ur = &U[(size_t)r * w];
          for (int c = 0; c < w; ++c) {
            Gr[c] += xv * ((float)qgi[c] * sgv[c]);
            Ur[c] += xv * ((float)qui[c] * suv[c]);
          }
        }
      }
      for (int r = 0; r < nb; ++r)
        for (int c = 0; c < w; ++c) {
          float gv = G[(size_t)r * w + c], uv = U[(size_t)r * w + c];
          size_t o = (size_t)(r0 + r) * f + c0 + c;
          h[o] = oracle_gelu_tanh(gv) * uv;
          if (g_out) g_out[o] = gv;
          if (u_out) u_out[o] = uv;
        }
    }
  });
  return 0;
}

/* Down projection of expert e [G3-MoE step 3 "-> linear_1"; G3-Q]:
     y[r,c] = sum_m h[r,m] * (q_down[e,m,c] * s_down[e,c])    (fp32, m ascending)
   h fp32 [n][f]; y fp32 [n][d]. */
int oracle_expert_down(const float* h, int n, const int8_t* w_down, const uint16_t* scales, int d,
                       int f, int E, int e, float* y, int nthreads) {
  if (n < 0 || d <= 0 || f <= 0 || e < 0 || e >= E) return -1;
  const int8_t* qd = w_down + (size_t)e * f * d;
  const uint16_t* sd = scales + (size_t)e * (2 * (size_t)f + d) + 2 * (size_t)f;
  const int RB = 16;
  parallel_chunks(d, thread_count(nthreads), [&](int c0, int c1) {
    int w = c1 - c0;
    std::vector<float> Y((size_t)RB * w), sdv(w);
    for (int c = 0; c < w; ++c) sdv[c] = bf16_value(sd[c0 + c]);
    for (int r0 = 0; r0 < n; r0 += RB) {
      int nb = std::min(RB, n - r0);
      std::fill(Y.begin(), Y.end(), 0.0f);
      for (int m = 0; m < f; ++m) {
        const int8_t* qdm = qd + (size_t)m * d + c0;
        for (int r = 0; r < nb; ++r) {
          float hv = h[(size_t)(r0 + r) * f + m];
          float* Yr = &Y[(size_t)r * w];
          for (int c = 0; c < w; ++c) Yr[c] += hv * ((float)qdm[c] * sdv[c]);
        }
      }
      for (int r = 0; r < nb; ++r)
        for (int c = 0; c < w; ++c) y[(size_t)(r0 + r) * d + c0 + c] = Y[(size_t)r * w + c];
    }
  });
  return 0;
}

/* The layer [G3-MoE steps 1-4]: route, run each selected expert on the tokens routed to it,
   then out[t] = 0 + w[t,0] * y_(t,0) + w[t,1] * y_(t,1) + ... (slots in order), where
   y_(t,j) is the output of expert ids[t,j] on token t. Padded tokens give +0.0 rows.
   The expert loop is blocked per expert over its tokens; every output element still has
   one fixed summation order, so the result does not depend on the thread count.
   ids/w (NULL = not wanted) receive the routing. Returns 0, or -1 on bad arguments. */
int oracle_forward(const uint16_t* x, const float* router_w, const float* router_bias,
                   const int8_t* w_gate, const int8_t* w_up, const int8_t* w_down,
                   const uint16_t* scales, const uint8_t* pad_mask, int T, int d, int f, int E,
                   int k, float* out, int32_t* ids_out, float* w_out, int nthreads) {
  if (T < 0 || d <= 0 || f <= 0 || E <= 0 || k <= 0 || k > E) return -1;
  std::vector<int32_t> ids((size_t)T * k);
  std::vector<float> w((size_t)T * k);
  if (oracle_route(x, router_w, router_bias, pad_mask, T, d, E, k, nullptr, nullptr, ids.data(),
                   w.data(), nullptr, nullptr) != 0)
    return -1;
  // y for every (t, j), computed per expert over the list of its tokens (t ascending).
  std::vector<float> ytj((size_t)T * k * d, 0.0f);
  for (int e = 0; e < E; ++e) {
    std::vector<int> tok, slot;
    for (int t = 0; t < T; ++t) {
      if (!is_real(pad_mask, t)) continue;
      for (int j = 0; j < k; ++j)
        if (ids[(size_t)t * k + j] == e) tok.push_back(t), slot.push_back(j);
    }
    const int BLK = 64;
    for (size_t b0 = 0; b0 < tok.size(); b0 += BLK) {
      int nb = (int)std::min<size_t>(BLK, tok.size() - b0);
      std::vector<uint16_t> xr((size_t)nb * d);
      for (int r = 0; r < nb; ++r)
        std::memcpy(&xr[(size_t)r * d], x + (size_t)tok[b0 + r] * d, sizeof(uint16_t) * d);
      std::vector<float> hr((size_t)nb * f), yr((size_t)nb * d);
      oracle_expert_hidden(xr.data(), nb, w_gate, w_up, scales, d, f, E, e, hr.data(), nullptr,
                           nullptr, nthreads);
      oracle_expert_down(hr.data(), nb, w_down, scales, d, f, E, e, yr.data(), nthreads);
      for (int r = 0; r < nb; ++r)
        std::memcpy(&ytj[((size_t)tok[b0 + r] * k + slot[b0 + r]) * d], &yr[(size_t)r * d],
                    sizeof(float) * d);
    }
  }
  for (int t = 0; t < T; ++t) {
    float* o = out + (size_t)t * d;
    if (!is_real(pad_mask, t)) {
      for (int c = 0; c < d; ++c) o[c] = 0.0f;
      continue;
    }
    for (int c = 0; c < d; ++c) {
      float acc = 0.0f;
      for (int j = 0; j < k; ++j) acc += w[(size_t)t * k + j] * ytj[((size_t)t * k + j) * d + c];
      o[c] = acc;
    }
  }
  // (an empty batch copies nothing: memcpy may not be handed the NULL data() of an empty vector)
  if (ids_out && !ids.empty()) std::memcpy(ids_out, ids.data(), sizeof(int32_t) * ids.size());
  if (w_out && !w.empty()) std::memcpy(w_out, w.data(), sizeof(float) * w.size());
  return 0;
}

/* The dense one-hot-gated formulation, written separately from oracle_forward
   [G3-MoE step 4 and the warning under it: every expert runs on every token, and the
   expert outputs are combined with one-hot selection masks scaled by the routing gate]:
     Y_all[t,e] = FFN_e(x[t]) for all E experts,  gate[t,e] = sum_j [ids[t,j] == e] w[t,j],
     out[t] = 0 + gate[t,0] Y_all[t,0] + ... + gate[t,E-1] Y_all[t,E-1].
   Its routing is its own code too. Token-at-a-time, column dot products; fp32. */
int oracle_forward_dense(const uint16_t* x, const float* router_w, const float* router_bias,
                         const int8_t* w_gate, const int8_t* w_up, const int8_t* w_down,
                         const uint16_t* scales, const uint8_t* pad_mask, int T, int d, int f,
                         int E, int k, float* out, int nthreads) {
  if (T < 0 || d <= 0 || f <= 0 || E <= 0 || k <= 0 || k > E) return -1;
  parallel_chunks(T, thread_count(nthreads), [&](int t0, int t1) {
    std::vector<float> xv(d), logit(E), prob(E), gate(E), hid(f), acc(d);
    std::vector<char> taken(E);
    for (int t = t0; t < t1; ++t) {
      float* o = out + (size_t)t * d;
      if (pad_mask && pad_mask[t] == 0) {
        std::fill(o, o + d, 0.0f);
        continue;
      }
      for (int i = 0; i < d; ++i) xv[i] = bf16_value(x[(size_t)t * d + i]);
      // routing probabilities
      for (int e = 0; e < E; ++e) {
        float s = 0.0f;
        for (int i = 0; i < d; ++i) s += xv[i] * router_w[(size_t)i * E + e];
        logit[e] = router_bias ? s + router_bias[e] : s;
      }
      float mx = *std::max_element(logit.begin(), logit.end());
      float z = 0.0f;
      for (int e = 0; e < E; ++e) z += (prob[e] = std::exp(logit[e] - mx));
      for (int e = 0; e < E; ++e) prob[e] /= z;
      // one-hot masks scaled by the gate: k rounds of "largest untaken, lowest index first"
      std::fill(gate.begin(), gate.end(), 0.0f);
      std::fill(taken.begin(), taken.end(), 0);
      for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e)
          if (!taken[e] && (best < 0 || prob[e] > prob[best])) best = e;
        taken[best] = 1;
        gate[best] += prob[best];
      }
      std::fill(acc.begin(), acc.end(), 0.0f);
      for (int e = 0; e < E; ++e) {
        const int8_t* qg = w_gate + (size_t)e * d * f;
        const int8_t* qu = w_up + (size_t)e * d * f;
        const int8_t* qd = w_down + (size_t)e * f * d;
        const uint16_t* sc = scales + (size_t)e * (2 * (size_t)f + d);
        for (int c = 0; c < f; ++c) {
          float sgc = bf16_value(sc[c]), suc = bf16_value(sc[f + c]);
          float gs = 0.0f, us = 0.0f;
          for (int i = 0; i < d; ++i) {
            gs += xv[i] * ((float)qg[(size_t)i * f + c] * sgc);
            us += xv[i] * ((float)qu[(size_t)i * f + c] * suc);
          }
          hid[c] = oracle_gelu_tanh(gs) * us;
        }
        for (int c = 0; c < d; ++c) {
          float sdc = bf16_value(sc[2 * (size_t)f + c]);
          float ys = 0.0f;
          for (int m = 0; m < f; ++m) ys += hid[m] * ((float)qd[(size_t)m * d + c] * sdc);
          acc[c] += gate[e] * ys;
        }
      }
      std::copy(acc.begin(), acc.end(), o);
    }
  });
  return 0;
}

/* Brute force in fp64 (every product, sum, exp and tanh in double), for tiny shapes:
   the same definition as oracle_forward, used to bound the fp32 oracle's rounding.
   Selection uses the fp64 probabilities. Outputs fp64 out [T][d]; ids [T][k] optional. */
int oracle_forward_f64(const uint16_t* x, const float* router_w, const float* router_bias,
                       const int8_t* w_gate, const int8_t* w_up, const int8_t* w_down,
                       const uint16_t* scales, const uint8_t* pad_mask, int T, int d, int f, int E,
                       int k, double* out, int32_t* ids_out) {
  if (T < 0 || d <= 0 || f <= 0 || E <= 0 || k <= 0 || k > E) return -1;
  std::vector<double> p(E), hid(f);
  std::vector<int> pick(k);
  for (int t = 0; t < T; ++t) {
    double* o = out + (size_t)t * d;
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    if (pad_mask && pad_mask[t] == 0) {
      if (ids_out)
        for (int j = 0; j < k; ++j) ids_out[(size_t)t * k + j] = -1;
      continue;
    }
    double mx = -INFINITY;
    for (int e = 0; e < E; ++e) {
      double s = router_bias ? (double)router_bias[e] : 0.0;
      for (int i = 0; i < d; ++i) s += (double)bf16_value(x[(size_t)t * d + i]) * router_w[(size_t)i * E + e];
      p[e] = s;
      mx = std::max(mx, s);
    }
    double z = 0.0;
    for (int e = 0; e < E; ++e) z += (p[e] = std::exp(p[e] - mx));
    for (int e = 0; e < E; ++e) p[e] /= z;
    // brute-force top-k: repeatedly the largest remaining, lowest index on ties
    std::vector<char> used(E, 0);
    for (int j = 0; j < k; ++j) {
      int b = -1;
      for (int e = 0; e < E; ++e)
        if (!used[e] && (b < 0 || p[e] > p[b])) b = e;
      used[b] = 1;
      pick[j] = b;
      if (ids_out) ids_out[(size_t)t * k + j] = b;
    }
    for (int j = 0; j < k; ++j) {
      int e = pick[j];
      const uint16_t* sc = scales + (size_t)e * (2 * (size_t)f + d);
      for (int c = 0; c < f; ++c) {
        double gs = 0.0, us = 0.0;
        for (int i = 0; i < d; ++i) {
          double xv = bf16_value(x[(size_t)t * d + i]);
          gs += xv * (double)w_gate[(size_t)e * d * f + (size_t)i * f + c] * bf16_value(sc[c]);
          us += xv * (double)w_up[(size_t)e * d * f + (size_t)i * f + c] * bf16_value(sc[f + c]);
        }
        double gelu = 0.5 * gs * (1.0 + std::tanh(0.79788456080286535588 * (gs + 0.044715 * gs * gs * gs)));
        hid[c] = gelu * us;
      }
      for (int c = 0; c < d; ++c) {
        double ys = 0.0;
        for (int m = 0; m < f; ++m)
          ys += hid[m] * (double)w_down[(size_t)e * f * d + (size_t)m * d + c] * bf16_value(sc[2 * (size_t)f + c]);
        o[c] += p[e] * ys;
      }
    }
  }
  return 0;
}

/* RMSNorm of one row, fp32: v * (1 / sqrt(mean(v^2) + eps)) * scale, the mean summed in
   index order. [G3-stack; FG4] (The sources give neither eps nor the scale's form: the
   reading taken is a learned per-feature fp32 scale and a caller-given eps.) */
void oracle_rms_norm_row(const float* v, const float* scale, float eps, int d, float* out) {
  float ss = 0.0f;
  for (int i = 0; i < d; ++i) ss += v[i] * v[i];
  const float r = 1.0f / std::sqrt(ss / (float)d + eps);
  for (int i = 0; i < d; ++i) out[i] = v[i] * r * scale[i];
}

/* The MoE block of a decoder layer [G3-stack; FG4]:
     x     = bf16(rms_norm(h; norm_pre))          (the MoE input, rounded to the bf16 fprop dtype)
     m     = moe(x, pad_mask)                    (oracle_forward)
     h_out = h + rms_norm(m; norm_post)          (fp32)
   h bf16 [T][d]; norm_pre, norm_post fp32 [d]; h_out fp32 [T][d]; x_out bf16 [T][d] or NULL.
   Padded tokens: m = 0, so h_out = h. */
int oracle_block_forward(const uint16_t* h, const float* norm_pre, const float* norm_post, float eps,
                         const float* router_w, const float* router_bias, const int8_t* w_gate,
                         const int8_t* w_up, const int8_t* w_down, const uint16_t* scales,
                         const uint8_t* pad_mask, int T, int d, int f, int E, int k, float* h_out,
                         uint16_t* x_out, int nthreads) {
  if (T < 0 || d <= 0 || f <= 0 || E <= 0 || k <= 0 || k > E) return -1;
  std::vector<uint16_t> x((size_t)T * d);
  std::vector<float> row(d), nrm(d);
  for (int t = 0; t < T; ++t) {
    for (int i = 0; i < d; ++i) row[i] = bf16_value(h[(size_t)t * d + i]);
    oracle_rms_norm_row(row.data(), norm_pre, eps, d, nrm.data());
    for (int i = 0; i < d; ++i) {
      uint32_t u;
      std::memcpy(&u, &nrm[i], 4);
      u += 0x7FFFu + ((u >> 16) & 1u);  // round to nearest even (finite values)
      x[(size_t)t * d + i] = (uint16_t)(u >> 16);
    }
  }
  std::vector<float> m((size_t)T * d);
  if (oracle_forward(x.data(), router_w, router_bias, w_gate, w_up, w_down, scales, pad_mask, T, d, f, E, k,
                     m.data(), nullptr, nullptr, nthreads) != 0)
    return -1;
  for (int t = 0; t < T; ++t) {
    oracle_rms_norm_row(&m[(size_t)t * d], norm_post, eps, d, nrm.data());
    for (int i = 0; i < d; ++i) h_out[(size_t)t * d + i] = bf16_value(h[(size_t)t * d + i]) + nrm[i];
  }
  if (x_out && !x.empty()) std::memcpy(x_out, x.data(), sizeof(uint16_t) * x.size());
  return 0;
}

}  // extern "C"
