// Launch policy of the expert kernels: which kernels run and how many parts the contractions
// are split into. The streaming kernels (T <= 160) read each touched expert's weights once
// per pass; a split only adds wavefronts (and fp32 partial sums) when the 256-column slabs
// alone would leave the chip under-filled, e.g. at one GPU's share of a tensor-parallel
// split over f. The prefill down kernel splits to fill a ragged last round of workgroups.
#pragma once

#include <algorithm>

#include "kernels.h"

namespace moe {

// Which expert kernels run: the streaming ones up to kDecodeMaxT tokens, but only when one
// expert matrix holds more than 2^23 weights. Smaller matrices are latency-bound in the
// streaming kernels (a few dozen wavefronts, each with a short chain of dependent steps) and
// the tiled kernels run them in narrow tiles over many more workgroups: d = 256, f = 512 at
// 64 tokens 39 -> 30 us per forward, d = 2048, f = 4096 (2^23) 3-29% faster from 8 to 160
// tokens; at 2^24 the streaming kernels are ahead again up to 128 tokens.
// Accepted trade-off: from 129 to 160 tokens a batch whose largest expert exceeds 48 rows
// takes a second streaming pass over that expert's weights; where the slabs fill only about
// one round of wavefronts (e.g. d = 4096, f = 8192 or f = 16384) the tiled kernels are then
// faster (311 vs 213 us and 546 vs 410 us at 160 tokens), but the host cannot see the row
// counts, and the Grok-1 shape and its tensor-parallel share do not lose there.
inline bool streaming_experts(int T, int d, int f) { return T <= kDecodeMaxT && (long)d * f > (1L << 23); }

// Small batches (T <= 160), targets measured on whole forward passes at the Grok-1 shape and
// at one GPU's tensor-parallel share: the down projection wants about 768 workgroups while
// each wavefront carries one 16-row tile (T <= 16: one wavefront per SIMD with a 4-step load
// ring, so that all of them are resident at once) and about 512 with two (longer streams win
// once the MFMA work per byte doubles), with parts of at least 1024 rows (shorter ones lose
// to their start-up). At most 16 parts (T = 1 at the Grok shape: 2 experts x 24 slabs x 16
// parts = 768 wavefronts, 233 -> 215 us per forward against 8 parts), each a whole number of
// 128-row steps.
// Large batches: the most parts the prefill down kernel may use. Launched with 2 or 4, it
// keeps 1, 2 or 4 on the device (from the live tile count, which only the device knows) and
// reports the choice to the combine. 4 where one part is expected to fill less than a round
// of 256 workgroups (about T * k / 256 + E / 2 row tiles x d / 256 column tiles; the kernel
// only takes 4 then) and the fp32 partials stay modest (T * k <= 8192 rows).
// The slab counts take the experts a batch can touch, min(E, T * k): at T = 1 only two stream.
inline int down_splits(int T, int d, int f, int E, int k) {
  if (T > kDecodeMaxT) {
    if (f < 8192) return 1;
    const long rows = (long)T * k;
    const long tiles = (rows + 255) / 256 + std::min<long>(E, rows) / 2;
    return rows <= 8192 && tiles * (d / 256) <= 256 && (f / 128) % 4 == 0 ? 4 : 2;
  }
  if (!streaming_experts(T, d, f)) {
    // small expert matrices in the tiled kernels: with few live tiles (about one row tile per
    // reachable expert x d / 256 column tiles) each workgroup would run the whole contraction
    // alone, one dependent slice after another; split it into up to 16 parts of at least 128
    // rows (two slices) while the parts still fit in one round of workgroups
    const long tiles = std::min<long>(E, (long)T * k) * (d / 256);
    int s = 1;
    while (s < 16 && tiles * 2 * s <= 256 && f / (2 * s) >= 128 && (f / 128) % (2 * s) == 0) s *= 2;
    return s;
  }
  const long slabs = (long)(d / 256) * std::min<long>(E, (long)T * k);
  const long target = T <= 16 ? 768 : 512;
  int s = 1;
  while (s < 16 && slabs * s < target && f / (2 * s) >= 1024 && (f / 128) % (2 * s) == 0) s *= 2;
  return s;
}

// gate/up: about 512 workgroups, parts of at least 768 rows of the contraction over d.
inline int gate_up_parts(int T, int d, int f, int E, int k) {
  if (!streaming_experts(T, d, f)) return 1;
  const long slabs = (long)(f / 256) * std::min<long>(E, (long)T * k);
  int s = 1;
  while (s < 8 && slabs * s < 512 && d / (2 * s) >= 768 && (d / 128) % (2 * s) == 0) s *= 2;
  return s;
}

}  // namespace moe
