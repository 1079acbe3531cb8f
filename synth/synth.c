/*
 * Seeded synthetic inputs for the top-2-of-8 MoE feed-forward layer.
 *
 * This module only draws numbers. It holds none of the layer's arithmetic and is
 * the one piece shared by the CPU checker and the GPU path (as data, never as code).
 *
 * Stream definition (counter-based, so results do not depend on thread count):
 *   mix64(z)      = SplitMix64 finaliser (Steele, Lea & Flood, "Fast splittable
 *                   pseudorandom number generators", OOPSLA 2014):
 *                   z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9
 *                   z = (z ^ (z >> 27)) * 0x94D049BB133111EB
 *                   z =  z ^ (z >> 31)
 *   stream key    = mix64(seed * G + mix64((set << 32) | tensor)),  G = 0x9E3779B97F4A7C15
 *   draw i        = mix64(key + (i + 1) * G)          (the i-th SplitMix64 output)
 *   uniform i     = (draw i >> 11) * 2^-53            in [0, 1)
 *
 * Distributions:
 *   normal       Box-Muller (1958), cosine branch only: element i uses uniforms 2i, 2i+1
 *   Student-t 4  Z / sqrt(V / 4), Z normal from uniforms 4i, 4i+1,
 *                V = -2 ln(u2 * u3) (chi-square with 4 dof) from uniforms 4i+2, 4i+3,
 *                then scaled by sqrt(1/2) to unit variance
 *   int8         (draw i >> 32) % 255 - 127, i.e. integers in [-127, 127]
 *   bf16         fp64 value -> fp32 (round to nearest even) -> bf16 (round to nearest even)
 *   pad mask     partial Fisher-Yates (Knuth, TAOCP vol. 2, Algorithm P) over [0, T):
 *                swap position i with i + draw(i) % (T - i), for i < n_pad; the first
 *                n_pad positions of the shuffled order are padded (mask 0), the rest 1
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint32_t set, uint32_t tensor) {
  return mix64(seed * GOLDEN + mix64(((uint64_t)set << 32) | tensor));
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

static inline double uni(uint64_t key, uint64_t i) {
  return (double)(draw(key, i) >> 11) * (1.0 / 9007199254740992.0);
}

uint16_t synth_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline double normal_at(uint64_t key, uint64_t i) {
  double u1 = 1.0 - uni(key, 2 * i); /* (0, 1] */
  double u2 = uni(key, 2 * i + 1);
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

static inline double student4_at(uint64_t key, uint64_t i) {
  double u0 = 1.0 - uni(key, 4 * i);
  double u1 = uni(key, 4 * i + 1);
  double z = sqrt(-2.0 * log(u0)) * cos(6.283185307179586476925 * u1);
  double u2 = 1.0 - uni(key, 4 * i + 2);
  double u3 = 1.0 - uni(key, 4 * i + 3);
  double v = -2.0 * log(u2 * u3);
  return z / sqrt(v / 4.0) * sqrt(0.5);
}

uint64_t synth_draw(uint64_t key, uint64_t i) { return draw(key, i); }
double synth_uniform(uint64_t key, uint64_t i) { return uni(key, i); }

/* Elements [start, start + n) of a normal(0, sigma^2) tensor, as bf16 bits. */
void synth_normal_bf16(uint16_t* out, uint64_t start, uint64_t n, uint64_t key, double sigma) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j)
    out[j] = synth_f32_to_bf16((float)(sigma * normal_at(key, start + (uint64_t)j)));
}

void synth_student4_bf16(uint16_t* out, uint64_t start, uint64_t n, uint64_t key) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j)
    out[j] = synth_f32_to_bf16((float)student4_at(key, start + (uint64_t)j));
}

void synth_normal_f32(float* out, uint64_t start, uint64_t n, uint64_t key, double sigma) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j) out[j] = (float)(sigma * normal_at(key, start + (uint64_t)j));
}

void synth_int8(int8_t* out, uint64_t start, uint64_t n, uint64_t key) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j)
    out[j] = (int8_t)((int)((draw(key, start + (uint64_t)j) >> 32) % 255u) - 127);
}

/* Uniforms [start, start + n) of a stream, as fp64 in [0, 1). */
void synth_uniform_f64(double* out, uint64_t start, uint64_t n, uint64_t key) {
  for (uint64_t j = 0; j < n; ++j) out[j] = uni(key, start + j);
}

/* mask[t] = 0 for n_pad seeded positions, 1 elsewhere. Returns 0, or -1 on bad sizes. */
int synth_pad_mask(uint8_t* mask, int T, int n_pad, uint64_t key) {
  if (T < 0 || n_pad < 0 || n_pad > T) return -1;
  int* order = (int*)malloc(sizeof(int) * (size_t)(T > 0 ? T : 1));
  if (!order) return -1;
  for (int t = 0; t < T; ++t) order[t] = t, mask[t] = 1;
  for (int i = 0; i < n_pad; ++i) {
    int j = i + (int)(draw(key, (uint64_t)i) % (uint64_t)(T - i));
    int tmp = order[i];
    order[i] = order[j];
    order[j] = tmp;
    mask[order[i]] = 0;
  }
  free(order);
  return 0;
}
