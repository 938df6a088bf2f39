/* Seeded input generation for the tree-verification workloads: SplitMix64
 * (Steele, Lea and Flood, OOPSLA 2014) used counter-style, and the Box-Muller
 * transform.  Holds no verification arithmetic.  Draw i of stream `key` is
 * mix(key + (i + 1) * GAMMA); a normal uses the two 32-bit halves of one draw. */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

void synth_u64(uint64_t key, int64_t start, int64_t n, uint64_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = mix64(key + (uint64_t)(start + i + 1) * GAMMA);
}

static inline double normal_at(uint64_t key, int64_t i) {
  const uint64_t r = mix64(key + (uint64_t)(i + 1) * GAMMA);
  const double u1 = ((double)(r >> 32) + 1.0) * (1.0 / 4294967296.0);
  const double u2 = (double)(r & 0xFFFFFFFFull) * (1.0 / 4294967296.0);
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

void synth_normal_f64(uint64_t key, int64_t n, double sigma, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = normal_at(key, i) * sigma;
}

void synth_normal_f32(uint64_t key, int64_t n, double sigma, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(normal_at(key, i) * sigma);
}

/* float32 value rounded to bfloat16, nearest-even (no NaN arises here). */
void synth_normal_bf16(uint64_t key, int64_t n, double sigma, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    const float f = (float)(normal_at(key, i) * sigma);
    uint32_t u;
    memcpy(&u, &f, 4);
    out[i] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
  }
}

/* Raw 16-bit cache contents for commit tests: an integer hash of (slab,
 * column, element) that reaches every bit pattern (NaN payloads included).
 * out is [n_slab][ncol][nel]; slabs[i] is the global slab index of row block i. */
void synth_commit_pattern(const int64_t* slabs, int64_t n_slab, int64_t ncol, int64_t nel, uint16_t* out) {
  for (int64_t s = 0; s < n_slab; ++s)
    for (int64_t c = 0; c < ncol; ++c)
      for (int64_t e = 0; e < nel; ++e) {
        int64_t h = (slabs[s] * 1000003 + c) * 131 + e;
        h ^= h >> 13;
        h = (h * 40503) & 0xFFFFFFFF;
        h ^= h >> 16;
        out[(s * ncol + c) * nel + e] = (uint16_t)(h & 0xFFFF);
      }
}
