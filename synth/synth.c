/*
 * Seeded synthetic inputs for the fused RMSNorm+MatMul workloads.
 *
 * This file holds input generation only: it draws the numbers that the
 * kernels and the CPU oracle both consume, and rounds them to the stored
 * dtype.  It contains none of the RMSNorm / matmul arithmetic.
 *
 * Generator (counter based, so any element can be drawn independently, in
 * any order, on any number of threads):
 *   mix(x)      = the SplitMix64 step (Vigna, "splitmix64.c", 2015): add the
 *                 golden gamma 0x9e3779b97f4a7c15 to the state x, then apply
 *                 the published xor-shift-multiply finaliser.  mix(1234567)
 *                 is 6457827717110365317, the first published output.
 *   base(t)     = mix(seed + t * 0xD1B54A32D192ED03)        one stream per tensor
 *   h(t,i,j)    = mix(base(t) ^ (2*i + j))
 *   u(t,i,j)    = ((h(t,i,j) >> 11) + 0.5) * 2^-53            uniform on (0,1)
 *   z(t,i)      = sqrt(-2 ln u(t,i,0)) * cos(2 pi u(t,i,1))   Box-Muller, one
 *                 normal per counter i
 * Streams: 1 = X, 2 = g, 3 = W / W1, 4 = W3, 5 = per-row scale, 6 = row pick,
 * 7.. = exact-arithmetic test inputs.
 *
 * Values are formed in double, rounded once to float, and (for bf16
 * workloads) rounded once more from float to bf16 with round-to-nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t mix(uint64_t x) {
  uint64_t z = x + 0x9e3779b97f4a7c15ULL;
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

static inline uint64_t base_of(uint64_t seed, int t) {
  return mix(seed + (uint64_t)t * 0xD1B54A32D192ED03ULL);
}

static inline uint64_t hash3(uint64_t b, int64_t i, int j) {
  return mix(b ^ (uint64_t)(2 * i + j));
}

static inline double unif(uint64_t h) {
  return ((double)(h >> 11) + 0.5) * 0x1.0p-53;
}

static inline double normal_at(uint64_t b, int64_t i) {
  double u0 = unif(hash3(b, i, 0));
  double u1 = unif(hash3(b, i, 1));
  return sqrt(-2.0 * log(u0)) * cos(6.283185307179586476925287 * u1);
}

uint64_t synth_mix(uint64_t x) { return mix(x); }

/* h(t,i,j) for i in [i0, i0+n). */
void synth_hash(uint64_t seed, int t, int64_t i0, int64_t n, int j, uint64_t* out) {
  uint64_t b = base_of(seed, t);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = hash3(b, i0 + i, j);
}

/* u(t,i,j) for i in [i0, i0+n). */
void synth_uniform(uint64_t seed, int t, int64_t i0, int64_t n, int j, double* out) {
  uint64_t b = base_of(seed, t);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = unif(hash3(b, i0 + i, j));
}

/* out[r*cols + c] = (float)(row_scale[r] * (add + mul * z(t, R*cols + c)))
   where R = row_idx[r] (or r when row_idx is NULL), so any subset of rows of a
   larger tensor can be drawn on its own.  row_scale may be NULL (all ones). */
void synth_normal_f32(uint64_t seed, int t, int64_t rows, int64_t cols, double mul,
                      double add, const double* row_scale, const int64_t* row_idx,
                      float* out) {
  uint64_t b = base_of(seed, t);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double s = row_scale ? row_scale[r] : 1.0;
    int64_t R = row_idx ? row_idx[r] : r;
    for (int64_t c = 0; c < cols; ++c) {
      out[r * cols + c] = (float)(s * (add + mul * normal_at(b, R * cols + c)));
    }
  }
}

/* Exact-arithmetic inputs: values are small integers (times a power of two)
   so every product and partial sum is exact in fp32 and in bf16 x bf16
   products, whatever the summation order.
     kind 0: +-1 with equal probability                       (X)
     kind 1: 1 or 2 with equal probability                    (g)
     kind 2: 0 with probability 1-density, else one of
             {-2,-1,1,2} with equal probability                (W)  */
void synth_exact_f32(uint64_t seed, int t, int64_t n, int kind, double density, float* out) {
  uint64_t b = base_of(seed, t);
  uint64_t thresh = (uint64_t)(density * 18446744073709551616.0 * 0.999999999);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint64_t h = hash3(b, i, 0);
    float v;
    if (kind == 0) {
      v = (h >> 63) ? -1.0f : 1.0f;
    } else if (kind == 1) {
      v = (h >> 63) ? 2.0f : 1.0f;
    } else {
      uint64_t h2 = hash3(b, i, 1);
      if (h2 >= thresh) {
        v = 0.0f;
      } else {
        static const float vals[4] = {-2.0f, -1.0f, 1.0f, 2.0f};
        v = vals[h >> 62];
      }
    }
    out[i] = v;
  }
}

/* float -> bf16 bits, round to nearest even; NaN stays NaN (quiet). */
void synth_f32_to_bf16(const float* in, uint16_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u;
    memcpy(&u, &in[i], 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) {
      out[i] = (uint16_t)((u >> 16) | 0x0040u);
    } else {
      uint32_t lsb = (u >> 16) & 1u;
      out[i] = (uint16_t)((u + 0x7fffu + lsb) >> 16);
    }
  }
}

/* bf16 bits -> float (exact). */
void synth_bf16_to_f32(const uint16_t* in, float* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u = (uint32_t)in[i] << 16;
    memcpy(&out[i], &u, 4);
  }
}
