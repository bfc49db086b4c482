/*
 * gen.c -- seeded synthetic inputs for the K-Means workloads.
 *
 * This module holds none of the clustering arithmetic: it only draws points.
 * Both the HIP library's tests/benchmark and the CPU oracle read the bytes it
 * writes, so the two sides always see identical inputs.
 *
 * Random numbers: Philox4x32-10, the counter-based generator of Salmon,
 * Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
 * (SC'11): ten rounds of two 32x32->64 multiplies with the published
 * multipliers and Weyl key increments.  Every value is a pure function of
 * (seed, stream tag, index), so any row can be regenerated on its own and
 * generation parallelises with no shared state.  Normal deviates come from
 * the Box-Muller transform on 53-bit uniforms in (0, 1).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void mulhilo32(uint32_t a, uint32_t b, uint32_t* hi, uint32_t* lo) {
  uint64_t p = (uint64_t)a * (uint64_t)b;
  *hi = (uint32_t)(p >> 32);
  *lo = (uint32_t)p;
}

/* One Philox4x32 block: 10 rounds, key bumped between rounds. */
void synth_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int r = 0; r < 10; ++r) {
    uint32_t hi0, lo0, hi1, lo1;
    mulhilo32(PHILOX_M0, c0, &hi0, &lo0);
    mulhilo32(PHILOX_M1, c2, &hi1, &lo1);
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += PHILOX_W0;
    k1 += PHILOX_W1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Stream tags keep the independent draws apart. */
enum { TAG_CENTER = 0x43454e54u, TAG_POINT = 0x504f494eu, TAG_COMP = 0x434f4d50u, TAG_PICK = 0x5049434bu };

static inline void block(uint64_t seed, uint32_t tag, uint64_t i, uint32_t j, uint32_t out[4]) {
  uint32_t ctr[4] = {(uint32_t)i, (uint32_t)(i >> 32), j, tag};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32) ^ tag};
  synth_philox4x32_10(ctr, key, out);
}

/* 53-bit uniform strictly inside (0, 1). */
static inline double u53(uint32_t a, uint32_t b) {
  uint64_t m = ((uint64_t)(a >> 5) << 26) | (uint64_t)(b >> 6);
  return ((double)m + 0.5) * (1.0 / 9007199254740992.0);
}

static inline void normal2(uint64_t seed, uint32_t tag, uint64_t i, uint32_t j, double* z0, double* z1) {
  uint32_t r[4];
  block(seed, tag, i, j, r);
  double u1 = u53(r[0], r[1]), u2 = u53(r[2], r[3]);
  double rad = sqrt(-2.0 * log(u1));
  double th = 6.283185307179586 * u2;
  *z0 = rad * cos(th);
  *z1 = rad * sin(th);
}

/* Raw 64 random bits number n of stream (seed, TAG_PICK): used to sample indices. */
uint64_t synth_bits64(uint64_t seed, uint64_t n) {
  uint32_t r[4];
  block(seed, TAG_PICK, n, 0, r);
  return ((uint64_t)r[0] << 32) | r[1];
}

/* Standard normal number n of stream (seed, tag); exposed for the generator's own tests. */
double synth_normal(uint64_t seed, uint32_t tag, uint64_t n) {
  double z0, z1;
  normal2(seed, tag, n >> 1, 0, &z0, &z1);
  return (n & 1) ? z1 : z0;
}

/* Component centers: M x D, centre m = scale * N(0, I); kind 1 normalises to unit length. */
void synth_centers(uint64_t seed, int64_t M, int64_t D, int kind, double scale, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    double* c = out + m * D;
    for (int64_t j = 0; j < D; j += 2) {
      double z0, z1;
      normal2(seed, TAG_CENTER, (uint64_t)m, (uint32_t)(j >> 1), &z0, &z1);
      c[j] = scale * z0;
      if (j + 1 < D) c[j + 1] = scale * z1;
    }
    if (kind == 1) {
      double s = 0.0;
      for (int64_t j = 0; j < D; ++j) s += c[j] * c[j];
      double inv = 1.0 / sqrt(s);
      for (int64_t j = 0; j < D; ++j) c[j] *= inv;
    }
  }
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40); /* quiet NaN */
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/*
 * Rows [row0, row0 + nrows) of a mixture.  Row i picks component m_i
 * (uniform when cdf == NULL, else the first m with u < cdf[m]), then
 * x_i = center[m_i] + sigma * N(0, I) (kind 1: then scaled to unit length).
 * Values are computed in fp64, rounded to fp32, and for out_dtype 1 (bf16)
 * rounded once more to bfloat16 (nearest, ties to even).  out_dtype 0 writes
 * fp32.  comp_out (nullable) receives m_i.
 */
int synth_points(uint64_t seed, const double* centers, int64_t M, int64_t D, int kind, double sigma,
                 const double* cdf, int out_dtype, void* out, int64_t row0, int64_t nrows, int32_t* comp_out) {
  if (out_dtype != 0 && out_dtype != 1) return -1;
#pragma omp parallel
  {
    double* x = (double*)malloc(sizeof(double) * (size_t)(D + 1));
#pragma omp for schedule(static, 256)
    for (int64_t r = 0; r < nrows; ++r) {
      uint64_t i = (uint64_t)(row0 + r);
      uint32_t cr[4];
      block(seed, TAG_COMP, i, 0, cr);
      int64_t m;
      if (!cdf) {
        uint64_t bits = ((uint64_t)cr[0] << 32) | cr[1];
        m = (int64_t)(((unsigned __int128)bits * (uint64_t)M) >> 64);
      } else {
        double u = u53(cr[0], cr[1]);
        int64_t lo = 0, hi = M - 1;
        while (lo < hi) {
          int64_t mid = (lo + hi) / 2;
          if (u < cdf[mid]) hi = mid; else lo = mid + 1;
        }
        m = lo;
      }
      if (comp_out) comp_out[r] = (int32_t)m;
      const double* c = centers + m * D;
      for (int64_t j = 0; j < D; j += 2) {
        double z0, z1;
        normal2(seed, TAG_POINT, i, (uint32_t)(j >> 1), &z0, &z1);
        x[j] = c[j] + sigma * z0;
        if (j + 1 < D) x[j + 1] = c[j + 1] + sigma * z1;
      }
      if (kind == 1) {
        double s = 0.0;
        for (int64_t j = 0; j < D; ++j) s += x[j] * x[j];
        double inv = 1.0 / sqrt(s);
        for (int64_t j = 0; j < D; ++j) x[j] *= inv;
      }
      if (out_dtype == 0) {
        float* o = (float*)out + r * D;
        for (int64_t j = 0; j < D; ++j) o[j] = (float)x[j];
      } else {
        uint16_t* o = (uint16_t*)out + r * D;
        for (int64_t j = 0; j < D; ++j) o[j] = f32_to_bf16_rne((float)x[j]);
      }
    }
    free(x);
  }
  return 0;
}

int synth_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
