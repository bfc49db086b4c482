/*
 * kmref.c -- the fp64 CPU oracle for exact Lloyd K-Means.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the HIP library; the two meet only at the seeded input bytes.
 *
 * Citations name the page "Flash-KMeans: Fast and Memory-Efficient Exact
 * K-Means" (gist.science summary of paper 2603.09229): "tech §n" is a section
 * of its technical summary, "pop §n" a section of its popular explainer.
 *
 * What is computed.  The page states that Flash-KMeans changes neither the
 * K-Means formula nor introduces any approximation (tech §2 opening, tech §3
 * "mathematical exactness", pop §4).  So the oracle is plain Lloyd K-Means,
 * written from its definition:
 *   assign:  a_i = argmin_k  sum_j (x_ij - c_kj)^2          (direct difference)
 *   update:  c_k = (1/n_k) sum_{i : a_i = k} x_i,   n_k = #{i : a_i = k}
 * The page does not fix the metric, the tie rule or what an empty cluster
 * does; this library's convention is: squared Euclidean distance, ties go to
 * the lowest centroid index, and an empty cluster keeps its previous centroid.
 *
 * Arithmetic: everything in fp64, summation over j ascending and over points
 * in ascending point index, no FMA contraction (built with -ffp-contract=off,
 * no fast-math).  Input points are decoded exactly from their stored type.
 *
 * Precision reading for 16-bit inputs: the page does not say in what
 * precision the contraction runs.  This library rounds the fp32 centroid
 * state once per assignment to the storage type of X (round to nearest, ties
 * to even) and computes distances against those rounded centroids;
 * kmref_quantize() applies that rounding and the distance is then exact
 * fp64 arithmetic on the rounded values.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { KMREF_X_F32 = 0, KMREF_X_BF16 = 1, KMREF_X_F16 = 2, KMREF_X_F64 = 3 };

/* ---- exact decoding of the stored point values ------------------------- */

static double decode_f32(uint32_t bits) {
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static double decode_bf16(uint16_t h) { return decode_f32((uint32_t)h << 16); }

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double decode_f16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-14 * 2^-10 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(m | 0x400), e - 25); /* (1.m) * 2^(e-15), 10 fraction bits */
  return sign ? -v : v;
}

static double load_x(const void* X, int dtype, int64_t idx) {
  switch (dtype) {
    case KMREF_X_F32: {
      uint32_t b;
      memcpy(&b, (const char*)X + 4 * idx, 4);
      return decode_f32(b);
    }
    case KMREF_X_BF16: return decode_bf16(((const uint16_t*)X)[idx]);
    case KMREF_X_F16: return decode_f16(((const uint16_t*)X)[idx]);
    default: return ((const double*)X)[idx];
  }
}

int kmref_decode(const void* X, int dtype, int64_t n, double* out) {
  if (dtype < 0 || dtype > 3) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = load_x(X, dtype, i);
  return 0;
}

/* ---- rounding to a binary floating-point format ------------------------ */

/*
 * Round x to the nearest value of a binary format with a p-bit significand
 * (hidden bit included), minimum normal exponent emin and maximum exponent
 * emax, ties to even; values beyond the largest finite number round to
 * infinity as IEEE 754 round-to-nearest prescribes.  Written from the IEEE
 * definition: find the exponent of x, clamp it to emin for subnormals, round
 * x / ulp to the nearest integer (ties to even), scale back.
 *   binary32: p=24, emin=-126, emax=127
 *   bfloat16: p=8,  emin=-126, emax=127
 *   binary16: p=11, emin=-14,  emax=15
 */
double kmref_round(double x, int p, int emin, int emax) {
  if (x != x || x == 0.0 || isinf(x)) return x;
  int e;
  frexp(x, &e); /* x = f * 2^e, 0.5 <= |f| < 1, so the leading bit has weight 2^(e-1) */
  int lead = e - 1;
  if (lead < emin) lead = emin;
  double ulp = ldexp(1.0, lead - (p - 1));
  double q = x / ulp; /* exact: power-of-two scaling */
  double r = nearbyint(q); /* default rounding mode: nearest, ties to even */
  double y = r * ulp;
  /* largest finite: (2 - 2^(1-p)) * 2^emax; the overflow threshold is that plus half an ulp */
  double maxf = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
  double thresh = maxf + ldexp(1.0, emax - p);
  if (fabs(x) >= thresh) return x > 0 ? INFINITY : -INFINITY;
  if (fabs(y) > maxf) return x > 0 ? maxf : -maxf; /* cannot happen below thresh; kept for clarity */
  return y;
}

/* Q(C): the centroids as the contraction sees them, for X of type dtype. */
void kmref_quantize(const double* C, int64_t n, int dtype, double* out) {
  for (int64_t i = 0; i < n; ++i) {
    double c = C[i];
    switch (dtype) {
      case KMREF_X_BF16: out[i] = kmref_round(c, 8, -126, 127); break;
      case KMREF_X_F16: out[i] = kmref_round(c, 11, -14, 15); break;
      default: out[i] = c; break;
    }
  }
}

/* ---- assignment -------------------------------------------------------- */

/*
 * Nearest-centroid assignment (tech §2.1 describes the fused form; the value
 * it must produce is the plain argmin).  For each point i, scan k ascending
 * from (best = +inf, idx = 0) and replace only on a strictly smaller distance,
 * which gives the lowest index among equal minima; a NaN distance never wins.
 * d1[i] = distance to a_i, d2[i] = smallest distance over k != a_i (+inf if
 * K == 1).  Either output pointer may be NULL.
 */
void kmref_assign(const void* X, int dtype, int64_t N, int64_t D,
                  const double* C, int64_t K, int32_t* a, double* d1, double* d2) {
#pragma omp parallel
  {
    double* x = (double*)malloc(sizeof(double) * (size_t)(D > 0 ? D : 1));
#pragma omp for schedule(dynamic, 64)
    for (int64_t i = 0; i < N; ++i) {
      for (int64_t j = 0; j < D; ++j) x[j] = load_x(X, dtype, i * D + j);
      double best = INFINITY, second = INFINITY;
      int64_t idx = 0;
      for (int64_t k = 0; k < K; ++k) {
        const double* c = C + k * D;
        double d = 0.0;
        for (int64_t j = 0; j < D; ++j) {
          double diff = x[j] - c[j];
          d += diff * diff;
        }
        if (d < best) {
          second = best;
          best = d;
          idx = k;
        } else if (d < second) {
          second = d;
        }
      }
      a[i] = (int32_t)idx;
      if (d1) d1[i] = best;
      if (d2) d2[i] = second;
    }
    free(x);
  }
}

/* ---- update ------------------------------------------------------------ */

/*
 * Mean of the assigned points (the update step that tech §2.2 reorganises
 * without changing its value).  n_k counts the points with a_i == k; s_k sums
 * them in fp64 in ascending point index; c_k = s_k / n_k when n_k > 0, else
 * c_k keeps C_prev[k] (copied bit for bit).  Assignments outside [0, K) are
 * ignored.  Cnew may alias Cprev.
 *
 * To visit each cluster's points in ascending index on several threads, the
 * points are first listed per cluster by a stable counting pass; the sum
 * itself is the plain definition.
 */
void kmref_update(const void* X, int dtype, int64_t N, int64_t D, const int32_t* a,
                  int64_t K, const double* Cprev, double* Cnew, int64_t* counts) {
  int64_t* start = (int64_t*)calloc((size_t)K + 1, sizeof(int64_t));
  int64_t* order = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
  int64_t* fill = (int64_t*)malloc(sizeof(int64_t) * (size_t)(K > 0 ? K : 1));
  for (int64_t i = 0; i < N; ++i)
    if (a[i] >= 0 && a[i] < K) start[a[i] + 1]++;
  for (int64_t k = 0; k < K; ++k) start[k + 1] += start[k];
  for (int64_t k = 0; k < K; ++k) fill[k] = start[k];
  for (int64_t i = 0; i < N; ++i)
    if (a[i] >= 0 && a[i] < K) order[fill[a[i]]++] = i;

#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(D > 0 ? D : 1));
#pragma omp for schedule(dynamic, 16)
    for (int64_t k = 0; k < K; ++k) {
      int64_t n = start[k + 1] - start[k];
      if (counts) counts[k] = n;
      if (n == 0) {
        if (Cnew != Cprev) memcpy(Cnew + k * D, Cprev + k * D, sizeof(double) * (size_t)D);
        continue;
      }
      for (int64_t j = 0; j < D; ++j) s[j] = 0.0;
      for (int64_t p = start[k]; p < start[k + 1]; ++p) {
        int64_t i = order[p];
        for (int64_t j = 0; j < D; ++j) s[j] += load_x(X, dtype, i * D + j);
      }
      for (int64_t j = 0; j < D; ++j) Cnew[k * D + j] = s[j] / (double)n;
    }
    free(s);
  }
  free(start);
  free(order);
  free(fill);
}

/* ---- Lloyd iterations -------------------------------------------------- */

/*
 * T iterations of Lloyd (one iteration = assign, then update; exactly T, no
 * early exit -- the page names no stopping rule and an iteration after
 * convergence changes nothing).  C0 is the fp32 initial centroid state.
 *   contract = 1: the centroid state between iterations is fp32 (each new
 *                 mean is rounded to binary32), as in the GPU library.
 *   contract = 0: the state stays fp64 (pure Lloyd in exact-as-possible
 *                 arithmetic; used for the monotonicity pins).
 * Before each assignment the centroids go through kmref_quantize (rounded to
 * the storage type of X).  Outputs: C_out (K*D) = C^T; a_out (N) and
 * counts_out (K) from the T-th assignment; J[t] = sum_i d_i of assignment t
 * (each may be NULL).  Returns 0, or -1 on allocation failure.
 */
int kmref_fit(const void* X, int dtype, int64_t N, int64_t D, int64_t K,
              const float* C0, int T, int contract, double* C_out, int32_t* a_out,
              int64_t* counts_out, double* J) {
  size_t kd = (size_t)K * (size_t)D;
  double* C = (double*)malloc(sizeof(double) * (kd ? kd : 1));
  double* Cq = (double*)malloc(sizeof(double) * (kd ? kd : 1));
  int32_t* a = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
  double* d1 = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
  int64_t* cnt = (int64_t*)malloc(sizeof(int64_t) * (size_t)(K > 0 ? K : 1));
  if (!C || !Cq || !a || !d1 || !cnt) {
    free(C); free(Cq); free(a); free(d1); free(cnt);
    return -1;
  }
  for (size_t i = 0; i < kd; ++i) C[i] = (double)C0[i];
  for (int64_t k = 0; k < K; ++k) cnt[k] = 0;
  for (int t = 0; t < T; ++t) {
    kmref_quantize(C, (int64_t)kd, dtype, Cq);
    kmref_assign(X, dtype, N, D, Cq, K, a, d1, NULL);
    if (J) {
      double s = 0.0;
      for (int64_t i = 0; i < N; ++i) s += d1[i];
      J[t] = s;
    }
    kmref_update(X, dtype, N, D, a, K, C, C, cnt);
    if (contract)
      for (size_t i = 0; i < kd; ++i) C[i] = kmref_round(C[i], 24, -126, 127);
  }
  if (C_out) memcpy(C_out, C, sizeof(double) * kd);
  if (a_out && T > 0) memcpy(a_out, a, sizeof(int32_t) * (size_t)N);
  if (counts_out) memcpy(counts_out, cnt, sizeof(int64_t) * (size_t)K);
  free(C); free(Cq); free(a); free(d1); free(cnt);
  return 0;
}

int kmref_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
