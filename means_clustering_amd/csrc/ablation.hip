// Ablation baselines: the two designs Flash-KMeans replaces, written for the
// same GPU so their cost can be measured next to the library's kernels.
// Not used by the library itself.
//
// Citations name the page "Flash-KMeans: Fast and Memory-Efficient Exact
// K-Means" (gist.science summary of paper 2603.09229); "tech §n" is a section
// of its technical summary.
//
//   * Materialised assignment (tech §1: the N x K distance matrix written to
//     and read back from HBM dominates the assign stage): the same MFMA
//     scores as FlashAssign, x.c - |c|^2/2 with the accumulator seeded by the
//     bias and the depth blocks in the same order (so every score is bit for
//     bit the one FlashAssign computes), are written to an N x K fp32 array;
//     a second kernel reads each row back and takes the argmax (lowest index
//     on ties).
//   * Atomic scatter update (tech §1: point-parallel atomics on hot clusters
//     serialise): every point adds its row into its cluster's fp32 sum and
//     count with device atomics, then the sums are divided.  The summation
//     order depends on scheduling, so results are not reproducible bit for bit.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/kmeans_ablation.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

enum { A_F32 = 0, A_BF16 = 1, A_F16 = 2 };

__device__ __forceinline__ uint32_t to16(float f, int dt) {
  if (dt == A_BF16) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
  }
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ float from16(uint32_t h, int dt) {
  return dt == A_BF16 ? __uint_as_float(h << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Rounded centroids (K x Dp, 16-bit, zero-padded to Dp = 16 * KB) and their
// biases -|c|^2/2 in the order FlashAssign's preparation sums them: per
// 8-value piece (depth block kb, half h) in element order, pieces summed per
// block in order, then blocks in the order of the four-wavefront split.
__global__ void abl_prep_kernel(const float* __restrict__ C, int64_t K, int D, int KB, int dt,
                                uint16_t* __restrict__ cq, float* __restrict__ bias) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  const int Dp = 16 * KB;
  float half[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (int kb = 0; kb < KB; ++kb) {
    for (int h = 0; h < 2; ++h) {
      float ss = half[h][kb & 3];
      for (int e = 0; e < 8; ++e) {
        const int d = kb * 16 + h * 8 + e;
        const float c = d < D ? C[k * D + d] : 0.0f;
        const uint32_t q = to16(c, dt);
        cq[k * Dp + d] = (uint16_t)q;
        const float f = from16(q, dt);
        ss = fmaf(f, f, ss);
      }
      half[h][kb & 3] = ss;
    }
  }
  // wavefront partials in wavefront order, then the two halves of the row
  float t0 = 0.f, t1 = 0.f;
  for (int w = 0; w < 4; ++w) {
    t0 = w == 0 ? half[0][0] : t0 + half[0][w];
    t1 = w == 0 ? half[1][0] : t1 + half[1][w];
  }
  bias[k] = -0.5f * (t0 + t1);
}

template <int DT>
__device__ __forceinline__ f32x16_t mma(u32x4_t a, u32x4_t b, f32x16_t c) {
  if constexpr (DT == A_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
}

// One wavefront per 32 points x 32 centroids tile: S[p][k] for the tile.
template <int DT>
__global__ __launch_bounds__(256) void abl_scores_kernel(const uint16_t* __restrict__ X, int64_t N, int D,
                                                         const uint16_t* __restrict__ cq, const float* __restrict__ bias,
                                                         int64_t K, int KB, float* __restrict__ S) {
  const int lane = threadIdx.x & 63, h = lane >> 5, col = lane & 31;
  const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t ngroups = (K + 31) / 32;
  const int64_t pb = tile / ngroups, g = tile % ngroups;
  if (pb * 32 >= N) return;
  const int64_t p = pb * 32 + col;             // this lane's point (B column)
  const int64_t crow = g * 32 + col;           // this lane's centroid row (A row)
  const int Dp = 16 * KB;
  f32x16_t acc;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t k = g * 32 + 8 * j + 4 * h + r;
      acc[4 * j + r] = k < K ? bias[k] : -INFINITY;
    }
  for (int kb = 0; kb < KB; ++kb) {
    uint32_t a[4] = {0, 0, 0, 0}, b[4] = {0, 0, 0, 0};
    if (crow < K) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        a[e] = (uint32_t)cq[crow * Dp + kb * 16 + h * 8 + 2 * e] |
               ((uint32_t)cq[crow * Dp + kb * 16 + h * 8 + 2 * e + 1] << 16);
    }
    if (p < N) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = kb * 16 + h * 8 + e;
        const uint32_t v = d < D ? (uint32_t)X[p * D + d] : 0u;
        b[e >> 1] |= v << (16 * (e & 1));
      }
    }
    acc = mma<DT>(u32x4_t{a[0], a[1], a[2], a[3]}, u32x4_t{b[0], b[1], b[2], b[3]}, acc);
  }
  if (p < N) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t k = g * 32 + 8 * j + 4 * h + r;
        if (k < K) S[p * K + k] = acc[4 * j + r];
      }
  }
}

// One wavefront per row of S: lowest index of the largest score.
__global__ __launch_bounds__(256) void abl_argmax_kernel(const float* __restrict__ S, int64_t N, int64_t K,
                                                         int32_t* __restrict__ assign) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= N) return;
  float best = -INFINITY;
  int64_t bi = INT64_MAX;
  for (int64_t k = lane; k < K; k += 64) {
    const float v = S[row * K + k];
    if (v > best) {  // within a lane k ascends, so the first maximum is kept
      best = v;
      bi = k;
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    const float ob = __shfl_xor(best, off);
    const int64_t oi = __shfl_xor(bi, off);
    if (ob > best || (ob == best && oi < bi)) {
      best = ob;
      bi = oi;
    }
  }
  if (lane == 0) assign[row] = bi == INT64_MAX ? 0 : (int32_t)bi;
}

__global__ void abl_zero_kernel(float* __restrict__ s, int64_t n, int32_t* __restrict__ c, int64_t k) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) s[i] = 0.0f;
  if (i < k) c[i] = 0;
}

// One thread per (point, column): device atomics on the cluster's sum (and count).
template <int ES>
__global__ void abl_scatter_kernel(const uint8_t* __restrict__ X, int dt, int64_t N, int D,
                                   const int32_t* __restrict__ assign, int64_t K, float* __restrict__ sums,
                                   int32_t* __restrict__ counts) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t i = t / D;
  const int c = (int)(t % D);
  if (i >= N) return;
  const int32_t a = assign[i];
  if (a < 0 || a >= K) return;
  float x;
  if (ES == 4)
    x = reinterpret_cast<const float*>(X)[i * D + c];
  else
    x = from16(reinterpret_cast<const uint16_t*>(X)[i * D + c], dt == A_BF16 ? A_BF16 : A_F16);
  atomicAdd(&sums[(int64_t)a * D + c], x);
  if (c == 0) atomicAdd(&counts[a], 1);
}

__global__ void abl_divide_kernel(const float* __restrict__ sums, const int32_t* __restrict__ counts, int64_t K,
                                  int D, const float* __restrict__ C_prev, float* __restrict__ C_new) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= K * D) return;
  const int32_t n = counts[i / D];
  C_new[i] = n > 0 ? sums[i] / (float)n : C_prev[i];
}

}  // namespace

extern "C" {

// Scratch for the materialised assignment: N*K floats of scores, then the
// rounded centroids and biases.  0 for unsupported arguments.
size_t kmeans_abl_materialized_bytes(int64_t N, int64_t D, int64_t K) {
  if (N < 1 || D < 1 || D > 512 || K < 1) return 0;
  const int64_t KB = (D + 15) / 16;
  return (size_t)N * (size_t)K * 4 + (size_t)K * (size_t)(16 * KB) * 2 + (size_t)K * 4 + 1024;
}

// Materialised assignment for 16-bit X (dt 1 bf16, 2 fp16): same scores as
// FlashAssign, written to HBM as an N x K matrix, then an argmax pass.
// Returns 0, or a HIP error code / -1 for bad arguments.  Asynchronous on `stream`.
int kmeans_abl_assign_materialized(const void* X, int dt, int64_t N, int64_t D, const float* C, int64_t K,
                                   int32_t* assign, void* scratch, size_t scratch_bytes, void* stream) {
  if ((dt != A_BF16 && dt != A_F16) || !X || !C || !assign || !scratch || N < 1 || D < 1 || D > 512 || K < 1)
    return -1;
  if (scratch_bytes < kmeans_abl_materialized_bytes(N, D, K) || scratch_bytes == 0) return -1;
  hipStream_t s = (hipStream_t)stream;
  const int KB = (int)((D + 15) / 16);
  float* S = (float*)scratch;
  uint8_t* rest = (uint8_t*)scratch + (((size_t)N * (size_t)K * 4 + 255) / 256) * 256;
  uint16_t* cq = (uint16_t*)rest;
  float* bias = (float*)(rest + (((size_t)K * (size_t)(16 * KB) * 2 + 255) / 256) * 256);
  hipLaunchKernelGGL(abl_prep_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, s, C, K, (int)D, KB, dt, cq,
                     bias);
  const int64_t tiles = ((N + 31) / 32) * ((K + 31) / 32);
  const dim3 grid((unsigned)((tiles + 3) / 4));
  if (dt == A_BF16)
    hipLaunchKernelGGL(abl_scores_kernel<A_BF16>, grid, dim3(256), 0, s, (const uint16_t*)X, N, (int)D, cq, bias, K,
                       KB, S);
  else
    hipLaunchKernelGGL(abl_scores_kernel<A_F16>, grid, dim3(256), 0, s, (const uint16_t*)X, N, (int)D, cq, bias, K,
                       KB, S);
  hipLaunchKernelGGL(abl_argmax_kernel, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s, (const float*)S, N, K,
                     assign);
  return (int)hipGetLastError();
}

// Scratch for the atomic update: K*D float sums and K counts.
size_t kmeans_abl_atomic_bytes(int64_t D, int64_t K) {
  if (D < 1 || K < 1) return 0;
  return (size_t)K * (size_t)D * 4 + (size_t)K * 4 + 512;
}

// Atomic scatter update (dt 0 fp32, 1 bf16, 2 fp16): C_new = sums / counts,
// empty clusters keep C_prev; ids outside [0, K) ignored.  counts_out
// (device int32[K]) receives the counts.  Asynchronous on `stream`.
int kmeans_abl_update_atomic(const void* X, int dt, int64_t N, int64_t D, const int32_t* assign, int64_t K,
                             const float* C_prev, float* C_new, int32_t* counts_out, void* scratch, size_t scratch_bytes,
                             void* stream) {
  if (dt < 0 || dt > 2 || N < 0 || D < 1 || K < 1 || !C_prev || !C_new || !counts_out || !scratch ||
      C_new == C_prev)
    return -1;
  if (N > 0 && (!X || !assign)) return -1;
  if (scratch_bytes < kmeans_abl_atomic_bytes(D, K)) return -1;
  hipStream_t s = (hipStream_t)stream;
  float* sums = (float*)scratch;
  const int64_t kd = K * D;
  hipLaunchKernelGGL(abl_zero_kernel, dim3((unsigned)((kd + 255) / 256)), dim3(256), 0, s, sums, kd, counts_out, K);
  if (N > 0) {
    const int64_t threads = N * D;
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (dt == A_F32)
      hipLaunchKernelGGL(abl_scatter_kernel<4>, grid, dim3(256), 0, s, (const uint8_t*)X, dt, N, (int)D, assign, K,
                         sums, counts_out);
    else
      hipLaunchKernelGGL(abl_scatter_kernel<2>, grid, dim3(256), 0, s, (const uint8_t*)X, dt, N, (int)D, assign, K,
                         sums, counts_out);
  }
  hipLaunchKernelGGL(abl_divide_kernel, dim3((unsigned)((kd + 255) / 256)), dim3(256), 0, s, (const float*)sums,
                     (const int32_t*)counts_out, K, (int)D, C_prev, C_new);
  return (int)hipGetLastError();
}

}  // extern "C"
