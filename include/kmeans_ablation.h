/*
 * kmeans_ablation.h -- comparison baselines for the two designs Flash-KMeans
 * replaces, built for the same GPU so their cost can be measured next to the
 * library's kernels (libkm_ablation.so; not used by libkmeans_amd.so).
 *
 * Citations name the page "Flash-KMeans: Fast and Memory-Efficient Exact
 * K-Means" (gist.science summary of paper 2603.09229): "tech §n" is a section
 * of its technical summary.
 *
 * Conventions: device pointers, row-major, caller-owned; `scratch` is device
 * memory of at least the size the matching *_bytes function returns (0 there
 * means unsupported arguments).  Calls are asynchronous on `stream` (a
 * hipStream_t, NULL for the default stream) and return 0, -1 for invalid
 * arguments (checked before any HIP call), or a HIP error code.
 */
#ifndef KMEANS_ABLATION_H
#define KMEANS_ABLATION_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Scratch for kmeans_abl_assign_materialized: N*K fp32 scores + rounded centroids + biases. */
size_t kmeans_abl_materialized_bytes(int64_t N, int64_t D, int64_t K);

/*
 * Assignment through the full N x K score matrix (tech §1: materialising the
 * distance matrix makes the assign stage HBM-bound): the scores
 * x.c - |c|^2/2 are computed exactly as FlashAssign computes them (16-bit
 * centroids rounded to nearest even, MFMA with the bias as the starting
 * accumulator, same depth order), written to HBM, then read back by a
 * per-row argmax (lowest index on ties).  The assignment therefore equals
 * FlashAssign's bit for bit.
 *   X       device, N x D, dt 1 = bf16 or 2 = fp16    (read)
 *   C       device K x D fp32 centroids               (read)
 *   assign  device int32[N]                           (written)
 * Limits: 1 <= N, 1 <= D <= 512, 1 <= K; N*K*4 bytes of scratch.
 */
int kmeans_abl_assign_materialized(const void* X, int dt, int64_t N, int64_t D, const float* C, int64_t K,
                                   int32_t* assign, void* scratch, size_t scratch_bytes, void* stream);

/* Scratch for kmeans_abl_update_atomic: K*D fp32 sums. */
size_t kmeans_abl_atomic_bytes(int64_t D, int64_t K);

/*
 * Point-parallel atomic scatter update (tech §1: atomics on hot clusters
 * serialise): every (point, column) adds into its cluster's fp32 sum with a
 * device atomic, every point adds 1 to its count, then C_new = sum / count
 * (empty clusters keep C_prev).  Ids outside [0, K) are ignored.  The order of
 * the additions depends on scheduling (not reproducible bit for bit).
 *   X         device N x D, dt 0 = fp32, 1 = bf16, 2 = fp16  (read)
 *   assign    device int32[N]                                (read)
 *   C_prev    device K x D fp32                              (read)
 *   C_new     device K x D fp32 (may not alias C_prev)       (written)
 *   counts    device int32[K]                                (written)
 */
int kmeans_abl_update_atomic(const void* X, int dt, int64_t N, int64_t D, const int32_t* assign, int64_t K,
                             const float* C_prev, float* C_new, int32_t* counts, void* scratch, size_t scratch_bytes,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KMEANS_ABLATION_H */
