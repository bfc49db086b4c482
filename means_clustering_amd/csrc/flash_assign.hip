// Centroid preparation and FlashAssign: the fused, materialisation-free
// nearest-centroid step of exact Lloyd K-Means on gfx950 matrix cores.
//
// Citations name the page "Flash-KMeans: Fast and Memory-Efficient Exact
// K-Means" (gist.science summary of paper 2603.09229); "tech §n" is a section
// of its technical summary.
//
// What is computed (tech §2.1): for every point x_i the index of the nearest
// centroid under squared Euclidean distance, lowest index on ties, without
// ever writing the N x K distance matrix (tech §1, §2.1: HBM traffic falls
// from O(NK) to O(Nd + Kd)).  Because ||x||^2 is common to every candidate,
//     argmin_k ||x - c_k||^2 = argmax_k ( x . c_k - ||c_k||^2 / 2 ),
// so the kernel seeds each MFMA accumulator with -||c_k||^2/2 and lets the
// matrix cores produce the score directly; only the running max/argmax costs
// vector ALU work.  The optional distance output adds ||x||^2 back.
//
// Precision: 16-bit X runs on v_mfma_f32_32x32x16_{bf16,f16} (fp32
// accumulation); the fp32 centroid state is rounded to X's type once per call
// (round to nearest, ties to even) and ||c||^2 is taken from the rounded
// values, so every candidate is scored against exactly the centroid the
// contraction saw.  fp32 X runs on v_mfma_f32_16x16x4_f32.
//
// Structure (tech §2.1 "online argmin", "tiled streaming", "double buffering",
// re-designed for CDNA4):
//   * 16-bit X uses v_mfma_f32_32x32x16 (32 centroids x 32 points per
//     instruction; on gfx950 the 16x16x32 shape runs at half this rate);
//     fp32 X uses v_mfma_f32_16x16x4_f32;
//   * a wavefront owns NB point groups and keeps their operand fragments in
//     VGPRs for the whole centroid sweep (X is read from HBM exactly once);
//   * centroids stream through LDS in tiles of CT groups, double-buffered:
//     tile t+1 is copied from L2/HBM straight into the other LDS buffer
//     (global_load_lds, no registers) while tile t feeds the matrix cores
//     (one barrier a tile); fp32 X stages tiles through registers;
//   * the accumulator of each MFMA chain starts at the centroid's bias, so
//     the matrix cores deliver the score and the vector ALUs only keep the
//     running (best score, selector) per lane in registers;
//   * the lanes that hold the same point merge once at the end (ties go to
//     the lowest centroid index);
//   * warm start: inside a Lloyd loop the previous iteration's argsort says
//     which centroid each point had.  Points are then taken in that sorted
//     order, so the 32 points of a block mostly share their previous
//     centroid; the block first scores the group of 32 centroids holding it
//     (exact MFMA values), which gives every point a score its final best
//     must reach, and the sweep then needs only the group maxima, scanning a
//     point group's scores exactly when some lane's maximum beats the lane's
//     running best.
//     The result is the same argmax as the full scan, bit for bit.
#include <math.h>

#include "frag_emit.hpp"
#include "km_internal.hpp"

namespace km {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- prep ----

// One workgroup (4 wavefronts) per centroid group: wavefront w quantises the
// group's depth blocks w, w+4, ... into fragment blocks; the partial sums of
// squares of the quantised values meet in LDS, and -||Q(c)||^2/2 (fp32) is
// written in the order the FlashAssign lanes read it.  Padding rows get zero
// fragments and a bias of -inf, so they can never be selected.
// Batched: workgroup w prepares group w % groups of problem w / groups, whose
// centroids start K*D floats and whose fragments start f_stride slots further.
__global__ __launch_bounds__(256) void prep_kernel(const float* __restrict__ C, int64_t K, int D, int dt, AssignCfg cfg,
                                                   int64_t groups, u32x4_t* __restrict__ frag, int64_t f_stride) {
  __shared__ float part[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t bz = (int64_t)blockIdx.x / groups;
  const int64_t g = (int64_t)blockIdx.x - bz * groups;
  C += bz * K * D;
  frag += bz * f_stride;
  const bool wide = cfg.rows == 32;
  const int rsel = wide ? (lane & 31) : (lane & 15);
  const int piece = wide ? (lane >> 5) : (lane >> 4);  // which 8 (wide) or 4 (narrow) depth values
  const int64_t row = g * cfg.rows + rsel;
  const bool live = row < K;
  u32x4_t* gdst = frag + (g / cfg.CT) * cfg.tile_slots() + (g % cfg.CT) * cfg.group_slots();
  float ss = 0.0f;
  for (int kb = wave; kb < cfg.KB; kb += 4) {
    uint32_t w[4];
    if (wide) {
      const int d0 = kb * kFragDepth + piece * 8;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int da = d0 + 2 * e, db = da + 1;
        const float ca = (live && da < D) ? C[row * D + da] : 0.0f;
        const float cb = (live && db < D) ? C[row * D + db] : 0.0f;
        const uint32_t qa = dt == DT_BF16 ? f32_to_bf16_bits(ca) : f32_to_f16_bits(ca);
        const uint32_t qb = dt == DT_BF16 ? f32_to_bf16_bits(cb) : f32_to_f16_bits(cb);
        const float fa = dt == DT_BF16 ? bf16_bits_to_f32(qa) : f16_bits_to_f32(qa);
        const float fb = dt == DT_BF16 ? bf16_bits_to_f32(qb) : f16_bits_to_f32(qb);
        ss = fmaf(fa, fa, ss);
        ss = fmaf(fb, fb, ss);
        w[e] = qa | (qb << 16);
      }
    } else {
      const int d0 = kb * kFragDepth + piece * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = d0 + e;
        const float c = (live && d < D) ? C[row * D + d] : 0.0f;
        ss = fmaf(c, c, ss);
        w[e] = __float_as_uint(c);
      }
    }
    gdst[kb * 64 + lane] = u32x4_t{w[0], w[1], w[2], w[3]};
  }
  part[wave][lane] = ss;
  __syncthreads();
  if (wave == 0) {
    // fixed order: the four wavefronts, then the lanes that hold the same row
    float t = part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane];
    if (wide) {
      t += __shfl_xor(t, 32);
    } else {
      t += __shfl_xor(t, 16);
      t += __shfl_xor(t, 32);
    }
    float* bias = reinterpret_cast<float*>(gdst + cfg.KB * 64);
    if (piece == 0) {
      const float b = live ? -0.5f * t : -INFINITY;
      if (wide) {  // lane half h reads rows 8j + 4h + r as its 16 accumulator values
        const int j = rsel >> 3, h = (rsel >> 2) & 1, r = rsel & 3;
        bias[h * 16 + j * 4 + r] = b;
      } else {  // lane quad q reads rows 4q .. 4q+3
        bias[rsel] = b;
      }
    }
  }
}

hipError_t launch_prep(const AssignGeom& g, const float* C, void* frag, hipStream_t stream, int64_t B) {
  const int64_t groups = g.groups();
  if (B < 1 || groups * B >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prep_kernel, dim3((unsigned)(groups * B)), dim3(256), 0, stream, C, g.K, (int)g.D, g.dt, g.cfg,
                     groups, (u32x4_t*)frag, (int64_t)(g.frag_bytes() / 16));
  return hipGetLastError();
}

// ------------------------------------------------------- point fragments ----

// 16 bytes of row p, elements [d0, d0 + 16/ES); zero beyond D or N.
template <int ES>
__device__ __forceinline__ u32x4_t load_point_frag(const uint8_t* __restrict__ X, int64_t p, int64_t N, int D, int d0,
                                                   bool vec_ok) {
  constexpr int EPL = 16 / ES;
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (p >= N || d0 >= D) return v;
  const uint8_t* row = X + (size_t)p * (size_t)D * ES;
  if (vec_ok && d0 + EPL <= D) return *reinterpret_cast<const u32x4_t*>(row + (size_t)d0 * ES);
  uint32_t w[4] = {0, 0, 0, 0};
  if (ES == 4) {
    const uint32_t* r = reinterpret_cast<const uint32_t*>(row);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (d0 + e < D) w[e] = r[d0 + e];
  } else {
    const uint16_t* r = reinterpret_cast<const uint16_t*>(row);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (d0 + e < D) w[e >> 1] |= (uint32_t)r[d0 + e] << (16 * (e & 1));
  }
  return u32x4_t{w[0], w[1], w[2], w[3]};
}

template <int DT>
__device__ __forceinline__ float sumsq16(u32x4_t v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = DT == DT_BF16 ? bf16_bits_to_f32(w[e] & 0xffffu) : f16_bits_to_f32(w[e] & 0xffffu);
    const float b = DT == DT_BF16 ? bf16_bits_to_f32(w[e] >> 16) : f16_bits_to_f32(w[e] >> 16);
    s = fmaf(a, a, s);
    s = fmaf(b, b, s);
  }
  return s;
}

template <int DT>
__device__ __forceinline__ f32x16_t mma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  if constexpr (DT == DT_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
}

// ------------------------------------------------- FlashAssign, 16-bit X ----
//
// MFMA 32x32x16 layout: lane l supplies A row (l % 32) and B column (l % 32),
// 8 depth values each (the same depth values for A and B, so the contraction
// is exact whatever order the hardware sums them in); the result lane l holds
// column (l % 32) and rows 8j + 4(l/32) + r as accumulator element 4j + r.
// So a lane scores one point against 16 centroids per instruction group, in
// ascending centroid order, and lanes l and l ^ 32 share the point.

// Running-argmax update with one score: if v > best then (best, rel) = (v, E).
// Three VALU instructions: the comparison lands in VCC and the element index
// E is an inline constant, so no selector has to be copied into a vector
// register.  `rel` counts from the base of the group being scanned (callers
// rebase it by -16 per group).  A NaN score never wins ("not greater than").
//
// The compiler's hazard checker does not look inside inline asm, so an asm
// instruction must never be the first reader of a fresh MFMA result (the
// hardware does not wait for the matrix core there).  Every accumulator is
// therefore first read by compiled code (argmax_update_c, fold_first, which
// the compiler spaces correctly after the MFMA), and every asm read of it
// depends on that code's result, so it comes later still.
template <int E>
__device__ __forceinline__ void argmax_update(float v, float& best, int& rel) {
  asm("v_cmp_ngt_f32 vcc, %2, %0\n\t"
      "v_cndmask_b32 %0, %2, %0, vcc\n\t"
      "v_cndmask_b32 %1, %3, %1, vcc"
      : "+v"(best), "+v"(rel)
      : "v"(v), "I"(E)
      : "vcc");
}

// The same update in compiled code (the first read of an accumulator).
template <int E>
__device__ __forceinline__ void argmax_update_c(float v, float& best, int& rel) {
  const bool gt = v > best;
  best = gt ? v : best;
  rel = gt ? E : rel;
}

template <int E, int NB>
__device__ __forceinline__ void argmax_all(const f32x16_t (&in)[NB], float (&best)[NB], int (&rel)[NB]) {
#pragma unroll
  for (int g = 0; g < NB; ++g) argmax_update<E>(in[g][E], best[g], rel[g]);
}

// Elements [E0, E1) of the previous group's scores.
template <int E0, int E1, int NB>
__device__ __forceinline__ void argmax_range(const f32x16_t (&in)[NB], float (&best)[NB], int (&rel)[NB]) {
  if constexpr (E0 < E1 && E0 < 16) {
    argmax_all<E0, NB>(in, best, rel);
    argmax_range<E0 + 1, E1, NB>(in, best, rel);
  }
}

// Elements [0, E1) of a group whose scores have not been read yet: the first
// in compiled code, the rest in asm.
template <int E1, int NB>
__device__ __forceinline__ void argmax_range_first(const f32x16_t (&in)[NB], float (&best)[NB], int (&rel)[NB]) {
#pragma unroll
  for (int g = 0; g < NB; ++g) argmax_update_c<0>(in[g][0], best[g], rel[g]);
  argmax_range<1, E1, NB>(in, best, rel);
}

__device__ __forceinline__ f32x16_t bias_of(const u32x4_t* bp) {
  const u32x4_t b0 = bp[0], b1 = bp[1], b2 = bp[2], b3 = bp[3];
  return f32x16_t{__uint_as_float(b0.x), __uint_as_float(b0.y), __uint_as_float(b0.z), __uint_as_float(b0.w),
                  __uint_as_float(b1.x), __uint_as_float(b1.y), __uint_as_float(b1.z), __uint_as_float(b1.w),
                  __uint_as_float(b2.x), __uint_as_float(b2.y), __uint_as_float(b2.z), __uint_as_float(b2.w),
                  __uint_as_float(b3.x), __uint_as_float(b3.y), __uint_as_float(b3.z), __uint_as_float(b3.w)};
}

__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// The largest float strictly below v (-inf for -inf and NaN).
__device__ __forceinline__ float float_below(float v) {
  if (!(v > -INFINITY)) return -INFINITY;
  if (v == 0.0f) return -__uint_as_float(1u);
  const uint32_t u = __float_as_uint(v);
  return __uint_as_float(v > 0.0f ? u - 1u : u + 1u);
}

// Lazy running argmax, fast part: fold a share of the previous group's 16
// scores into a running group maximum m (exact, 1 instruction per 2 scores).
template <int E0, int E1, int NB>
__device__ __forceinline__ void fold_range(const f32x16_t (&in)[NB], float (&m)[NB]) {
  if constexpr (E0 < E1 && E0 < 16) {
    if constexpr (E0 + 1 < E1 && E0 + 1 < 16) {
#pragma unroll
      for (int g = 0; g < NB; ++g) m[g] = max3f(m[g], in[g][E0], in[g][E0 + 1]);
      fold_range<E0 + 2, E1, NB>(in, m);
    } else {
#pragma unroll
      for (int g = 0; g < NB; ++g) m[g] = max3f(m[g], in[g][E0], in[g][E0]);
      fold_range<E0 + 1, E1, NB>(in, m);
    }
  }
}

// Start of a fold over a group whose scores have not been read yet (compiled
// code; a NaN score is ignored like v_max3_f32 ignores it).
template <int NB>
__device__ __forceinline__ void fold_first(const f32x16_t (&in)[NB], float (&m)[NB]) {
#pragma unroll
  for (int g = 0; g < NB; ++g) m[g] = fmaxf(in[g][0], in[g][1]);
}

// Lazy running argmax, slow part: a point group's scores are scanned exactly
// only when some lane's group maximum beats its running best, each point
// group on its own (a block where one point moves scans that point's group of
// 32, not the wavefront's every point group).  The result is the same as
// scanning every group exactly: a group whose maximum does not exceed the best
// cannot change the lowest-index argmax.
template <int E0, int E1>
__device__ __forceinline__ void argmax_one(const f32x16_t& in, float& best, int& rel) {
  if constexpr (E0 < E1 && E0 < 16) {
    argmax_update<E0>(in[E0], best, rel);
    argmax_one<E0 + 1, E1>(in, best, rel);
  }
}

template <int NB>
__device__ __forceinline__ void lazy_resolve(const f32x16_t (&in)[NB], const float (&m)[NB], float (&best)[NB],
                                             int (&rel)[NB]) {
#pragma unroll
  for (int g = 0; g < NB; ++g)
    if (__builtin_amdgcn_ballot_w64(m[g] > best[g])) argmax_one<0, 16>(in[g], best[g], rel[g]);
}

// Deferred argmax (the single-accumulator kernel), per group: a lane keeps only its best score and the first
// group that reached it (one comparison and two selects, no branch); which of
// that group's 32 centroids it was is settled once, after the sweep, by
// resolve_deferred.  A group whose maximum does not beat the running best
// cannot hold the lowest-index argmax, so the result is the full scan's.
template <int NB>
__device__ __forceinline__ void defer_take(const float (&m)[NB], float (&best)[NB], int (&qsel)[NB], int q) {
#pragma unroll
  for (int g = 0; g < NB; ++g) {
    const bool up = m[g] > best[g];
    best[g] = up ? m[g] : best[g];
    qsel[g] = up ? q : qsel[g];
  }
}

// After a deferred sweep each lane holds its best score `v` and the first
// group `q` that reached it (INT32_MAX: none).  The two lanes of a point
// agree on the point's maximum and on the first group holding it; the
// wavefront then scores each distinct such group again with the sweep's own
// MFMA chain (bias first, depth blocks in order, the same operands), which
// reproduces those scores bit for bit, and the lowest row whose score equals
// the maximum is the point's centroid.  After a warm start the 32 points of a
// block mostly share one winning group, so this takes one or two rounds.
// Returns the centroid index within the sweep (INT32_MAX: none); v becomes
// the point's maximum.
template <int DT, int KB>
__device__ __forceinline__ int resolve_deferred(float& v, int q, const u32x4_t (&xb)[KB],
                                                const u32x4_t* __restrict__ frag, int64_t TS, int64_t GS, int CT,
                                                int lane, int h) {
  const float ov = __shfl_xor(v, 32);
  const int oq = __shfl_xor(q, 32);
  const float vm = fmaxf(v, ov);
  const int qa = v == vm ? q : INT32_MAX, qb = ov == vm ? oq : INT32_MAX;
  const int qw = vm > -INFINITY ? (qa < qb ? qa : qb) : INT32_MAX;
  v = vm;
  int k = INT32_MAX;
  uint64_t pending = __builtin_amdgcn_ballot_w64(qw != INT32_MAX);
  while (pending) {
    const int qq = __builtin_amdgcn_readlane(qw, (int)__builtin_ctzll(pending));
    const u32x4_t* grp = frag + (int64_t)(qq / CT) * TS + (int64_t)(qq % CT) * GS;
    f32x16_t sc = bias_of(grp + KB * 64 + h * 4);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sc = mma32<DT>(grp[kb * 64 + lane], xb[kb], sc);
    int r = INT32_MAX;  // lowest row of this lane's half scoring the maximum
#pragma unroll
    for (int e = 15; e >= 0; --e) r = sc[e] == vm ? (e >> 2) * 8 + h * 4 + (e & 3) : r;
    const bool mine = qw == qq;
    const int kk = mine && r != INT32_MAX ? qq * 32 + r : INT32_MAX;
    const int ok = __shfl_xor(kk, 32);
    if (mine) k = kk < ok ? kk : ok;
    pending &= ~__builtin_amdgcn_ballot_w64(mine);
  }
  return k;
}

// One pipeline stage: the MFMAs of one 32-centroid group into `out`, depth
// block by depth block, each block fenced together with its share of the
// running-argmax update over the previous group's scores `in`, so the matrix
// cores and the vector ALUs of one wavefront overlap.  `a0`/`bias` hold the
// group's first A fragment and its bias (fetched by the caller); the next
// depth block's fragment is fetched one step ahead.
template <int KB, int NB, int KBI, bool LAZY>
__device__ __forceinline__ void epilogue_share(const f32x16_t (&in)[NB], float (&best)[NB], int (&rel)[NB],
                                               float (&m)[NB]) {
  constexpr int per = (16 + KB - 1) / KB;  // epilogue elements per depth block
  if constexpr (LAZY) {
    if constexpr (KBI == 0) {  // elements 0 and 1 (and the rest of the share) of a fresh group
      fold_first<NB>(in, m);
      fold_range<2, per, NB>(in, m);
    } else {
      fold_range<(KBI * per > 2 ? KBI * per : 2), (KBI + 1) * per, NB>(in, m);
    }
  } else {
    if constexpr (KBI == 0)
      argmax_range_first<per, NB>(in, best, rel);
    else
      argmax_range<KBI * per, (KBI + 1) * per, NB>(in, best, rel);
  }
}

template <int DT, int KB, int NB, bool LAZY, bool epi, int KBI = 0>
__device__ __forceinline__ void pipeline_steps(const u32x4_t* __restrict__ grp, int lane, u32x4_t a,
                                               const f32x16_t& bias, const u32x4_t (&xb)[NB][KB],
                                               f32x16_t (&out)[NB], const f32x16_t (&in)[NB], float (&best)[NB],
                                               int (&rel)[NB], float (&m)[NB]) {
  if constexpr (KBI < KB) {
    u32x4_t a_next;
    if constexpr (KBI + 1 < KB) a_next = grp[(KBI + 1) * 64 + lane];
    if constexpr (epi) {
      if constexpr (KBI == 0) {
#pragma unroll
        for (int g = 0; g < NB; ++g) rel[g] -= 16;  // selectors now count from this group's base
      }
      epilogue_share<KB, NB, KBI, LAZY>(in, best, rel, m);
    }
#pragma unroll
    for (int g = 0; g < NB; ++g) out[g] = mma32<DT>(a, xb[g][KBI], KBI == 0 ? bias : out[g]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (KBI + 1 < KB)
      pipeline_steps<DT, KB, NB, LAZY, epi, KBI + 1>(grp, lane, a_next, bias, xb, out, in, best, rel, m);
    else if constexpr (epi && LAZY)
      lazy_resolve<NB>(in, m, best, rel);
  }
}

// Copy one centroid tile (TS 16-byte slots) from global memory straight into
// LDS: each lane moves 16 bytes per instruction, and a wavefront fills 64
// consecutive slots starting at a wave-uniform LDS address, so no VGPRs hold
// the data in flight.  Completion is awaited with s_waitcnt before the
// barrier that publishes the tile.
template <int TS, int NTHR>
__device__ __forceinline__ void tile_dma(const u32x4_t* __restrict__ src, u32x4_t* lds_tile, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < TS / NTHR; ++i) {
    const int base = i * NTHR + wave * 64;
    __builtin_amdgcn_global_load_lds((const void*)(src + base + lane),
                                     (__attribute__((address_space(3))) void*)(lds_tile + base), 16, 0, 0);
  }
}

template <int NB>
__device__ __forceinline__ void drain_epilogue(const f32x16_t (&in)[NB], float (&best)[NB], int (&rel)[NB]) {
#pragma unroll
  for (int g = 0; g < NB; ++g) rel[g] -= 16;
  argmax_range_first<16, NB>(in, best, rel);
}

// WARM: points are visited in the order perm[0..N) and prev[i] is the
// previous centroid of point perm[i] (both from the previous iteration's
// argsort); the sweep starts from a bound taken from that centroid's group.
template <int DT, int KB, bool LAZY, bool WARM, bool SPLIT>
__global__ __launch_bounds__(wide_cfg(KB).W * 64) __attribute__((amdgpu_waves_per_eu(wide_wpe(KB)))) void flash_assign_wide_kernel(
    const uint8_t* __restrict__ X, int64_t N, int D, bool vec_ok, const u32x4_t* __restrict__ frag, int ntiles,
    int32_t* __restrict__ assign, float* __restrict__ min_dist, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ prev, int64_t K, Batch bt) {
  constexpr AssignCfg cfg = wide_cfg(KB);
  constexpr int NB = cfg.NB, CT = cfg.CT, W = cfg.W;
  constexpr int GS = (int)cfg.group_slots();
  constexpr int TS = (int)cfg.tile_slots();
  constexpr int NTHR = W * 64;
  constexpr bool FOLD = LAZY || WARM;
  static_assert(TS % NTHR == 0 && TS >= CT * GS, "tile padding");
  static_assert(CT % 2 == 0, "groups alternate between two accumulator sets");
  __shared__ u32x4_t lds[2][TS];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 31;
  const int h = lane >> 5;
  const uint32_t bz = blockIdx.x / bt.bpp;  // problem of this workgroup (0 unless batched)
  const int64_t wbase = ((int64_t)(blockIdx.x - bz * bt.bpp) * W + wave) * (NB * 32);
  X += (int64_t)bz * bt.x_stride;
  frag += (int64_t)bz * bt.f_stride;
  assign += (int64_t)bz * N;
  if (min_dist) min_dist += (int64_t)bz * N;
  const int32_t id_base = (int32_t)bz * bt.id_mul;
  const int sp = SPLIT ? (int)blockIdx.y : 0;  // centroid range of a split sweep
  if constexpr (SPLIT) {
    frag += (int64_t)sp * bt.split_tiles * TS;
    ntiles = ntiles - sp * bt.split_tiles < bt.split_tiles ? ntiles - sp * bt.split_tiles : bt.split_tiles;
  }

  // the point each lane scores, per point group (its row of X, or N past the end)
  int64_t pt[NB];
#pragma unroll
  for (int g = 0; g < NB; ++g) {
    const int64_t slot = wbase + g * 32 + col;
    if constexpr (WARM)
      pt[g] = slot < N ? (int64_t)perm[slot] : N;
    else
      pt[g] = slot;
  }

  // Point fragments: read once from HBM, kept in VGPRs for the whole sweep.
  u32x4_t xb[NB][KB];
#pragma unroll
  for (int g = 0; g < NB; ++g)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) xb[g][kb] = load_point_frag<2>(X, pt[g], N, D, kb * kFragDepth + h * 8, vec_ok);

  // best score per point group and lane; `rel` = selected element counted
  // from the base of the group most recently scanned (rebased by -16 a group;
  // the start value stays far below any real selection)
  float best[NB];
  int rel[NB];
#pragma unroll
  for (int g = 0; g < NB; ++g) {
    best[g] = -INFINITY;
    rel[g] = -(1 << 30);
  }

  if constexpr (WARM) {
    // Score the block against the group of its first point's previous
    // centroid.  The best of those 32 exact scores is reached by the final
    // answer, so the running best starts just below it: a group can then
    // hold the answer only if its maximum exceeds the running best, and the
    // group that supplied the bound is itself scanned exactly in its turn.
#pragma unroll
    for (int g = 0; g < NB; ++g) {
      const int64_t s0 = wbase + g * 32 < N ? wbase + g * 32 : N - 1;
      int64_t k0 = prev[s0];
      k0 = k0 < 0 ? 0 : (k0 >= K ? K - 1 : k0);
      const int64_t q0 = k0 >> 5;
      const u32x4_t* grp = frag + (q0 / CT) * TS + (q0 % CT) * GS;
      f32x16_t sc = bias_of(grp + KB * 64 + h * 4);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sc = mma32<DT>(grp[kb * 64 + lane], xb[g][kb], sc);
      float mx = fmaxf(sc[0], sc[1]);  // compiled code: the compiler waits for the MFMA results
#pragma unroll
      for (int e = 2; e < 16; ++e) mx = fmaxf(mx, sc[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      best[g] = float_below(mx);
    }
  }

  // tile 0 into LDS
  tile_dma<TS, NTHR>(frag, &lds[0][0], wave, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Group q's scores land in acc0 (q even) or acc1 (q odd); the stage that
  // computes group q also folds group q-1 into the running argmax.
  f32x16_t acc0[NB], acc1[NB];
  float m[NB];  // running maximum of the group being folded (lazy argmax)
  for (int t = 0; t < ntiles; ++t) {
    const u32x4_t* tile = &lds[t & 1][0];
    // the next tile streams into the other buffer while this one is used
    if (t + 1 < ntiles) tile_dma<TS, NTHR>(frag + (size_t)(t + 1) * TS, &lds[(t + 1) & 1][0], wave, lane);
#pragma unroll
    for (int c = 0; c < CT; c += 2) {
      const u32x4_t* g0 = tile + c * GS;
      const u32x4_t* g1 = g0 + GS;
      const u32x4_t a00 = g0[lane];
      const f32x16_t bias0 = bias_of(g0 + KB * 64 + h * 4);
      if (c == 0 && t == 0)
        pipeline_steps<DT, KB, NB, FOLD, false>(g0, lane, a00, bias0, xb, acc0, acc1, best, rel, m);
      else
        pipeline_steps<DT, KB, NB, FOLD, true>(g0, lane, a00, bias0, xb, acc0, acc1, best, rel, m);
      const u32x4_t a10 = g1[lane];
      const f32x16_t bias1 = bias_of(g1 + KB * 64 + h * 4);
      pipeline_steps<DT, KB, NB, FOLD, true>(g1, lane, a10, bias1, xb, acc1, acc0, best, rel, m);
    }
    if (t + 1 < ntiles) {
      __builtin_amdgcn_s_waitcnt(0);  // this wave's part of the next tile has landed
      __syncthreads();                // ... and everyone's; this tile is no longer read
    }
  }
  drain_epilogue<NB>(acc1, best, rel);

  const int last_base = (ntiles * CT - 1) * 16;  // selector base of the final group
#pragma unroll
  for (int g = 0; g < NB; ++g) {
    float b = best[g];
    const int sg = last_base + rel[g];
    const bool none = b == -INFINITY || rel[g] <= -(1 << 30);  // nothing selected (NaN scores)
    int k = none ? INT32_MAX : (sg >> 4) * 32 + ((sg & 15) >> 2) * 8 + h * 4 + (sg & 3);
    const float ob = __shfl_xor(b, 32);
    const int ok = __shfl_xor(k, 32);
    if (ob > b || (ob == b && ok < k)) {
      b = ob;
      k = ok;
    }
    float xn = 0.0f;  // ||x||^2, only for the distance output
    if (min_dist || (SPLIT && bt.part_xn)) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) xn += sumsq16<DT>(xb[g][kb]);
      xn += __shfl_xor(xn, 32);
    }
    const int64_t p = pt[g];
    if constexpr (SPLIT) {  // one range of a split sweep: its best, in problem indices
      if (h == 0 && p < N) {
        const int64_t o = (int64_t)bz * N + p;
        bt.part_s[sp * bt.part_stride + o] = b;
        bt.part_k[sp * bt.part_stride + o] = k == INT32_MAX ? INT32_MAX : k + sp * bt.split_tiles * CT * 32;
        if (sp == 0 && bt.part_xn) bt.part_xn[o] = xn;
      }
      continue;
    }
    if (k == INT32_MAX) k = 0;  // no finite score (NaN input): index 0
    if (h == 0 && p < N) {
      assign[p] = k + id_base;
      if (min_dist) min_dist[p] = fmaxf(xn - 2.0f * b, 0.0f);
    }
  }
}

// Single-accumulator variant for long sweeps (D <= 128; layout in wide8_cfg).
// Per group of 32 centroids a wavefront loads the group's bias straight into
// its accumulators, runs the KB-step MFMA chain for all of its point groups,
// then updates the running argmax from those accumulators while the other
// wavefront on the SIMD keeps the matrix cores busy.
template <int DT, int KB, bool LAZY, bool WARM, bool SPLIT>
__global__ __launch_bounds__(wide8_cfg(KB).W * 64) __attribute__((amdgpu_waves_per_eu(KM_W8_WPE))) void flash_assign_w8_kernel(
    const uint8_t* __restrict__ X, int64_t N, int D, bool vec_ok, const u32x4_t* __restrict__ frag, int ntiles,
    int32_t* __restrict__ assign, float* __restrict__ min_dist, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ prev, int64_t K, Batch bt) {
  constexpr AssignCfg cfg = wide8_cfg(KB);
  constexpr int NB = cfg.NB, CT = cfg.CT, W = cfg.W;
  constexpr int GS = (int)cfg.group_slots();
  constexpr int TS = (int)cfg.tile_slots();
  constexpr int NTHR = W * 64;
  constexpr bool FOLD = LAZY || WARM;
  static_assert(TS % NTHR == 0 && TS >= CT * GS, "tile padding");
  __shared__ u32x4_t lds[2][TS];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 31;
  const int h = lane >> 5;
  const uint32_t bz = blockIdx.x / bt.bpp;  // problem of this workgroup (0 unless batched)
  const int64_t wbase = ((int64_t)(blockIdx.x - bz * bt.bpp) * W + wave) * (NB * 32);
  X += (int64_t)bz * bt.x_stride;
  frag += (int64_t)bz * bt.f_stride;
  assign += (int64_t)bz * N;
  if (min_dist) min_dist += (int64_t)bz * N;
  const int32_t id_base = (int32_t)bz * bt.id_mul;
  const int sp = SPLIT ? (int)blockIdx.y : 0;  // centroid range of a split sweep
  if constexpr (SPLIT) {
    frag += (int64_t)sp * bt.split_tiles * TS;
    ntiles = ntiles - sp * bt.split_tiles < bt.split_tiles ? ntiles - sp * bt.split_tiles : bt.split_tiles;
  }

  // the point each lane scores (its row of X, or N past the end); looked up
  // again at the end rather than kept live through the sweep
  auto point_of = [&](int g) -> int64_t {
    const int64_t slot = wbase + g * 32 + col;
    if constexpr (WARM)
      return slot < N ? (int64_t)perm[slot] : N;
    else
      return slot;
  };

  u32x4_t xb[NB][KB];
#pragma unroll
  for (int g = 0; g < NB; ++g) {
    const int64_t p = point_of(g);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) xb[g][kb] = load_point_frag<2>(X, p, N, D, kb * kFragDepth + h * 8, vec_ok);
  }

  float best[NB];
  int rel[NB];  // exact scan: selected element from the last group's base; folded: first group reaching best
#pragma unroll
  for (int g = 0; g < NB; ++g) {
    best[g] = -INFINITY;
    rel[g] = FOLD ? INT32_MAX : -(1 << 30);
  }

  if constexpr (WARM) {
    // bound from the group of the block's first point's previous centroid (see the four-wavefront kernel)
#pragma unroll
    for (int g = 0; g < NB; ++g) {
      const int64_t s0 = wbase + g * 32 < N ? wbase + g * 32 : N - 1;
      int64_t k0 = prev[s0];
      k0 = k0 < 0 ? 0 : (k0 >= K ? K - 1 : k0);
      const int64_t q0 = k0 >> 5;
      const u32x4_t* grp = frag + (q0 / CT) * TS + (q0 % CT) * GS;
      f32x16_t sc = bias_of(grp + KB * 64 + h * 4);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sc = mma32<DT>(grp[kb * 64 + lane], xb[g][kb], sc);
      float mx = fmaxf(sc[0], sc[1]);
#pragma unroll
      for (int e = 2; e < 16; ++e) mx = fmaxf(mx, sc[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      best[g] = float_below(mx);
    }
  }

  tile_dma<TS, NTHR>(frag, &lds[0][0], wave, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  f32x16_t acc[NB];
  for (int t = 0; t < ntiles; ++t) {
    const u32x4_t* tile = &lds[t & 1][0];
    if (t + 1 < ntiles) tile_dma<TS, NTHR>(frag + (size_t)(t + 1) * TS, &lds[(t + 1) & 1][0], wave, lane);
#pragma unroll 2
    for (int c = 0; c < CT; ++c) {
      const u32x4_t* grp = tile + c * GS;
#pragma unroll
      for (int g = 0; g < NB; ++g) acc[g] = bias_of(grp + KB * 64 + h * 4);
      u32x4_t a = grp[lane];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        u32x4_t an;
        if (kb + 1 < KB) an = grp[(kb + 1) * 64 + lane];
#pragma unroll
        for (int g = 0; g < NB; ++g) acc[g] = mma32<DT>(a, xb[g][kb], acc[g]);
        if (kb + 1 < KB) a = an;
      }
      if constexpr (FOLD) {
        float m[NB];
        fold_first<NB>(acc, m);
        fold_range<2, 16, NB>(acc, m);
        defer_take<NB>(m, best, rel, t * CT + c);
      } else {
#pragma unroll
        for (int g = 0; g < NB; ++g) rel[g] -= 16;  // selectors now count from this group's base
        argmax_range_first<16, NB>(acc, best, rel);
      }
    }
    if (t + 1 < ntiles) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  const int last_base = (ntiles * CT - 1) * 16;
#pragma unroll
  for (int g = 0; g < NB; ++g) {
    float b = best[g];
    int k;
    if constexpr (FOLD) {
      k = resolve_deferred<DT, KB>(b, rel[g], xb[g], frag, TS, GS, CT, lane, h);
    } else {
      const int sg = last_base + rel[g];
      const bool none = b == -INFINITY || rel[g] <= -(1 << 30);
      k = none ? INT32_MAX : (sg >> 4) * 32 + ((sg & 15) >> 2) * 8 + h * 4 + (sg & 3);
      const float ob = __shfl_xor(b, 32);
      const int ok = __shfl_xor(k, 32);
      if (ob > b || (ob == b && ok < k)) {
        b = ob;
        k = ok;
      }
    }
    float xn = 0.0f;
    if (min_dist || (SPLIT && bt.part_xn)) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) xn += sumsq16<DT>(xb[g][kb]);
      xn += __shfl_xor(xn, 32);
    }
    const int64_t p = point_of(g);
    if constexpr (SPLIT) {  // one range of a split sweep: its best, in problem indices
      if (h == 0 && p < N) {
        const int64_t o = (int64_t)bz * N + p;
        bt.part_s[sp * bt.part_stride + o] = b;
        bt.part_k[sp * bt.part_stride + o] = k == INT32_MAX ? INT32_MAX : k + sp * bt.split_tiles * CT * 32;
        if (sp == 0 && bt.part_xn) bt.part_xn[o] = xn;
      }
      continue;
    }
    if (k == INT32_MAX) k = 0;
    if (h == 0 && p < N) {
      assign[p] = k + id_base;
      if (min_dist) min_dist[p] = fmaxf(xn - 2.0f * b, 0.0f);
    }
  }
}

// --------------------------------------------------- FlashAssign, fp32 X ----
//
// MFMA 16x16x4 f32 layout: lane l supplies A row (l % 16) and B column
// (l % 16), one depth value each; a fragment holds the four depth values of
// four consecutive instructions.  The result lane l holds column (l % 16) and
// rows 4(l/16) + r; lanes l, l^16, l^32, l^48 share the point.

__device__ __forceinline__ f32x4_t mma16_f32(u32x4_t a, u32x4_t b, f32x4_t c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  return c;
}

template <int KB, bool HALF, bool THIN, bool SPLIT>
__global__ __launch_bounds__(narrow_cfg(KB, HALF, THIN).W * 64) void flash_assign_narrow_kernel(
    const uint8_t* __restrict__ X, int64_t N, int D, bool vec_ok, const u32x4_t* __restrict__ frag, int ntiles,
    int32_t* __restrict__ assign, float* __restrict__ min_dist, Batch bt) {
  constexpr AssignCfg cfg = narrow_cfg(KB, HALF, THIN);
  constexpr int NB = cfg.NB, CT = cfg.CT, W = cfg.W;
  constexpr int GS = (int)cfg.group_slots();
  constexpr int TS = (int)cfg.tile_slots();
  constexpr int NTHR = W * 64;
  constexpr int CPT = TS / NTHR;
  static_assert(TS % NTHR == 0 && TS >= CT * GS, "tile padding");
  __shared__ u32x4_t lds[2][TS];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int quad = lane >> 4;
  const uint32_t bz = blockIdx.x / bt.bpp;  // problem of this workgroup (0 unless batched)
  const int64_t wbase = ((int64_t)(blockIdx.x - bz * bt.bpp) * W + wave) * (NB * 16);
  X += (int64_t)bz * bt.x_stride;
  frag += (int64_t)bz * bt.f_stride;
  assign += (int64_t)bz * N;
  if (min_dist) min_dist += (int64_t)bz * N;
  const int32_t id_base = (int32_t)bz * bt.id_mul;
  const int sp = SPLIT ? (int)blockIdx.y : 0;  // centroid range of a split sweep
  if constexpr (SPLIT) {
    frag += (int64_t)sp * bt.split_tiles * TS;
    ntiles = ntiles - sp * bt.split_tiles < bt.split_tiles ? ntiles - sp * bt.split_tiles : bt.split_tiles;
  }

  u32x4_t xb[NB][KB];
  float xn[NB];
#pragma unroll
  for (int g = 0; g < NB; ++g) {
    const int64_t p = wbase + g * 16 + col;
    float s = 0.0f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      xb[g][kb] = load_point_frag<4>(X, p, N, D, kb * kFragDepth + quad * 4, vec_ok);
      const u32x4_t v = xb[g][kb];
      s = fmaf(__uint_as_float(v.x), __uint_as_float(v.x), s);
      s = fmaf(__uint_as_float(v.y), __uint_as_float(v.y), s);
      s = fmaf(__uint_as_float(v.z), __uint_as_float(v.z), s);
      s = fmaf(__uint_as_float(v.w), __uint_as_float(v.w), s);
    }
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    xn[g] = s;
  }

  float best[NB];
  int sel[NB];
#pragma unroll
  for (int g = 0; g < NB; ++g) {
    best[g] = -INFINITY;
    sel[g] = -1;
  }

  u32x4_t stage[CPT];
  {
    const u32x4_t* src = frag + threadIdx.x;
#pragma unroll
    for (int i = 0; i < CPT; ++i) stage[i] = src[i * NTHR];
#pragma unroll
    for (int i = 0; i < CPT; ++i) lds[0][i * NTHR + threadIdx.x] = stage[i];
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < ntiles;
    if (more) {
      const u32x4_t* src = frag + (size_t)(t + 1) * TS + threadIdx.x;
#pragma unroll
      for (int i = 0; i < CPT; ++i) stage[i] = src[i * NTHR];
    }
#pragma unroll 2
    for (int c = 0; c < CT; ++c) {
      const u32x4_t* grp = &lds[buf][c * GS];
      u32x4_t a[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) a[kb] = grp[kb * 64 + lane];
      const f32x4_t bias4 = __builtin_bit_cast(f32x4_t, grp[KB * 64 + quad]);
      const int s0 = (t * CT + c) * 4;  // wave-uniform selector of this 16-centroid group
#pragma unroll
      for (int g = 0; g < NB; ++g) {
        f32x4_t acc = bias4;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) acc = mma16_f32(a[kb], xb[g][kb], acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (acc[i] > best[g]) {
            best[g] = acc[i];
            sel[g] = s0 + i;
          }
        }
      }
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) lds[buf ^ 1][i * NTHR + threadIdx.x] = stage[i];
    }
    __syncthreads();
  }

#pragma unroll
  for (int g = 0; g < NB; ++g) {
    float b = best[g];
    int k = sel[g] < 0 ? INT32_MAX : (sel[g] >> 2) * 16 + quad * 4 + (sel[g] & 3);
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float ob = __shfl_xor(b, off);
      const int ok = __shfl_xor(k, off);
      if (ob > b || (ob == b && ok < k)) {
        b = ob;
        k = ok;
      }
    }
    const int64_t p = wbase + g * 16 + col;
    if constexpr (SPLIT) {  // one range of a split sweep: its best, in problem indices
      if (quad == 0 && p < N) {
        const int64_t o = (int64_t)bz * N + p;
        bt.part_s[sp * bt.part_stride + o] = b;
        bt.part_k[sp * bt.part_stride + o] = k == INT32_MAX ? INT32_MAX : k + sp * bt.split_tiles * CT * 16;
        if (sp == 0 && bt.part_xn) bt.part_xn[o] = xn[g];
      }
      continue;
    }
    if (k == INT32_MAX) k = 0;
    if (quad == 0 && p < N) {
      assign[p] = k + id_base;
      if (min_dist) min_dist[p] = fmaxf(xn[g] - 2.0f * b, 0.0f);
    }
  }
}

// --------------------------------------------------------------- launch ----

static bool same_cfg(const AssignCfg& a, const AssignCfg& b) {
  return a.rows == b.rows && a.KB == b.KB && a.NB == b.NB && a.CT == b.CT && a.W == b.W;
}

// How a sweep is split over centroid ranges (S == 1: not split).
struct SplitPlan {
  int64_t S = 1;
  int32_t tiles = 0;
  float* s = nullptr;
  int32_t* k = nullptr;
  float* xn = nullptr;
  int64_t stride = 0;
};

// Workgroups per problem times problems; the batch strides follow from the shape.
static Batch make_batch(const AssignGeom& g, int64_t N, int64_t blocks, int32_t id_mul, const SplitPlan& sp) {
  Batch b;
  b.bpp = (uint32_t)blocks;
  b.id_mul = id_mul;
  b.x_stride = N * g.D * (int64_t)dtype_size(g.dt);
  b.f_stride = (int64_t)(g.frag_bytes() / 16);
  b.split_tiles = sp.S > 1 ? sp.tiles : 0;
  b.part_s = sp.S > 1 ? sp.s : nullptr;
  b.part_k = sp.k;
  b.part_xn = sp.xn;
  b.part_stride = sp.stride;
  return b;
}

// ------------------------------------------------- FlashAssign, deep rows ----
//
// Rows too long to keep a point's whole operand in registers (16-bit X beyond
// kMaxD16 values, fp32 X beyond kMaxD32): the same fused distance + argmin,
// with the depth walked in chunks.  A workgroup (four wavefronts, two point
// groups each) sweeps tiles of kDeepCT centroid groups; for each tile the
// depth is taken kDeepKC fragment blocks (64 values) at a time: the tile's
// centroid fragments of that chunk are copied into LDS (double-buffered,
// global_load_lds), the points' fragments of that chunk are loaded into
// registers one step ahead, and the MFMAs accumulate every (point, centroid)
// score of the tile over the whole depth in registers.  When a tile's last
// chunk is done its scores (bias-seeded, as in the other kernels) update the
// running best per lane, ascending centroid order, strict comparison; the
// lanes holding one point merge at the end with the lower index winning ties.
// No N x K array exists anywhere: a tile's scores live in registers only.
// The points' operands are re-read once per tile (from L2 / the last-level
// cache), the price of rows that do not fit in registers.
template <int DT>
struct DeepOps;
template <>
struct DeepOps<DT_BF16> {
  using acc_t = f32x16_t;
  static constexpr int kRows = 32, kE = 16, kES = 2;
  static __device__ __forceinline__ acc_t mma(u32x4_t a, u32x4_t b, acc_t c) { return mma32<DT_BF16>(a, b, c); }
  static __device__ __forceinline__ acc_t bias(const u32x4_t* grp_bias, int piece) { return bias_of(grp_bias + piece * 4); }
  static __device__ __forceinline__ float sumsq(u32x4_t v) { return sumsq16<DT_BF16>(v); }
  static __device__ __forceinline__ int row_of(int e, int piece) { return (e >> 2) * 8 + piece * 4 + (e & 3); }
};
template <>
struct DeepOps<DT_F16> {
  using acc_t = f32x16_t;
  static constexpr int kRows = 32, kE = 16, kES = 2;
  static __device__ __forceinline__ acc_t mma(u32x4_t a, u32x4_t b, acc_t c) { return mma32<DT_F16>(a, b, c); }
  static __device__ __forceinline__ acc_t bias(const u32x4_t* grp_bias, int piece) { return bias_of(grp_bias + piece * 4); }
  static __device__ __forceinline__ float sumsq(u32x4_t v) { return sumsq16<DT_F16>(v); }
  static __device__ __forceinline__ int row_of(int e, int piece) { return (e >> 2) * 8 + piece * 4 + (e & 3); }
};
template <>
struct DeepOps<DT_F32> {
  using acc_t = f32x4_t;
  static constexpr int kRows = 16, kE = 4, kES = 4;
  static __device__ __forceinline__ acc_t mma(u32x4_t a, u32x4_t b, acc_t c) { return mma16_f32(a, b, c); }
  static __device__ __forceinline__ acc_t bias(const u32x4_t* grp_bias, int piece) {
    return __builtin_bit_cast(f32x4_t, grp_bias[piece]);
  }
  static __device__ __forceinline__ float sumsq(u32x4_t v) {
    float s = 0.0f;
    s = fmaf(__uint_as_float(v.x), __uint_as_float(v.x), s);
    s = fmaf(__uint_as_float(v.y), __uint_as_float(v.y), s);
    s = fmaf(__uint_as_float(v.z), __uint_as_float(v.z), s);
    s = fmaf(__uint_as_float(v.w), __uint_as_float(v.w), s);
    return s;
  }
  static __device__ __forceinline__ int row_of(int e, int piece) { return piece * 4 + e; }
};

template <int DT, bool SPLIT>
__global__ __launch_bounds__(kDeepW * 64) void flash_assign_deep_kernel(
    const uint8_t* __restrict__ X, int64_t N, int D, bool vec_ok, const u32x4_t* __restrict__ frag, int ntiles, int KB,
    int32_t* __restrict__ assign, float* __restrict__ min_dist, Batch bt) {
  using Ops = DeepOps<DT>;
  using acc_t = typename Ops::acc_t;
  constexpr int ROWS = Ops::kRows, E = Ops::kE, ES = Ops::kES;
  constexpr int NB = kDeepNB, CT = kDeepCT, W = kDeepW, KC = kDeepKC;
  constexpr int PIECE_LANES = ROWS;              // lanes l and l + ROWS (.. ) hold one point
  constexpr int PIECE_VALS = ROWS / 4;           // depth values per lane per block: 8 or 4
  const AssignCfg cfg = deep_cfg(DT, KB);
  const int64_t GS = cfg.group_slots();
  const int64_t TS = cfg.tile_slots();
  const int NC = (KB + KC - 1) / KC;  // depth chunks
  __shared__ u32x4_t lds[2][CT * KC][64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane % PIECE_LANES;
  const int piece = lane / PIECE_LANES;
  const uint32_t bz = blockIdx.x / bt.bpp;
  const int64_t wbase = ((int64_t)(blockIdx.x - bz * bt.bpp) * W + wave) * (NB * ROWS);
  X += (int64_t)bz * bt.x_stride;
  frag += (int64_t)bz * bt.f_stride;
  assign += (int64_t)bz * N;
  if (min_dist) min_dist += (int64_t)bz * N;
  const int32_t id_base = (int32_t)bz * bt.id_mul;
  const int sp = SPLIT ? (int)blockIdx.y : 0;
  if constexpr (SPLIT) {
    frag += (int64_t)sp * bt.split_tiles * TS;
    ntiles = ntiles - sp * bt.split_tiles < bt.split_tiles ? ntiles - sp * bt.split_tiles : bt.split_tiles;
  }
  int64_t pt[NB];
#pragma unroll
  for (int g = 0; g < NB; ++g) pt[g] = wbase + g * ROWS + col;

  // centroid fragments of step s (tile s / NC, depth chunk s % NC) into LDS buffer `buf`: each wavefront
  // copies whole fragment blocks (64 slots), wave-uniform destinations
  auto stage_centroids = [&](int s, int buf) {
    const int t = s / NC, kb0 = (s % NC) * KC;
#pragma unroll
    for (int j = 0; j < CT * KC / W; ++j) {
      const int i = j * W + wave;  // (group, block) pair
      const int g = i / KC, kk = i % KC;
      if (kb0 + kk < KB)
        __builtin_amdgcn_global_load_lds((const void*)(frag + (int64_t)t * TS + g * GS + (int64_t)(kb0 + kk) * 64 + lane),
                                         (__attribute__((address_space(3))) void*)&lds[buf][i][0], 16, 0, 0);
    }
  };
  // point fragments of depth chunk c into registers (zero beyond D and N)
  auto load_points = [&](int c, u32x4_t (&xb)[NB][KC]) {
    const int kb0 = c * KC;
#pragma unroll
    for (int g = 0; g < NB; ++g)
#pragma unroll
      for (int kk = 0; kk < KC; ++kk)
        xb[g][kk] = load_point_frag<ES>(X, pt[g], N, D, (kb0 + kk) * kFragDepth + piece * PIECE_VALS, vec_ok);
  };

  float best[NB], xn[NB];
  int32_t bidx[NB];
#pragma unroll
  for (int g = 0; g < NB; ++g) {
    best[g] = -INFINITY;
    bidx[g] = INT32_MAX;
    xn[g] = 0.0f;
  }
  const int steps = ntiles * NC;
  u32x4_t xb[NB][KC], xnx[NB][KC];
  acc_t acc[NB][CT];
  if (steps > 0) {
    stage_centroids(0, 0);
    load_points(0, xb);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  for (int s = 0; s < steps; ++s) {
    const int buf = s & 1;
    const int t = s / NC, c = s % NC;
    if (s + 1 < steps) {  // the next step's operands stream in while this one computes
      stage_centroids(s + 1, buf ^ 1);
      load_points((s + 1) % NC, xnx);
    }
    if (c == 0) {
#pragma unroll
      for (int g = 0; g < CT; ++g) {
        const acc_t b = Ops::bias(frag + (int64_t)t * TS + g * GS + (int64_t)KB * 64, piece);
#pragma unroll
        for (int q = 0; q < NB; ++q) acc[q][g] = b;
      }
    }
    if (t == 0) {  // ||x||^2 from the first tile's pass over the depth
#pragma unroll
      for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) xn[q] += Ops::sumsq(xb[q][kk]);
    }
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      if (c * KC + kk < KB) {
#pragma unroll
        for (int g = 0; g < CT; ++g) {
          const u32x4_t a = lds[buf][g * KC + kk][lane];
#pragma unroll
          for (int q = 0; q < NB; ++q) acc[q][g] = Ops::mma(a, xb[q][kk], acc[q][g]);
        }
      }
    }
    if (c == NC - 1) {  // the tile's scores are complete: running best, ascending centroid order
#pragma unroll
      for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int g = 0; g < CT; ++g)
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float v = acc[q][g][e];
            if (v > best[q]) {
              best[q] = v;
              bidx[q] = (t * CT + g) * ROWS + Ops::row_of(e, piece);
            }
          }
    }
    if (s + 1 < steps) {
      __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of the next step have landed
      __syncthreads();                // ... and everyone's; this buffer is no longer read
#pragma unroll
      for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) xb[q][kk] = xnx[q][kk];
    }
  }

#pragma unroll
  for (int q = 0; q < NB; ++q) {
    float b = best[q], x2 = xn[q];
    int32_t k = bidx[q];
#pragma unroll
    for (int off = PIECE_LANES; off < 64; off <<= 1) {
      const float ob = __shfl_xor(b, off);
      const int32_t ok = __shfl_xor(k, off);
      if (ob > b || (ob == b && ok < k)) {
        b = ob;
        k = ok;
      }
      x2 += __shfl_xor(x2, off);
    }
    const int64_t p = pt[q];
    if constexpr (SPLIT) {
      if (piece == 0 && p < N) {
        const int64_t o = (int64_t)bz * N + p;
        bt.part_s[sp * bt.part_stride + o] = b;
        bt.part_k[sp * bt.part_stride + o] = k == INT32_MAX ? INT32_MAX : k + sp * bt.split_tiles * CT * ROWS;
        if (sp == 0 && bt.part_xn) bt.part_xn[o] = x2;
      }
      continue;
    }
    if (k == INT32_MAX) k = 0;  // no finite score (NaN input): index 0
    if (piece == 0 && p < N) {
      assign[p] = k + id_base;
      if (min_dist) min_dist[p] = fmaxf(x2 - 2.0f * b, 0.0f);
    }
  }
}

template <int DT>
static hipError_t launch_deep(const AssignGeom& g, const void* X, int64_t N, const void* frag, int32_t* assign,
                              float* min_dist, int64_t B, int32_t id_mul, const SplitPlan& sp, hipStream_t s) {
  const AssignCfg cfg = deep_cfg(DT, g.cfg.KB);
  if (!same_cfg(g.cfg, cfg)) return hipErrorInvalidValue;
  const int64_t pts = (int64_t)cfg.W * cfg.NB * cfg.rows;
  const int64_t blocks = (N + pts - 1) / pts;
  const int64_t nsteps = g.ntiles() * ((cfg.KB + kDeepKC - 1) / kDeepKC);  // (tile, depth chunk) steps
  if (blocks * B >= ((int64_t)1 << 31) || nsteps >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const int es = dtype_size(g.dt);
  const bool vec_ok = (((uintptr_t)X) % 16 == 0) && ((g.D * es) % 16 == 0);
  const dim3 grid((unsigned)(blocks * B), (unsigned)sp.S), block(cfg.W * 64);
  const Batch bt = make_batch(g, N, blocks, id_mul, sp);
  if (sp.S > 1)
    hipLaunchKernelGGL((flash_assign_deep_kernel<DT, true>), grid, block, 0, s, (const uint8_t*)X, N, (int)g.D, vec_ok,
                       (const u32x4_t*)frag, (int)g.ntiles(), cfg.KB, assign, min_dist, bt);
  else
    hipLaunchKernelGGL((flash_assign_deep_kernel<DT, false>), grid, block, 0, s, (const uint8_t*)X, N, (int)g.D, vec_ok,
                       (const u32x4_t*)frag, (int)g.ntiles(), cfg.KB, assign, min_dist, bt);
  return hipGetLastError();
}

// The best of a split sweep's ranges per point, taken in range order with
// the kernels' own rule (a higher score wins; on equal scores the lower
// index), so the result is the unsplit sweep's.
__global__ __launch_bounds__(256) void assign_merge_kernel(const float* __restrict__ part_s,
                                                           const int32_t* __restrict__ part_k,
                                                           const float* __restrict__ part_xn, int64_t total, int64_t N,
                                                           int S, int32_t id_mul, int32_t* __restrict__ assign,
                                                           float* __restrict__ min_dist) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  float b = -INFINITY;
  int32_t k = INT32_MAX;
  for (int r = 0; r < S; ++r) {
    const float v = part_s[r * total + i];
    const int32_t kk = part_k[r * total + i];
    if (v > b || (v == b && kk < k)) {
      b = v;
      k = kk;
    }
  }
  if (k == INT32_MAX) k = 0;  // no finite score (NaN input): index 0
  assign[i] = k + (int32_t)(i / N) * id_mul;
  if (min_dist) min_dist[i] = fmaxf(part_xn[i] - 2.0f * b, 0.0f);
}

template <int DT, int KB>
static hipError_t launch_wide8(const AssignGeom& g, const void* X, int64_t N, const void* frag, int32_t* assign,
                               float* min_dist, const int32_t* perm, const int32_t* prev, int64_t B, int32_t id_mul,
                               const SplitPlan& sp, hipStream_t s) {
  constexpr AssignCfg cfg = wide8_cfg(KB);
  if (!same_cfg(g.cfg, cfg)) return hipErrorInvalidValue;
  const int64_t pts = (int64_t)cfg.W * cfg.NB * 32;
  const int64_t blocks = (N + pts - 1) / pts;
  if (blocks * B >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const bool vec_ok = (((uintptr_t)X) % 16 == 0) && ((g.D * 2) % 16 == 0);
  const dim3 grid((unsigned)(blocks * B), (unsigned)sp.S), block(cfg.W * 64);
  const Batch bt = make_batch(g, N, blocks, id_mul, sp);
  const uint8_t* x = (const uint8_t*)X;
  const u32x4_t* f = (const u32x4_t*)frag;
  const int nt = (int)g.ntiles();
  if (sp.S > 1 && g.lazy)  // (split sweeps are cold)
    hipLaunchKernelGGL((flash_assign_w8_kernel<DT, KB, true, false, true>), grid, block, 0, s, x, N, (int)g.D, vec_ok, f,
                       nt, assign, min_dist, nullptr, nullptr, g.K, bt);
  else if (sp.S > 1)
    hipLaunchKernelGGL((flash_assign_w8_kernel<DT, KB, false, false, true>), grid, block, 0, s, x, N, (int)g.D, vec_ok,
                       f, nt, assign, min_dist, nullptr, nullptr, g.K, bt);
  else if (perm)
    hipLaunchKernelGGL((flash_assign_w8_kernel<DT, KB, true, true, false>), grid, block, 0, s, x, N, (int)g.D, vec_ok, f,
                       nt, assign, min_dist, perm, prev, g.K, bt);
  else if (g.lazy)
    hipLaunchKernelGGL((flash_assign_w8_kernel<DT, KB, true, false, false>), grid, block, 0, s, x, N, (int)g.D, vec_ok, f,
                       nt, assign, min_dist, perm, prev, g.K, bt);
  else
    hipLaunchKernelGGL((flash_assign_w8_kernel<DT, KB, false, false, false>), grid, block, 0, s, x, N, (int)g.D, vec_ok,
                       f, nt, assign, min_dist, perm, prev, g.K, bt);
  return hipGetLastError();
}

template <int DT, int KB>
static hipError_t launch_wide(const AssignGeom& g, const void* X, int64_t N, const void* frag, int32_t* assign,
                              float* min_dist, const int32_t* perm, const int32_t* prev, int64_t B, int32_t id_mul,
                              const SplitPlan& sp, hipStream_t s) {
  if constexpr (KB <= kWide8MaxKB) {
    if (same_cfg(g.cfg, wide8_cfg(KB)))
      return launch_wide8<DT, KB>(g, X, N, frag, assign, min_dist, perm, prev, B, id_mul, sp, s);
  }
  constexpr AssignCfg cfg = wide_cfg(KB);
  // The centroid fragments were laid out with the caller's geometry: it must be
  // the one this kernel was compiled for (both come from one header).
  if (!same_cfg(g.cfg, cfg)) return hipErrorInvalidValue;
  const int64_t pts = (int64_t)cfg.W * cfg.NB * 32;
  const int64_t blocks = (N + pts - 1) / pts;
  if (blocks * B >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const bool vec_ok = (((uintptr_t)X) % 16 == 0) && ((g.D * 2) % 16 == 0);
  const dim3 grid((unsigned)(blocks * B), (unsigned)sp.S), block(cfg.W * 64);
  const Batch bt = make_batch(g, N, blocks, id_mul, sp);
  const uint8_t* x = (const uint8_t*)X;
  const u32x4_t* f = (const u32x4_t*)frag;
  const int nt = (int)g.ntiles();
  if (sp.S > 1 && g.lazy)  // (split sweeps are cold)
    hipLaunchKernelGGL((flash_assign_wide_kernel<DT, KB, true, false, true>), grid, block, 0, s, x, N, (int)g.D, vec_ok, f,
                       nt, assign, min_dist, nullptr, nullptr, g.K, bt);
  else if (sp.S > 1)
    hipLaunchKernelGGL((flash_assign_wide_kernel<DT, KB, false, false, true>), grid, block, 0, s, x, N, (int)g.D, vec_ok,
                       f, nt, assign, min_dist, nullptr, nullptr, g.K, bt);
  else if (perm)
    hipLaunchKernelGGL((flash_assign_wide_kernel<DT, KB, true, true, false>), grid, block, 0, s, x, N, (int)g.D, vec_ok, f,
                       nt, assign, min_dist, perm, prev, g.K, bt);
  else if (g.lazy)
    hipLaunchKernelGGL((flash_assign_wide_kernel<DT, KB, true, false, false>), grid, block, 0, s, x, N, (int)g.D, vec_ok, f,
                       nt, assign, min_dist, perm, prev, g.K, bt);
  else
    hipLaunchKernelGGL((flash_assign_wide_kernel<DT, KB, false, false, false>), grid, block, 0, s, x, N, (int)g.D, vec_ok,
                       f, nt, assign, min_dist, perm, prev, g.K, bt);
  return hipGetLastError();
}

template <int KB>
static hipError_t launch_narrow(const AssignGeom& g, const void* X, int64_t N, const void* frag, int32_t* assign,
                                float* min_dist, int64_t B, int32_t id_mul, const SplitPlan& sp, hipStream_t s) {
  if constexpr (KB <= kNarrowHalfMaxKB) {
    const bool thin = same_cfg(g.cfg, narrow_cfg(KB, true, true));
    if (thin || same_cfg(g.cfg, narrow_cfg(KB, true))) {
      const AssignCfg cfg = g.cfg;
      const int64_t pts = (int64_t)cfg.W * cfg.NB * 16;
      const int64_t blocks = (N + pts - 1) / pts;
      if (blocks * B >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
      const bool vec_ok = (((uintptr_t)X) % 16 == 0) && ((g.D * 4) % 16 == 0);
      const dim3 grid((unsigned)(blocks * B), (unsigned)sp.S), block(cfg.W * 64);
      const Batch bt = make_batch(g, N, blocks, id_mul, sp);
      const uint8_t* x = (const uint8_t*)X;
      const u32x4_t* f = (const u32x4_t*)frag;
      const int nt = (int)g.ntiles();
      if (thin && sp.S > 1)
        hipLaunchKernelGGL((flash_assign_narrow_kernel<KB, true, true, true>), grid, block, 0, s, x, N, (int)g.D,
                           vec_ok, f, nt, assign, min_dist, bt);
      else if (thin)
        hipLaunchKernelGGL((flash_assign_narrow_kernel<KB, true, true, false>), grid, block, 0, s, x, N, (int)g.D,
                           vec_ok, f, nt, assign, min_dist, bt);
      else if (sp.S > 1)
        hipLaunchKernelGGL((flash_assign_narrow_kernel<KB, true, false, true>), grid, block, 0, s, x, N, (int)g.D,
                           vec_ok, f, nt, assign, min_dist, bt);
      else
        hipLaunchKernelGGL((flash_assign_narrow_kernel<KB, true, false, false>), grid, block, 0, s, x, N, (int)g.D,
                           vec_ok, f, nt, assign, min_dist, bt);
      return hipGetLastError();
    }
  }
  constexpr AssignCfg cfg = narrow_cfg(KB);
  if (!same_cfg(g.cfg, cfg)) return hipErrorInvalidValue;
  const int64_t pts = (int64_t)cfg.W * cfg.NB * 16;
  const int64_t blocks = (N + pts - 1) / pts;
  if (blocks * B >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const bool vec_ok = (((uintptr_t)X) % 16 == 0) && ((g.D * 4) % 16 == 0);
  const dim3 grid((unsigned)(blocks * B), (unsigned)sp.S), block(cfg.W * 64);
  const Batch bt = make_batch(g, N, blocks, id_mul, sp);
  if (sp.S > 1)
    hipLaunchKernelGGL((flash_assign_narrow_kernel<KB, false, false, true>), grid, block, 0, s, (const uint8_t*)X, N,
                       (int)g.D, vec_ok, (const u32x4_t*)frag, (int)g.ntiles(), assign, min_dist, bt);
  else
    hipLaunchKernelGGL((flash_assign_narrow_kernel<KB, false, false, false>), grid, block, 0, s, (const uint8_t*)X, N,
                       (int)g.D, vec_ok, (const u32x4_t*)frag, (int)g.ntiles(), assign, min_dist, bt);
  return hipGetLastError();
}

template <int DT>
static hipError_t dispatch_wide(const AssignGeom& g, const void* X, int64_t N, const void* frag, int32_t* assign,
                                float* min_dist, const int32_t* perm, const int32_t* prev, int64_t B, int32_t id_mul,
                                const SplitPlan& sp, hipStream_t s) {
  switch (g.cfg.KB) {
#define KM_CASE(n) \
  case n: return launch_wide<DT, n>(g, X, N, frag, assign, min_dist, perm, prev, B, id_mul, sp, s);
    KM_CASE(1) KM_CASE(2) KM_CASE(3) KM_CASE(4) KM_CASE(5) KM_CASE(6) KM_CASE(7) KM_CASE(8)
    KM_CASE(10) KM_CASE(12) KM_CASE(14) KM_CASE(16) KM_CASE(20) KM_CASE(24) KM_CASE(28) KM_CASE(32)
#undef KM_CASE
    default: return hipErrorInvalidValue;
  }
}

static hipError_t launch_sweep(const AssignGeom& g, const void* X, int64_t N, const void* frag, int32_t* assign,
                               float* min_dist, hipStream_t stream, const int32_t* perm, const int32_t* prev,
                               int64_t B, int32_t id_mul, const SplitPlan& sp) {
  if (is_deep_cfg(g.dt, g.cfg)) {  // (cold order: the warm start only reorders work)
    switch (g.dt) {
      case DT_BF16: return launch_deep<DT_BF16>(g, X, N, frag, assign, min_dist, B, id_mul, sp, stream);
      case DT_F16: return launch_deep<DT_F16>(g, X, N, frag, assign, min_dist, B, id_mul, sp, stream);
      case DT_F32: return launch_deep<DT_F32>(g, X, N, frag, assign, min_dist, B, id_mul, sp, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (g.dt) {
    case DT_BF16: return dispatch_wide<DT_BF16>(g, X, N, frag, assign, min_dist, perm, prev, B, id_mul, sp, stream);
    case DT_F16: return dispatch_wide<DT_F16>(g, X, N, frag, assign, min_dist, perm, prev, B, id_mul, sp, stream);
    case DT_F32:
      switch (g.cfg.KB) {
#define KM_CASE(n) \
  case n: return launch_narrow<n>(g, X, N, frag, assign, min_dist, B, id_mul, sp, stream);
        KM_CASE(1) KM_CASE(2) KM_CASE(3) KM_CASE(4) KM_CASE(5) KM_CASE(6) KM_CASE(7) KM_CASE(8)
        KM_CASE(9) KM_CASE(10) KM_CASE(11) KM_CASE(12) KM_CASE(13) KM_CASE(14) KM_CASE(15) KM_CASE(16)
#undef KM_CASE
        default: return hipErrorInvalidValue;
      }
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_flash_assign(const AssignGeom& g, const void* X, int64_t N, const void* frag, int32_t* assign,
                               float* min_dist, hipStream_t stream, const int32_t* perm, const int32_t* prev,
                               int64_t B, int32_t id_mul, void* split_ws) {
  if (N == 0) return hipSuccess;
  if ((perm == nullptr) != (prev == nullptr)) return hipErrorInvalidValue;
  if (B < 1 || (perm && B != 1)) return hipErrorInvalidValue;  // the warm order is per problem
  SplitPlan sp;
  const int64_t st = split_ws ? assign_split_tiles(g, N, B) : 0;
  if (st == 0) return launch_sweep(g, X, N, frag, assign, min_dist, stream, perm, prev, B, id_mul, sp);
  // Split sweep: every range of every row block writes its best to the
  // scratch, then one pass merges the ranges.  (The warm start only reorders
  // the work; it is not used here.)
  if ((uintptr_t)split_ws % 16 != 0) return hipErrorInvalidValue;
  const int64_t total = B * N;
  sp.S = (g.ntiles() + st - 1) / st;
  sp.tiles = (int32_t)st;
  sp.stride = total;
  sp.s = (float*)split_ws;
  sp.k = (int32_t*)(sp.s + sp.S * total);
  sp.xn = min_dist ? (float*)(sp.k + sp.S * total) : nullptr;
  hipError_t e = launch_sweep(g, X, N, frag, assign, nullptr, stream, nullptr, nullptr, B, id_mul, sp);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(assign_merge_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, sp.s, sp.k,
                     sp.xn, total, N, (int)sp.S, id_mul, assign, min_dist);
  return hipGetLastError();
}

}  // namespace km
