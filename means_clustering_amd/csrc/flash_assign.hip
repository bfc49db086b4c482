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
// Precision: 16-bit X runs on v_mfma_f32_16x16x32_{bf16,f16} (fp32
// accumulation); the fp32 centroid state is rounded to X's type once per call
// (round to nearest, ties to even) and ||c||^2 is taken from the rounded
// values, so every candidate is scored against exactly the centroid the
// contraction saw.  fp32 X runs on v_mfma_f32_16x16x4_f32.
//
// Structure (tech §2.1 "online argmin", "tiled streaming", "double buffering",
// re-designed for CDNA4):
//   * a wavefront owns NB x 16 points and keeps their operand fragments in
//     VGPRs for the whole centroid sweep (X is read from HBM exactly once);
//   * centroids stream through LDS in tiles of CT x 16, double-buffered:
//     tile t+1 is fetched from L2/HBM into registers while tile t feeds the
//     matrix cores, then stored to the other LDS buffer (one barrier a tile);
//   * each lane keeps (best score, tile-relative selector) for its points in
//     registers; the four lanes that hold the same point merge once at the
//     end, so ties resolve to the lowest centroid index.
#include <math.h>

#include "km_internal.hpp"

namespace km {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // keep NaN quiet
  u += 0x7fffu + ((u >> 16) & 1u);                                // round to nearest, ties to even
  return u >> 16;
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // IEEE conversion, round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Value of the centroid coordinate as the contraction sees it.
__device__ __forceinline__ float quantize(float c, int dt) {
  if (dt == DT_BF16) return bf16_bits_to_f32(f32_to_bf16_bits(c));
  if (dt == DT_F16) return f16_bits_to_f32(f32_to_f16_bits(c));
  return c;
}

// ---------------------------------------------------------------- prep ----

// One thread per 16-byte fragment (group g, depth block kb, lane).  Group g
// occupies KB*64 + 4 consecutive 16-byte slots: its fragments, then its 16
// bias values (written by prep_bias_kernel).
__global__ void prep_frag_kernel(const float* __restrict__ C, int64_t K, int64_t D, int dt, int KB,
                                 int64_t total, uint4* __restrict__ frag) {
  int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= total) return;
  const int lane = (int)(tid & 63);
  const int64_t t2 = tid >> 6;
  const int kb = (int)(t2 % KB);
  const int64_t g = t2 / KB;
  const int64_t CT = assign_cfg(KB).CT;
  const int64_t slot = (g / CT) * tile_slots(KB) + (g % CT) * group_slots(KB) + (int64_t)kb * 64 + lane;
  const int64_t k = g * kGroupRows + (lane & 15);
  uint32_t w[4];
  if (dt == DT_F32) {
    const int64_t d0 = (int64_t)kb * 16 + (lane >> 4) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t d = d0 + e;
      w[e] = __float_as_uint((k < K && d < D) ? C[k * D + d] : 0.0f);
    }
  } else {
    const int64_t d0 = (int64_t)kb * 32 + (lane >> 4) * 8;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t lo = 0, hi = 0;
      const int64_t da = d0 + 2 * e, db = d0 + 2 * e + 1;
      const float ca = (k < K && da < D) ? C[k * D + da] : 0.0f;
      const float cb = (k < K && db < D) ? C[k * D + db] : 0.0f;
      lo = dt == DT_BF16 ? f32_to_bf16_bits(ca) : f32_to_f16_bits(ca);
      hi = dt == DT_BF16 ? f32_to_bf16_bits(cb) : f32_to_f16_bits(cb);
      w[e] = lo | (hi << 16);
    }
  }
  frag[slot] = make_uint4(w[0], w[1], w[2], w[3]);
}

// bias_k = -||Q(c_k)||^2 / 2 in fp32 (ascending coordinate order), -inf for
// padding rows; stored after the fragments of its group, 16 floats a group.
__global__ void prep_bias_kernel(const float* __restrict__ C, int64_t K, int64_t D, int dt, int KB, int64_t Kpad,
                                 float* __restrict__ frag_f) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= Kpad) return;
  const int64_t g = k / kGroupRows;
  const int64_t CT = assign_cfg(KB).CT;
  float* dst = frag_f + ((g / CT) * tile_slots(KB) + (g % CT) * group_slots(KB) + (int64_t)KB * 64) * 4 +
               (k % kGroupRows);
  if (k >= K) {
    *dst = -INFINITY;
    return;
  }
  float s = 0.0f;
  for (int64_t d = 0; d < D; ++d) {
    const float q = quantize(C[k * D + d], dt);
    s = fmaf(q, q, s);
  }
  *dst = -0.5f * s;
}

hipError_t launch_prep(const float* C, int64_t K, int64_t D, int dt, int KB, int64_t Kpad, void* frag,
                       hipStream_t stream) {
  const int64_t total = (Kpad / kGroupRows) * KB * 64;
  const int tpb = 256;
  hipLaunchKernelGGL(prep_frag_kernel, dim3((unsigned)((total + tpb - 1) / tpb)), dim3(tpb), 0, stream, C, K, D,
                     dt, KB, total, (uint4*)frag);
  hipLaunchKernelGGL(prep_bias_kernel, dim3((unsigned)((Kpad + tpb - 1) / tpb)), dim3(tpb), 0, stream, C, K, D, dt,
                     KB, Kpad, (float*)frag);
  return hipGetLastError();
}

// ---------------------------------------------------------- FlashAssign ----

template <int DT>
struct FragTraits;
template <>
struct FragTraits<DT_BF16> {
  static constexpr int EPL = 8, FB = 32, ES = 2;
  static __device__ __forceinline__ f32x4_t mma(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  }
  static __device__ __forceinline__ float sumsq(u32x4_t v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = bf16_bits_to_f32(w[e] & 0xffffu), b = bf16_bits_to_f32(w[e] >> 16);
      s = fmaf(a, a, s);
      s = fmaf(b, b, s);
    }
    return s;
  }
};
template <>
struct FragTraits<DT_F16> {
  static constexpr int EPL = 8, FB = 32, ES = 2;
  static __device__ __forceinline__ f32x4_t mma(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
  }
  static __device__ __forceinline__ float sumsq(u32x4_t v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = f16_bits_to_f32(w[e] & 0xffffu), b = f16_bits_to_f32(w[e] >> 16);
      s = fmaf(a, a, s);
      s = fmaf(b, b, s);
    }
    return s;
  }
};
template <>
struct FragTraits<DT_F32> {
  static constexpr int EPL = 4, FB = 16, ES = 4;
  static __device__ __forceinline__ f32x4_t mma(u32x4_t a, u32x4_t b, f32x4_t c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ float sumsq(u32x4_t v) {
    const float a = __uint_as_float(v.x), b = __uint_as_float(v.y), c = __uint_as_float(v.z),
                d = __uint_as_float(v.w);
    float s = 0.0f;
    s = fmaf(a, a, s);
    s = fmaf(b, b, s);
    s = fmaf(c, c, s);
    s = fmaf(d, d, s);
    return s;
  }
};

// 16 bytes of point p, depth values [d0, d0 + EPL); zero beyond D or N.
template <int DT>
__device__ __forceinline__ u32x4_t load_point_frag(const uint8_t* __restrict__ X, int64_t p, int64_t N, int D, int d0,
                                                 bool vec_ok) {
  using T = FragTraits<DT>;
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (p >= N || d0 >= D) return v;
  const uint8_t* row = X + (size_t)p * (size_t)D * T::ES;
  if (vec_ok && d0 + T::EPL <= D) return *reinterpret_cast<const u32x4_t*>(row + (size_t)d0 * T::ES);
  uint32_t w[4] = {0, 0, 0, 0};
  if (T::ES == 4) {
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

template <int DT, int KB, int NB, int W, int CT>
__global__ __launch_bounds__(W * 64) void flash_assign_kernel(const uint8_t* __restrict__ X, int64_t N, int D,
                                                              bool vec_ok, const u32x4_t* __restrict__ frag,
                                                              int ntiles, int32_t* __restrict__ assign,
                                                              float* __restrict__ min_dist) {
  using T = FragTraits<DT>;
  constexpr int GS = (int)group_slots(KB);  // 16-byte slots per centroid group: fragments, then 16 biases
  constexpr int TS = (int)tile_slots(KB);   // slots per tile, a multiple of the thread count
  constexpr int NTHR = W * 64;
  constexpr int CPT = TS / NTHR;            // 16-byte copies per thread per tile
  static_assert(TS % NTHR == 0 && TS >= CT * GS, "tile padding");
  __shared__ u32x4_t lds[2][TS];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int quad = lane >> 4;
  const int64_t wbase = ((int64_t)blockIdx.x * W + wave) * (NB * 16);

  // Point fragments: read once from HBM, kept in VGPRs for the whole sweep.
  u32x4_t xb[NB][KB];
  float xn[NB];
#pragma unroll
  for (int g = 0; g < NB; ++g) {
    const int64_t p = wbase + g * 16 + col;
    float s = 0.0f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      xb[g][kb] = load_point_frag<DT>(X, p, N, D, kb * T::FB + quad * T::EPL, vec_ok);
      s += T::sumsq(xb[g][kb]);
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
    if (more) {  // next tile in flight while this one feeds the matrix cores
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
        for (int kb = 0; kb < KB; ++kb) acc = T::mma(a[kb], xb[g][kb], acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (acc[i] > best[g]) {  // strict: the first (lowest) index among equals stays
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

  // Merge the four lanes that hold the same point; ties go to the lower index.
#pragma unroll
  for (int g = 0; g < NB; ++g) {
    float b = best[g];
    int k = sel[g] < 0 ? INT32_MAX : (sel[g] >> 2) * kGroupRows + quad * 4 + (sel[g] & 3);
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float ob = __shfl_xor(b, off);
      const int ok = __shfl_xor(k, off);
      if (ob > b || (ob == b && ok < k)) {
        b = ob;
        k = ok;
      }
    }
    if (k == INT32_MAX) k = 0;  // no finite score (NaN input): index 0
    const int64_t p = wbase + g * 16 + col;
    if (quad == 0 && p < N) {
      assign[p] = k;
      if (min_dist) min_dist[p] = fmaxf(xn[g] - 2.0f * b, 0.0f);
    }
  }
}

template <int DT, int KB>
static hipError_t launch_fa(const void* X, int64_t N, int64_t D, const void* frag, int64_t Kpad, int32_t* assign,
                            float* min_dist, hipStream_t stream) {
  constexpr int NB = assign_cfg(KB).NB;
  constexpr int CT = assign_cfg(KB).CT;
  constexpr int W = assign_cfg(KB).W;
  const int64_t pts = (int64_t)W * NB * 16;
  const int64_t nblk = (N + pts - 1) / pts;
  const int ntiles = (int)(Kpad / (CT * kGroupRows));
  const bool vec_ok = (((uintptr_t)X) % 16 == 0) && ((D * FragTraits<DT>::ES) % 16 == 0);
  hipLaunchKernelGGL((flash_assign_kernel<DT, KB, NB, W, CT>), dim3((unsigned)nblk), dim3(W * 64), 0, stream,
                     (const uint8_t*)X, N, (int)D, vec_ok, (const u32x4_t*)frag, ntiles, assign, min_dist);
  return hipGetLastError();
}

template <int DT>
static hipError_t dispatch_kb(int KB, const void* X, int64_t N, int64_t D, const void* frag, int64_t Kpad,
                              int32_t* assign, float* min_dist, hipStream_t s) {
  switch (KB) {
#define KM_CASE(n) \
  case n: return launch_fa<DT, n>(X, N, D, frag, Kpad, assign, min_dist, s);
    KM_CASE(1) KM_CASE(2) KM_CASE(3) KM_CASE(4) KM_CASE(5) KM_CASE(6) KM_CASE(7) KM_CASE(8)
    KM_CASE(9) KM_CASE(10) KM_CASE(11) KM_CASE(12) KM_CASE(13) KM_CASE(14) KM_CASE(15) KM_CASE(16)
#undef KM_CASE
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_flash_assign(const void* X, int dt, int64_t N, int64_t D, int KB, const void* frag,
                               int64_t Kpad, int32_t* assign, float* min_dist, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  switch (dt) {
    case DT_BF16: return dispatch_kb<DT_BF16>(KB, X, N, D, frag, Kpad, assign, min_dist, stream);
    case DT_F16: return dispatch_kb<DT_F16>(KB, X, N, D, frag, Kpad, assign, min_dist, stream);
    case DT_F32: return dispatch_kb<DT_F32>(KB, X, N, D, frag, Kpad, assign, min_dist, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace km
