// gen_gpu.hip -- the synthetic mixture generator of gen.c, run on the GPU.
//
// Holds none of the clustering arithmetic: it only draws points.  Same
// definition as the host generator (Philox4x32-10 of Salmon et al., SC'11,
// keyed by (seed, stream tag, index); 53-bit uniforms; Box-Muller normals in
// fp64; fp64 -> fp32 -> bf16 round-to-nearest-even), written again here for
// the device so that a billion-row dataset takes seconds instead of minutes.
// Built with -ffp-contract=off so every fp64 operation rounds exactly as in the
// host version; the only possible difference is the last bit of the device
// log/cos/sin, which survives the two roundings to 16 bits with negligible
// probability (a GPU test compares both generators bit for bit).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;  // Philox4x32 multipliers
constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;  // Weyl key increments
constexpr uint32_t kTagPoint = 0x504f494eu, kTagComp = 0x434f4d50u;

struct U4 {
  uint32_t v[4];
};

__device__ __forceinline__ U4 philox(uint64_t seed, uint32_t tag, uint64_t i, uint32_t j) {
  uint32_t c0 = (uint32_t)i, c1 = (uint32_t)(i >> 32), c2 = j, c3 = tag;
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32) ^ tag;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t hi0 = __umulhi(kM0, c0), lo0 = kM0 * c0;
    const uint32_t hi1 = __umulhi(kM1, c2), lo1 = kM1 * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += kW0;
    k1 += kW1;
  }
  return U4{{c0, c1, c2, c3}};
}

__device__ __forceinline__ double u53(uint32_t a, uint32_t b) {
  const uint64_t m = ((uint64_t)(a >> 5) << 26) | (uint64_t)(b >> 6);
  return ((double)m + 0.5) * (1.0 / 9007199254740992.0);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// One thread per row; D <= 512.
__global__ __launch_bounds__(256) void points_kernel(uint64_t seed, const double* __restrict__ centers, int64_t M,
                                                     int D, int kind, double sigma, const double* __restrict__ cdf,
                                                     int out_dtype, void* __restrict__ out, int64_t row0,
                                                     int64_t nrows, int32_t* __restrict__ comp_out) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= nrows) return;
  const uint64_t i = (uint64_t)(row0 + r);
  const U4 cr = philox(seed, kTagComp, i, 0);
  int64_t m;
  if (!cdf) {
    const uint64_t bits = ((uint64_t)cr.v[0] << 32) | cr.v[1];
    m = (int64_t)__umul64hi(bits, (uint64_t)M);
  } else {
    const double u = u53(cr.v[0], cr.v[1]);
    int64_t lo = 0, hi = M - 1;
    while (lo < hi) {
      const int64_t mid = (lo + hi) / 2;
      if (u < cdf[mid]) hi = mid;
      else lo = mid + 1;
    }
    m = lo;
  }
  if (comp_out) comp_out[r] = (int32_t)m;
  const double* c = centers + m * D;
  double inv = 1.0;
  if (kind == 1) {  // first pass: the squared norm, in the same order as the host
    double s = 0.0;
    for (int j = 0; j < D; j += 2) {
      const U4 b = philox(seed, kTagPoint, i, (uint32_t)(j >> 1));
      const double u1 = u53(b.v[0], b.v[1]), u2 = u53(b.v[2], b.v[3]);
      const double rad = sqrt(-2.0 * log(u1));
      const double th = 6.283185307179586 * u2;
      const double x0 = c[j] + sigma * (rad * cos(th));
      s += x0 * x0;
      if (j + 1 < D) {
        const double x1 = c[j + 1] + sigma * (rad * sin(th));
        s += x1 * x1;
      }
    }
    inv = 1.0 / sqrt(s);
  }
  for (int j = 0; j < D; j += 2) {
    const U4 b = philox(seed, kTagPoint, i, (uint32_t)(j >> 1));
    const double u1 = u53(b.v[0], b.v[1]), u2 = u53(b.v[2], b.v[3]);
    const double rad = sqrt(-2.0 * log(u1));
    const double th = 6.283185307179586 * u2;
    double x0 = c[j] + sigma * (rad * cos(th));
    double x1 = (j + 1 < D) ? c[j + 1] + sigma * (rad * sin(th)) : 0.0;
    if (kind == 1) {
      x0 *= inv;
      x1 *= inv;
    }
    if (out_dtype == 0) {
      float* o = (float*)out + r * D;
      o[j] = (float)x0;
      if (j + 1 < D) o[j + 1] = (float)x1;
    } else {
      uint16_t* o = (uint16_t*)out + r * D;
      o[j] = bf16_rne((float)x0);
      if (j + 1 < D) o[j + 1] = bf16_rne((float)x1);
    }
  }
}

}  // namespace

// Rows [row0, row0 + nrows) of the mixture into device memory `out` (same
// contract as synth_points in gen.c; centers and cdf are device arrays).
// Returns 0, -1 for a bad argument, or the HIP error of the launch.
extern "C" int synth_points_device(uint64_t seed, const double* centers, int64_t M, int64_t D, int kind,
                                   double sigma, const double* cdf, int out_dtype, void* out, int64_t row0,
                                   int64_t nrows, int32_t* comp_out, void* stream) {
  if ((out_dtype != 0 && out_dtype != 1) || D < 1 || D > 512 || M < 1 || nrows < 0 || row0 < 0) return -1;
  if (nrows == 0) return 0;
  const int64_t blocks = (nrows + 255) / 256;
  hipLaunchKernelGGL(points_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, (uint64_t)seed,
                     centers, M, (int)D, kind, sigma, cdf, out_dtype, out, row0, nrows, comp_out);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;
}
