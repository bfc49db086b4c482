// Same-run peak probes for the roofline denominators: the sustained matrix-core
// rate of the MFMA shape FlashAssign uses, device memory copy and read
// bandwidth, and LDS read bandwidth per compute unit.
// Not part of the clustering path; the benchmark reports these next to the
// datasheet peaks, because on a power-limited part the sustained matrix-core
// rate with real-valued operands sits well below the datasheet figure.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;  // independent accumulators per wavefront

// Pseudo-random 16-bit values in [-1, 1) from a 32-bit integer hash (operands
// with real bit activity: zero operands draw less power and run faster).
__device__ __forceinline__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

template <bool BF16>
__device__ __forceinline__ uint32_t rand_pair(uint32_t seed) {
  const uint32_t h = hash32(seed);
  // exponent 126 or 127 (|x| in [0.5, 2)), random sign and mantissa
  const uint32_t lo = BF16 ? (0x3f00u | (h & 0x807fu)) : (0x3800u | (h & 0x83ffu));
  const uint32_t hi = BF16 ? (0x3f00u | ((h >> 16) & 0x807fu)) : (0x3800u | ((h >> 16) & 0x83ffu));
  return lo | (hi << 16);
}

template <bool BF16>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int reps, float* __restrict__ out) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  u32x4_t a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = u32x4_t{rand_pair<BF16>(t * 32 + i * 8), rand_pair<BF16>(t * 32 + i * 8 + 1),
                   rand_pair<BF16>(t * 32 + i * 8 + 2), rand_pair<BF16>(t * 32 + i * 8 + 3)};
    b[i] = u32x4_t{rand_pair<BF16>(t * 32 + i * 8 + 4), rand_pair<BF16>(t * 32 + i * 8 + 5),
                   rand_pair<BF16>(t * 32 + i * 8 + 6), rand_pair<BF16>(t * 32 + i * 8 + 7)};
  }
  f32x16_t acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16_t{};
  for (int r = 0; r < reps; ++r) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < kChains; ++c) {
        if constexpr (BF16)
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[(i + c) & 3]),
                                                           __builtin_bit_cast(bf16x8_t, b[i]), acc[c], 0, 0, 0);
        else
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a[(i + c) & 3]),
                                                          __builtin_bit_cast(f16x8_t, b[i]), acc[c], 0, 0, 0);
      }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][threadIdx.x & 15];
  out[t] = s;
}

// Four 16-byte vectors in flight per thread: consecutive wavefront-wide 1 KiB pieces.
__global__ __launch_bounds__(256) void copy_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                   int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256 * 4;
  for (int64_t i0 = (int64_t)blockIdx.x * 1024 + threadIdx.x; i0 < n; i0 += stride) {
    u32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i0 + u * 256 < n) v[u] = src[i0 + u * 256];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i0 + u * 256 < n) dst[i0 + u * 256] = v[u];
  }
}

__global__ __launch_bounds__(256) void read_kernel(const u32x4_t* __restrict__ src, int64_t n,
                                                   uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * 256 * 4;
  uint32_t x = 0;
  for (int64_t i0 = (int64_t)blockIdx.x * 1024 + threadIdx.x; i0 < n; i0 += stride) {
    u32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = i0 + u * 256 < n ? src[i0 + u * 256] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 4; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = x;
}

// LDS reads: every lane reads 16 bytes a step, consecutive lanes on
// consecutive addresses (no bank conflicts; `stride` 256 slots between a
// lane's steps), eight reads in flight, from a 64 KiB buffer; each wavefront
// records the shader clocks its loop took.
__global__ __launch_bounds__(256) void lds_read_kernel(int iters, int stride, int64_t* __restrict__ clocks,
                                                       u32x4_t* __restrict__ out) {
  __shared__ u32x4_t buf[4096];
  const int t = threadIdx.x;
  for (int i = t; i < 4096; i += 256) buf[i] = u32x4_t{(uint32_t)i, (uint32_t)i * 3u, (uint32_t)i * 5u, (uint32_t)i * 7u};
  __syncthreads();
  const int lane = t & 63, wave = t >> 6;
  const int base = (wave * 64 + lane) & 4095;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  const int64_t c0 = clock64();
  for (int i = 0; i < iters; i += 8) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = buf[(base + (i + u) * stride) & 4095];
    acc += (v[0] + v[1]) + (v[2] + v[3]) + (v[4] + v[5]) + (v[6] + v[7]);
    // the addresses repeat and nothing writes the buffer in the loop: keep the
    // compiler from reusing earlier loads instead of reading LDS again
    __asm__ volatile("" ::: "memory");
  }
  const int64_t c1 = clock64();
  if (lane == 0) clocks[blockIdx.x * 4 + wave] = c1 - c0;
  out[blockIdx.x * 256 + t] = acc;
}

}  // namespace

extern "C" {

// Sustained dense rate of v_mfma_f32_32x32x16_{bf16,f16} (fp32 accumulation)
// with pseudo-random operands: `blocks` workgroups of 4 wavefronts, each
// wavefront running 8 independent accumulator chains for `reps` x 32 MFMAs.
// `scratch` holds blocks * 256 floats (device).  Returns 0 and the rate in
// TFLOP/s, or the HIP error code.  Synchronous.
int km_peak_mfma(int bf16, int blocks, int reps, float* scratch, double* tflops) {
  if (blocks < 1 || reps < 1 || !scratch || !tflops) return (int)hipErrorInvalidValue;
  hipEvent_t e0, e1;
  hipError_t e = hipEventCreate(&e0);
  if (e != hipSuccess) return (int)e;
  if ((e = hipEventCreate(&e1)) != hipSuccess) return (int)e;
  auto launch = [&](int r) {
    if (bf16)
      hipLaunchKernelGGL(mfma_loop_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, 0, r, scratch);
    else
      hipLaunchKernelGGL(mfma_loop_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, 0, r, scratch);
  };
  launch(4);  // warm-up
  hipEventRecord(e0, 0);
  launch(reps);
  hipEventRecord(e1, 0);
  e = hipEventSynchronize(e1);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (e != hipSuccess) return (int)e;
  const double flops = (double)blocks * 4.0 * reps * 4.0 * kChains * 2.0 * 32 * 32 * 16;
  *tflops = flops / (ms * 1e-3) / 1e12;
  return 0;
}

// Device-to-device copy of `bytes` (a multiple of 16, 16-byte aligned
// pointers) repeated `reps` times; returns bytes read + written per second in
// GB/s.  Synchronous.
int km_peak_copy(const void* src, void* dst, int64_t bytes, int reps, double* gbps) {
  if (!src || !dst || bytes <= 0 || bytes % 16 || reps < 1 || !gbps) return (int)hipErrorInvalidValue;
  const int64_t n = bytes / 16;
  hipEvent_t e0, e1;
  hipError_t e = hipEventCreate(&e0);
  if (e != hipSuccess) return (int)e;
  if ((e = hipEventCreate(&e1)) != hipSuccess) return (int)e;
  const unsigned grid = 4096;
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, 0, (const u32x4_t*)src, (u32x4_t*)dst, n);
  hipEventRecord(e0, 0);
  for (int r = 0; r < reps; ++r)
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, 0, (const u32x4_t*)src, (u32x4_t*)dst, n);
  hipEventRecord(e1, 0);
  e = hipEventSynchronize(e1);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (e != hipSuccess) return (int)e;
  *gbps = 2.0 * (double)bytes * reps / (ms * 1e-3) / 1e9;
  return 0;
}

// Streaming read of `bytes` (multiple of 16, 16-byte aligned) repeated `reps`
// times; `scratch` holds 256 * 4096 uint32 (device).  Returns bytes read per
// second in GB/s.  Synchronous.
int km_peak_read(const void* src, int64_t bytes, int reps, void* scratch, double* gbps) {
  if (!src || !scratch || bytes <= 0 || bytes % 16 || reps < 1 || !gbps) return (int)hipErrorInvalidValue;
  const int64_t n = bytes / 16;
  hipEvent_t e0, e1;
  hipError_t e = hipEventCreate(&e0);
  if (e != hipSuccess) return (int)e;
  if ((e = hipEventCreate(&e1)) != hipSuccess) return (int)e;
  const unsigned grid = 4096;
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, 0, (const u32x4_t*)src, n, (uint32_t*)scratch);
  hipEventRecord(e0, 0);
  for (int r = 0; r < reps; ++r)
    hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, 0, (const u32x4_t*)src, n, (uint32_t*)scratch);
  hipEventRecord(e1, 0);
  e = hipEventSynchronize(e1);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (e != hipSuccess) return (int)e;
  *gbps = (double)bytes * reps / (ms * 1e-3) / 1e9;
  return 0;
}

// LDS read bandwidth: two workgroups of 4 wavefronts per compute unit (8
// wavefronts, 128 KiB of LDS), each wavefront reading `iters` x 1 KiB
// (`iters` a multiple of 8).  `scratch` holds 2 * cus * (4 * 8 + 256 * 16)
// bytes (device).  Returns the bytes read per shader clock per compute unit
// (from the median wavefront's clock count) and the aggregate rate in TB/s.
// Synchronous.
int km_peak_lds(int iters, void* scratch, int64_t scratch_bytes, double* bytes_per_clock_cu, double* tbps) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return (int)e;
  const int blocks = 2 * cus;
  if (iters < 8 || iters % 8 || !scratch || !bytes_per_clock_cu || !tbps ||
      scratch_bytes < (int64_t)blocks * (4 * 8 + 256 * 16))
    return (int)hipErrorInvalidValue;
  int64_t* clocks = static_cast<int64_t*>(scratch);
  u32x4_t* out = reinterpret_cast<u32x4_t*>(static_cast<char*>(scratch) + (int64_t)blocks * 4 * 8);
  hipEvent_t e0, e1;
  if ((e = hipEventCreate(&e0)) != hipSuccess) return (int)e;
  if ((e = hipEventCreate(&e1)) != hipSuccess) return (int)e;
  hipLaunchKernelGGL(lds_read_kernel, dim3((unsigned)blocks), dim3(256), 0, 0, 64, 256, clocks, out);  // warm-up
  hipEventRecord(e0, 0);
  hipLaunchKernelGGL(lds_read_kernel, dim3((unsigned)blocks), dim3(256), 0, 0, iters, 256, clocks, out);
  hipEventRecord(e1, 0);
  e = hipEventSynchronize(e1);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (e != hipSuccess) return (int)e;
  int64_t* host = new int64_t[(size_t)blocks * 4];
  e = hipMemcpy(host, clocks, sizeof(int64_t) * blocks * 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess) {
    // median by counting (blocks * 4 values)
    const int n = blocks * 4;
    int64_t med = host[0];
    for (int i = 0; i < n; ++i) {
      int below = 0, equal = 0;
      for (int j = 0; j < n; ++j) {
        below += host[j] < host[i];
        equal += host[j] == host[i];
      }
      if (below <= n / 2 && n / 2 < below + equal) {
        med = host[i];
        break;
      }
    }
    *bytes_per_clock_cu = med > 0 ? 8.0 * iters * 1024.0 / (double)med : 0.0;
    *tbps = (double)blocks * 4 * iters * 1024.0 / (ms * 1e-3) / 1e12;
  }
  delete[] host;
  return (int)e;
}

}  // extern "C"
