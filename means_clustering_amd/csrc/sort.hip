// Explicit inverse map of Sort-Inverse Update: a stable LSD radix argsort of
// the assignment vector, and the cluster segment boundaries of the result.
//
// Citations name the page "Flash-KMeans: Fast and Memory-Efficient Exact
// K-Means" (gist.science summary of paper 2603.09229); "tech §n" is a section
// of its technical summary.
//
// tech §2.2 sorts the assignment vector (argsort) so that the points of each
// cluster become contiguous; the update then reduces contiguous segments
// instead of scattering.  Here the sort is an LSD radix sort over the bits of
// the largest cluster id, at most 8 bits a pass, passes of balanced width.
// Nothing in it uses a global atomic, so a hot cluster (many points with one
// id) costs no contention: inside a wavefront, lanes with equal digits are
// found with ballots, the lowest such lane (the "leader") advances the wave's
// private LDS counter for that digit once for the whole group, and per-block
// digit counts become global destinations through an exclusive scan.  Every
// step is a deterministic function of the input, and equal ids keep ascending
// point order (stable), which fixes the summation order of the update.
#include "km_internal.hpp"

namespace km {

constexpr int kSortWaves = kSortThreads / 64;
constexpr int kRounds = kSortItems;  // a wave handles kRounds x 64 consecutive keys

// Lanes of this wavefront whose `bits`-bit digit equals this lane's (active lanes only).
__device__ __forceinline__ uint64_t match_digit(uint32_t d, int bits, bool active) {
  uint64_t m = __ballot(active);
  for (int b = 0; b < bits; ++b) {
    const bool bit = (d >> b) & 1u;
    const uint64_t v = __ballot(active && bit);
    m &= bit ? v : ~v;
  }
  return m;
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Key and value of sorted-input position pos for this pass.  Pass 0 reads the
// caller's assignment vector: ids outside [0, K) become K-1 with the invalid
// flag in the value, and the value is the point index itself.
__device__ __forceinline__ void load_kv(const int32_t* __restrict__ keys, const int32_t* __restrict__ vals,
                                        bool first, int64_t pos, int64_t K, int32_t& key, int32_t& val) {
  key = keys[pos];
  if (first) {
    val = (int32_t)pos;
    if ((uint32_t)key >= (uint32_t)K) {
      key = (int32_t)(K - 1);
      val = (int32_t)((uint32_t)pos | kInvalidFlag);
    }
  } else {
    val = vals[pos];
  }
}

// Per-block digit counts: counts[d * nblk + b].
__global__ __launch_bounds__(kSortThreads) void radix_count_kernel(const int32_t* __restrict__ keys, int64_t N,
                                                                   int64_t K, int first, int shift, int bits,
                                                                   int64_t nblk, uint32_t* __restrict__ counts) {
  __shared__ uint32_t cnt[kSortWaves][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int R = 1 << bits;
  for (int i = threadIdx.x; i < kSortWaves * 256; i += kSortThreads) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const int64_t b = blockIdx.x;
  const int64_t base = b * kSortBlock + (int64_t)wave * (kRounds * 64);
  for (int r = 0; r < kRounds; ++r) {
    const int64_t pos = base + r * 64 + lane;
    const bool active = pos < N;
    uint32_t d = 0;
    if (active) {
      int32_t key = keys[pos];
      if (first && (uint32_t)key >= (uint32_t)K) key = (int32_t)(K - 1);
      d = ((uint32_t)key >> shift) & (uint32_t)(R - 1);
    }
    const uint64_t m = match_digit(d, bits, active);
    if (active && lanes_below(m) == 0) cnt[wave][d] += (uint32_t)__popcll(m);  // one leader per digit
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  for (int d = threadIdx.x; d < R; d += kSortThreads) {
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) s += cnt[w][d];
    counts[(int64_t)d * nblk + b] = s;
  }
}

// Stable scatter: destination = scanned block base + earlier waves + rank in wave.
__global__ __launch_bounds__(kSortThreads) void radix_scatter_kernel(const int32_t* __restrict__ keys_in,
                                                                     const int32_t* __restrict__ vals_in, int64_t N,
                                                                     int64_t K, int first, int shift, int bits,
                                                                     int64_t nblk,
                                                                     const uint32_t* __restrict__ offsets,
                                                                     int32_t* __restrict__ keys_out,
                                                                     int32_t* __restrict__ vals_out) {
  __shared__ uint32_t cnt[kSortWaves][256];
  __shared__ uint32_t gbase[256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int R = 1 << bits;
  for (int i = threadIdx.x; i < kSortWaves * 256; i += kSortThreads) (&cnt[0][0])[i] = 0;
  const int64_t b = blockIdx.x;
  for (int d = threadIdx.x; d < R; d += kSortThreads) gbase[d] = offsets[(int64_t)d * nblk + b];
  __syncthreads();

  const int64_t base = b * kSortBlock + (int64_t)wave * (kRounds * 64);
  int32_t key[kRounds], val[kRounds];
  uint32_t rank[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int64_t pos = base + r * 64 + lane;
    const bool active = pos < N;
    key[r] = 0;
    val[r] = 0;
    uint32_t d = 0;
    if (active) {
      load_kv(keys_in, vals_in, first, pos, K, key[r], val[r]);
      d = ((uint32_t)key[r] >> shift) & (uint32_t)(R - 1);
    }
    const uint64_t m = match_digit(d, bits, active);
    const uint32_t below = lanes_below(m);
    uint32_t before = 0;
    if (active) before = cnt[wave][d];
    __builtin_amdgcn_wave_barrier();
    if (active && below == 0) cnt[wave][d] = before + (uint32_t)__popcll(m);
    __builtin_amdgcn_wave_barrier();
    rank[r] = before + below;
  }
  __syncthreads();
  // exclusive prefix over waves for every digit, plus the block's global base
  for (int d = threadIdx.x; d < R; d += kSortThreads) {
    uint32_t run = gbase[d];
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) {
      const uint32_t c = cnt[w][d];
      cnt[w][d] = run;
      run += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int64_t pos = base + r * 64 + lane;
    if (pos < N) {
      const uint32_t d = ((uint32_t)key[r] >> shift) & (uint32_t)(R - 1);
      const uint32_t dst = cnt[wave][d] + rank[r];
      if (dst < (uint64_t)N) {  // always true for a consistent scan; keeps any inconsistency in bounds
        keys_out[dst] = key[r];
        vals_out[dst] = val[r];
      }
    }
  }
}

// ------------------------------------------------------------------- scan --

constexpr int kScanThreads = 1024;
constexpr int kScanItems = 16;
constexpr int64_t kScanTile = (int64_t)kScanThreads * kScanItems;

// Exclusive scan of v[] across the block (each thread holds kScanItems
// consecutive values); returns the block total.
__device__ uint32_t block_exclusive_scan(uint32_t (&v)[kScanItems], uint32_t carry, uint32_t* lds_waves) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) {
    const uint32_t t = v[i];
    v[i] = s;
    s += t;
  }
  uint32_t x = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) lds_waves[wave] = x;
  __syncthreads();
  if (wave == 0) {
    constexpr int NW = kScanThreads / 64;
    uint32_t w = lane < NW ? lds_waves[lane] : 0;
    uint32_t z = w;
#pragma unroll
    for (int off = 1; off < NW; off <<= 1) {
      const uint32_t y = __shfl_up(z, off);
      if (lane >= off) z += y;
    }
    if (lane < NW) lds_waves[NW + lane] = z - w;  // exclusive wave prefix
    if (lane == NW - 1) lds_waves[2 * NW] = z;    // block total
  }
  __syncthreads();
  const uint32_t pre = carry + lds_waves[kScanThreads / 64 + wave] + (x - s);
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) v[i] += pre;
  const uint32_t total = lds_waves[2 * (kScanThreads / 64)];
  __syncthreads();
  return total;
}

// Sum of each tile of kScanTile values.
__global__ __launch_bounds__(kScanThreads) void scan_reduce_kernel(const uint32_t* __restrict__ a, int64_t n,
                                                                   uint32_t* __restrict__ part) {
  __shared__ uint32_t lds[2 * (kScanThreads / 64) + 1];
  uint32_t v[kScanItems];
  const int64_t base = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kScanItems;
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) v[i] = base + i < n ? a[base + i] : 0u;
  const uint32_t total = block_exclusive_scan(v, 0u, lds);
  if (threadIdx.x == 0) part[blockIdx.x] = total;
}

// In-place exclusive scan of a[0..n) by one block, tile after tile with a carry.
__global__ __launch_bounds__(kScanThreads) void scan_single_kernel(uint32_t* __restrict__ a, int64_t n) {
  __shared__ uint32_t lds[2 * (kScanThreads / 64) + 1];
  uint32_t carry = 0;
  for (int64_t t0 = 0; t0 < n; t0 += kScanTile) {
    uint32_t v[kScanItems];
    const int64_t base = t0 + (int64_t)threadIdx.x * kScanItems;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) v[i] = base + i < n ? a[base + i] : 0u;
    const uint32_t total = block_exclusive_scan(v, carry, lds);
#pragma unroll
    for (int i = 0; i < kScanItems; ++i)
      if (base + i < n) a[base + i] = v[i];
    carry += total;
  }
}

// In-place exclusive scan of each tile, offset by the scanned tile sums.
__global__ __launch_bounds__(kScanThreads) void scan_apply_kernel(uint32_t* __restrict__ a, int64_t n,
                                                                  const uint32_t* __restrict__ part) {
  __shared__ uint32_t lds[2 * (kScanThreads / 64) + 1];
  uint32_t v[kScanItems];
  const int64_t base = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kScanItems;
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) v[i] = base + i < n ? a[base + i] : 0u;
  block_exclusive_scan(v, part[blockIdx.x], lds);
#pragma unroll
  for (int i = 0; i < kScanItems; ++i)
    if (base + i < n) a[base + i] = v[i];
}

static hipError_t launch_scan(uint32_t* a, int64_t n, uint32_t* part, hipStream_t s) {
  if (n <= 4 * kScanTile) {
    hipLaunchKernelGGL(scan_single_kernel, dim3(1), dim3(kScanThreads), 0, s, a, n);
    return hipGetLastError();
  }
  const int64_t tiles = (n + kScanTile - 1) / kScanTile;
  hipLaunchKernelGGL(scan_reduce_kernel, dim3((unsigned)tiles), dim3(kScanThreads), 0, s, (const uint32_t*)a, n,
                     part);
  hipLaunchKernelGGL(scan_single_kernel, dim3(1), dim3(kScanThreads), 0, s, part, tiles);
  hipLaunchKernelGGL(scan_apply_kernel, dim3((unsigned)tiles), dim3(kScanThreads), 0, s, a, n,
                     (const uint32_t*)part);
  return hipGetLastError();
}

int64_t scan_part_len(int64_t n) { return (n + kScanTile - 1) / kScanTile + 1; }

hipError_t launch_argsort(const SortGeom& g, const int32_t* keys_in, int32_t* key_a, int32_t* val_a,
                          int32_t* key_b, int32_t* val_b, int32_t* key_final, int32_t* val_final, uint32_t* counts,
                          uint32_t* scan_part, hipStream_t stream) {
  if (g.N == 0) return hipSuccess;
  const int32_t* kin = keys_in;
  const int32_t* vin = nullptr;
  int shift = 0;
  for (int p = 0; p < g.npass; ++p) {
    const int bits = g.bits[p];
    const int first = p == 0;
    const bool last = p == g.npass - 1;
    int32_t* kout = last ? key_final : (p % 2 == 0 ? key_a : key_b);
    int32_t* vout = last ? val_final : (p % 2 == 0 ? val_a : val_b);
    hipLaunchKernelGGL(radix_count_kernel, dim3((unsigned)g.nblk), dim3(kSortThreads), 0, stream, kin, g.N, g.K,
                       first, shift, bits, g.nblk, counts);
    hipError_t e = launch_scan(counts, ((int64_t)1 << bits) * g.nblk, scan_part, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(radix_scatter_kernel, dim3((unsigned)g.nblk), dim3(kSortThreads), 0, stream, kin, vin, g.N,
                       g.K, first, shift, bits, g.nblk, (const uint32_t*)counts, kout, vout);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    kin = kout;
    vin = vout;
    shift += bits;
  }
  return hipSuccess;
}

// --------------------------------------------------------------- segments --

// off[k] for every k in (key[i-1], key[i]] is i; key[-1] = -1, key[N] = K.
__global__ void boundaries_kernel(const int32_t* __restrict__ keys, int64_t N, int64_t K, int32_t* __restrict__ off) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i > N) return;
  int64_t prev = i == 0 ? -1 : (int64_t)keys[i - 1];
  int64_t cur = i == N ? K : (int64_t)keys[i];
  prev = prev < -1 ? -1 : (prev > K ? K : prev);  // sorted ids lie in [0, K); clamping keeps writes in bounds
  cur = cur < -1 ? -1 : (cur > K ? K : cur);
  for (int64_t k = prev + 1; k <= cur; ++k) off[k] = (int32_t)i;
}

hipError_t launch_boundaries(const int32_t* sorted_keys, int64_t N, int64_t K, int32_t* off, hipStream_t stream) {
  const int tpb = 256;
  hipLaunchKernelGGL(boundaries_kernel, dim3((unsigned)((N + 1 + tpb - 1) / tpb)), dim3(tpb), 0, stream, sorted_keys,
                     N, K, off);
  return hipGetLastError();
}

}  // namespace km
