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
// the largest cluster id, at most 6 bits a pass, passes of balanced width.
// No global atomic anywhere, so a hot cluster (many points with one id) costs
// no contention in memory.  Per pass: a count of each block's digits (an LDS
// histogram per wavefront), the exclusive scan of those counts over (digit,
// block) (small tables: summed by every scatter workgroup itself; larger
// ones: each digit's row scanned by one workgroup, the scatter adding the
// totals of the smaller digits), and the scatter.  Ranking inside a block of 256 x IT keys (IT = 8, 16 or 32 by N):
// every thread owns IT consecutive keys and a private 16-bit counter per
// digit in LDS; counting its own keys in order gives each key its rank among
// the thread's keys of that digit, and one exclusive scan over the counters in
// (digit, thread) order turns them into block-wide ranks that keep the input
// order of equal digits (stable).  Every step is a deterministic function of
// the input, which fixes the summation order of the update.
#include "block_rank.hpp"
#include "km_internal.hpp"

namespace km {

// Keys (and values) of this thread: IT consecutive positions.
// Pass 0 reads the caller's assignment vector: ids outside [0, K) become K-1
// with the invalid flag in the value, and the value is the point index itself.
template <int IT>
__device__ __forceinline__ void load_block_keys(const int32_t* __restrict__ keys, const int32_t* __restrict__ vals,
                                                bool first, int64_t N, int64_t K, int64_t base,
                                                int32_t (&key)[IT], int32_t (&val)[IT],
                                                bool (&valid)[IT], bool want_vals) {
  const int64_t p0 = base + (int64_t)threadIdx.x * IT;
  if (p0 + IT <= N && ((reinterpret_cast<uintptr_t>(keys + p0) & 15) == 0)) {
    const int4* k4 = reinterpret_cast<const int4*>(keys + p0);
#pragma unroll
    for (int i = 0; i < IT / 4; ++i) {
      const int4 v = k4[i];
      key[4 * i] = v.x;
      key[4 * i + 1] = v.y;
      key[4 * i + 2] = v.z;
      key[4 * i + 3] = v.w;
    }
    if (want_vals && !first) {
      const int4* v4 = reinterpret_cast<const int4*>(vals + p0);
#pragma unroll
      for (int i = 0; i < IT / 4; ++i) {
        const int4 v = v4[i];
        val[4 * i] = v.x;
        val[4 * i + 1] = v.y;
        val[4 * i + 2] = v.z;
        val[4 * i + 3] = v.w;
      }
    }
#pragma unroll
    for (int i = 0; i < IT; ++i) valid[i] = true;
  } else {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int64_t pos = p0 + i;
      valid[i] = pos < N;
      key[i] = valid[i] ? keys[pos] : 0;
      if (want_vals && !first) val[i] = valid[i] ? vals[pos] : 0;
    }
  }
  if (first) {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int64_t pos = p0 + i;
      val[i] = (int32_t)pos;
      if ((uint32_t)key[i] >= (uint32_t)K) {
        key[i] = (int32_t)(K - 1);
        val[i] = (int32_t)((uint32_t)pos | kInvalidFlag);
      }
    }
  }
}

// Per-block digit counts: counts[d * nblk + b].  A histogram in LDS, one per
// wavefront (integer additions, so the order of the atomics does not matter,
// and a hot digit contends within one wavefront only).
template <int BITS, int IT>
__global__ __launch_bounds__(kRadixThreads) void radix_count_kernel(const int32_t* __restrict__ keys, int64_t N,
                                                                    int64_t K, int first, int shift, int64_t nblk,
                                                                    uint32_t* __restrict__ counts) {
  constexpr int R = 1 << BITS;
  constexpr int NW = kRadixThreads / 64;
  __shared__ uint32_t hist[NW][R];
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < NW * R; i += kRadixThreads) hist[i / R][i % R] = 0u;
  __syncthreads();
  const int64_t b = blockIdx.x;
  int32_t key[IT], val[IT];
  bool valid[IT];
  load_block_keys<IT>(keys, nullptr, first, N, K, b * (kRadixThreads * IT), key, val, valid, false);
#pragma unroll
  for (int i = 0; i < IT; ++i)
    if (valid[i]) atomicAdd(&hist[wave][((uint32_t)key[i] >> shift) & (uint32_t)(R - 1)], 1u);
  __syncthreads();
  for (int dd = threadIdx.x; dd < R; dd += kRadixThreads) {
    uint32_t c = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) c += hist[w][dd];
    counts[(int64_t)dd * nblk + b] = c;
  }
}

// Destination base of each digit for block b straight from the raw (digit,
// block) counts, for small count tables: the keys of smaller digits anywhere,
// plus the keys of the same digit in earlier blocks.  Thread t adds up digit
// t / S over blocks t % S, t % S + S, ... (S = threads per digit), so a
// wavefront reads runs of S consecutive counts; 32 of a thread's loads are
// in flight at once (a workgroup waits on this before it can place a key).
template <int R>
__device__ __forceinline__ void digit_bases(const uint32_t* __restrict__ counts, int64_t nblk, int64_t b,
                                            uint32_t* part_pre, uint32_t* part_all, uint32_t* tot,
                                            uint32_t* gbase) {
  constexpr int S = kRadixThreads / R;
  const int d = threadIdx.x / S, r = threadIdx.x % S;
  const uint32_t* row = counts + (int64_t)d * nblk;
  uint32_t pre = 0, all = 0;
#pragma unroll 32
  for (int64_t j = r; j < nblk; j += S) {
    const uint32_t c = row[j];
    all += c;
    pre += j < b ? c : 0u;
  }
  part_pre[threadIdx.x] = pre;
  part_all[threadIdx.x] = all;
  __syncthreads();
  if (threadIdx.x < R) {
    uint32_t p = 0, a = 0;
    for (int q = 0; q < S; ++q) {
      p += part_pre[threadIdx.x * S + q];
      a += part_all[threadIdx.x * S + q];
    }
    gbase[threadIdx.x] = p;
    tot[threadIdx.x] = a;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t run = 0;
    for (int dd = 0; dd < R; ++dd) {
      const uint32_t a = tot[dd];
      gbase[dd] += run;
      run += a;
    }
  }
  __syncthreads();
}

// How a scatter workgroup finds the destination base of each digit of its block.
enum ScatterBases {
  kBasesScanned = 0,  // the whole (digit, block) table was scanned: the entry itself
  kBasesRaw = 1,      // raw counts: the workgroup sums the table itself (small tables)
  kBasesPerDigit = 2  // each digit's row scanned by itself, row totals in `tot`: entry + earlier digits' totals
};

// Stable scatter: destination = scanned global base of (digit, block) + rank
// within the digit.  The block's keys and values are first placed in LDS in
// sorted order (reusing the counter space: both at once in blocks of up to
// 4,096 keys, else keys, then values), then written out with consecutive
// lanes on consecutive block positions, so each digit's run leaves as
// contiguous stores rather than scattered words.
static_assert(kRadixPadded >= kRadixThreads * kRadixMaxItems, "staging reuses the counter space");
static_assert((1 << kMaxDigitBits) <= 64, "one wavefront adds up the digit totals");
template <int BITS, int IT, int BASES>
__global__ __launch_bounds__(kRadixThreads) void radix_scatter_kernel(const int32_t* __restrict__ keys_in,
                                                                      const int32_t* __restrict__ vals_in, int64_t N,
                                                                      int64_t K, int first, int shift, int64_t nblk,
                                                                      const uint32_t* __restrict__ offsets,
                                                                      const uint32_t* __restrict__ tot,
                                                                      int32_t* __restrict__ keys_out,
                                                                      int32_t* __restrict__ vals_out) {
  constexpr int R = 1 << BITS;
  __shared__ uint32_t ctr[kRadixPadded];
  __shared__ uint32_t wsum[kRadixThreads / 64];
  __shared__ uint32_t start[R + 1];
  __shared__ uint32_t gbase[R];
  const int64_t b = blockIdx.x;
  if constexpr (BASES == kBasesRaw) {  // `offsets` holds the raw counts
    digit_bases<R>(offsets, nblk, b, ctr, ctr + kRadixThreads, ctr + 2 * kRadixThreads, gbase);
  } else if constexpr (BASES == kBasesPerDigit) {
    if (threadIdx.x < 64) {  // one wavefront: exclusive prefix of the digit totals, plus this block's entry
      const int dd = threadIdx.x;
      const uint32_t v = dd < R ? tot[dd] : 0u;
      uint32_t x = v;
#pragma unroll
      for (int off = 1; off < R; off <<= 1) {
        const uint32_t y = __shfl_up(x, off);
        if (dd >= off) x += y;
      }
      if (dd < R) gbase[dd] = (x - v) + offsets[(int64_t)dd * nblk + b];
    }
  } else {
    for (int dd = threadIdx.x; dd < R; dd += kRadixThreads) gbase[dd] = offsets[(int64_t)dd * nblk + b];
  }
  int32_t key[IT], val[IT];
  bool valid[IT];
  load_block_keys<IT>(keys_in, vals_in, first, N, K, b * (kRadixThreads * IT), key, val, valid, true);
  uint32_t d[IT], rank[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) d[i] = ((uint32_t)key[i] >> shift) & (uint32_t)(R - 1);
  block_rank<BITS, IT>(d, valid, ctr, wsum, start, rank);
  const uint32_t nkeys = start[R];
  int32_t* stage = reinterpret_cast<int32_t*>(ctr);
  if constexpr (2 * kRadixThreads * IT <= kRadixPadded) {
    // keys and values staged side by side in sorted order, then written out in one round
    int32_t* sval = stage + kRadixThreads * IT;
#pragma unroll
    for (int i = 0; i < IT; ++i)
      if (valid[i]) {
        stage[rank[i]] = key[i];
        sval[rank[i]] = val[i];
      }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const uint32_t p = (uint32_t)(i * kRadixThreads + threadIdx.x);
      if (p < nkeys) {
        const int32_t k = stage[p];
        const uint32_t dg = ((uint32_t)k >> shift) & (uint32_t)(R - 1);
        const uint32_t dst = gbase[dg] + (p - start[dg]);
        if (dst < (uint64_t)N) {  // always true for a consistent scan
          keys_out[dst] = k;
          vals_out[dst] = sval[p];
        }
      }
    }
    return;
  }
  // keys in sorted order; remember each striped position's destination
#pragma unroll
  for (int i = 0; i < IT; ++i)
    if (valid[i]) stage[rank[i]] = key[i];
  __syncthreads();
  uint32_t dst[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const uint32_t p = (uint32_t)(i * kRadixThreads + threadIdx.x);
    dst[i] = 0xffffffffu;
    if (p < nkeys) {
      const int32_t k = stage[p];
      const uint32_t dg = ((uint32_t)k >> shift) & (uint32_t)(R - 1);
      dst[i] = gbase[dg] + (p - start[dg]);
      if (dst[i] < (uint64_t)N) keys_out[dst[i]] = k;  // always true for a consistent scan
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < IT; ++i)
    if (valid[i]) stage[rank[i]] = val[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const uint32_t p = (uint32_t)(i * kRadixThreads + threadIdx.x);
    if (p < nkeys && dst[i] < (uint64_t)N) vals_out[dst[i]] = stage[p];
  }
}

// Wave-ranked variant of the stable scatter, for digits of up to 8 bits.
// Wavefront w of the block takes the 64 * IT consecutive keys from position
// w * 64 * IT, 64 at a time (step j: positions j * 64 + lane).  In each step
// the lanes holding the same digit find each other with one ballot per digit
// bit; a key's rank is the wave's running count of its digit (one LDS word
// per digit and wave, advanced by the highest such lane) plus the number of
// such lanes below it.  The waves' counts then become per-wave offsets inside
// each digit, the digit totals the block's digit starts.  Steps run in
// position order and lanes in position order, so equal digits keep their
// input order (stable).  No per-thread counters and no serial chain of LDS
// read-modify-writes per key.
template <int BITS, int IT, int BASES>
__global__ __launch_bounds__(kRadixThreads) void radix_scatter_wave_kernel(const int32_t* __restrict__ keys_in,
                                                                           const int32_t* __restrict__ vals_in,
                                                                           int64_t N, int64_t K, int first, int shift,
                                                                           int64_t nblk,
                                                                           const uint32_t* __restrict__ offsets,
                                                                           const uint32_t* __restrict__ tot,
                                                                           int32_t* __restrict__ keys_out,
                                                                           int32_t* __restrict__ vals_out) {
  constexpr int R = 1 << BITS;
  constexpr int NW = kRadixThreads / 64;
  constexpr int BLK = kRadixThreads * IT;
  static_assert(R <= kRadixThreads, "a thread per digit");
  static_assert(BLK >= 3 * kRadixThreads, "the raw-count bases use the staging space");
  __shared__ int32_t stage[BLK];
  __shared__ uint32_t whist[NW * R];
  __shared__ uint32_t wsum[kRadixThreads / 64];
  __shared__ uint32_t start[R + 1];
  __shared__ uint32_t gbase[R];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int64_t b = blockIdx.x;
  if constexpr (BASES == kBasesRaw) {  // `offsets` holds the raw counts; the staging space is free until the keys
    uint32_t* scr = reinterpret_cast<uint32_t*>(stage);
    digit_bases<R>(offsets, nblk, b, scr, scr + kRadixThreads, scr + 2 * kRadixThreads, gbase);
  } else if constexpr (BASES == kBasesPerDigit) {  // exclusive prefix of the digit totals, plus this block's entry
    uint32_t excl;
    block_scan_excl(t < R ? tot[t] : 0u, excl, wsum);
    if (t < R) gbase[t] = excl + offsets[(int64_t)t * nblk + b];
  } else {
    for (int dd = t; dd < R; dd += kRadixThreads) gbase[dd] = offsets[(int64_t)dd * nblk + b];
  }
  for (int i = t; i < NW * R; i += kRadixThreads) whist[i] = 0u;

  // this wavefront's keys (and values; the first pass makes them from the positions)
  const int64_t p0 = b * BLK + (int64_t)wave * 64 * IT + lane;
  int32_t key[IT], val[IT];
#pragma unroll
  for (int j = 0; j < IT; ++j) {
    const int64_t pos = p0 + (int64_t)j * 64;
    const bool ok = pos < N;
    key[j] = ok ? keys_in[pos] : 0;
    if (first) {
      val[j] = (int32_t)pos;
      if (ok && (uint32_t)key[j] >= (uint32_t)K) {
        key[j] = (int32_t)(K - 1);
        val[j] = (int32_t)((uint32_t)pos | kInvalidFlag);
      }
    } else {
      val[j] = ok ? vals_in[pos] : 0;
    }
  }
  __syncthreads();  // counters zeroed

  uint32_t* hist = whist + wave * R;
  const uint64_t lower = (1ull << lane) - 1ull;  // lanes below this one
  uint32_t rank[IT];
#pragma unroll
  for (int j = 0; j < IT; ++j) {
    const bool ok = p0 + (int64_t)j * 64 < N;
    const uint32_t dg = ((uint32_t)key[j] >> shift) & (uint32_t)(R - 1);
    uint64_t peers = __ballot(ok);
#pragma unroll
    for (int bit = 0; bit < BITS; ++bit) {
      const bool on = (dg >> bit) & 1u;
      const uint64_t m = __ballot(on);
      peers &= on ? m : ~m;
    }
    const uint32_t below = (uint32_t)__popcll(peers & lower);
    rank[j] = 0;
    if (ok) {
      const uint32_t c = hist[dg];
      rank[j] = c + below;
      if (below + 1 == (uint32_t)__popcll(peers)) hist[dg] = c + below + 1;  // the digit's highest lane
    }
  }
  __syncthreads();
  // each digit: the waves' counts become offsets inside the digit; the totals become the digit starts
  uint32_t total = 0;
  if (t < R) {
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t c = whist[w * R + t];
      whist[w * R + t] = total;
      total += c;
    }
  }
  uint32_t excl;
  const uint32_t nkeys = block_scan_excl(total, excl, wsum);
  if (t < R) start[t] = excl;
  if (t == 0) start[R] = nkeys;
  __syncthreads();
  // keys in sorted order; remember each striped position's destination
#pragma unroll
  for (int j = 0; j < IT; ++j) {
    if (p0 + (int64_t)j * 64 < N) {
      const uint32_t dg = ((uint32_t)key[j] >> shift) & (uint32_t)(R - 1);
      rank[j] += start[dg] + hist[dg];
      stage[rank[j]] = key[j];
    }
  }
  __syncthreads();
  uint32_t dst[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const uint32_t p = (uint32_t)(i * kRadixThreads + t);
    dst[i] = 0xffffffffu;
    if (p < nkeys) {
      const int32_t k = stage[p];
      const uint32_t dg = ((uint32_t)k >> shift) & (uint32_t)(R - 1);
      dst[i] = gbase[dg] + (p - start[dg]);
      if (dst[i] < (uint64_t)N) keys_out[dst[i]] = k;  // always true for a consistent scan
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < IT; ++j)
    if (p0 + (int64_t)j * 64 < N) stage[rank[j]] = val[j];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const uint32_t p = (uint32_t)(i * kRadixThreads + t);
    if (p < nkeys && dst[i] < (uint64_t)N) vals_out[dst[i]] = stage[p];
  }
}

// ------------------------------------------------------------------- scan --
//
// Exclusive scan of the (digit, block) counts.  A tile is 1024 threads x 4
// consecutive values, loaded and stored as one 16-byte vector per thread
// (a wavefront touches 1 KiB of contiguous memory per instruction).

constexpr int kScanThreads = 1024;
constexpr int64_t kScanTile = (int64_t)kScanThreads * 4;

// Exclusive scan of one value per thread across the 1024-thread block; returns the total.
__device__ uint32_t scan_block(uint32_t v, uint32_t& excl, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (wave == 0) {
    constexpr int NW = kScanThreads / 64;
    const uint32_t w = lane < NW ? wsum[lane] : 0u;
    uint32_t z = w;
#pragma unroll
    for (int off = 1; off < NW; off <<= 1) {
      const uint32_t y = __shfl_up(z, off);
      if (lane >= off) z += y;
    }
    if (lane < NW) wsum[NW + lane] = z - w;  // exclusive prefix of each wavefront
    if (lane == NW - 1) wsum[2 * NW] = z;    // block total
  }
  __syncthreads();
  excl = wsum[kScanThreads / 64 + wave] + x - v;
  const uint32_t total = wsum[2 * (kScanThreads / 64)];
  __syncthreads();
  return total;
}

__device__ __forceinline__ uint4 load4(const uint32_t* a, int64_t i, int64_t n) {
  if (i + 4 <= n) return *reinterpret_cast<const uint4*>(a + i);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (i < n) v.x = a[i];
  if (i + 1 < n) v.y = a[i + 1];
  if (i + 2 < n) v.z = a[i + 2];
  return v;
}

__device__ __forceinline__ void store4(uint32_t* a, int64_t i, int64_t n, uint4 v) {
  if (i + 4 <= n) {
    *reinterpret_cast<uint4*>(a + i) = v;
    return;
  }
  if (i < n) a[i] = v.x;
  if (i + 1 < n) a[i + 1] = v.y;
  if (i + 2 < n) a[i + 2] = v.z;
}

// Scan one tile in place with carry-in `carry`; returns the tile total.
__device__ uint32_t scan_tile(uint32_t* a, int64_t n, int64_t t0, uint32_t carry, uint32_t* wsum) {
  const int64_t i = t0 + (int64_t)threadIdx.x * 4;
  uint4 v = load4(a, i, n);
  const uint32_t s = v.x + v.y + v.z + v.w;
  uint32_t excl;
  const uint32_t total = scan_block(s, excl, wsum);
  const uint32_t b = carry + excl;
  const uint4 o = make_uint4(b, b + v.x, b + v.x + v.y, b + v.x + v.y + v.z);
  store4(a, i, n, o);
  return total;
}

// Sum of each tile.
__global__ __launch_bounds__(kScanThreads) void scan_reduce_kernel(const uint32_t* __restrict__ a, int64_t n,
                                                                   uint32_t* __restrict__ part) {
  __shared__ uint32_t wsum[2 * (kScanThreads / 64) + 1];
  const int64_t i = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * 4;
  const uint4 v = load4(a, i, n);
  uint32_t excl;
  const uint32_t total = scan_block(v.x + v.y + v.z + v.w, excl, wsum);
  if (threadIdx.x == 0) part[blockIdx.x] = total;
}

// In-place exclusive scan of a[0..n) by one block, tile after tile.
__global__ __launch_bounds__(kScanThreads) void scan_single_kernel(uint32_t* __restrict__ a, int64_t n) {
  __shared__ uint32_t wsum[2 * (kScanThreads / 64) + 1];
  uint32_t carry = 0;
  for (int64_t t0 = 0; t0 < n; t0 += kScanTile) carry += scan_tile(a, n, t0, carry, wsum);
}

// In-place exclusive scan of each digit's row of the (digit, block) count
// table, one workgroup per digit, tile after tile (a thread takes 4
// consecutive entries, loaded one by one: rows need not be 16-byte aligned);
// the row's total goes to tot[digit].
__global__ __launch_bounds__(kScanThreads) void digit_scan_kernel(uint32_t* __restrict__ counts, int64_t nblk,
                                                                  uint32_t* __restrict__ tot) {
  __shared__ uint32_t wsum[2 * (kScanThreads / 64) + 1];
  uint32_t* row = counts + (int64_t)blockIdx.x * nblk;
  uint32_t carry = 0;
  for (int64_t t0 = 0; t0 < nblk; t0 += kScanTile) {
    const int64_t i = t0 + (int64_t)threadIdx.x * 4;
    uint32_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = i + j < nblk ? row[i + j] : 0u;
    uint32_t excl;
    const uint32_t total = scan_block(v[0] + v[1] + v[2] + v[3], excl, wsum);
    uint32_t run = carry + excl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (i + j < nblk) row[i + j] = run;
      run += v[j];
    }
    carry += total;
  }
  if (threadIdx.x == 0) tot[blockIdx.x] = carry;
}

// In-place exclusive scan of each tile, offset by the scanned tile sums.
__global__ __launch_bounds__(kScanThreads) void scan_apply_kernel(uint32_t* __restrict__ a, int64_t n,
                                                                  const uint32_t* __restrict__ part) {
  __shared__ uint32_t wsum[2 * (kScanThreads / 64) + 1];
  scan_tile(a, n, (int64_t)blockIdx.x * kScanTile, part[blockIdx.x], wsum);
}

// Up to this many entries one block scans tile after tile (a kernel launch
// costs more than the few extra tiles); beyond it, reduce / scan / apply.
// (measured on gfx950: 16 tiles (64 digits x 1024 blocks) take 19.6 us in one
// block, 8 us in three launches; 4 tiles are faster in one block)
#ifndef KM_SCAN_SINGLE_TILES
#define KM_SCAN_SINGLE_TILES 8
#endif
constexpr int64_t kScanSingleMax = KM_SCAN_SINGLE_TILES * kScanTile;

static hipError_t launch_scan(uint32_t* a, int64_t n, uint32_t* part, hipStream_t s) {
  if (n <= kScanSingleMax) {
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

// Count tables up to this many entries skip the scan: every scatter workgroup
// derives its own destinations from the raw counts (reads the whole table).
#ifndef KM_SCAN_FUSE_TILES
#define KM_SCAN_FUSE_TILES 4
#endif
constexpr int64_t kScanFuseMax = KM_SCAN_FUSE_TILES * kScanTile;

// Scratch of the count scans: the tile sums of a whole-table scan, or the digit totals of per-digit scans.
int64_t scan_part_len(int64_t n) {
  const int64_t tiles = (n + kScanTile - 1) / kScanTile + 1;
  return tiles > (1 << kMaxWaveDigitBits) ? tiles : (1 << kMaxWaveDigitBits);
}

template <int B, int IT>
static void count_pass(const SortGeom& g, const int32_t* kin, int first, int shift, uint32_t* counts, hipStream_t s) {
  hipLaunchKernelGGL((radix_count_kernel<B, IT>), dim3((unsigned)g.nblk), dim3(kRadixThreads), 0, s, kin, g.N, g.K,
                     first, shift, g.nblk, counts);
}

template <int B, int IT, int BASES>
static void scatter_launch(const SortGeom& g, const int32_t* kin, const int32_t* vin, int first, int shift,
                           const uint32_t* counts, const uint32_t* tot, int32_t* kout, int32_t* vout, hipStream_t s) {
  const dim3 grid((unsigned)g.nblk), block(kRadixThreads);
  if constexpr (B <= kMaxDigitBits) {
    if (!g.wave_rank) {
      hipLaunchKernelGGL((radix_scatter_kernel<B, IT, BASES>), grid, block, 0, s, kin, vin, g.N, g.K, first, shift,
                         g.nblk, counts, tot, kout, vout);
      return;
    }
  }
  hipLaunchKernelGGL((radix_scatter_wave_kernel<B, IT, BASES>), grid, block, 0, s, kin, vin, g.N, g.K, first, shift,
                     g.nblk, counts, tot, kout, vout);
}

template <int B, int IT>
static void scatter_pass(const SortGeom& g, const int32_t* kin, const int32_t* vin, int first, int shift,
                         const uint32_t* counts, const uint32_t* tot, int bases, int32_t* kout, int32_t* vout,
                         hipStream_t s) {
  if (bases == kBasesRaw)
    scatter_launch<B, IT, kBasesRaw>(g, kin, vin, first, shift, counts, tot, kout, vout, s);
  else if (bases == kBasesPerDigit)
    scatter_launch<B, IT, kBasesPerDigit>(g, kin, vin, first, shift, counts, tot, kout, vout, s);
  else
    scatter_launch<B, IT, kBasesScanned>(g, kin, vin, first, shift, counts, tot, kout, vout, s);
}

#define KM_SORT_DISPATCH(CALL)                                                               \
  switch (g.items * 16 + bits) {                                                             \
    case 8 * 16 + 1: CALL(1, 8); break;                                                      \
    case 8 * 16 + 2: CALL(2, 8); break;                                                      \
    case 8 * 16 + 3: CALL(3, 8); break;                                                      \
    case 8 * 16 + 4: CALL(4, 8); break;                                                      \
    case 8 * 16 + 5: CALL(5, 8); break;                                                      \
    case 8 * 16 + 6: CALL(6, 8); break;                                                      \
    case 8 * 16 + 7: CALL(7, 8); break;                                                      \
    case 8 * 16 + 8: CALL(8, 8); break;                                                      \
    case 16 * 16 + 1: CALL(1, 16); break;                                                    \
    case 16 * 16 + 2: CALL(2, 16); break;                                                    \
    case 16 * 16 + 3: CALL(3, 16); break;                                                    \
    case 16 * 16 + 4: CALL(4, 16); break;                                                    \
    case 16 * 16 + 5: CALL(5, 16); break;                                                    \
    case 16 * 16 + 6: CALL(6, 16); break;                                                    \
    case 16 * 16 + 7: CALL(7, 16); break;                                                    \
    case 16 * 16 + 8: CALL(8, 16); break;                                                    \
    case 32 * 16 + 1: CALL(1, 32); break;                                                    \
    case 32 * 16 + 2: CALL(2, 32); break;                                                    \
    case 32 * 16 + 3: CALL(3, 32); break;                                                    \
    case 32 * 16 + 4: CALL(4, 32); break;                                                    \
    case 32 * 16 + 5: CALL(5, 32); break;                                                    \
    case 32 * 16 + 6: CALL(6, 32); break;                                                    \
    case 32 * 16 + 7: CALL(7, 32); break;                                                    \
    case 32 * 16 + 8: CALL(8, 32); break;                                                    \
    default: return hipErrorInvalidValue;                                                    \
  }

static hipError_t launch_pass_count(const SortGeom& g, int bits, const int32_t* kin, int first, int shift,
                                    uint32_t* counts, hipStream_t s) {
#define KM_CALL(B, IT) count_pass<B, IT>(g, kin, first, shift, counts, s)
  KM_SORT_DISPATCH(KM_CALL)
#undef KM_CALL
  return hipGetLastError();
}

static hipError_t launch_pass_scatter(const SortGeom& g, int bits, const int32_t* kin, const int32_t* vin, int first,
                                      int shift, const uint32_t* counts, const uint32_t* tot, int bases,
                                      int32_t* kout, int32_t* vout, hipStream_t s) {
#define KM_CALL(B, IT) scatter_pass<B, IT>(g, kin, vin, first, shift, counts, tot, bases, kout, vout, s)
  KM_SORT_DISPATCH(KM_CALL)
#undef KM_CALL
  return hipGetLastError();
}
#undef KM_SORT_DISPATCH

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
    hipError_t e = launch_pass_count(g, bits, kin, first, shift, counts, stream);
    if (e != hipSuccess) return e;
    // A small count table is summed by every scatter workgroup itself, which saves the scan's launch.  A larger
    // one is scanned digit by digit, one launch of a workgroup per digit, the scatter adding the digits' totals
    // (measured on gfx950: 2^23 keys in two 6-bit passes sort 6% faster than with the whole table scanned in
    // three launches, 2^26 keys 0.5%), or, as the planner's alternative, as a whole.
    const int64_t entries = ((int64_t)1 << bits) * g.nblk;
    int bases = kBasesScanned;
    if (g.scan_mode == 2 || (g.scan_mode == 0 && entries > kScanFuseMax)) {
      hipLaunchKernelGGL(digit_scan_kernel, dim3(1u << bits), dim3(kScanThreads), 0, stream, counts, g.nblk,
                         scan_part);
      bases = kBasesPerDigit;
    } else if (entries <= kScanFuseMax) {
      bases = kBasesRaw;
    } else {
      e = launch_scan(counts, entries, scan_part, stream);
      if (e != hipSuccess) return e;
    }
    e = launch_pass_scatter(g, bits, kin, vin, first, shift, counts, scan_part, bases, kout, vout, stream);
    if (e != hipSuccess) return e;
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
