// Sort-Inverse Update for small problems: codebooks of at most 64 clusters
// per problem, and a few problems of at most 16384 points with at most 2048
// clusters in all -- the shape of many small K-Means problems called back to
// back or batched.
//
// Citations name the page "Flash-KMeans: Fast and Memory-Efficient Exact
// K-Means" (gist.science summary of paper 2603.09229); "tech §n" is a section
// of its technical summary.
//
// Same idea as tech §2.2 (make each cluster's points contiguous, then reduce
// contiguous runs with no atomics), kept on chip.  A few problems of at most
// 16384 points take one workgroup per cluster (or per 2 or 4 clusters),
// which lists its own points in index order (small_owner_kernel, below).
// Otherwise, with K <= 64 the whole cluster id is one 6-bit radix digit: one
// workgroup ranks
// the ids of a chunk (2048 points, 512 for small calls) stably (512: wavefront
// ballots and LDS histograms; 2048: the radix sort's block rank), lays the
// chunk's point indices out in cluster order in LDS, and then lets each lane
// group walk whole clusters of the chunk in that order, 16 rows in flight.
// No global sort, no carries: a cluster's chunk sum is complete in one lane
// group.  When a problem has one chunk the means are written right away (one
// launch for the whole update); otherwise the chunk sums are added chunk by
// chunk in a second launch.  The order of every addition is fixed
// (chunk, then point index), so results are deterministic.
#include "block_rank.hpp"
#include "frag_emit.hpp"
#include "km_internal.hpp"
#include "rows.hpp"

namespace km {

// Points per workgroup: 2048 (8 ids a thread), or 512 (2 a thread) when that
// many chunks would leave most CUs idle: the walk after the rank is
// latency-bound, so a lone small problem finishes sooner spread thinner.
// (8192-point chunks were slower on c1-shaped problems, alone and batched.)
constexpr int kSmallChunk = kRadixThreads * 8;
constexpr int kSmallChunkThin = kRadixThreads * 2;
static_assert(kSmallMaxK <= (1 << kMaxDigitBits), "one radix digit holds every id");

// 512-point chunks when 2048-point chunks would give fewer workgroups than compute units
static int small_it(int64_t B, int64_t N) {
  return B * ((N + kSmallChunk - 1) / kSmallChunk) < device_info().cus ? 2 : 8;
}

struct SmallParams {
  const uint8_t* X;     // B x N x D
  int dt;
  int64_t N;            // points per problem
  int D;
  int64_t K;            // clusters per problem
  bool vec_ok;
  const int32_t* ids;   // B x N; problem b's ids are b * id_mul + k
  int64_t id_mul;
  int64_t P;            // chunks per problem
  int Dc;
  const float* C_prev;  // B x K x D
  float* C_new;
  int32_t* counts;      // B x K, nullable
  float* part_sum;      // (B * P) x K x Dc (P > 1)
  int32_t* part_cnt;    // (B * P) x K
  // fp32 X, P > 1: the chunk-sum step also writes each new centroid's MFMA
  // fragment and bias for the next assignment (frag == NULL: it does not)
  uint32_t* frag;       // 16-byte slots, problem b at b * f_stride
  int64_t f_stride;
  AssignCfg cfg;
};

// Sum of the rows srow[s0 .. s1) (lane j: its 16-byte column chunk).  The
// U indices of a round are read from LDS first and the row loads are
// unconditional (the tail repeats the last row and skips its add), so a
// round's U loads leave back to back.  VEC: rows are whole 16-byte chunks.
template <int ES, bool VEC, int U>
__device__ __forceinline__ void walk_rows(const uint8_t* __restrict__ Xb, const int32_t* srow, int s0, int s1, int D,
                                          int dt, int j, float (&acc)[16 / ES]) {
  constexpr int EPL = 16 / ES;
  for (int p = s0; p < s1; p += U) {
    int32_t r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = srow[p + u < s1 ? p + u : s1 - 1];
    u32x4_r xr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (VEC)
        xr[u] = *reinterpret_cast<const u32x4_r*>(Xb + ((size_t)r[u] * (size_t)D + (size_t)(j * EPL)) * ES);
      else
        xr[u] = load_chunk<ES>(Xb, r[u], D, j * EPL, false);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (p + u < s1) {
        float f[EPL];
        widen(xr[u], dt, f);
#pragma unroll
        for (int x = 0; x < EPL; ++x) acc[x] += f[x];
      }
    }
  }
}

// Stable rank of a chunk's ids (all below 64): rank = ids smaller than this one
// anywhere in the chunk + equal ids at earlier positions (position = thread *
// IT + i), the same order as the radix sort's block rank.  Equal ids earlier in
// the wavefront come from six bit-sliced ballots per key slot; the wavefronts'
// id counts (LDS histograms, integer atomics) give the rest.  start[0..64] is
// left holding each id's first position.
template <int IT>
__device__ __forceinline__ void small_rank(const uint32_t (&d)[IT], const bool (&valid)[IT], uint32_t* hist,
                                           uint32_t* start, uint32_t (&rank)[IT]) {
  constexpr int NW = kRadixThreads / 64;
  constexpr int R = 1 << kMaxDigitBits;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < NW * R; i += kRadixThreads) hist[i] = 0u;
  const uint64_t below = (1ull << lane) - 1ull;
  uint32_t inwave[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) inwave[i] = 0;
#pragma unroll
  for (int j = 0; j < IT; ++j) {  // key slot j of every lane: the lanes whose key there equals each own key
    const uint64_t vm = __builtin_amdgcn_ballot_w64(valid[j]);
    uint64_t bal[kMaxDigitBits];
#pragma unroll
    for (int b = 0; b < kMaxDigitBits; ++b) bal[b] = __builtin_amdgcn_ballot_w64(valid[j] && ((d[j] >> b) & 1u));
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      uint64_t m = vm;
#pragma unroll
      for (int b = 0; b < kMaxDigitBits; ++b) m &= ((d[i] >> b) & 1u) ? bal[b] : ~bal[b];
      inwave[i] += (uint32_t)__popcll(m & below) + ((j < i && valid[j] && d[j] == d[i]) ? 1u : 0u);
    }
  }
  __syncthreads();  // histograms cleared
#pragma unroll
  for (int i = 0; i < IT; ++i)
    if (valid[i]) atomicAdd(&hist[wave * R + d[i]], 1u);
  __syncthreads();
  if (threadIdx.x < R) {  // per id: counts of earlier wavefronts, and the chunk total
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t h = hist[w * R + threadIdx.x];
      hist[w * R + threadIdx.x] = s;
      s += h;
    }
    start[threadIdx.x + 1] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {  // exclusive scan of the totals over ids
    uint32_t run = 0;
    start[0] = 0;
    for (int k = 0; k < R; ++k) {
      run += start[k + 1];
      start[k + 1] = run;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < IT; ++i)
    if (valid[i]) rank[i] = start[d[i]] + hist[wave * R + d[i]] + inwave[i];
}

template <int ES, int G, int IT>
__global__ __launch_bounds__(kRadixThreads) void small_update_kernel(SmallParams S) {
  constexpr int kSmallIT = IT;
  constexpr int kChunk = kRadixThreads * IT;
  constexpr int EPL = 16 / ES;
  constexpr int NG = kRadixThreads / G;  // lane groups
  constexpr int U = IT == 2 ? 8 : 16;    // rows in flight per lane group (measured: 8 for a lone problem, 16 batched)
  __shared__ uint32_t start[(1 << kMaxDigitBits) + 1];
  __shared__ int32_t srow[kChunk];
  const int64_t b = blockIdx.x / S.P, c = blockIdx.x - b * S.P;
  const int64_t c0 = c * kChunk;
  const int64_t n = S.N - c0 < kChunk ? S.N - c0 : kChunk;
  const int32_t* ids = S.ids + b * S.N + c0;
  const int64_t id0 = b * S.id_mul;

  uint32_t d[kSmallIT], rank[kSmallIT];
  bool valid[kSmallIT];
#pragma unroll
  for (int i = 0; i < kSmallIT; ++i) {
    const int64_t pos = (int64_t)threadIdx.x * kSmallIT + i;
    const int64_t k = pos < n ? (int64_t)ids[pos] - id0 : -1;
    valid[i] = k >= 0 && k < S.K;  // ids outside [0, K) are ignored
    d[i] = valid[i] ? (uint32_t)k : 0u;
  }
  if constexpr (IT <= 2) {  // 512 ids: ballots (the general block rank clears and scans 16K counters)
    __shared__ uint32_t hist[(kRadixThreads / 64) << kMaxDigitBits];
    small_rank<IT>(d, valid, hist, start, rank);
  } else {  // more ids a thread: the ballots would outgrow the scalar registers
    __shared__ uint32_t ctr[kRadixPadded];
    __shared__ uint32_t wsum[kRadixThreads / 64];
    block_rank<kMaxDigitBits, IT>(d, valid, ctr, wsum, start, rank);
  }
#pragma unroll
  for (int i = 0; i < kSmallIT; ++i)
    if (valid[i]) srow[rank[i]] = (int32_t)(c0 + (int64_t)threadIdx.x * kSmallIT + i);
  __syncthreads();

  const int g = threadIdx.x / G, j = threadIdx.x % G;
  const uint8_t* Xb = S.X + (size_t)b * (size_t)S.N * (size_t)S.D * ES;
  for (int64_t k = g; k < S.K; k += NG) {
    const int s0 = (int)start[k], s1 = (int)start[k + 1];
    float acc[EPL];
#pragma unroll
    for (int x = 0; x < EPL; ++x) acc[x] = 0.0f;
    if (S.vec_ok && (j + 1) * EPL <= S.D)
      walk_rows<ES, true, U>(Xb, srow, s0, s1, S.D, S.dt, j, acc);
    else if (j * EPL < S.D)
      walk_rows<ES, false, U>(Xb, srow, s0, s1, S.D, S.dt, j, acc);
    const int32_t cnt = s1 - s0;
    if (S.P == 1) {  // the chunk is the whole problem: its means (an empty cluster keeps its centroid)
      const int64_t row = (b * S.K + k) * S.D;
#pragma unroll
      for (int x = 0; x < EPL; ++x) {
        const int col = j * EPL + x;
        if (col < S.D) S.C_new[row + col] = cnt > 0 ? acc[x] / (float)cnt : S.C_prev[row + col];
      }
      if (j == 0 && S.counts) S.counts[b * S.K + k] = cnt;
    } else {
      float4* dst = reinterpret_cast<float4*>(S.part_sum + ((b * S.P + c) * S.K + k) * S.Dc + j * EPL);
#pragma unroll
      for (int x = 0; x < EPL; x += 4) dst[x / 4] = make_float4(acc[x], acc[x + 1], acc[x + 2], acc[x + 3]);
      if (j == 0) S.part_cnt[(b * S.P + c) * S.K + k] = cnt;
    }
  }
}

// One wavefront per (problem, cluster): the chunk sums of a cluster, added in
// a fixed order.  Lanes form R rows of DL lanes (DL = D rounded up to a power
// of two, at most 64); row r takes chunks r, r + R, ... in ascending order,
// 8 in flight, and the rows then meet in a fixed shuffle tree.
__global__ __launch_bounds__(256) void small_combine_kernel(SmallParams S, int64_t nclusters, int DL) {
  __shared__ float rows[4][kMaxD32];  // fp32 rows for the fragments
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t q = (int64_t)blockIdx.x * 4 + wv;  // b * K + k
  const bool active = q < nclusters;                 // (every wavefront reaches the barrier below)
  const int64_t b = active ? q / S.K : 0, k = active ? q - b * S.K : 0;
  constexpr int kMaxCols = 512 / 64;  // columns per lane at most (D <= 512 with DL = 64)
  const int R = 64 / DL, r = lane / DL, cl = lane % DL;
  float acc[kMaxCols];
#pragma unroll
  for (int x = 0; x < kMaxCols; ++x) acc[x] = 0.0f;
  int32_t cnt = 0;
  constexpr int UNR = 8;  // chunks in flight per row
  for (int64_t c0 = r; active && c0 < S.P; c0 += (int64_t)R * UNR) {
    float v[UNR][kMaxCols];
    int32_t n[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t cu = c0 + (int64_t)u * R;
      const int64_t c = cu < S.P ? cu : S.P - 1;  // the tail reloads the last chunk, not added
      const float* src = S.part_sum + ((b * S.P + c) * S.K + k) * S.Dc;
#pragma unroll
      for (int x = 0; x < kMaxCols; ++x) {
        const int col = cl + DL * x;
        v[u][x] = col < S.D ? src[col] : 0.0f;
      }
      n[u] = S.part_cnt[(b * S.P + c) * S.K + k];
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (c0 + (int64_t)u * R < S.P) {
#pragma unroll
        for (int x = 0; x < kMaxCols; ++x) acc[x] += v[u][x];
        cnt += n[u];
      }
    }
  }
  for (int off = DL; off < 64; off <<= 1) {
#pragma unroll
    for (int x = 0; x < kMaxCols; ++x) acc[x] += __shfl_xor(acc[x], off);
    cnt += __shfl_xor(cnt, off);
  }
  const int64_t row = q * S.D;
  if (active && r == 0) {
#pragma unroll
    for (int x = 0; x < kMaxCols; ++x) {
      const int col = cl + DL * x;
      if (col < S.D) {
        const float c = cnt > 0 ? acc[x] / (float)cnt : S.C_prev[row + col];
        S.C_new[row + col] = c;
        if (S.frag) rows[wv][col] = c;
      }
    }
    if (cl == 0 && S.counts) S.counts[q] = cnt;
  }
  if (!S.frag) return;  // (uniform)
  __syncthreads();
  if (active) emit_fragment_row(rows[wv], S.D, S.dt, S.cfg, S.frag + 4 * b * S.f_stride, k);
}

// A few small problems (N <= 16384, at most owner_max_groups() workgroups of R
// consecutive clusters, R = 1, 2 or 4): one workgroup per (problem, R
// clusters).  It reads all of the problem's ids at once, lists each of its
// clusters' points in ascending index order in LDS (per-thread match counts,
// one block scan per cluster), and then, cluster after cluster, lets each lane
// group sum one contiguous block of that cluster's list, adds the lane
// groups' sums in order and writes the mean (an empty cluster keeps its
// centroid), the count and, when asked, the centroid's operand fragment for
// the next assignment.  One launch and no chunk sums; every addition in a
// fixed order, the same for every R.
constexpr int kOwnerMaxN = 16384;
constexpr int kOwnerIPT = kOwnerMaxN / kRadixThreads;  // ids per thread
#ifndef KM_OWNER_MAX_GROUPS_PER_CU
#define KM_OWNER_MAX_GROUPS_PER_CU 2  // (measured on gfx950, 256 compute units, with c1-shaped problems: 1.44x
                                      //  faster than chunk sums for 1 to 4 problems, 1.25x for 8; 0.93x for 16,
                                      //  0.72x for 256)
#endif
static int64_t owner_max_groups() { return KM_OWNER_MAX_GROUPS_PER_CU * (int64_t)device_info().cus; }
#ifndef KM_OWNER_MAX_R
#define KM_OWNER_MAX_R 4  // (measured on gfx950, single problems of 600 to 2,048 clusters: 1.1-2.2x faster than
                          //  the sorted path with 2 or 4 clusters a workgroup, 0.87-1.0x with 8)
#endif
constexpr int kOwnerMaxR = KM_OWNER_MAX_R;  // clusters per workgroup, at most (1, 2, 4 or 8)

// clusters per workgroup for B problems of K clusters (0: the layout does not apply).  Several clusters a
// workgroup only above kSmallMaxK clusters a problem: at most kSmallMaxK the chunk-sum layout takes over
// beyond owner_max_groups() one-cluster workgroups (where it measured faster, 16 or more c1-shaped problems),
// and the 2- and 4-cluster workgroups were measured against the sorted path only.
static int owner_r(int64_t B, int64_t K) {
  const int rmax = K > kSmallMaxK ? kOwnerMaxR : 1;
  for (int r = 1; r <= rmax; r *= 2)
    if (B * ((K + r - 1) / r) <= owner_max_groups()) return r;
  return 0;
}

template <int ES, int G, int R>
__global__ __launch_bounds__(kRadixThreads) void small_owner_kernel(SmallParams S) {
  constexpr int EPL = 16 / ES;
  constexpr int NG = kRadixThreads / G;  // lane groups
  constexpr int GE = G * EPL;            // columns a lane group holds
  __shared__ int32_t list[kOwnerMaxN];
  __shared__ uint32_t wsum[kRadixThreads / 64];
  __shared__ float part[NG * GE];
  __shared__ float part2[kRadixThreads];  // stage-one sums, TPC x GE (below)
  __shared__ float row[kMaxD16];
  const int64_t nq = (S.K + R - 1) / R;  // workgroups per problem
  const int64_t b = blockIdx.x / nq, k0 = (blockIdx.x - b * nq) * R;
  const int32_t want0 = (int32_t)(b * S.id_mul + k0);  // id of cluster k0 + r: want0 + r
  const int32_t* ids = S.ids + b * S.N;
  const int64_t p0 = (int64_t)threadIdx.x * kOwnerIPT;
  int32_t v[kOwnerIPT];
  if (p0 + kOwnerIPT <= S.N && (reinterpret_cast<uintptr_t>(ids + p0) & 15) == 0) {
    const int4* v4 = reinterpret_cast<const int4*>(ids + p0);
#pragma unroll
    for (int i = 0; i < kOwnerIPT / 4; ++i) {
      const int4 w = v4[i];
      v[4 * i] = w.x;
      v[4 * i + 1] = w.y;
      v[4 * i + 2] = w.z;
      v[4 * i + 3] = w.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kOwnerIPT; ++i) v[i] = p0 + i < S.N ? ids[p0 + i] : want0 + R;  // want0 + R: no match
  }
  uint32_t m[R];
#pragma unroll
  for (int r = 0; r < R; ++r) m[r] = 0;
#pragma unroll
  for (int i = 0; i < kOwnerIPT; ++i) {
    const uint32_t rel = (uint32_t)v[i] - (uint32_t)want0;  // (modular: any id outside the R is >= R)
#pragma unroll
    for (int r = 0; r < R; ++r) m[r] += rel == (uint32_t)r ? 1u : 0u;
  }
  // cluster r's list: [lb[r], lb[r] + tot[r]) of `list`, in point order
  uint32_t off[R], tot[R], lb[R];
  uint32_t at = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    tot[r] = block_scan_excl(m[r], off[r], wsum);
    lb[r] = at;
    off[r] += at;
    at += tot[r];
  }
#pragma unroll
  for (int i = 0; i < kOwnerIPT; ++i) {
    const uint32_t rel = (uint32_t)v[i] - (uint32_t)want0;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (rel == (uint32_t)r) list[off[r]++] = (int32_t)(p0 + i);
  }
  __syncthreads();

  const int g = threadIdx.x / G, j = threadIdx.x % G;
  const uint8_t* Xb = S.X + (size_t)b * (size_t)S.N * (size_t)S.D * ES;
#pragma unroll 1
  for (int r = 0; r < R; ++r) {
    const int64_t k = k0 + r;
    if (k >= S.K) break;  // (uniform)
    const uint32_t total = tot[r];
    const int32_t* cl = list + lb[r];
    const int per = (int)((total + NG - 1) / NG);
    const int s0 = g * per < (int)total ? g * per : (int)total;
    const int s1 = s0 + per < (int)total ? s0 + per : (int)total;
    float acc[EPL];
#pragma unroll
    for (int x = 0; x < EPL; ++x) acc[x] = 0.0f;
    if (S.vec_ok && (j + 1) * EPL <= S.D)
      walk_rows<ES, true, 8>(Xb, cl, s0, s1, S.D, S.dt, j, acc);
    else if (j * EPL < S.D)
      walk_rows<ES, false, 8>(Xb, cl, s0, s1, S.D, S.dt, j, acc);
#pragma unroll
    for (int x = 0; x < EPL; ++x) part[g * GE + j * EPL + x] = acc[x];
    __syncthreads();
    // The lane groups' sums of a column, in two fixed stages when the
    // workgroup has threads to spare: TPC threads per column each add every
    // TPC-th lane group, then one thread adds those TPC partial sums in order.
    constexpr int TPC0 = kRadixThreads / GE;
    constexpr int TPC = TPC0 < 2 ? 1 : (TPC0 > NG ? NG : TPC0);
    if constexpr (TPC > 1) {
      const int c = threadIdx.x % GE, t = threadIdx.x / GE;
      if (t < TPC) {
        float u = 0.0f;
        for (int gg = t; gg < NG; gg += TPC) u += part[gg * GE + c];
        part2[t * GE + c] = u;
      }
      __syncthreads();
    }
    const int64_t q = b * S.K + k;
    const int64_t base = q * S.D;
    for (int c = threadIdx.x; c < S.D; c += kRadixThreads) {
      float sum = 0.0f;
      if constexpr (TPC > 1) {
#pragma unroll
        for (int t = 0; t < TPC; ++t) sum += part2[t * GE + c];
      } else {
        for (int gg = 0; gg < NG; ++gg) sum += part[gg * GE + c];
      }
      const float mean = total > 0 ? sum / (float)total : S.C_prev[base + c];
      S.C_new[base + c] = mean;
      if (c < kMaxD16) row[c] = mean;
    }
    if (threadIdx.x == 0 && S.counts) S.counts[q] = (int32_t)total;
    __syncthreads();  // row complete; part and part2 free for the next cluster
    if (S.frag) {     // (uniform)
      if (threadIdx.x < 64) emit_fragment_row(row, S.D, S.dt, S.cfg, S.frag + 4 * b * S.f_stride, k);
      __syncthreads();  // row read before the next cluster writes it
    }
  }
}

int64_t small_chunks(int64_t N) { return (N + kSmallChunkThin - 1) / kSmallChunkThin; }  // at most

bool small_owner_fits(int64_t B, int64_t N, int64_t K) {
  return B >= 1 && K >= 1 && N <= kOwnerMaxN && owner_r(B, K) > 0;
}

hipError_t launch_small_update(const SmallArgs& a, hipStream_t stream) {
  if (a.N == 0 || a.B == 0) return hipSuccess;
  const bool owner = small_owner_fits(a.B, a.N, a.K);
  if (a.K < 1 || (a.K > kSmallMaxK && !owner) || a.D < 1 || deep_rows(a.dt, a.D)) return hipErrorInvalidValue;
  SmallParams S;
  S.X = (const uint8_t*)a.X;
  S.dt = a.dt;
  S.N = a.N;
  S.D = (int)a.D;
  S.K = a.K;
  const int es = dtype_size(a.dt);
  S.vec_ok = (((uintptr_t)a.X) % 16 == 0) && ((a.D * es) % 16 == 0);
  S.ids = a.ids;
  S.id_mul = a.id_mul;
  const int it = small_it(a.B, a.N);
  S.P = (a.N + kRadixThreads * it - 1) / (kRadixThreads * it);
  S.Dc = (int)reduce_dc(a.dt, a.D);
  S.C_prev = a.C_prev;
  S.C_new = a.C_new;
  S.counts = a.counts;
  S.part_sum = a.part_sum;
  S.part_cnt = a.part_cnt;
  S.frag = nullptr;
  S.f_stride = 0;
  S.cfg = a.cfg;
  if (owner) {  // one workgroup per cluster, one launch
    const bool emit = a.frag != nullptr;
    if (emit) {
      S.frag = (uint32_t*)a.frag;
      S.f_stride = a.f_stride;
    }
    if (a.emitted) *a.emitted = emit;
    const int es_ = dtype_size(a.dt);
    const int64_t nch_ = (a.D + 16 / es_ - 1) / (16 / es_);
    int g_ = 1;
    while (g_ < nch_ && g_ < 64) g_ <<= 1;
    const int r_ = owner_r(a.B, a.K);
    const dim3 og((unsigned)(a.B * ((a.K + r_ - 1) / r_))), ob(kRadixThreads);
    bool done = false;
#define KM_OWNER_R(ES_, G_, R_)                                                                \
  if (!done && es_ == ES_ && g_ == G_ && r_ == R_) {                                           \
    hipLaunchKernelGGL((small_owner_kernel<ES_, G_, R_>), og, ob, 0, stream, S);               \
    done = true;                                                                               \
  }
#define KM_OWNER(ES_, G_) KM_OWNER_R(ES_, G_, 1) KM_OWNER_R(ES_, G_, 2) KM_OWNER_R(ES_, G_, 4) KM_OWNER_R(ES_, G_, 8)
    KM_OWNER(2, 1) KM_OWNER(2, 2) KM_OWNER(2, 4) KM_OWNER(2, 8) KM_OWNER(2, 16) KM_OWNER(2, 32) KM_OWNER(2, 64)
    KM_OWNER(4, 1) KM_OWNER(4, 2) KM_OWNER(4, 4) KM_OWNER(4, 8) KM_OWNER(4, 16) KM_OWNER(4, 32) KM_OWNER(4, 64)
#undef KM_OWNER
#undef KM_OWNER_R
    return done ? hipGetLastError() : hipErrorInvalidValue;
  }
  const int64_t grid = a.B * S.P;
  if (grid >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const int epl = 16 / es;
  const int64_t nch = (a.D + epl - 1) / epl;
  int g = 1;
  while (g < nch && g < 64) g <<= 1;
  bool launched = false;
#define KM_SMALL(ES_, G_)                                                                                     \
  if (!launched && es == ES_ && g == G_) {                                                                    \
    if (it == 2)                                                                                              \
      hipLaunchKernelGGL((small_update_kernel<ES_, G_, 2>), dim3((unsigned)grid), dim3(kRadixThreads), 0,      \
                         stream, S);                                                                          \
    else                                                                                                      \
      hipLaunchKernelGGL((small_update_kernel<ES_, G_, 8>), dim3((unsigned)grid), dim3(kRadixThreads), 0,      \
                         stream, S);                                                                          \
    launched = true;                                                                                          \
  }
  KM_SMALL(2, 1) KM_SMALL(2, 2) KM_SMALL(2, 4) KM_SMALL(2, 8) KM_SMALL(2, 16) KM_SMALL(2, 32) KM_SMALL(2, 64)
  KM_SMALL(4, 1) KM_SMALL(4, 2) KM_SMALL(4, 4) KM_SMALL(4, 8) KM_SMALL(4, 16) KM_SMALL(4, 32) KM_SMALL(4, 64)
#undef KM_SMALL
  if (!launched) return hipErrorInvalidValue;
  if (a.emitted) *a.emitted = false;
  if (S.P > 1) {
    if (a.frag && a.dt == DT_F32 && a.cfg.rows == 16 && a.D <= kMaxD32) {
      S.frag = (uint32_t*)a.frag;
      S.f_stride = a.f_stride;
      if (a.emitted) *a.emitted = true;
    }
    const int64_t nq = a.B * a.K;
    int dl = 1;
    while (dl < a.D && dl < 64) dl <<= 1;
    hipLaunchKernelGGL(small_combine_kernel, dim3((unsigned)((nq + 3) / 4)), dim3(256), 0, stream, S, nq, dl);
  }
  return hipGetLastError();
}

}  // namespace km
