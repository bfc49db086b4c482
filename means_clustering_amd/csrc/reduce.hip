// Segmented reduction of Sort-Inverse Update, boundary fix-up, finalisation
// and the fp64 objective.
//
// Citations name the page "Flash-KMeans: Fast and Memory-Efficient Exact
// K-Means" (gist.science summary of paper 2603.09229); "tech §n" is a section
// of its technical summary.
//
// tech §2.2: after the argsort, the points of a cluster are contiguous in the
// sorted order, so each worker reduces contiguous same-cluster segments on
// chip and touches global memory only at segment boundaries.  Re-designed for
// CDNA4 with no atomics at all:
//   * the sorted order is cut into tiles (kSegTile positions, fewer for a
//     small N); one "lane group" (G lanes, 16 bytes of a row each) walks a
//     tile in order, gathering X[perm[i]] rows and accumulating in fp32
//     registers;
//   * a segment that starts and ends inside the tile is finished right there
//     (mean written, or added to the running totals when streaming);
//   * a segment cut by a tile edge leaves a partial sum in one of the tile's
//     two carry slots (slot 0: the tile's first id, slot 1: its last id);
//   * the fix-up pass gives every cut segment one workgroup that adds its
//     carry pieces in a fixed order (strided per thread row, then a fixed
//     tree), so results do not depend on scheduling.
// Atomic count: zero, against the page's O((K + N/B_N) d) boundary atomics.
#include "frag_emit.hpp"
#include "km_internal.hpp"
#include "rows.hpp"

namespace km {

static int64_t reduce_lanes(int dt, int64_t D) {  // G: lanes holding one row (16 bytes each)
  const int64_t epl = dt == DT_F32 ? 4 : 8;
  const int64_t nch = (D + epl - 1) / epl;
  int64_t g = 1;
  while (g < nch && g < 64) g <<= 1;
  return g;
}

int64_t reduce_tpb(int dt, int64_t D) { return 256 / reduce_lanes(dt, D); }

static bool seg_fine(int G, int64_t N) {
  const int ov = plan_override().reduce_tile;
  return ov == 2 || (ov != 1 && N * G * 16 <= seg_fine_max_bytes());
}

int64_t reduce_tile(int dt, int64_t D, int64_t N) {
  const int G = (int)reduce_lanes(dt, D);
  return seg_fine(G, N) ? seg_tile_fine(G) : kSegTile;
}

int64_t reduce_carry_tiles(int dt, int64_t D, int64_t N) {
  const int G = (int)reduce_lanes(dt, D);
  const int64_t fine = seg_tile_fine(G);
  if (seg_fine(G, N)) return (N + fine - 1) / fine;
  const int64_t coarse = (N + kSegTile - 1) / kSegTile;
  if (plan_override().reduce_tile == 1) return coarse;
  const int64_t most_fine_n = seg_fine_max_bytes() / (16 * G);  // largest short-tile N
  const int64_t most_fine = (most_fine_n + fine - 1) / fine;
  return coarse > most_fine ? coarse : most_fine;
}

// A carry piece holds one column strip of a row: G lanes x 16 bytes (rows
// longer than 64 such pieces are reduced strip by strip, see reduce_strips).
int64_t reduce_dc(int dt, int64_t D) {
  const int64_t epl = dt == DT_F32 ? 4 : 8;
  return reduce_lanes(dt, D) * epl;
}

// Column strips of the segmented reduction: rows of at most 64 16-byte pieces
// (512 16-bit / 256 fp32 values) are one strip; longer rows are cut into
// strips of that width, each reduced by its own segmented-reduction and
// fix-up launches over the same sorted order (the sorted ids and indices are
// re-read per strip, a small fraction of the row bytes).
int64_t reduce_strips(int dt, int64_t D) {
  const int64_t w = reduce_dc(dt, D);
  return (D + w - 1) / w;
}

struct SegParams {
  const uint8_t* X;  // this strip's first column of row 0
  int dt;
  int64_t N;
  int D;             // columns of this strip
  int64_t ldx;       // row stride of X and of the centroid arrays, in elements (the full D)
  bool first_strip;  // counts are added to running totals by the first strip only
  int64_t K;
  bool vec_ok;  // X rows and the output rows are whole 16-byte pieces, 16-byte aligned
  const int32_t* keys;
  const int32_t* vals;
  int32_t* off;  // K+1 cluster offsets, written by the segmented reduction
  float* carry_sum;
  int32_t* carry_cnt;
  float* group_sum;   // [blocks][Dc]: a segment-reduce workgroup's slot-0 pieces, summed, when its positions hold one id
  int32_t* group_cnt;
  int tpb;            // tiles per segment-reduce workgroup
  int tile;           // sorted positions per tile (reduce_tile)
  // mean mode, optional: FlashAssign's operand fragments of the new centroids
  // (cluster k is centroid k % kper of problem k / kper, whose fragments start
  // f_stride 16-byte slots further), written by the fix-up
  uint32_t* frag;
  int64_t f_stride, kper;
  AssignCfg cfg;
  int Dc;
  int mode;
  int cpw;  // fix-up: clusters screened per wavefront (1: a wavefront per cluster)
  const float* C_prev;
  float* C_new;
  int32_t* counts;
  float* acc_sum;
  int64_t* acc_cnt;
};

// Write a finished segment (or a carry piece) held by one lane group.  A
// segment is finished here when it both starts and ends inside this tile
// (`complete`, known from the id changes the walk has seen).  A lane's EPL
// consecutive values leave as 16-byte stores: always for a carry piece, and
// for a finished mean when the rows are whole 16-byte pieces with 16-byte
// aligned outputs (VEC) and span at least 8 lanes (measured on gfx950: one
// 4-byte store per value, strided over the row, made c3's 65,536 short
// segments cost 1.4x; narrower rows would lose a wavefront per SIMD to the
// extra registers).
template <int EPL, int CPL, int G, bool VEC>
__device__ __forceinline__ void flush_piece(const SegParams& P, int64_t tile, int32_t first_key, int32_t k,
                                            bool complete, const float (&acc)[CPL][EPL], int32_t cnt, int j) {
  static_assert(EPL % 4 == 0, "a lane's values are whole 16-byte pieces");
  if (k < 0 || k >= P.K) return;  // sorted ids lie in [0, K)
  if (complete) {
    if (P.mode == MODE_MEAN) {
      if (j == 0 && P.counts) P.counts[k] = cnt;
      const float fcnt = (float)cnt;
#pragma unroll
      for (int q = 0; q < CPL; ++q) {
        const int c0 = (j + q * G) * EPL;
        if (VEC && G >= 8 && cnt > 0 && c0 + EPL <= P.D) {
          float4* dst = reinterpret_cast<float4*>(P.C_new + (int64_t)k * P.ldx + c0);
#pragma unroll
          for (int x = 0; x < EPL; x += 4)
            dst[x / 4] = make_float4(acc[q][x] / fcnt, acc[q][x + 1] / fcnt, acc[q][x + 2] / fcnt,
                                     acc[q][x + 3] / fcnt);
        } else {
#pragma unroll
          for (int x = 0; x < EPL; ++x) {
            const int c = c0 + x;
            if (c < P.D) {
              const int64_t o = (int64_t)k * P.ldx + c;
              P.C_new[o] = cnt > 0 ? acc[q][x] / fcnt : P.C_prev[o];
            }
          }
        }
      }
    } else {
      if (j == 0 && P.first_strip) P.acc_cnt[k] += cnt;
#pragma unroll
      for (int q = 0; q < CPL; ++q) {
        const int c0 = (j + q * G) * EPL;
#pragma unroll
        for (int x = 0; x < EPL; ++x) {
          const int c = c0 + x;
          if (c < P.D) P.acc_sum[(int64_t)k * P.ldx + c] += acc[q][x];
        }
      }
    }
  } else {  // cut by a tile edge: leave a carry piece (Dc floats, 16-byte aligned)
    const int slot = k == first_key ? 0 : 1;
    float* dst = P.carry_sum + (tile * 2 + slot) * (int64_t)P.Dc;
    if (j == 0) P.carry_cnt[tile * 2 + slot] = cnt;
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      float4* d4 = reinterpret_cast<float4*>(dst + (j + q * G) * EPL);
#pragma unroll
      for (int x = 0; x < EPL; x += 4) d4[x / 4] = make_float4(acc[q][x], acc[q][x + 1], acc[q][x + 2], acc[q][x + 3]);
    }
  }
}

// VEC: X rows are whole, 16-byte aligned chunks (vector loads without a per-row fallback).
// FINE: short tiles (seg_tile_fine) with more rows in flight, for small N.
template <int ES, int CPL, int G, bool VEC, bool FINE>
__global__ __launch_bounds__(256) void segment_reduce_kernel(SegParams P) {
  static_assert(CPL == 1, "a lane holds one 16-byte column chunk");
  constexpr int EPL = 16 / ES;
  // The ids and point indices of a whole chunk of the tile (KPL per lane, up
  // to 16) are read in one round trip; the chunk's rows then go out U at a
  // time in a fully unrolled walk, so the next rows can be in flight while
  // the current ones are added.
  constexpr int TILE = FINE ? seg_tile_fine(G) : kSegTile;
  constexpr int KPL = TILE / G < 16 ? TILE / G : 16;
  constexpr int BATCH = G * KPL;
  // rows in flight per lane group: with kSegTile-long tiles, half the lane
  // group's width, at least 2 (measured on gfx950: more rows cost occupancy
  // at large N, c2 G=16 best at 8, c4 G=8 at 4); with short tiles (small N,
  // occupancy to spare) up to KM_SEG_FINE_U, so a lane group needs few rounds
  constexpr int UC = G / 2 < 2 ? 2 : (G / 2 > KM_SEG_U ? KM_SEG_U : G / 2);
  constexpr int UF = KM_SEG_FINE_U < BATCH ? KM_SEG_FINE_U : BATCH;
  constexpr int U = FINE ? UF : UC;
  static_assert(U >= 1 && BATCH % U == 0 && TILE % BATCH == 0, "rows in flight divide the chunk");
  const int j = threadIdx.x % G;
  const int lgbase = (threadIdx.x & 63) & ~(G - 1);
  constexpr int T = 256 / G;  // tiles per workgroup
  const int64_t tile = (int64_t)blockIdx.x * T + threadIdx.x / G;
  const int64_t ps = tile * TILE;
  // A workgroup whose positions all hold one id sums its tiles' pieces at the
  // end (one piece for the fix-up instead of T); it keeps every thread until then.
  const int64_t bps = (int64_t)blockIdx.x * T * TILE;
  const int64_t bpe = bps + (int64_t)T * TILE < P.N ? bps + (int64_t)T * TILE : P.N;
  const bool solid = P.keys[bps] == P.keys[bpe - 1];
  if (ps >= P.N && !solid) return;
  if (ps < P.N) {
    const int64_t pe = ps + TILE < P.N ? ps + TILE : P.N;
    const int32_t first_key = P.keys[ps];
    const int32_t before_key = ps > 0 ? P.keys[ps - 1] : -1;   // id just before the tile
    const int32_t after_key = pe < P.N ? P.keys[pe] : -1;      // id just after the tile

    // Cluster offsets: off[k] = first sorted position with id >= k.  Every id
    // change between positions p-1 and p is seen by exactly one lane group
    // (the one whose tile holds p), which writes off[(id before, id at p]] = p.
    auto write_offsets = [&](int64_t a, int64_t b, int64_t p) {
      if (j != 0) return;
      a = a < -1 ? -1 : (a >= P.K ? P.K : a);  // sorted ids lie in [0, K); clamping keeps writes in bounds
      b = b < -1 ? -1 : (b >= P.K ? P.K : b);
      for (int64_t k = a + 1; k <= b; ++k) P.off[k] = (int32_t)p;
    };
    if (before_key != first_key) write_offsets(before_key, first_key, ps);

    float acc[CPL][EPL];
#pragma unroll
    for (int q = 0; q < CPL; ++q)
#pragma unroll
      for (int x = 0; x < EPL; ++x) acc[q][x] = 0.0f;
    int32_t cnt = 0;
    int32_t cur = first_key;
    bool started = before_key != first_key;  // the current segment began inside this tile

    for (int64_t p0 = ps; p0 < pe; p0 += BATCH) {
      // lane j holds positions p0 + j + G*m, m < KPL
      int32_t kj[KPL], vj[KPL];
#pragma unroll
      for (int m = 0; m < KPL; ++m) {
        const int64_t mypos = p0 + j + (int64_t)G * m;
        kj[m] = mypos < pe ? P.keys[mypos] : 0;
        vj[m] = mypos < pe ? P.vals[mypos] : (int32_t)kInvalidFlag;
      }
#pragma unroll
      for (int b0 = 0; b0 < BATCH; b0 += U) {
        if (p0 + b0 >= pe) break;
        u32x4_r xr[U][CPL];
        int32_t kk[U];
        bool ok[U], in[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int b = b0 + u;  // batch position: lane b % G, slot b / G
          const int32_t v = __shfl(vj[b / G], lgbase + b % G);
          kk[u] = __shfl(kj[b / G], lgbase + b % G);
          in[u] = p0 + b < pe;
          const int64_t row = (int64_t)((uint32_t)v & ~kInvalidFlag);
          ok[u] = in[u] && v >= 0 && row < P.N;
#pragma unroll
          for (int q = 0; q < CPL; ++q) {
            const int c0 = (j + q * G) * EPL;
            if constexpr (VEC) {  // whole 16-byte chunks: one unconditional load, masked after
              const int64_t rr = ok[u] ? row : 0;
              const int cc = c0 < P.D ? c0 : 0;
              const u32x4_r w = *reinterpret_cast<const u32x4_r*>(P.X + ((size_t)rr * (size_t)P.ldx + (size_t)cc) * ES);
              xr[u][q] = (ok[u] && c0 < P.D) ? w : u32x4_r{0u, 0u, 0u, 0u};
            } else {
              xr[u][q] = ok[u] ? load_chunk<ES>(P.X, row, P.D, c0, false, P.ldx) : u32x4_r{0u, 0u, 0u, 0u};
            }
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (in[u]) {
            if (kk[u] != cur) {  // the current segment ends inside the tile
              write_offsets(cur, kk[u], p0 + b0 + u);
              flush_piece<EPL, CPL, G, VEC>(P, tile, first_key, cur, started, acc, cnt, j);
              cur = kk[u];
              cnt = 0;
              started = true;
#pragma unroll
              for (int q = 0; q < CPL; ++q)
#pragma unroll
                for (int x = 0; x < EPL; ++x) acc[q][x] = 0.0f;
            }
            cnt += ok[u] ? 1 : 0;
#pragma unroll
            for (int q = 0; q < CPL; ++q) {
              float f[EPL];
              widen(xr[u][q], P.dt, f);
#pragma unroll
              for (int x = 0; x < EPL; ++x) acc[q][x] += f[x];
            }
          }
        }
      }
    }
    flush_piece<EPL, CPL, G, VEC>(P, tile, first_key, cur, started && after_key != cur, acc, cnt, j);
    if (pe == P.N) write_offsets(cur, P.K, P.N);  // ids after the last one start (and end) at N
  }
  if (!solid) return;
  __syncthreads();  // the workgroup's pieces are stored
  if (threadIdx.x >= 64) return;
  // wavefront 0: rows of G lanes take the tiles r, r + R, ... in order, then a fixed tree
  constexpr int R = 64 / G;
  const int r = threadIdx.x / G;
  const int64_t t_end = (bpe + TILE - 1) / TILE;
  float sum[EPL];
#pragma unroll
  for (int x = 0; x < EPL; ++x) sum[x] = 0.0f;
  int32_t n = 0;
  for (int64_t t = (int64_t)blockIdx.x * T + r; t < t_end; t += R) {
    const float4* src = reinterpret_cast<const float4*>(P.carry_sum + (t * 2) * (int64_t)P.Dc + j * EPL);
#pragma unroll
    for (int x = 0; x < EPL; x += 4) {
      const float4 w = src[x / 4];
      sum[x] += w.x;
      sum[x + 1] += w.y;
      sum[x + 2] += w.z;
      sum[x + 3] += w.w;
    }
    n += P.carry_cnt[t * 2];
  }
  for (int off = G; off < 64; off <<= 1) {
#pragma unroll
    for (int x = 0; x < EPL; ++x) sum[x] += __shfl_xor(sum[x], off);
    n += __shfl_xor(n, off);
  }
  if (r == 0) {
    float4* dst = reinterpret_cast<float4*>(P.group_sum + (int64_t)blockIdx.x * P.Dc + j * EPL);
#pragma unroll
    for (int x = 0; x < EPL; x += 4) dst[x / 4] = make_float4(sum[x], sum[x + 1], sum[x + 2], sum[x + 3]);
    if (j == 0) P.group_cnt[blockIdx.x] = n;
  }
}

// Segments cut by tile edges are summed from their pieces; empty clusters
// keep their centroid.  One wavefront per cluster.  The pieces of cluster k,
// tiles t0..t1, are taken as: the head tiles up to the end of t0's
// segment-reduce workgroup, then every whole workgroup up to the one holding
// t1 (one piece each, summed by that workgroup since all its positions hold
// k), then the tail tiles of t1's workgroup.
// Lanes split into R rows x (Dc/4) float4 columns; row r takes items r,
// r + R, ... of that list in order and the rows are combined by a fixed
// shuffle tree, so the order of additions never depends on scheduling.
// Cluster k's segment [s, e) of the sorted positions and its tiles t0..t1.
struct FixupSeg {
  int64_t s, e, t0, t1;
  bool valid, cut;
};

__device__ __forceinline__ FixupSeg fixup_seg(const SegParams& P, int64_t k) {
  FixupSeg g;
  const bool active = k < P.K;
  g.s = active ? P.off[k] : 0;
  g.e = active ? P.off[k + 1] : 0;
  g.valid = active && g.s >= 0 && g.e <= P.N && g.s <= g.e;  // offsets are monotone in [0, N]
  g.t0 = g.s / P.tile;
  g.t1 = g.e > g.s ? (g.e - 1) / P.tile : g.t0;
  g.cut = g.valid && g.s < g.e && g.t0 != g.t1;  // otherwise empty, or finished by segment_reduce_kernel
  return g;
}

// One wavefront completes cluster k: an empty cluster keeps its centroid, a
// segment cut by tile edges is summed from its pieces (row: the wavefront's
// LDS row, filled with the new mean when fragments are written).
template <int CPL, int UNR>  // UNR: carry pieces in flight per lane
__device__ __forceinline__ void fixup_one(const SegParams& P, const FixupSeg& g, int64_t k, int lane, float* row) {
  const int gc = P.Dc / 4;                    // float4 columns of a carry piece (power of two, <= 128)
  const int lpr = gc < 64 ? gc : 64;          // lanes per row
  const int R = 64 / lpr;                     // rows
  constexpr int cpl = CPL;
  const int r = lane / lpr, c0 = lane % lpr;
  const int64_t s = g.s, e = g.e, t0 = g.t0, t1 = g.t1;
  if (g.valid && s == e && P.mode == MODE_MEAN) {  // empty: keeps its centroid
    if (lane == 0 && P.counts) P.counts[k] = 0;
    if (P.C_new != P.C_prev)
      for (int c = lane; c < P.D; c += 64) P.C_new[k * P.ldx + c] = P.C_prev[k * P.ldx + c];
  }
  if (g.cut) {
    // item list: head tiles [t0, hb), whole groups [g0, g1), tail tiles [tb, t1]
    const int64_t T = P.tpb;
    int64_t hb = (t0 / T + 1) * T;
    const int64_t tb = (t1 / T) * T;
    int64_t g0 = hb / T, g1 = tb / T;
    if (hb > tb) {  // t0 and t1 in the same or adjacent groups: tiles only
      hb = t1 + 1;
      g0 = g1 = 0;
    }
    const int64_t nh = hb - t0, ng = g1 - g0, nt = hb > tb ? 0 : t1 - tb + 1;
    const int64_t nitems = nh + ng + nt;
    float a[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    int32_t n = 0;
    for (int64_t ib = r; ib < nitems; ib += (int64_t)R * UNR) {
      float4 v[UNR][2];
      int32_t cc[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int64_t it = ib + (int64_t)u * R;
        cc[u] = 0;
        v[u][0] = v[u][1] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (it < nitems) {
          const float* piece;
          if (it < nh || it >= nh + ng) {
            const int64_t t = it < nh ? t0 + it : tb + (it - nh - ng);
            const int slot = (t == t0 && s != t0 * P.tile) ? 1 : 0;
            piece = P.carry_sum + (t * 2 + slot) * (int64_t)P.Dc;
            cc[u] = P.carry_cnt[t * 2 + slot];
          } else {
            const int64_t gi = g0 + (it - nh);
            piece = P.group_sum + gi * (int64_t)P.Dc;
            cc[u] = P.group_cnt[gi];
          }
#pragma unroll
          for (int cl = 0; cl < cpl; ++cl) v[u][cl] = *reinterpret_cast<const float4*>(piece + (c0 + cl * lpr) * 4);
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {  // ascending item order within the row
#pragma unroll
        for (int cl = 0; cl < 2; ++cl) {
          a[cl][0] += v[u][cl].x;
          a[cl][1] += v[u][cl].y;
          a[cl][2] += v[u][cl].z;
          a[cl][3] += v[u][cl].w;
        }
        n += cc[u];
      }
    }
    for (int off = lpr; off < 64; off <<= 1) {  // fixed tree over the rows
#pragma unroll
      for (int cl = 0; cl < 2; ++cl)
#pragma unroll
        for (int x = 0; x < 4; ++x) a[cl][x] += __shfl_xor(a[cl][x], off);
      n += __shfl_xor(n, off);
    }
    if (r == 0) {
#pragma unroll
      for (int cl = 0; cl < cpl; ++cl)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int c = (c0 + cl * lpr) * 4 + x;
          if (c >= P.D) continue;
          const int64_t o = k * P.ldx + c;
          if (P.mode == MODE_MEAN) {
            const float m = n > 0 ? a[cl][x] / (float)n : P.C_prev[o];
            P.C_new[o] = m;
            if (P.frag) row[c] = m;
          } else {
            P.acc_sum[o] += a[cl][x];
          }
        }
      if (c0 == 0) {
        if (P.mode == MODE_MEAN) {
          if (P.counts) P.counts[k] = n;
        } else if (P.first_strip) {
          P.acc_cnt[k] += n;
        }
      }
    }
  }
}

// Without fragments to write (P.cpw > 1), a wavefront screens P.cpw
// consecutive clusters, one lane each, and completes only those that are cut
// or empty, one after another: at 65,536 clusters of ~16 points most
// segments were finished by the segmented reduction, and a wavefront per
// cluster cost more to launch than the work (measured on gfx950 at c3's
// shape: see fixup_cpw).  With fragments every cluster's row is needed:
// one wavefront per cluster.
template <int CPL, int UNR>  // float4 columns per lane: 2 only when a piece has 128 of them
__global__ __launch_bounds__(256) void fixup_kernel(SegParams P) {
  __shared__ float rows[4][kMaxD16];  // each wavefront's final row, for the operand fragments
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* row = rows[wave];
  if (P.cpw > 1) {  // (uniform; never with fragments)
    const int64_t k0 = ((int64_t)blockIdx.x * 4 + wave) * P.cpw;
    bool need = false;
    if (lane < P.cpw) {
      const FixupSeg g = fixup_seg(P, k0 + lane);
      need = g.cut || (g.valid && g.s == g.e && P.mode == MODE_MEAN);
    }
    uint64_t m = __ballot(need);
    while (m) {  // wave-uniform
      const int i = __builtin_ctzll(m);
      m &= m - 1;
      fixup_one<CPL, UNR>(P, fixup_seg(P, k0 + i), k0 + i, lane, row);
    }
    return;
  }
  const int64_t k = (int64_t)blockIdx.x * 4 + wave;
  // (no early return: with fragments to write every wavefront meets the barrier below)
  const FixupSeg g = fixup_seg(P, k);
  fixup_one<CPL, UNR>(P, g, k, lane, row);
  if (!P.frag) return;  // (uniform: mean mode with a fragment buffer)
  // The new centroid's row: from the sums above, else as the segmented
  // reduction (finished clusters) or the empty rule (C_prev) left it.
  if (g.valid && !g.cut) {
    const float* src = g.s == g.e ? P.C_prev : P.C_new;
    for (int c = lane; c < P.D; c += 64) row[c] = src[k * P.ldx + c];
  }
  __syncthreads();
  if (g.valid) {
    const int64_t b = k / P.kper;
    emit_fragment_row(row, P.D, P.dt, P.cfg, P.frag + 4 * b * P.f_stride, k - b * P.kper);
  }
}

static SegParams make_params(const ReduceArgs& a) {
  SegParams P;
  const int es = dtype_size(a.dt);
  const int64_t sw = reduce_dc(a.dt, a.D);  // strip width in columns
  const int64_t c0 = a.strip * sw;          // first column of this strip
  P.X = (const uint8_t*)a.X + c0 * es;
  P.dt = a.dt;
  P.N = a.N;
  P.D = (int)(a.D - c0 < sw ? a.D - c0 : sw);
  P.ldx = a.D;
  P.first_strip = a.strip == 0;
  P.K = a.K;
  P.vec_ok = (((uintptr_t)a.X) % 16 == 0) && ((a.D * es) % 16 == 0);
  P.keys = a.keys;
  P.vals = a.vals;
  P.off = a.off;
  P.carry_sum = a.carry_sum;
  P.carry_cnt = a.carry_cnt;
  P.group_sum = a.group_sum;
  P.group_cnt = a.group_cnt;
  P.tpb = (int)reduce_tpb(a.dt, a.D);
  P.tile = (int)reduce_tile(a.dt, a.D, a.N);
  P.frag = a.mode == MODE_MEAN && reduce_strips(a.dt, a.D) == 1 ? (uint32_t*)a.frag : nullptr;
  P.f_stride = a.f_stride;
  P.kper = a.kper > 0 ? a.kper : a.K;
  P.cfg = a.cfg;
  P.Dc = (int)reduce_dc(a.dt, a.D);
  P.mode = a.mode;
  P.cpw = 1;
  P.C_prev = a.C_prev ? a.C_prev + c0 : nullptr;
  P.C_new = a.C_new ? a.C_new + c0 : nullptr;
  P.counts = a.counts;
  P.acc_sum = a.acc_sum ? a.acc_sum + c0 : nullptr;
  P.acc_cnt = a.acc_cnt;
  auto al16 = [](const void* q) { return q == nullptr || ((uintptr_t)q) % 16 == 0; };
  P.vec_ok = P.vec_ok && al16(P.C_new) && al16(P.C_prev) && al16(P.acc_sum);
  return P;
}

template <int ES, int CPL, int G>
static void launch_seg(const SegParams& P, hipStream_t s) {
  const int64_t ntiles = (P.N + P.tile - 1) / P.tile;
  const int64_t per_block = 256 / G;
  const dim3 grid((unsigned)((ntiles + per_block - 1) / per_block));
  const bool fine = seg_fine(G, P.N);  // (P.tile is reduce_tile of the same N)
  if (P.vec_ok && fine)
    hipLaunchKernelGGL((segment_reduce_kernel<ES, CPL, G, true, true>), grid, dim3(256), 0, s, P);
  else if (P.vec_ok)
    hipLaunchKernelGGL((segment_reduce_kernel<ES, CPL, G, true, false>), grid, dim3(256), 0, s, P);
  else if (fine)
    hipLaunchKernelGGL((segment_reduce_kernel<ES, CPL, G, false, true>), grid, dim3(256), 0, s, P);
  else
    hipLaunchKernelGGL((segment_reduce_kernel<ES, CPL, G, false, false>), grid, dim3(256), 0, s, P);
}

hipError_t launch_segment_reduce(const ReduceArgs& a, hipStream_t stream) {
  if (a.N == 0) return hipSuccess;
  if (a.strip < 0 || a.strip >= reduce_strips(a.dt, a.D)) return hipErrorInvalidValue;
  const SegParams P = make_params(a);
  const int es = dtype_size(a.dt);
  // every strip of a row takes the lane-group width of a whole strip (a narrower last strip leaves lanes idle),
  // so all strips share one tile length and carry layout
  const int g = (int)reduce_lanes(a.dt, a.D);
#define KM_SEG(ES_, G_) \
  if (es == ES_ && g == G_) { launch_seg<ES_, 1, G_>(P, stream); return hipGetLastError(); }
  KM_SEG(2, 1) KM_SEG(2, 2) KM_SEG(2, 4) KM_SEG(2, 8) KM_SEG(2, 16) KM_SEG(2, 32) KM_SEG(2, 64)
  KM_SEG(4, 1) KM_SEG(4, 2) KM_SEG(4, 4) KM_SEG(4, 8) KM_SEG(4, 16) KM_SEG(4, 32) KM_SEG(4, 64)
#undef KM_SEG
  return hipErrorInvalidValue;
}

// Clusters screened per fix-up wavefront when no fragments are written: enough
// wavefronts for 8 per compute unit, at most 64 clusters each (measured on
// gfx950 at c3's shape, 65,536 clusters: 26.8 us with a wavefront per
// cluster; 28.6, 19.2, 20.3, 21.0 and 25.7 us with 4, 8, 16, 32 and 64
// wavefronts per compute unit).
static int fixup_cpw(int64_t K) {
  const int64_t target = 8 * device_info().cus;
  const int64_t c = K / (target > 0 ? target : 1);
  return c < 1 ? 1 : (c > 64 ? 64 : (int)c);
}

hipError_t launch_fixup(const ReduceArgs& a, hipStream_t stream) {
  if (a.K == 0) return hipSuccess;
  SegParams P = make_params(a);
  P.cpw = P.frag ? 1 : fixup_cpw(a.K);
  const bool wide = P.Dc / 4 > 64;
  const int64_t waves = (a.K + P.cpw - 1) / P.cpw;
  const dim3 grid((unsigned)((waves + 3) / 4));
  // Carry pieces in flight per lane: 8 where a row of lanes spans at least 32 float4 columns (two rows or one a
  // wavefront), else 4 (measured on gfx950: c2, D = 128, 12.4 -> 10.8 us with 8; c4, D = 64, four rows a
  // wavefront, 14.3 -> 18.4 us with 8).
  const bool deep = P.Dc / 4 >= 32;
  if (wide)
    hipLaunchKernelGGL((fixup_kernel<2, 8>), grid, dim3(256), 0, stream, P);
  else if (deep)
    hipLaunchKernelGGL((fixup_kernel<1, 8>), grid, dim3(256), 0, stream, P);
  else
    hipLaunchKernelGGL((fixup_kernel<1, 4>), grid, dim3(256), 0, stream, P);
  return hipGetLastError();
}

// ------------------------------------------------------------- streaming --

__global__ void finalize_accum_kernel(const float* __restrict__ acc_sum, const int64_t* __restrict__ acc_cnt,
                                      int64_t K, int64_t D, float* __restrict__ C, int32_t* __restrict__ counts) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= K * D) return;
  const int64_t k = i / D;
  const int64_t n = acc_cnt[k];
  if (n > 0) C[i] = acc_sum[i] / (float)n;
  if (counts && i % D == 0) counts[k] = (int32_t)n;
}

hipError_t launch_finalize_accum(const float* acc_sum, const int64_t* acc_cnt, int64_t K, int64_t D, float* C,
                                 int32_t* counts, hipStream_t stream) {
  const int64_t n = K * D;
  const int tpb = 256;
  hipLaunchKernelGGL(finalize_accum_kernel, dim3((unsigned)((n + tpb - 1) / tpb)), dim3(tpb), 0, stream, acc_sum,
                     acc_cnt, K, D, C, counts);
  return hipGetLastError();
}

__global__ void zero_kernel(uint32_t* __restrict__ p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// Fill with zeros by a kernel (never hipMemsetAsync, so callers may capture it in a graph).
hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream) {
  const int64_t words = (int64_t)(bytes / 4);
  if (words == 0) return hipSuccess;
  int64_t blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint32_t*)p, words);
  return hipGetLastError();
}

// ------------------------------------------------------------- objective --

constexpr int kObjThreads = 256;
constexpr int kObjItems = 16;

__global__ __launch_bounds__(kObjThreads) void objective_partial_kernel(const float* __restrict__ v, int64_t n,
                                                                        double* __restrict__ part) {
  __shared__ double red[kObjThreads];
  const int64_t base = ((int64_t)blockIdx.x * kObjThreads + threadIdx.x) * kObjItems;
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < kObjItems; ++i)
    if (base + i < n) s += (double)v[base + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int st = kObjThreads / 2; st > 0; st >>= 1) {
    if ((int)threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(kObjThreads) void objective_final_kernel(const double* __restrict__ part, int64_t np,
                                                                      double* __restrict__ out, int accumulate) {
  __shared__ double red[kObjThreads];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < np; i += kObjThreads) s += part[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int st = kObjThreads / 2; st > 0; st >>= 1) {
    if ((int)threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = (accumulate ? out[0] : 0.0) + red[0];
}

int64_t objective_partials(int64_t n) {
  const int64_t per = (int64_t)kObjThreads * kObjItems;
  return (n + per - 1) / per + 1;
}

hipError_t launch_objective(const float* v, int64_t n, double* partials, double* out, int accumulate,
                            hipStream_t stream) {
  const int64_t per = (int64_t)kObjThreads * kObjItems;
  const int64_t np = (n + per - 1) / per;
  if (np > 0)
    hipLaunchKernelGGL(objective_partial_kernel, dim3((unsigned)np), dim3(kObjThreads), 0, stream, v, n, partials);
  hipLaunchKernelGGL(objective_final_kernel, dim3(1), dim3(kObjThreads), 0, stream, (const double*)partials, np, out,
                     accumulate);
  return hipGetLastError();
}

// One workgroup per problem: a strided fp64 sum per thread, then a fixed tree.
__global__ __launch_bounds__(kObjThreads) void objective_batched_kernel(const float* __restrict__ v, int64_t n,
                                                                        double* __restrict__ out) {
  __shared__ double red[kObjThreads];
  const float* vb = v + (int64_t)blockIdx.x * n;
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += kObjThreads) s += (double)vb[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int st = kObjThreads / 2; st > 0; st >>= 1) {
    if ((int)threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

hipError_t launch_objective_batched(const float* v, int64_t B, int64_t n, double* out, hipStream_t stream) {
  if (B < 1 || B >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(objective_batched_kernel, dim3((unsigned)B), dim3(kObjThreads), 0, stream, v, n, out);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void local_ids_kernel(const int32_t* __restrict__ ids, int64_t total, int64_t n,
                                                        int64_t K, int32_t* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256)
    out[i] = (int32_t)((int64_t)ids[i] - (i / n) * K);
}

hipError_t launch_local_ids(const int32_t* ids, int64_t B, int64_t n, int64_t K, int32_t* out, hipStream_t stream) {
  const int64_t total = B * n;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(local_ids_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, ids, total, n, K, out);
  return hipGetLastError();
}

}  // namespace km
