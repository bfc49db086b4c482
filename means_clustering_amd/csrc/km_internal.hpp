// Internal declarations shared by the HIP translation units of the K-Means
// library (gfx950 / MI355X only).  Nothing here is part of the C ABI.
//
// Citations name the page "Flash-KMeans: Fast and Memory-Efficient Exact
// K-Means" (gist.science summary of paper 2603.09229); "tech §n" is a section
// of its technical summary.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace km {

enum Dtype : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

inline int dtype_size(int dt) { return dt == DT_F32 ? 4 : 2; }

// ---------------------------------------------------------------------------
// Centroid fragments.  The contraction x . c runs on the matrix cores with the
// centroids as the A operand and the points as the B operand.  Two layouts:
//   * 16-bit X ("wide"): v_mfma_f32_32x32x16_{bf16,f16}; a centroid group is
//     32 rows, a fragment block covers 32 rows x 16 depth values (lane l:
//     row l % 32, depth 16*kb + 8*(l/32) .. +7, 16 bytes);
//   * fp32 X ("narrow"): four v_mfma_f32_16x16x4_f32; a group is 16 rows, a
//     fragment block covers 16 rows x 16 depth values (lane l: row l % 16,
//     depth 16*kb + 4*(l/16) .. +3, 16 bytes).
// A group is stored as its KB fragment blocks (64 lanes x 16 bytes each),
// then its bias values -||c||^2/2 (32 or 16 floats, in the order the lanes
// read them).  Groups are packed into tiles of CT groups, each tile padded to
// a whole number of 16-byte copies per thread, so streaming a tile into LDS
// is one contiguous, unconditional copy and every LDS read is lane-linear.
// ---------------------------------------------------------------------------
constexpr int kFragDepth = 16;     // depth values per fragment block (both layouts)
constexpr int kPadK = 128;         // 16-bit X: K is padded to a multiple of this (>= any tile)
constexpr int kMaxD16 = 512;       // longest 16-bit rows kept whole in registers / one lane group
constexpr int kMaxD32 = 256;       // ... fp32 rows
constexpr int64_t kMaxD = (int64_t)1 << 24;  // longest rows accepted at all (32-bit index arithmetic)
// Rows longer than the register-resident limit take the depth-tiled FlashAssign
// (both operands staged per depth chunk) and a segmented reduction in column
// strips of kMaxD16 / kMaxD32 values.
inline bool deep_rows(int dt, int64_t D) { return D > (dt == DT_F32 ? kMaxD32 : kMaxD16); }

// ---------------------------------------------------------------------------
// The device a plan is made for.  The launch shapes below follow from the
// number of compute units (how many workgroups fill the GPU) and from the
// size of the last-level cache (below which a gathered walk over the rows is
// bound by latency rather than bandwidth).  Both are read once per device:
// hipDeviceGetAttribute, and the KFD topology for the last-level cache, which
// HIP does not report.  A query that no device answers (a workspace-size call
// on a machine without a GPU) gets the MI355X values.
// ---------------------------------------------------------------------------
struct DeviceInfo {
  int cus;            // compute units (256 on MI355X)
  int64_t lds_bytes;  // LDS per compute unit (160 KiB)
  int64_t l2_bytes;   // L2 as HIP reports it (4 MiB, per XCD)
  int64_t llc_bytes;  // last-level cache (256 MiB Infinity Cache); the L2 if no larger level is found
  bool queried;       // false: the MI355X defaults
  const char* llc_from;  // where llc_bytes came from: "KFD topology", "gfx950", "L2" or "defaults"
};
const DeviceInfo& device_info();  // of the calling thread's current device

// Overrides of the planner's choices, for the planner study: 0 keeps the
// planner's choice.  Process-wide; set between calls, not during one.
struct PlanOverride {
  int assign_kernel;  // 1 pipelined four-wavefront kernel, 2 single-accumulator kernel (16-bit X, D <= 128)
  int assign_fold;    // 1 exact argmax per score, 2 folded argmax (cold launches, 16-bit X)
  int assign_split;   // 1 never split the centroid sweep; n >= 2 split it into n ranges where it can be
  int reduce_tile;    // 1 long (128-position) segment tiles, 2 short ones
  int radix_items;    // keys per thread of the argsort: 8, 16 or 32
  int small_update;   // 1 no on-chip small-codebook update (always the sorted path)
  int sort_scan;      // 1 scan larger argsort count tables as a whole, 2 scan every count table digit by digit
  int sort_rank;      // 1 per-thread digit counters in the argsort's scatter, 2 wavefront ballots
  int radix_bits;     // widest digit of an argsort pass, 5 to 8 (above 6: wavefront ballots)
};
PlanOverride plan_override();

// Launch shape of one FlashAssign instantiation.
struct AssignCfg {
  int rows;   // centroids per group (32 wide, 16 narrow)
  int KB;     // fragment blocks per group
  int NB;     // point groups per wavefront (32 points wide, 16 narrow)
  int CT;     // centroid groups per LDS tile
  int W;      // wavefronts per workgroup
  constexpr int64_t bias_slots() const { return rows / 4; }
  constexpr int64_t group_slots() const { return (int64_t)KB * 64 + bias_slots(); }
  constexpr int64_t tile_slots() const {
    return (CT * group_slots() + W * 64 - 1) / (W * 64) * (W * 64);
  }
};

// Depth blocks actually instantiated for 16-bit X (D padded up to 16 * one of these).
constexpr int kWideKB[] = {1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 14, 16, 20, 24, 28, 32};

// Build-time knobs for tile sweeps (defaults are the shipped configuration).
#ifndef KM_WIDE_NB_SMALL
#define KM_WIDE_NB_SMALL 2  // point groups per wavefront for D <= 64
#endif
#ifndef KM_WIDE_NB_MID
#define KM_WIDE_NB_MID 2    // ... for 64 < D <= 128
#endif
#ifndef KM_WIDE_W
#define KM_WIDE_W 4         // wavefronts per workgroup
#endif
#ifndef KM_WIDE_CT
#define KM_WIDE_CT 2        // centroid groups per LDS tile for 64 < D <= 256 (even, divides 4)
#endif
#ifndef KM_WIDE_CT_SMALL
#define KM_WIDE_CT_SMALL 4  // ... for D <= 64
#endif
#ifndef KM_WIDE_WPE_SMALL
#define KM_WIDE_WPE_SMALL 3  // wavefronts per SIMD the four-wavefront kernel's registers are sized for, D <= 64
#endif
// (measured on gfx950: D = 64 fits 4 wavefronts per SIMD in 128 VGPRs and runs ~1.5% faster than with the
// compiler's default split at 2; D = 128 showed no difference, so it keeps the default)
constexpr int wide_wpe(int KB) { return KB <= 4 ? KM_WIDE_WPE_SMALL : 1; }
constexpr AssignCfg wide_cfg(int KB) {
  return AssignCfg{32, KB, KB <= 4 ? KM_WIDE_NB_SMALL : (KB <= 8 ? KM_WIDE_NB_MID : (KB <= 16 ? 2 : 1)),
                   KB <= 4 ? KM_WIDE_CT_SMALL : (KB <= 16 ? KM_WIDE_CT : 2), KM_WIDE_W};
}
// Single-accumulator layout for long centroid sweeps (D <= 128, at least 256
// groups of 32): four point groups per wavefront (each centroid fragment read
// from LDS feeds four MFMAs), two wavefronts per SIMD, tiles of 4 (D <= 128)
// or 8 (D <= 64) groups.  On gfx950 the matrix cores sustain more with fewer
// wavefronts holding more independent accumulators than with many wavefronts
// interleaving single chains; for short sweeps the pipelined four-wavefront
// kernel measured as fast or faster.
#ifndef KM_WIDE8
#define KM_WIDE8 1  // 0: always use the four-wavefront layout (for comparisons)
#endif
#ifndef KM_W8_NB
#define KM_W8_NB 4         // point groups per wavefront (64 < D <= 128)
#endif
#ifndef KM_W8_NB_SMALL
#define KM_W8_NB_SMALL 4   // ... (D <= 64)
#endif
#ifndef KM_W8_CT
#define KM_W8_CT 4         // groups per tile (64 < D <= 128)
#endif
#ifndef KM_W8_CT_SMALL
#define KM_W8_CT_SMALL 8   // ... (D <= 64)
#endif
#ifndef KM_W8_W
#define KM_W8_W 4          // wavefronts per workgroup
#endif
#ifndef KM_W8_WPE
#define KM_W8_WPE 2        // wavefronts per SIMD the register budget is sized for
#endif
constexpr int kWide8MaxKB = KM_WIDE8 ? 8 : 0;
constexpr AssignCfg wide8_cfg(int KB) {
  return AssignCfg{32, KB, KB <= 4 ? KM_W8_NB_SMALL : KM_W8_NB, KB <= 4 ? KM_W8_CT_SMALL : KM_W8_CT, KM_W8_W};
}
// Depth-tiled layout (deep_rows): tiles of 4 groups (128 centroids of 16-bit X,
// 64 of fp32), two point groups per wavefront, four wavefronts; the depth is
// walked in chunks of 4 fragment blocks (64 values).
constexpr int kDeepCT = 4, kDeepNB = 2, kDeepW = 4, kDeepKC = 4;
constexpr AssignCfg deep_cfg(int dt, int KB) {
  return AssignCfg{dt == DT_F32 ? 16 : 32, KB, kDeepNB, kDeepCT, kDeepW};
}
inline bool is_deep_cfg(int dt, const AssignCfg& c) { return c.KB > (dt == DT_F32 ? kMaxD32 : kMaxD16) / kFragDepth; }
// fp32 X.  `half`: tiles of half as many groups, so that a small K (e.g. 64)
// is not padded up to a whole 128-centroid tile.  `thin`: one point group per
// wavefront, for calls too small to fill the GPU otherwise (with half tiles).
constexpr AssignCfg narrow_cfg(int KB, bool half = false, bool thin = false) {
  return AssignCfg{16, KB, thin ? 1 : (KB <= 4 ? 4 : (KB <= 8 ? 2 : 1)),
                   (KB <= 2 ? 8 : (KB <= 4 ? 4 : (KB <= 8 ? 2 : 1))) / (half && KB <= 8 ? 2 : 1), 4};
}
constexpr int kNarrowHalfMaxKB = 8;
// fp32: one point group per wavefront when the usual layout would give fewer workgroups than compute units

inline int wide_kb(int64_t D) {
  const int need = (int)((D + kFragDepth - 1) / kFragDepth);
  for (int kb : kWideKB)
    if (kb >= need) return kb;
  return -1;
}
inline int64_t pad_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

struct AssignGeom {
  int dt;
  int64_t N, D, K;
  int64_t Kpad;    // K rounded up to a whole number of tiles
  AssignCfg cfg;
  bool lazy;       // argmax by group maxima first (pays off when the centroid sweep is long)
  int64_t groups() const { return Kpad / cfg.rows; }
  int64_t ntiles() const { return groups() / cfg.CT; }
  size_t frag_bytes() const { return (size_t)ntiles() * (size_t)cfg.tile_slots() * 16; }
};

#ifndef KM_LAZY_MIN_GROUPS
#define KM_LAZY_MIN_GROUPS 256  // cold launches fold the argmax from this many centroid groups of 32
#endif

// B: problems launched together (batched calls), for the choice of a thin layout.
inline AssignGeom make_assign_geom(int64_t N, int64_t D, int64_t K, int dt, int64_t B = 1) {
  AssignGeom g;
  g.dt = dt;
  g.N = N;
  g.D = D;
  g.K = K;
  g.Kpad = pad_up(K, kPadK);
  if (deep_rows(dt, D)) {
    g.cfg = deep_cfg(dt, (int)((D + kFragDepth - 1) / kFragDepth));
    g.Kpad = pad_up(K, (int64_t)g.cfg.rows * g.cfg.CT);
    g.lazy = false;
    return g;
  }
  if (dt == DT_F32) {
    const int kb = (int)((D + kFragDepth - 1) / kFragDepth);
    const AssignCfg full = narrow_cfg(kb), half = narrow_cfg(kb, true);
    const int64_t kp_full = pad_up(K, (int64_t)full.rows * full.CT);
    const int64_t kp_half = pad_up(K, (int64_t)half.rows * half.CT);
    const bool use_half = kb <= kNarrowHalfMaxKB && kp_half < kp_full;
    g.cfg = use_half ? half : full;
    g.Kpad = use_half ? kp_half : kp_full;
    const int64_t pts = (int64_t)half.W * half.NB * 16;
    if (use_half && B * ((N + pts - 1) / pts) < device_info().cus) g.cfg = narrow_cfg(kb, true, true);
  } else {
    const int kb = wide_kb(D);
    const AssignCfg c8 = wide8_cfg(kb);
    const int ov = plan_override().assign_kernel;
    const bool w8_ok = kb <= kWide8MaxKB && K >= 2 * (int64_t)c8.rows * c8.CT;
    if (w8_ok && (ov == 2 || (ov != 1 && pad_up(K, kPadK) / 32 >= 256))) {
      g.cfg = c8;
      g.Kpad = pad_up(K, (int64_t)c8.rows * c8.CT);
    } else {
      g.cfg = wide_cfg(kb);
    }
  }
  // Folded argmax (a max3 per two scores, then the index settled after the
  // sweep) against an exact compare-and-select per score: the fold pays off
  // with many groups (measured on gfx950: better from about 256 groups of 32);
  // warm-started launches always fold.
  const int fold = plan_override().assign_fold;
  g.lazy = dt != DT_F32 && (fold == 2 || (fold != 1 && g.groups() >= KM_LAZY_MIN_GROUPS));
  return g;
}

// ---------------------------------------------------------------------------
// Sort-inverse update geometry.
// ---------------------------------------------------------------------------
#ifndef KM_SEG_TILE
#define KM_SEG_TILE 128   // sorted positions per segment tile
#endif
#ifndef KM_SEG_U
#define KM_SEG_U 16       // most rows in flight per lane group in the segmented reduction
#endif
// Short segment tiles while N rows of G 16-byte pieces fit in half the last-level cache.
inline int64_t seg_fine_max_bytes() { return device_info().llc_bytes / 2; }
#ifndef KM_SEG_FINE_U
#define KM_SEG_FINE_U 16  // rows in flight per lane with short segment tiles
#endif
constexpr int kRadixThreads = 256;
constexpr int kRadixMaxItems = 32;           // consecutive keys per thread: 8, 16 or 32 (block positions fit in 16 bits)
// Keys per thread for N keys: 8192-key blocks from 8 blocks per compute
// unit, 4096-key blocks from one per compute unit, else 2048-key blocks
// (measured on gfx950 by the planner study, whole fits: 2^20 keys 0.2-1.1%
// faster in 4096-key blocks than in 2048, 2^23 keys 1% faster in 4096 than in
// 8192, 2^26 keys fastest in 8192-key blocks).
inline int radix_items(int64_t N) {
  const int ov = plan_override().radix_items;
  if (ov == 8 || ov == 16 || ov == 32) return ov;
  const int64_t cus = device_info().cus;
  return N >= 8 * cus * 8192 ? 32 : (N >= cus * 4096 ? 16 : 8);
}
constexpr int kMaxDigitBits = 6;             // digits of at most 64 values per pass (per-thread counters)
constexpr int kMaxWaveDigitBits = 8;         // ... of at most 256 values (wavefront ballots)
constexpr int kSegTile = KM_SEG_TILE;
// Short segment tiles, used while N rows of G lanes (16 bytes each) take at
// most seg_fine_max_bytes() (half the last-level cache), where the
// walk is bound by memory latency: 16 positions (8 for rows of one lane, G
// for rows of more than 16), so that the positions spread over many
// workgroups and each lane group has its whole tile in flight at once.  A
// larger N keeps kSegTile positions per tile, with fewer carry pieces for
// the fix-up (measured on gfx950: short tiles gain 1.1-10x below that size
// and lose up to 10% above it).
constexpr int seg_tile_fine(int G) { return G == 1 ? 8 : (G > 16 ? G : 16); }
constexpr uint32_t kInvalidFlag = 0x80000000u;  // marks a point whose cluster id was out of range

struct SortGeom {
  int64_t N;
  int64_t K;
  int kbits;        // bits of the largest valid id (K - 1), at least 1
  int npass;        // radix passes
  int bits[6];      // digit width of each pass
  int items;        // keys per thread (radix_items)
  int64_t nblk;     // key blocks of kRadixThreads * items keys
  int64_t count_len;  // max over passes of (2^bits * nblk)
  int scan_mode;    // count-table scans: 0 per digit (small tables: summed by the scatter), 1 whole table, 2 per digit
  bool wave_rank;   // scatter ranks keys by wavefront ballots (always for digits of more than kMaxDigitBits)
};

// Several independent problems of one shape in one launch.  Workgroup w works
// on problem b = w / bpp; that problem's X, centroid fragments and outputs
// start b * x_stride bytes, b * f_stride fragment slots and b * N entries
// further, and its cluster ids are written as b * id_mul + k.
struct Batch {
  uint32_t bpp;      // workgroups per problem
  int32_t id_mul;
  int64_t x_stride;
  int64_t f_stride;
  // Centroid-range split (split_tiles == 0: none).  Workgroup row y =
  // blockIdx.y sweeps tiles [y * split_tiles, (y + 1) * split_tiles) and
  // writes, per point o = b * N + p, its best score to part_s[y * part_stride
  // + o] and that centroid's index in the problem to part_k[...] (INT32_MAX:
  // none); row 0 also writes ||x||^2 to part_xn[o] when part_xn is set.
  int32_t split_tiles;
  float* part_s;
  int32_t* part_k;
  float* part_xn;
  int64_t part_stride;
};

// FlashAssign splits the centroid sweep over several workgroups per row block
// when the row blocks alone (B problems of N points, fewer than
// KM_SPLIT_MAX_BLOCKS_PER_CU workgroups per compute unit) would leave most of
// the GPU idle: up to KM_SPLIT_TARGET_BLOCKS_PER_CU workgroups per compute
// unit in all, each sweeping at least KM_SPLIT_MIN_TILES tiles, at most 64
// ranges; a merge pass then takes the best of the ranges in index order (the
// result is unchanged).  Measured on gfx950 (256 compute units): 2-19x faster
// sweeps for N up to 65,536 with 4,096 to 65,536 centroids; 16 workgroups per
// compute unit and 4 tiles beat 4 or 8 per compute unit and 8 tiles in most shapes.
#ifndef KM_SPLIT_MAX_BLOCKS_PER_CU
#define KM_SPLIT_MAX_BLOCKS_PER_CU 2
#endif
#ifndef KM_SPLIT_TARGET_BLOCKS_PER_CU
#define KM_SPLIT_TARGET_BLOCKS_PER_CU 16
#endif
#ifndef KM_SPLIT_MIN_TILES
#define KM_SPLIT_MIN_TILES 4
#endif
// tiles per range, 0 when the sweep is not split
inline int64_t assign_split_tiles(const AssignGeom& g, int64_t N, int64_t B) {
  const int64_t pts = (int64_t)g.cfg.W * g.cfg.NB * g.cfg.rows;
  const int64_t blocks = B * ((N + pts - 1) / pts);
  const int ov = plan_override().assign_split;
  if (N <= 0 || ov == 1) return 0;
  const int64_t nt = g.ntiles();
  if (ov >= 2) {  // a forced number of ranges (at least one tile each, at most 64)
    const int64_t S = ov < nt ? (ov < 64 ? ov : 64) : nt;
    return S < 2 ? 0 : (nt + S - 1) / S;
  }
  const int64_t cus = device_info().cus;
  if (blocks >= KM_SPLIT_MAX_BLOCKS_PER_CU * cus) return 0;
  int64_t S = (KM_SPLIT_TARGET_BLOCKS_PER_CU * cus + blocks - 1) / blocks;
  if (S > nt / KM_SPLIT_MIN_TILES) S = nt / KM_SPLIT_MIN_TILES;
  if (S > 64) S = 64;
  return S < 2 ? 0 : (nt + S - 1) / S;
}
inline int64_t assign_splits(const AssignGeom& g, int64_t N, int64_t B) {
  const int64_t st = assign_split_tiles(g, N, B);
  return st ? (g.ntiles() + st - 1) / st : 1;
}
// scratch of a split sweep: scores and indices per range and point, ||x||^2 per point
inline size_t assign_split_bytes(const AssignGeom& g, int64_t N, int64_t B) {
  const int64_t S = assign_splits(g, N, B);
  return S > 1 ? (size_t)(B * N) * (size_t)(8 * S + 4) + 256 : 0;
}

// ---------------------------------------------------------------------------
// Launchers (all asynchronous on `stream`; they return the launch status).
// ---------------------------------------------------------------------------
// B problems: C holds B x K x D floats, frag B x frag_bytes().
hipError_t launch_prep(const AssignGeom& g, const float* C, void* frag, hipStream_t stream, int64_t B = 1);

// perm/prev (both or neither): visit points in the order perm[0..N), where
// prev[i] is the previous centroid of point perm[i]; the result is the same,
// only faster when the assignment changes little (16-bit X only; ignored for
// fp32 X).  B > 1 (no perm/prev): B problems of N points each, X holding
// B x N rows and assign/min_dist B x N entries; ids are written as b*id_mul + k.
// split_ws (optional, assign_split_bytes(g, N, B) bytes, 16-byte aligned):
// scratch that lets a short sweep over many centroids split its centroid range
// (then perm/prev are not used).
hipError_t launch_flash_assign(const AssignGeom& g, const void* X, int64_t N, const void* frag, int32_t* assign,
                               float* min_dist, hipStream_t stream, const int32_t* perm = nullptr,
                               const int32_t* prev = nullptr, int64_t B = 1, int32_t id_mul = 0,
                               void* split_ws = nullptr);

// Radix argsort of cluster ids.  keys_in: the assignment vector.  The passes
// ping-pong through (key_a, val_a) and (key_b, val_b); the last pass writes
// (key_final, val_final), which must not be the last pass's input: use set a
// when npass is odd, set b when it is even, or caller memory.  Afterwards
// key_final holds the ids in ascending order and val_final the point index of
// each (stable: equal ids keep ascending point order); ids outside [0, K) are
// sorted as K-1 with kInvalidFlag set in their value.
hipError_t launch_argsort(const SortGeom& g, const int32_t* keys_in, int32_t* key_a, int32_t* val_a,
                          int32_t* key_b, int32_t* val_b, int32_t* key_final, int32_t* val_final, uint32_t* counts,
                          uint32_t* scan_part, hipStream_t stream);
int64_t scan_part_len(int64_t n);

// off[k] = first sorted position whose id >= k, k in [0, K]; off[K] = N.
hipError_t launch_boundaries(const int32_t* sorted_keys, int64_t N, int64_t K, int32_t* off,
                             hipStream_t stream);

enum ReduceMode : int { MODE_MEAN = 0, MODE_ACCUM = 1 };

struct ReduceArgs {
  const void* X;
  int dt;
  int64_t N, D, K;
  const int32_t* keys;
  const int32_t* vals;
  int32_t* off;         // K+1 cluster offsets (written by launch_segment_reduce, read by launch_fixup)
  float* carry_sum;     // [ntiles][2][Dc]
  int32_t* carry_cnt;   // [ntiles][2]
  float* group_sum;     // [ceil(ntiles / reduce_tpb)][Dc]: per segment-reduce workgroup whose positions hold one id
  int32_t* group_cnt;
  int mode;
  const float* C_prev;  // MODE_MEAN
  float* C_new;         // MODE_MEAN
  int32_t* counts;      // MODE_MEAN, nullable
  float* acc_sum;       // MODE_ACCUM: K x D running sums
  int64_t* acc_cnt;     // MODE_ACCUM: K running counts
  int64_t strip = 0;    // column strip (reduce_strips(dt, D) of them; one launch pair per strip)
  // MODE_MEAN, optional: the fix-up also writes FlashAssign's operand
  // fragments of C_new (cluster k = centroid k % kper of problem k / kper,
  // problem fragments f_stride 16-byte slots apart, geometry cfg)
  void* frag = nullptr;
  int64_t f_stride = 0, kper = 0;
  AssignCfg cfg{};
};

int64_t reduce_dc(int dt, int64_t D);   // padded length of a carry piece (one column strip)
int64_t reduce_strips(int dt, int64_t D);  // column strips of a row
int64_t reduce_tpb(int dt, int64_t D);  // tiles per segment-reduce workgroup
int64_t reduce_tile(int dt, int64_t D, int64_t N);         // sorted positions per segment tile for N positions
int64_t reduce_carry_tiles(int dt, int64_t D, int64_t N);  // most segment tiles of any N' <= N positions
hipError_t launch_segment_reduce(const ReduceArgs& a, hipStream_t stream);
hipError_t launch_fixup(const ReduceArgs& a, hipStream_t stream);
// Small codebooks (K <= kSmallMaxK per problem, or small_owner_fits; mean mode): the update of B
// problems of N points each in one launch (two when a problem spans several
// chunks of 512 or 2048 points), sort and reduction on chip.  ids[b*N + i] = b*id_mul + k.
constexpr int64_t kSmallMaxK = 64;
struct SmallArgs {
  const void* X;        // B x N x D
  int dt;
  int64_t B, N, D, K;   // per problem
  const int32_t* ids;
  int64_t id_mul;
  const float* C_prev;  // B x K x D
  float* C_new;         // may alias C_prev
  int32_t* counts;      // B x K, nullable
  float* part_sum;      // B * small_chunks(N) * K * reduce_dc(dt, D) floats
  int32_t* part_cnt;    // B * small_chunks(N) * K
  // optional: FlashAssign's centroid fragments for the next assignment,
  // written along with the means by the one-launch layout (any X) and by the
  // chunk-sum combine pass (fp32 X); *emitted says whether they were
  void* frag;           // B x frag_bytes of geometry cfg (NULL: none)
  int64_t f_stride;     // 16-byte slots per problem
  AssignCfg cfg;
  bool* emitted;
};
int64_t small_chunks(int64_t N);  // chunks per problem, at most
// Whether B problems of N points and K clusters each take the one-launch
// layout of one workgroup per 1, 2 or 4 clusters (then also for K above
// kSmallMaxK): N <= 16384 and at most 512 such workgroups.
bool small_owner_fits(int64_t B, int64_t N, int64_t K);
hipError_t launch_small_update(const SmallArgs& a, hipStream_t stream);
hipError_t launch_finalize_accum(const float* acc_sum, const int64_t* acc_cnt, int64_t K, int64_t D,
                                 float* C, int32_t* counts, hipStream_t stream);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream);

// Objective: out[0] (+)= sum of v[0..n) in fp64 with a fixed reduction order.
int64_t objective_partials(int64_t n);
hipError_t launch_objective(const float* v, int64_t n, double* partials, double* out, int accumulate,
                            hipStream_t stream);
// out[b] = sum of v[b*n .. (b+1)*n) in fp64 with a fixed reduction order, b < B.
hipError_t launch_objective_batched(const float* v, int64_t B, int64_t n, double* out, hipStream_t stream);
// out[i] = ids[i] - (i / n) * K for i < B*n: composite ids of a batch back to per-problem ids.
hipError_t launch_local_ids(const int32_t* ids, int64_t B, int64_t n, int64_t K, int32_t* out, hipStream_t stream);

}  // namespace km
