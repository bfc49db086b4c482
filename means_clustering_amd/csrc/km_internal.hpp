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
// centroids as the A operand (16 rows) and the points as the B operand (16
// columns).  A "fragment block" is what one wavefront feeds one group of
// MFMAs: 64 lanes x 16 bytes, covering 16 centroids x FB depth values, where
// FB = 32 for 16-bit data (v_mfma_f32_16x16x32_{bf16,f16}: 8 values per lane)
// and FB = 16 for fp32 (four v_mfma_f32_16x16x4_f32: 4 values per lane).
// Lane l holds centroid (l % 16) and depth values [FB*kb + EPL*(l/16), +EPL).
// Fragments are stored [group g][depth block kb][lane][16 bytes], so a
// centroid tile is one contiguous run of bytes: copying it to LDS and reading
// it back are both lane-linear 16-byte accesses.
// ---------------------------------------------------------------------------
constexpr int kGroupRows = 16;     // centroids per fragment group
constexpr int kPadK = 128;         // K is padded to a multiple of this (>= any tile)
constexpr int kMaxKB = 16;         // depth blocks supported: D <= 512 (16-bit), D <= 256 (fp32)

inline int frag_depth(int dt) { return dt == DT_F32 ? 16 : 32; }
inline int64_t pad_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// FlashAssign launch shape for a given number of depth blocks KB:
//   NB  16-point groups per wavefront (register-resident point fragments),
//   CT  16-centroid groups per LDS tile,
//   W   wavefronts per workgroup.
struct AssignCfg {
  int NB, CT, W;
};
constexpr AssignCfg assign_cfg(int KB) {
  return AssignCfg{KB <= 4 ? 4 : (KB <= 8 ? 2 : 1), KB <= 2 ? 8 : (KB <= 4 ? 4 : (KB <= 8 ? 2 : 1)), 4};
}
// 16-byte slots of one centroid group: KB*64 fragments, then 4 slots of bias.
constexpr int64_t group_slots(int KB) { return (int64_t)KB * 64 + 4; }
// 16-byte slots of one tile, padded so every thread of the block copies the
// same number of slots.
constexpr int64_t tile_slots(int KB) {
  return (assign_cfg(KB).CT * group_slots(KB) + assign_cfg(KB).W * 64 - 1) / (assign_cfg(KB).W * 64) *
         (assign_cfg(KB).W * 64);
}

struct AssignGeom {
  int dt;
  int64_t N, D, K;
  int KB;          // depth blocks = ceil(D / FB)
  int64_t Kpad;    // K rounded up to kPadK
  int64_t ntiles() const { return Kpad / ((int64_t)assign_cfg(KB).CT * kGroupRows); }
  size_t frag_bytes() const { return (size_t)ntiles() * (size_t)tile_slots(KB) * 16; }
};

// ---------------------------------------------------------------------------
// Sort-inverse update geometry.
// ---------------------------------------------------------------------------
constexpr int kSortThreads = 256;            // 4 wavefronts
constexpr int kSortItems = 16;               // keys per thread
constexpr int kSortBlock = kSortThreads * kSortItems;  // 4096 keys per block
constexpr int kSegTile = 256;                // sorted positions per segment tile
constexpr uint32_t kInvalidFlag = 0x80000000u;  // marks a point whose cluster id was out of range

struct SortGeom {
  int64_t N;
  int64_t K;
  int kbits;        // bits of the largest valid id (K - 1), at least 1
  int npass;        // radix passes
  int bits[4];      // digit width of each pass
  int64_t nblk;     // key blocks of kSortBlock
  int64_t count_len;  // max over passes of (2^bits * nblk)
};

// ---------------------------------------------------------------------------
// Launchers (all asynchronous on `stream`; they return the launch status).
// ---------------------------------------------------------------------------
hipError_t launch_prep(const float* C, int64_t K, int64_t D, int dt, int KB, int64_t Kpad, void* frag,
                       hipStream_t stream);

hipError_t launch_flash_assign(const void* X, int dt, int64_t N, int64_t D, int KB, const void* frag, int64_t Kpad,
                               int32_t* assign, float* min_dist, hipStream_t stream);

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
  const int32_t* off;
  float* carry_sum;     // [ntiles][2][Dc]
  int32_t* carry_cnt;   // [ntiles][2]
  int mode;
  const float* C_prev;  // MODE_MEAN
  float* C_new;         // MODE_MEAN
  int32_t* counts;      // MODE_MEAN, nullable
  float* acc_sum;       // MODE_ACCUM: K x D running sums
  int64_t* acc_cnt;     // MODE_ACCUM: K running counts
};

int64_t reduce_dc(int dt, int64_t D);  // padded row length of a carry piece
hipError_t launch_segment_reduce(const ReduceArgs& a, hipStream_t stream);
hipError_t launch_fixup(const ReduceArgs& a, hipStream_t stream);
hipError_t launch_finalize_accum(const float* acc_sum, const int64_t* acc_cnt, int64_t K, int64_t D,
                                 float* C, int32_t* counts, hipStream_t stream);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream);

// Objective: out[0] (+)= sum of v[0..n) in fp64 with a fixed reduction order.
int64_t objective_partials(int64_t n);
hipError_t launch_objective(const float* v, int64_t n, double* partials, double* out, int accumulate,
                            hipStream_t stream);

}  // namespace km
