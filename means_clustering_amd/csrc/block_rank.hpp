// Stable rank of a block's keys by one radix digit, in LDS (shared by the
// radix argsort and the small-K update).  Internal to the library.
#pragma once

#include "km_internal.hpp"

namespace km {

// ----------------------------------------------------------- block rank --

constexpr int kRadixWords = (1 << kMaxDigitBits) * kRadixThreads / 2;  // 16-bit counters, two a word
constexpr int kRadixPadded = kRadixWords + kRadixWords / 32;             // + one pad word per 32

// LDS word of the counter of (digit d, thread t): counters are laid out in
// (digit, thread) order, two to a 32-bit word, with one pad word after every
// 32 so the raking scan's per-thread chunks fall in different banks.
__device__ __forceinline__ int ctr_word(int f) {
  const int w = f >> 1;
  return w + (w >> 5);
}

__device__ __forceinline__ uint32_t ctr_get(const uint32_t* ctr, int f) {
  return (ctr[ctr_word(f)] >> (16 * (f & 1))) & 0xffffu;
}

// Exclusive scan of one value per thread across the block; returns the total.
__device__ __forceinline__ uint32_t block_scan_excl(uint32_t v, uint32_t& excl, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kRadixThreads / 64; ++w) {
    const uint32_t sw = wsum[w];
    if (w < wave) before += sw;
    total += sw;
  }
  excl = before + x - v;
  __syncthreads();
  return total;
}

// Stable ranks of this block's keys by BITS-bit digit.  d[i] is the digit of
// the thread's i-th key (valid[i] false: not a key).  On return rank[i] is
// the key's position in the block sorted by digit, and start[dd] (LDS, R+1
// entries) the first position of digit dd.
template <int BITS, int IT>
__device__ __forceinline__ void block_rank(const uint32_t (&d)[IT], const bool (&valid)[IT], uint32_t* ctr,
                                           uint32_t* wsum, uint32_t* start, uint32_t (&rank)[IT]) {
  constexpr int R = 1 << BITS;
  constexpr int T = kRadixThreads;
  const int t = threadIdx.x;
  for (int i = t; i < kRadixPadded; i += T) ctr[i] = 0;
  __syncthreads();
  // count own keys in order: rank among this thread's keys of the same digit
  uint16_t* c16 = reinterpret_cast<uint16_t*>(ctr);
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    if (valid[i]) {
      const int f = (int)d[i] * T + t;
      const int h = ctr_word(f) * 2 + (f & 1);
      const uint32_t c = c16[h];
      rank[i] = c;
      c16[h] = (uint16_t)(c + 1);
    }
  }
  __syncthreads();
  // raking exclusive scan over the R*T counters in (digit, thread) order:
  // thread t owns the flat counters [t*R, t*R + R)
  constexpr int CH = R;  // counters per thread
  uint32_t loc[CH];
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    loc[j] = ctr_get(ctr, t * CH + j);
    sum += loc[j];
  }
  uint32_t excl;
  block_scan_excl(sum, excl, wsum);
  uint32_t run = excl;
#pragma unroll
  for (int j = 0; j < CH; j += 2) {
    const uint32_t lo = run;
    run += loc[j];
    const uint32_t hi = run;
    run += loc[j + 1];
    ctr[ctr_word(t * CH + j)] = lo | (hi << 16);  // block positions fit in 16 bits
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < IT; ++i)
    if (valid[i]) rank[i] += ctr_get(ctr, (int)d[i] * T + t);
  for (int dd = t; dd < R; dd += T) start[dd] = ctr_get(ctr, dd * T);
  if (t == T - 1) start[R] = run;  // the last thread's running sum is the block's key count
  __syncthreads();
}

}  // namespace km
