// Loading a 16-byte piece of an X row and widening it to fp32 (shared by the
// segmented reduction and the small-K update).  Internal to the library.
#pragma once

#include "km_internal.hpp"

namespace km {

typedef unsigned u32x4_r __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void widen(const u32x4_r& v, int dt, float* out) {
  if (dt == DT_F32) {
    out[0] = __uint_as_float(v.x);
    out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z);
    out[3] = __uint_as_float(v.w);
  } else if (dt == DT_BF16) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[2 * e] = __uint_as_float(w[e] << 16);
      out[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  } else {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e] & 0xffffu));
      out[2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e] >> 16));
    }
  }
}

// 16 bytes of row `row`, elements [c0, c0 + EPL), zero beyond D; rows are
// `ld` elements apart (ld = 0: D).
template <int ES>
__device__ __forceinline__ u32x4_r load_chunk(const uint8_t* __restrict__ X, int64_t row, int D, int c0, bool vec_ok,
                                              int64_t ld = 0) {
  constexpr int EPL = 16 / ES;
  u32x4_r v = {0u, 0u, 0u, 0u};
  if (c0 >= D) return v;
  const uint8_t* r = X + (size_t)row * (size_t)(ld ? ld : D) * ES;
  if (vec_ok && c0 + EPL <= D) return *reinterpret_cast<const u32x4_r*>(r + (size_t)c0 * ES);
  uint32_t w[4] = {0, 0, 0, 0};
  if (ES == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (c0 + e < D) w[e] = reinterpret_cast<const uint32_t*>(r)[c0 + e];
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (c0 + e < D) w[e >> 1] |= (uint32_t)reinterpret_cast<const uint16_t*>(r)[c0 + e] << (16 * (e & 1));
  }
  return u32x4_r{w[0], w[1], w[2], w[3]};
}

}  // namespace km
