// Conversion of centroids to FlashAssign's matrix-core operands, shared by
// the centroid preparation and by the update kernels that write the
// operands of the centroids they have just formed (so a fit needs no separate
// preparation launch per iteration).  Internal to the library.
#pragma once

#include "km_internal.hpp"

namespace km {

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // keep NaN quiet
  u += 0x7fffu + ((u >> 16) & 1u);                                // round to nearest, ties to even
  return u >> 16;
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // IEEE conversion, round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Writes centroid k's operand fragment and bias -||Q(c)||^2 / 2 from its
// final fp32 row `row` (D values, readable by every lane, e.g. in LDS) into
// `gbase` (the problem's fragment buffer, 16-byte slots, geometry cfg), bit
// for bit as the centroid preparation does it: the same rounding Q to X's
// type and the same summation order of the bias (fmaf chains over the depth
// blocks kb = w, w + 4, ... of each lane piece, w = 0..3 as the four
// preparation wavefronts, then those four in order, then the pieces of the
// row in the preparation's shuffle order).  One whole wavefront.
__device__ inline void emit_fragment_row(const float* row, int D, int dt, const AssignCfg& cfg, uint32_t* gbase,
                                         int64_t k) {
  const int lane = threadIdx.x & 63;
  const bool wide = cfg.rows == 32;
  const int npiece = wide ? 2 : 4;  // pieces of a depth block (8 or 4 values each)
  const int pv = wide ? 8 : 4;      // values per piece
  const int KB = cfg.KB;
  const int64_t g = k / cfg.rows;
  const int rsel = (int)(k % cfg.rows);
  uint32_t* gdst = gbase + 4 * ((g / cfg.CT) * cfg.tile_slots() + (g % cfg.CT) * cfg.group_slots());
  auto value = [&](int d) -> float {  // the value the matrix cores see
    const float c = d < D ? row[d] : 0.0f;
    if (!wide) return c;
    return dt == DT_BF16 ? bf16_bits_to_f32(f32_to_bf16_bits(c)) : f16_bits_to_f32(f32_to_f16_bits(c));
  };
  auto bits = [&](int d) -> uint32_t {
    const float c = d < D ? row[d] : 0.0f;
    if (!wide) return __float_as_uint(c);
    return dt == DT_BF16 ? f32_to_bf16_bits(c) : f32_to_f16_bits(c);
  };
  if (lane < npiece * KB) {  // lane = kb * npiece + p: piece p of depth block kb
    const int kb = lane / npiece, p = lane % npiece;
    const int d0 = kb * kFragDepth + p * pv;
    uint32_t w[4];
    if (wide) {
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = bits(d0 + 2 * e) | (bits(d0 + 2 * e + 1) << 16);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = bits(d0 + e);
    }
    uint32_t* dst = gdst + 4 * (kb * 64 + p * cfg.rows + rsel);
    dst[0] = w[0];
    dst[1] = w[1];
    dst[2] = w[2];
    dst[3] = w[3];
  }
  // chains: lane 4 p + w holds the chain of (wavefront w, piece p)
  float ss = 0.0f;
  if (lane < 4 * npiece) {
    const int w = lane & 3, p = lane >> 2;
    for (int kb = w; kb < KB; kb += 4) {
      const int d0 = kb * kFragDepth + p * pv;
      for (int e = 0; e < pv; ++e) {
        const float v = value(d0 + e);
        ss = fmaf(v, v, ss);
      }
    }
  }
  // lane p: T_p = ((S_0p + S_1p) + S_2p) + S_3p
  const int p = lane & 3;
  const float t = ((__shfl(ss, 4 * p) + __shfl(ss, 4 * p + 1)) + __shfl(ss, 4 * p + 2)) + __shfl(ss, 4 * p + 3);
  float tot;
  if (wide) {
    tot = __shfl(t, 0) + __shfl(t, 1);
  } else {
    const float t01 = __shfl(t, 0) + __shfl(t, 1), t23 = __shfl(t, 2) + __shfl(t, 3);
    tot = t01 + t23;
  }
  if (lane == 0) {
    float* bias = reinterpret_cast<float*>(gdst + 4 * (KB * 64));
    if (wide) {  // accumulator order of the lanes that read the bias
      const int j = rsel >> 3, h = (rsel >> 2) & 1, r = rsel & 3;
      bias[h * 16 + j * 4 + r] = -0.5f * tot;
    } else {
      bias[rsel] = -0.5f * tot;
    }
  }
}

}  // namespace km
