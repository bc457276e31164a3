// MXFP8 element and scale encoding (OCP Microscaling Formats v1.0): E4M3
// ("FN": bias 7, max 448, no infinities) elements with one E8M0 scale
// 2^(floor(log2 amax) - 8) per block of 32, written with exact operations
// only (power-of-two scaling, round-half-even to an integer, comparisons).
// Shared by every quantiser so they all produce the same bytes.
#pragma once

#include <math.h>

#include "common.h"

namespace moe {

// floor(log2 |a|) of a finite non-zero fp32 value, exact (subnormals included).
__device__ __forceinline__ int floor_log2_f32(float a) {
  const uint32_t u = __float_as_uint(a) & 0x7fffffffu;
  const int ef = static_cast<int>(u >> 23);
  if (ef != 0) return ef - 127;
  return -149 + (31 - __clz(static_cast<int>(u)));
}

// E8M0 code of the block scale for block maximum |v| = amax (amax >= 0).
__device__ __forceinline__ int mx_scale_code(float amax) {
  if (amax == 0.0f) return 0;
  const int c = floor_log2_f32(amax) - 8 + 127;
  return c < 0 ? 0 : (c > 254 ? 254 : c);
}

// E4M3 code of y (already divided by the block scale; exact in fp32).
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: subnormal spacing 2^-9
    code = static_cast<uint32_t>(rintf(a * 512.0f));   // 0..8 (8 is the smallest normal)
  } else {
    const int ex = floor_log2_f32(a);
    float r = rintf(ldexpf(a, 3 - ex));      // significand with 3 fraction bits, in [8, 16]
    int e2 = ex;
    if (r >= 16.0f) { r = 8.0f; e2 = ex + 1; }
    if (e2 > 8 || (e2 == 8 && r > 14.0f)) { e2 = 8; r = 14.0f; }  // saturate to 448
    code = static_cast<uint32_t>((e2 + 7) << 3) | static_cast<uint32_t>(r - 8.0f);
  }
  return sign | code;
}

// Scale code and the 32 E4M3 codes of one block (v[] in fp32).
__device__ __forceinline__ int mx_encode_block(const float (&v)[32], uint32_t (&w)[8]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int c = mx_scale_code(amax);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    w[i] = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[i] |= e4m3_encode(ldexpf(v[i * 4 + j], 127 - c)) << (8 * j);
  }
  return c;
}

}  // namespace moe
