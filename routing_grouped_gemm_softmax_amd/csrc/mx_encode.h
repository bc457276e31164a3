// MXFP8 element and scale encoding (OCP Microscaling Formats v1.0): E4M3
// ("FN": bias 7, max 448, no infinities) elements with one E8M0 scale
// 2^(floor(log2 amax) - 8) per block of 32. e4m3_encode spells the element
// rounding out with exact integer operations and serves every fp32 input; the
// quantisers of bf16 inputs use the hardware conversion (e4m3_encode4), which
// gives the same bytes on those. Shared by every quantiser so they all
// produce the same bytes.
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

// E4M3 code of y (already divided by the block scale; exact in fp32 and
// |y| < 512, which the block scale guarantees). Normal range (|y| >= 2^-6):
// round the fp32 significand to 3 bits, ties to even, by integer addition on
// the bit pattern, rebias the exponent (127 -> 7) and saturate at 448 (code
// 0x7E; 480 would be the NaN code). Below 2^-6 the E4M3 spacing is 2^-9:
// code = rint(|y| * 512), 0..8. The sign is kept.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a < 0x3C800000u) {
    code = static_cast<uint32_t>(rintf(__uint_as_float(a) * 512.0f));
  } else {
    const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
    code = min(r - 0x3C0u, 0x7Eu);
  }
  return sign | code;
}

// E4M3 codes of four values already divided by their block scale (|y| <
// 512), packed little-endian: the hardware conversion (round to nearest even)
// of each value clamped to +-448. On every such value that is a bf16 number
// times a power of two (all inputs here) this gives e4m3_encode's byte,
// signed zero included; the GPU tests pin it against the oracle's encoder.
__device__ __forceinline__ uint32_t e4m3_encode4(float a, float b, float c, float d) {
  auto sat = [](float y) { return __builtin_amdgcn_fmed3f(y, -448.0f, 448.0f); };
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), lo, true));
}

// Scale code and the 32 E4M3 codes of one block (v[] in fp32).
__device__ __forceinline__ int mx_encode_block(const float (&v)[32], uint32_t (&w)[8]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int c = mx_scale_code(amax);
  const int sh = 127 - c;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    w[i] = e4m3_encode4(ldexpf(v[i * 4], sh), ldexpf(v[i * 4 + 1], sh), ldexpf(v[i * 4 + 2], sh),
                        ldexpf(v[i * 4 + 3], sh));
  return c;
}

// Eight consecutive values of one block (block scale code c) -> 8 E4M3 bytes.
__device__ __forceinline__ uint2 mx_encode8(const float (&v)[8], int c) {
  const int sh = 127 - c;
  return make_uint2(e4m3_encode4(ldexpf(v[0], sh), ldexpf(v[1], sh), ldexpf(v[2], sh), ldexpf(v[3], sh)),
                    e4m3_encode4(ldexpf(v[4], sh), ldexpf(v[5], sh), ldexpf(v[6], sh), ldexpf(v[7], sh)));
}

// Block scale code of a 32-block held by 4 consecutive lanes (8 values each,
// lane groups aligned to 4): the maximum over the group, by two butterflies.
// Every lane of the wave must execute it.
__device__ __forceinline__ int mx_group4_code(const float (&v)[8]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
  return mx_scale_code(amax);
}

// The same for fp32 values, which carry more significand bits than the
// hardware conversion was checked on: four codes by the exact encoder.
__device__ __forceinline__ uint32_t mx_encode4_exact(const float (&v)[4], int c) {
  const int sh = 127 - c;
  return e4m3_encode(ldexpf(v[0], sh)) | (e4m3_encode(ldexpf(v[1], sh)) << 8) |
         (e4m3_encode(ldexpf(v[2], sh)) << 16) | (e4m3_encode(ldexpf(v[3], sh)) << 24);
}

// Eight consecutive fp32 values of one block (code c) -> 8 E4M3 bytes, exactly.
__device__ __forceinline__ uint2 mx_encode8_exact(const float (&v)[8], int c) {
  const float a[4] = {v[0], v[1], v[2], v[3]}, b[4] = {v[4], v[5], v[6], v[7]};
  return make_uint2(mx_encode4_exact(a, c), mx_encode4_exact(b, c));
}

// Scale code and the 32 E4M3 codes of one block of fp32 values (exact encoder).
__device__ __forceinline__ int mx_encode_block_exact(const float (&v)[32], uint32_t (&w)[8]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int c = mx_scale_code(amax);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q[4] = {v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
    w[i] = mx_encode4_exact(q, c);
  }
  return c;
}

// Block scale code of a 32-block of fp32 values held by 8 consecutive lanes
// (4 values each, lane groups aligned to 8): three butterflies. Every lane of
// the wave must execute it.
__device__ __forceinline__ int mx_group8_code(const float (&v)[4]) {
  float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
  amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 4, kWave));
  return mx_scale_code(amax);
}

}  // namespace moe
