// MXFP8 quantisation: E4M3 elements with one E8M0 scale per 32 elements.
//
// The pages only say that MXFP8 is supported and that it cuts data movement
// and compute ("Olmo-core 3 é lançado com infraestrutura para treinar modelos
// MoE", section "Otimizações e testes em escala de trilhões"; "Ai2 rilascia
// Olmo-Core 3...", section "Parallelismo, precisione e tecniche di memoria").
// The conversion follows the OCP Microscaling Formats (MX) v1.0 rule: the
// block scale is 2^(floor(log2 amax) - 8) (8 = exponent of the largest E4M3
// normal, 448 = 1.75 * 2^8), as an E8M0 code clamped to 0..254; each element
// v / scale is rounded to the nearest E4M3 ("FN": bias 7, no infinities)
// value, ties to even, saturating at +-448 and keeping the sign.
//
// The element encoder is written with exact operations only (power-of-two
// scaling, round-half-even to an integer, comparisons), so it is bit-exact.
#include <math.h>

#include "common.h"
#include "kernels.h"

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

// axis 0: one thread per block of 32 consecutive elements of a row.
__global__ __launch_bounds__(256) void mxfp8_rows_kernel(const bf16_t* __restrict__ in, int64_t nblocks,
                                                         uint8_t* __restrict__ q, uint8_t* __restrict__ scale) {
  const int64_t b = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const bf16_t* src = in + b * 32;
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float t[8];
    unpack16(ld16(src + i * 8), t);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[i * 8 + j] = t[j];
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int c = mx_scale_code(amax);
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    w[i] = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[i] |= e4m3_encode(ldexpf(v[i * 4 + j], 127 - c)) << (8 * j);
  }
  uint4* dst = reinterpret_cast<uint4*>(q + b * 32);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  scale[b] = static_cast<uint8_t>(c);
}

// axis 1: one thread per (32-row block, column); consecutive threads take
// consecutive columns so loads and byte stores are coalesced.
__global__ __launch_bounds__(256) void mxfp8_cols_kernel(const bf16_t* __restrict__ in, int64_t rows, int64_t cols,
                                                         uint8_t* __restrict__ q, uint8_t* __restrict__ scale) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= (rows / 32) * cols) return;
  const int64_t rb = i / cols, col = i % cols;
  const bf16_t* src = in + rb * 32 * cols + col;
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    v[r] = bf16_to_f32(src[r * cols]);
    amax = fmaxf(amax, fabsf(v[r]));
  }
  const int c = mx_scale_code(amax);
  uint8_t* dst = q + rb * 32 * cols + col;
#pragma unroll
  for (int r = 0; r < 32; ++r) dst[r * cols] = static_cast<uint8_t>(e4m3_encode(ldexpf(v[r], 127 - c)));
  scale[i] = static_cast<uint8_t>(c);
}

hipError_t launch_mxfp8_quantize(const void* in, int64_t rows, int64_t cols, int axis, uint8_t* q, uint8_t* scale,
                                 hipStream_t s) {
  const bf16_t* src = static_cast<const bf16_t*>(in);
  if (axis == 0) {
    const int64_t nb = rows * (cols / 32);
    hipLaunchKernelGGL(mxfp8_rows_kernel, dim3(static_cast<unsigned>((nb + 255) / 256)), dim3(256), 0, s, src, nb, q,
                       scale);
  } else {
    const int64_t n = (rows / 32) * cols;
    hipLaunchKernelGGL(mxfp8_cols_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, src, rows,
                       cols, q, scale);
  }
  return hipGetLastError();
}

}  // namespace moe
