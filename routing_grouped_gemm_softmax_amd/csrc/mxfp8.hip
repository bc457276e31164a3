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
#include "common.h"
#include "kernels.h"
#include "mx_encode.h"

namespace moe {

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
  uint32_t w[8];
  const int c = mx_encode_block(v, w);
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

// ---------------------------------------------------------------------------------
// Quantisers into the grouped GEMM's operand layout: E4M3 K-major, scales
// slab-major (per 64-k slab, 2 bytes per row: the slab's two 32-blocks).
// ---------------------------------------------------------------------------------

// K along the columns: in [R][C] -> q [R][C], s [C/64][R][2]. One thread per
// 64-column chunk of a row; consecutive threads take consecutive rows so the
// 2-byte scale pairs land contiguously. Batched (weights: one batch per expert).
__global__ __launch_bounds__(256) void mx_kmajor_kernel(const bf16_t* __restrict__ in, int R, int C, int64_t n,
                                                        int64_t in_bstride, uint8_t* __restrict__ q,
                                                        int64_t q_bstride, uint8_t* __restrict__ s,
                                                        int64_t s_bstride) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int64_t per = static_cast<int64_t>(R) * (C / 64);
  const int64_t b = i / per, rem = i % per;
  const int c64 = static_cast<int>(rem / R), r = static_cast<int>(rem % R);
  const bf16_t* src = in + b * in_bstride + static_cast<int64_t>(r) * C + c64 * 64;
  uint8_t* dq = q + b * q_bstride + static_cast<int64_t>(r) * C + c64 * 64;
  int code[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float v[32];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float t[8];
      unpack16(ld16(src + h * 32 + j * 8), t);
#pragma unroll
      for (int u = 0; u < 8; ++u) v[j * 8 + u] = t[u];
    }
    uint32_t w[8];
    code[h] = mx_encode_block(v, w);
    uint4* d4 = reinterpret_cast<uint4*>(dq + h * 32);
    d4[0] = make_uint4(w[0], w[1], w[2], w[3]);
    d4[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
  *reinterpret_cast<uint16_t*>(s + b * s_bstride + (static_cast<int64_t>(c64) * R + r) * 2) =
      static_cast<uint16_t>(code[0] | (code[1] << 8));
}

// K along the rows, written transposed: in [R][C] -> q [C][P], s [P/64][C][2],
// blocked inside row groups. With `offsets` (E+1 ints) and `poff` (the same
// groups padded to 64 rows, E+1 ints) group e's rows offsets[e].. land at
// q columns poff[e].. and the padding reads as zeros; without them the batch
// is one group of R rows (R a multiple of 64). One workgroup per (64 padded
// rows, 64 columns): the tile goes through LDS so loads and stores are
// row-contiguous.
__global__ __launch_bounds__(128) void mx_tgroup_kernel(const bf16_t* __restrict__ in, int R, int C,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ poff, int E,
                                                        int64_t in_bstride, uint8_t* __restrict__ q, int64_t P,
                                                        int64_t q_bstride, uint8_t* __restrict__ s,
                                                        int64_t s_bstride) {
  __shared__ __attribute__((aligned(16))) bf16_t tile[64][64 + 8];
  __shared__ int s_grp[2];
  const int tid = threadIdx.x, sb = blockIdx.x, cc = blockIdx.y, b = blockIdx.z;
  const int64_t p0 = static_cast<int64_t>(sb) * 64;
  int src0 = 0, valid = 0;
  if (poff == nullptr) {
    src0 = static_cast<int>(p0);
    valid = static_cast<int>(min(static_cast<int64_t>(64), static_cast<int64_t>(R) - p0));
  } else {
    // The group g with poff[g] <= p0 < poff[g+1] (at most one: empty groups
    // have poff[g] == poff[g+1]).
    if (tid == 0) s_grp[0] = -1;
    __syncthreads();
    for (int e = tid; e < E; e += 128)
      if (poff[e] <= p0 && p0 < poff[e + 1]) s_grp[0] = e;
    __syncthreads();
    const int g = s_grp[0];
    if (g < 0) return;  // past the last group: never read by the GEMM
    src0 = offsets[g] + static_cast<int>(p0 - poff[g]);
    valid = min(64, offsets[g + 1] - src0);
  }
  const bf16_t* src = in + static_cast<int64_t>(b) * in_bstride;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int id = tid + 128 * j, row = id >> 3, part = id & 7;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < valid) v = ld16(src + static_cast<int64_t>(src0 + row) * C + cc * 64 + part * 8);
    *reinterpret_cast<uint4*>(&tile[row][part * 8]) = v;
  }
  __syncthreads();
  const int c = tid & 63, blk = tid >> 6;
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = bf16_to_f32(tile[blk * 32 + i][c]);
  uint32_t w[8];
  const int code = mx_encode_block(v, w);
  const int64_t col = static_cast<int64_t>(cc) * 64 + c;
  uint4* dq = reinterpret_cast<uint4*>(q + static_cast<int64_t>(b) * q_bstride + col * P + p0 + blk * 32);
  dq[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dq[1] = make_uint4(w[4], w[5], w[6], w[7]);
  s[static_cast<int64_t>(b) * s_bstride + (static_cast<int64_t>(sb) * C + col) * 2 + blk] = static_cast<uint8_t>(code);
}

// poff[e] = sum over e' < e of ceil(n_e' / 64) * 64 (one wave; E <= 256).
__global__ __launch_bounds__(64) void mx_poff_kernel(const int32_t* __restrict__ offsets, int E,
                                                     int32_t* __restrict__ poff) {
  const int lane = threadIdx.x;
  int v[4], sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane * 4 + q;
    v[q] = e < E ? (offsets[e + 1] - offsets[e] + 63) / 64 * 64 : 0;
    sum += v[q];
  }
  int run = wave_exclusive_scan(sum);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane * 4 + q;
    if (e < E) poff[e] = run;
    run += v[q];
  }
  if (lane == 63) poff[E] = run;
}

hipError_t launch_mx_kmajor(const void* in, int R, int C, int batches, int64_t in_bstride, uint8_t* q,
                            int64_t q_bstride, uint8_t* s, int64_t s_bstride, hipStream_t st) {
  const int64_t n = static_cast<int64_t>(batches) * R * (C / 64);
  hipLaunchKernelGGL(mx_kmajor_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st,
                     static_cast<const bf16_t*>(in), R, C, n, in_bstride, q, q_bstride, s, s_bstride);
  return hipGetLastError();
}

hipError_t launch_mx_tgroup(const void* in, int R, int C, const int32_t* offsets, const int32_t* poff, int E,
                            int batches, int64_t in_bstride, uint8_t* q, int64_t P, int64_t q_bstride, uint8_t* s,
                            int64_t s_bstride, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(P / 64), static_cast<unsigned>(C / 64), static_cast<unsigned>(batches));
  hipLaunchKernelGGL(mx_tgroup_kernel, grid, dim3(128), 0, st, static_cast<const bf16_t*>(in), R, C, offsets, poff,
                     E, in_bstride, q, P, q_bstride, s, s_bstride);
  return hipGetLastError();
}

hipError_t launch_mx_poff(const int32_t* offsets, int E, int32_t* poff, hipStream_t st) {
  hipLaunchKernelGGL(mx_poff_kernel, dim3(1), dim3(64), 0, st, offsets, E, poff);
  return hipGetLastError();
}

}  // namespace moe
