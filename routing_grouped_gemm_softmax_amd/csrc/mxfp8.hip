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

// Blocks of 32 consecutive rows inside row groups [off[g], off[g+1]), each
// group's last block completed with zero rows (which change no scale): the
// layout of a weight-gradient operand, whose K runs over one expert's tokens.
// One workgroup per (32-row block of the group-major block list, 256
// columns): grid x over blocks, y over column tiles. Every workgroup scans the group sizes in LDS to find its block's
// group; workgroups past the last block exit. Offsets are clamped into
// [0, rows], so a malformed table cannot make an access out of bounds.
__global__ __launch_bounds__(256) void mxfp8_grouped_kernel(const bf16_t* __restrict__ in, int64_t rows, int64_t cols,
                                                            const int32_t* __restrict__ off, int G,
                                                            uint8_t* __restrict__ q, uint8_t* __restrict__ scale) {
  __shared__ int s_lo[256], s_hi[256], s_first[257];
  const int tid = threadIdx.x;
  // Group bounds and blocks per group (clamped), then a block-start scan.
  int nb = 0;
  if (tid < G) {
    const int64_t lo = min(max(static_cast<int64_t>(off[tid]), int64_t{0}), rows);
    const int64_t hi = min(max(static_cast<int64_t>(off[tid + 1]), lo), rows);
    s_lo[tid] = static_cast<int>(lo);
    s_hi[tid] = static_cast<int>(hi);
    nb = static_cast<int>((hi - lo + 31) / 32);
  }
  __shared__ int s_wave[4];
  const int lane = tid & 63, wave = tid >> 6;
  const int incl = wave_exclusive_scan(nb) + nb;
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += s_wave[w];
  if (tid < G) s_first[tid + 1] = base + incl;
  if (tid == 0) s_first[0] = 0;
  __syncthreads();
  const int b = blockIdx.x;
  if (b >= s_first[G]) return;  // uniform: past the last block
  int lo = 0, hi = G;           // s_first[lo] <= b < s_first[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_first[mid] <= b) lo = mid; else hi = mid;
  }
  const int64_t r0 = s_lo[lo] + static_cast<int64_t>(b - s_first[lo]) * 32;
  const int n = static_cast<int>(min(static_cast<int64_t>(32), s_hi[lo] - r0));
  const int64_t col = static_cast<int64_t>(blockIdx.y) * 256 + tid;
  if (col >= cols) return;
  const bf16_t* src = in + r0 * cols + col;
  float v[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    const float x = bf16_to_f32(src[min(r, n - 1) * cols]);  // rows past the group end: in bounds, zeroed
    v[r] = r < n ? x : 0.0f;
  }
  uint32_t w[8];
  const int c = mx_encode_block(v, w);
  uint8_t* dst = q + r0 * cols + col;
#pragma unroll
  for (int r = 0; r < 32; ++r)
    if (r < n) dst[r * cols] = static_cast<uint8_t>(w[r / 4] >> (8 * (r % 4)));
  scale[static_cast<int64_t>(b) * cols + col] = static_cast<uint8_t>(c);
}

hipError_t launch_mxfp8_quantize_grouped(const void* in, int64_t rows, int64_t cols, const int32_t* off, int G,
                                         uint8_t* q, uint8_t* scale, hipStream_t s) {
  const int64_t nb_max = rows / 32 + G;  // >= the sum over groups of ceil(n_g / 32)
  const dim3 grid(static_cast<unsigned>(nb_max), static_cast<unsigned>((cols + 255) / 256));
  hipLaunchKernelGGL(mxfp8_grouped_kernel, grid, dim3(256), 0, s, static_cast<const bf16_t*>(in), rows, cols, off, G,
                     q, scale);
  return hipGetLastError();
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

// K along the columns: in [R][C] -> q [R][C], s [C/64][R][2], batched (one
// batch per expert for the weights). A wave covers tiles of 8 rows x 64
// columns: lane l takes row l / 8, columns 8 (l % 8) .. +7, so each load is
// 8 rows x 128 contiguous bytes, the 4 lanes of a 32-block find its maximum
// by butterflies and each lane stores its 8 codes; lane 8r writes row r's two
// scale bytes. Each wave takes kTilesPerWave consecutive tiles (row-major:
// column slabs fastest), loading all of them before encoding any.
constexpr int kTilesPerWave = 4;
__global__ __launch_bounds__(256) void mx_kmajor_kernel(const bf16_t* __restrict__ in, int R, int C, int64_t ntiles,
                                                        int64_t in_bstride, uint8_t* __restrict__ q,
                                                        int64_t q_bstride, uint8_t* __restrict__ s,
                                                        int64_t s_bstride) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t per_batch = static_cast<int64_t>(R / 8) * (C / 64);
  const int rl = lane >> 3, ch = lane & 7;
  uint4 raw[kTilesPerWave];
#pragma unroll
  for (int u = 0; u < kTilesPerWave; ++u) {
    const int64_t t = wave * kTilesPerWave + u;
    if (t >= ntiles) continue;
    const int64_t b = t / per_batch, rem = t % per_batch;
    const int row = static_cast<int>(rem / (C / 64)) * 8 + rl, c64 = static_cast<int>(rem % (C / 64));
    raw[u] = ld16(in + b * in_bstride + static_cast<int64_t>(row) * C + c64 * 64 + ch * 8);
  }
#pragma unroll
  for (int u = 0; u < kTilesPerWave; ++u) {
    const int64_t t = wave * kTilesPerWave + u;
    if (t >= ntiles) continue;  // wave-uniform
    const int64_t b = t / per_batch, rem = t % per_batch;
    const int row = static_cast<int>(rem / (C / 64)) * 8 + rl, c64 = static_cast<int>(rem % (C / 64));
    float v[8];
    unpack16(raw[u], v);
    const int code = mx_group4_code(v);
    *reinterpret_cast<uint2*>(q + b * q_bstride + static_cast<int64_t>(row) * C + c64 * 64 + ch * 8) =
        mx_encode8(v, code);
    const int code_hi = __shfl(code, (lane & ~7) + 4, kWave);
    if (ch == 0)
      *reinterpret_cast<uint16_t*>(s + b * s_bstride + (static_cast<int64_t>(c64) * R + row) * 2) =
          static_cast<uint16_t>(code | (code_hi << 8));
  }
}

// K along the rows, written transposed: in [R][C] -> q [C][P], s [P/64][C][2],
// blocked inside row groups. With the block table `blk` (mx_blocks_kernel:
// for each 64-column block of q, its first source row and how many of its
// rows are real) group e's rows land at q columns poff[e].. (poff: the groups
// padded to 64 rows) and the padding reads as zeros; without it the batch is
// one group of R rows (R a multiple of 64). With qk != nullptr (bf16 input,
// one group only) the same pass also writes the columns-blocked copy qk
// [R][C], sk [C/64][R][2] (mx_kmajor_kernel's layout), so a weight is read
// once for both of its GEMM layouts. T is bf16_t (weights, xp) or float (the
// fp32 operands H, dO, dG | dU of an MXFP8 layer, encoded exactly).
//
// One workgroup per (128 padded rows, 64 columns), each 64-row half resolving
// its own group: the tile goes through LDS; each wave reads one 32-row block
// of all 64 columns (thread = one column, 32 conflict-free reads), encodes it
// into an LDS output tile [64 columns][128 bytes], which then leaves as full
// 128-byte rows of q.
template <typename T>
__global__ __launch_bounds__(256) void mx_tgroup_kernel(const T* __restrict__ in, int R, int C,
                                                        const int2* __restrict__ blk, int64_t in_bstride, uint8_t* __restrict__ q, int64_t P,
                                                        int64_t q_bstride, uint8_t* __restrict__ s,
                                                        int64_t s_bstride, uint8_t* __restrict__ qk,
                                                        uint8_t* __restrict__ sk) {
  constexpr bool kF32 = sizeof(T) == 4;
  constexpr int VE = 16 / sizeof(T);  // elements per 16-byte load
  constexpr int LPR = 64 / VE;        // lanes per 64-column row
  constexpr int RPP = 256 / LPR;      // rows per pass of the workgroup
  constexpr int NP = 128 / RPP;       // passes over the 128 rows
  constexpr int kLd = 64 + VE;        // elements per LDS input row (16-byte aligned rows)
  constexpr int kLdq = 128 + 16;      // bytes per LDS output row
  __shared__ __attribute__((aligned(16))) T tile[128][kLd];
  __shared__ __attribute__((aligned(16))) uint8_t qt[64][kLdq];
  __shared__ int s_src[2], s_valid[2];
  const int tid = threadIdx.x, b = blockIdx.z;
  const int64_t p0 = static_cast<int64_t>(blockIdx.x) * 128;
  const int c0 = blockIdx.y * 64;
  if (tid < 2) {
    const int64_t ph = p0 + 64 * tid;
    int src = 0, valid = 0;
    if (ph < P) {
      if (blk == nullptr) {
        src = static_cast<int>(ph);
        valid = static_cast<int>(min(static_cast<int64_t>(64), static_cast<int64_t>(R) - ph));
      } else {
        const int2 t = blk[ph >> 6];
        src = t.x;
        valid = t.y;
      }
    }
    s_src[tid] = src;
    s_valid[tid] = valid;
  }
  __syncthreads();
  const T* src = in + static_cast<int64_t>(b) * in_bstride;
  const int ch = tid % LPR;
  // All loads go out before any is used: rows past a group's end load row 0
  // (always in bounds) and are replaced by zeros.
  uint4 raw[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int r = i * RPP + tid / LPR, h = r >> 6, rr = r & 63;
    const int64_t row = rr < s_valid[h] ? s_src[h] + rr : 0;
    raw[i] = ld16(src + row * C + c0 + ch * VE);
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int r = i * RPP + tid / LPR, h = r >> 6, rr = r & 63;
    const bool ok = rr < s_valid[h];
    const uint4 v = make_uint4(ok ? raw[i].x : 0u, ok ? raw[i].y : 0u, ok ? raw[i].z : 0u, ok ? raw[i].w : 0u);
    *reinterpret_cast<uint4*>(&tile[r][ch * VE]) = v;
    if constexpr (!kF32) {
      if (qk != nullptr && p0 + r < P) {  // uniform per wave (a wave's 8 rows share a 64-row half)
        // Columns-blocked copy straight from the registers (one group: row p0 + r).
        float f[8];
        unpack16(v, f);
        const int code = mx_group4_code(f);
        const int64_t row = p0 + r;
        *reinterpret_cast<uint2*>(qk + static_cast<int64_t>(b) * q_bstride + row * C + c0 + ch * 8) =
            mx_encode8(f, code);
        const int code_hi = __shfl(code, (tid & 56) + 4, kWave);
        if (ch == 0)
          *reinterpret_cast<uint16_t*>(sk + static_cast<int64_t>(b) * s_bstride +
                                       (static_cast<int64_t>(c0 / 64) * R + row) * 2) =
              static_cast<uint16_t>(code | (code_hi << 8));
      }
    }
  }
  __syncthreads();
  {
    const int col = tid & 63, block = tid >> 6;
    float v[32];
    uint32_t w[8];
    int code;
    if constexpr (kF32) {
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = tile[block * 32 + i][col];
      code = mx_encode_block_exact(v, w);
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = bf16_to_f32(tile[block * 32 + i][col]);
      code = mx_encode_block(v, w);
    }
    uint4* d = reinterpret_cast<uint4*>(&qt[col][block * 32]);
    d[0] = make_uint4(w[0], w[1], w[2], w[3]);
    d[1] = make_uint4(w[4], w[5], w[6], w[7]);
    if (p0 + block * 32 < P) {
      const int64_t sb = (p0 >> 6) + (block >> 1);
      s[static_cast<int64_t>(b) * s_bstride + (sb * C + c0 + col) * 2 + (block & 1)] = static_cast<uint8_t>(code);
    }
  }
  __syncthreads();
  // 64 columns x 128 bytes -> q rows, 8 lanes per 128-byte row.
  const int64_t pvalid = min(static_cast<int64_t>(128), P - p0);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = i * 32 + (tid >> 3), c16 = tid & 7;
    if (c16 * 16 < pvalid)
      *reinterpret_cast<uint4*>(q + static_cast<int64_t>(b) * q_bstride + static_cast<int64_t>(c0 + row) * P + p0 +
                                c16 * 16) = *reinterpret_cast<const uint4*>(&qt[row][c16 * 16]);
  }
}

// K along the columns of an fp32 matrix [R][C] (an MXFP8 layer's dO) -> q
// [R][C], s [C/64][R][2]: 8 lanes per 32-block of a row, 4 values each,
// encoded exactly.
__global__ __launch_bounds__(256) void mx_kmajor_f32_kernel(const float* __restrict__ in, int R, int C, int64_t nblk,
                                                            uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const int64_t g = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 3;
  const int c = threadIdx.x & 7;
  const bool live = g < nblk;  // the same for the 8 lanes of a block
  const int64_t gg = live ? g : 0;
  const int64_t row = gg / (C / 32), cb = gg % (C / 32);
  float x[4];
  unpack16(ld16(in + row * C + cb * 32 + c * 4), x);
  const int code = mx_group8_code(x);  // every lane: butterflies
  if (live) {
    *reinterpret_cast<uint32_t*>(q + row * C + cb * 32 + c * 4) = mx_encode4_exact(x, code);
    if (c == 0) s[((cb >> 1) * R + row) * 2 + (cb & 1)] = static_cast<uint8_t>(code);
  }
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

// Block table of the grouped transposing quantiser: for padded 64-row block
// b (b < P/64), the group e with poff[e] <= 64 b < poff[e+1] (binary search;
// empty groups have poff[e] == poff[e+1]) gives x = offsets[e] + 64 b -
// poff[e], y = min(64, offsets[e+1] - x); blocks past the last group get y = 0.
__global__ __launch_bounds__(256) void mx_blocks_kernel(const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ poff, int E, int nblk,
                                                        int2* __restrict__ blk) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblk) return;
  const int p = b * 64;
  int2 t = make_int2(0, 0);
  if (p < poff[E]) {
    int lo = 0, hi = E;  // poff[lo] <= p < poff[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (poff[mid] <= p) lo = mid; else hi = mid;
    }
    t.x = offsets[lo] + (p - poff[lo]);
    t.y = min(64, offsets[lo + 1] - t.x);
  }
  blk[b] = t;
}

hipError_t launch_mx_blocks(const int32_t* offsets, const int32_t* poff, int E, int64_t P, void* blk, hipStream_t st) {
  const int nblk = static_cast<int>(P / 64);
  hipLaunchKernelGGL(mx_blocks_kernel, dim3((nblk + 255) / 256), dim3(256), 0, st, offsets, poff, E, nblk,
                     static_cast<int2*>(blk));
  return hipGetLastError();
}

hipError_t launch_mx_kmajor_f32(const void* in, int R, int C, uint8_t* q, uint8_t* s, hipStream_t st) {
  const int64_t nblk = static_cast<int64_t>(R) * (C / 32);
  hipLaunchKernelGGL(mx_kmajor_f32_kernel, dim3(static_cast<unsigned>((nblk * 8 + 255) / 256)), dim3(256), 0, st,
                     static_cast<const float*>(in), R, C, nblk, q, s);
  return hipGetLastError();
}

hipError_t launch_mx_kmajor(const void* in, int R, int C, int batches, int64_t in_bstride, uint8_t* q,
                            int64_t q_bstride, uint8_t* s, int64_t s_bstride, hipStream_t st) {
  const int64_t ntiles = static_cast<int64_t>(batches) * (R / 8) * (C / 64);
  const int64_t waves = (ntiles + kTilesPerWave - 1) / kTilesPerWave;
  hipLaunchKernelGGL(mx_kmajor_kernel, dim3(static_cast<unsigned>((waves + 3) / 4)), dim3(256), 0, st,
                     static_cast<const bf16_t*>(in), R, C, ntiles, in_bstride, q, q_bstride, s, s_bstride);
  return hipGetLastError();
}

hipError_t launch_mx_tgroup(const void* in, int R, int C, const void* blk, int batches, int64_t in_bstride,
                            uint8_t* q, int64_t P, int64_t q_bstride, uint8_t* s, int64_t s_bstride, hipStream_t st,
                            uint8_t* qk, uint8_t* sk) {
  const dim3 grid(static_cast<unsigned>((P + 127) / 128), static_cast<unsigned>(C / 64),
                  static_cast<unsigned>(batches));
  hipLaunchKernelGGL(mx_tgroup_kernel<bf16_t>, grid, dim3(256), 0, st, static_cast<const bf16_t*>(in), R, C,
                     static_cast<const int2*>(blk), in_bstride, q, P, q_bstride, s, s_bstride, qk, sk);
  return hipGetLastError();
}

hipError_t launch_mx_tgroup_f32(const void* in, int R, int C, const void* blk, uint8_t* q, int64_t P, uint8_t* s,
                                hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((P + 127) / 128), static_cast<unsigned>(C / 64), 1);
  hipLaunchKernelGGL(mx_tgroup_kernel<float>, grid, dim3(256), 0, st, static_cast<const float*>(in), R, C,
                     static_cast<const int2*>(blk), 0, q, P, 0, s, 0, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_mx_poff(const int32_t* offsets, int E, int32_t* poff, hipStream_t st) {
  hipLaunchKernelGGL(mx_poff_kernel, dim3(1), dim3(64), 0, st, offsets, E, poff);
  return hipGetLastError();
}

}  // namespace moe
