// Router: logits = x W_r, softmax, top-k, renormalised gates; and its backward.
//
// Each token activates k of the E experts ("Olmo-core 3 é lançado com
// infraestrutura para treinar modelos MoE", section "Mudança de arquitetura e
// ganhos de desempenho"); routing stays on the device so the host never waits
// for it ("Olmo-core 3 escala el entrenamiento de mixture-of-experts a billones
// de parámetros", section "Cómo funciona"). Softmax, top-k with ties to the
// lower index and gate renormalisation follow the layer specification.
//
// The router contraction has a narrow output (E <= 256 columns); it runs as a
// register-blocked fp32 FMA kernel: a workgroup owns 32 output rows x all E
// columns, stages 32-deep slices of both operands in LDS, every thread owns
// 4x4 output blocks and, when the output is narrow, a share of the reduction
// (combined in a fixed order at the end).
#include <math.h>

#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

constexpr int kRtm = 32;   // output rows per workgroup
constexpr int kRkc = 32;   // reduction slice staged in LDS
constexpr int kRouteTokChunk = 1024;  // tokens per partial sum of dW_r

// C[m][n] (fp32) = sum_{k in [k_begin, k_end)} A(m,k) * B[k][n], n < N (<= 256).
// A_KMAJOR: A is [M][K] row-major (x in the forward); else A is [K][M] (x in
// the weight gradient, where K runs over tokens). B is [K][N] row-major.
template <typename TA, typename TB, bool A_KMAJOR>
__global__ __launch_bounds__(256) void narrow_gemm_kernel(const TA* __restrict__ A, const TB* __restrict__ B,
                                                          float* __restrict__ C, int M, int N, int K,
                                                          int k_chunk, int64_t c_chunk_stride) {
  __shared__ __attribute__((aligned(16))) float As[kRkc][kRtm];
  __shared__ __attribute__((aligned(16))) float Bs[kRkc][256];
  __shared__ float red[256 * 16];
  const int tid = threadIdx.x;
  const int NP = (N + 3) & ~3;
  const int ngrp = NP / 4;
  const int nb = (kRtm / 4) * ngrp;                 // 4x4 blocks in the tile
  const int KS = nb >= 256 ? 1 : 256 / nb;          // reduction split inside the workgroup
  const int m0 = blockIdx.x * kRtm;
  const int k_begin = blockIdx.y * k_chunk;
  const int k_end = min(K, k_begin + k_chunk);
  C += static_cast<int64_t>(blockIdx.y) * c_chunk_stride;

  float acc[2][16];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[b][q] = 0.0f;
  const int ks = (nb >= 256) ? 0 : tid / nb;
  const int blk0 = (nb >= 256) ? tid : tid % nb;
  const bool active = (nb >= 256) || (tid < KS * nb);

  for (int kc = k_begin; kc < k_end; kc += kRkc) {
    // Stage A as As[k][m] and B as Bs[k][n], zero outside the valid ranges.
    for (int i = tid; i < kRtm * kRkc; i += 256) {
      int m, kk;
      if constexpr (A_KMAJOR) { m = i / kRkc; kk = i % kRkc; }
      else { kk = i / kRtm; m = i % kRtm; }
      const int gm = m0 + m, gk = kc + kk;
      float v = 0.0f;
      if (gm < M && gk < k_end)
        v = Elem<TA>::to_f32(A_KMAJOR ? A[static_cast<int64_t>(gm) * K + gk] : A[static_cast<int64_t>(gk) * M + gm]);
      As[kk][m] = v;
    }
    for (int i = tid; i < kRkc * NP; i += 256) {
      const int kk = i / NP, n = i % NP, gk = kc + kk;
      Bs[kk][n] = (n < N && gk < k_end) ? Elem<TB>::to_f32(B[static_cast<int64_t>(gk) * N + n]) : 0.0f;
    }
    __syncthreads();
    if (active) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int blk = blk0 + b * 256;
        if (blk < nb) {
          const int mg = blk / ngrp, ng = blk % ngrp;
          for (int kk = ks; kk < kRkc; kk += KS) {
            const float4 a4 = *reinterpret_cast<const float4*>(&As[kk][mg * 4]);
            const float4 b4 = *reinterpret_cast<const float4*>(&Bs[kk][ng * 4]);
            const float av[4] = {a4.x, a4.y, a4.z, a4.w};
            const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int j = 0; j < 4; ++j) acc[b][i * 4 + j] = fmaf(av[i], bv[j], acc[b][i * 4 + j]);
          }
        }
      }
    }
    __syncthreads();
  }

  if (KS == 1) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int blk = blk0 + b * 256;
      if (blk < nb) {
        const int mg = blk / ngrp, ng = blk % ngrp;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int m = m0 + mg * 4 + q / 4, n = ng * 4 + q % 4;
          if (m < M && n < N) C[static_cast<int64_t>(m) * N + n] = acc[b][q];
        }
      }
    }
  } else {
    // Combine the KS partial sums of each block in ks order.
    if (active) {
#pragma unroll
      for (int q = 0; q < 16; ++q) red[(ks * nb + blk0) * 16 + q] = acc[0][q];
    }
    __syncthreads();
    for (int o = tid; o < nb * 16; o += 256) {
      const int blk = o / 16, q = o % 16;
      float s = 0.0f;
      for (int j = 0; j < KS; ++j) s += red[(j * nb + blk) * 16 + q];
      const int mg = blk / ngrp, ng = blk % ngrp;
      const int m = m0 + mg * 4 + q / 4, n = ng * 4 + q % 4;
      if (m < M && n < N) C[static_cast<int64_t>(m) * N + n] = s;
    }
  }
}

// One wave per token: top-k and gates of the logits (topk.h).
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                   int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[4];
  bool live[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = q * 64 + lane;
    live[q] = e < E;
    v[q] = live[q] ? logits[static_cast<int64_t>(t) * E + e] : 0.0f;
  }
  float sel_v[8], g[8];
  int sel_i[8];
  wave_topk(v, live, k, lane, sel_v, sel_i);
  topk_gates(sel_v, k, g);
  if (lane < k) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j == lane) {
        topk_idx[static_cast<int64_t>(t) * k + j] = sel_i[j];
        topk_gate[static_cast<int64_t>(t) * k + j] = g[j];
      }
  }
}

// dlogits[t][e] = g_te (dgate_te - sum_j g_tj dgate_tj) on the chosen set, else 0.
__global__ void dlogits_kernel(const int32_t* __restrict__ idx, const float* __restrict__ gate,
                               const float* __restrict__ dgate, int T, int E, int k, float* __restrict__ dl) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(T) * E) return;
  const int t = static_cast<int>(i / E), e = static_cast<int>(i % E);
  const int32_t* it = idx + static_cast<int64_t>(t) * k;
  const float* gt = gate + static_cast<int64_t>(t) * k;
  const float* dt = dgate + static_cast<int64_t>(t) * k;
  float inner = 0.0f, out = 0.0f;
  for (int j = 0; j < k; ++j) inner = fmaf(gt[j], dt[j], inner);
  for (int j = 0; j < k; ++j)
    if (it[j] == e) out = gt[j] * (dt[j] - inner);
  dl[i] = out;
}

// dW_r[i][e] = sum over token chunks c (in order) of part[c][i][e].
template <typename T>
__global__ void reduce_chunks_kernel(const float* __restrict__ part, int nchunks, int64_t n, T* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  for (int c = 0; c < nchunks; ++c) s += part[c * n + i];
  out[i] = Elem<T>::from_f32(s);
}

hipError_t launch_route(const void* x, const void* w_router, bool is_f32, int T, int d, int E, int k,
                        float* logits, int32_t* topk_idx, float* topk_gate, hipStream_t s) {
  const dim3 grid((T + kRtm - 1) / kRtm, 1);
  if (is_f32)
    hipLaunchKernelGGL((narrow_gemm_kernel<float, float, true>), grid, dim3(256), 0, s,
                       static_cast<const float*>(x), static_cast<const float*>(w_router), logits, T, E, d, d, 0);
  else
    hipLaunchKernelGGL((narrow_gemm_kernel<bf16_t, bf16_t, true>), grid, dim3(256), 0, s,
                       static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(w_router), logits, T, E, d, d, 0);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, topk_idx, topk_gate);
  return hipGetLastError();
}

size_t route_bwd_workspace(int T, int d, int E) {
  const int nch = (T + kRouteTokChunk - 1) / kRouteTokChunk;
  return static_cast<size_t>(nch) * d * E * sizeof(float);
}

hipError_t launch_route_bwd(const void* x, const int32_t* topk_idx, const float* topk_gate,
                            const float* dgate, bool is_f32, int T, int d, int E, int k,
                            float* dlogits, void* dw_router, void* ws, hipStream_t s) {
  const int64_t te = static_cast<int64_t>(T) * E;
  hipLaunchKernelGGL(dlogits_kernel, dim3(static_cast<unsigned>((te + 255) / 256)), dim3(256), 0, s,
                     topk_idx, topk_gate, dgate, T, E, k, dlogits);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int nch = (T + kRouteTokChunk - 1) / kRouteTokChunk;
  float* part = static_cast<float*>(ws);
  const int64_t de = static_cast<int64_t>(d) * E;
  const dim3 grid((d + kRtm - 1) / kRtm, nch);
  if (is_f32)
    hipLaunchKernelGGL((narrow_gemm_kernel<float, float, false>), grid, dim3(256), 0, s,
                       static_cast<const float*>(x), dlogits, part, d, E, T, kRouteTokChunk, de);
  else
    hipLaunchKernelGGL((narrow_gemm_kernel<bf16_t, float, false>), grid, dim3(256), 0, s,
                       static_cast<const bf16_t*>(x), dlogits, part, d, E, T, kRouteTokChunk, de);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const unsigned rg = static_cast<unsigned>((de + 255) / 256);
  if (is_f32)
    hipLaunchKernelGGL(reduce_chunks_kernel<float>, dim3(rg), dim3(256), 0, s, part, nch, de,
                       static_cast<float*>(dw_router));
  else
    hipLaunchKernelGGL(reduce_chunks_kernel<bf16_t>, dim3(rg), dim3(256), 0, s, part, nch, de,
                       static_cast<bf16_t*>(dw_router));
  return hipGetLastError();
}

}  // namespace moe
