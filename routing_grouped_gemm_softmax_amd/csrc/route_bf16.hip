// bf16 router on the matrix cores: logits = x W_r with softmax top-k fused in,
// and the router weight gradient dW_r = x^T dlogits.
//
// Each token activates k of the E experts ("Olmo-core 3 é lançado com
// infraestrutura para treinar modelos MoE", section "Mudança de arquitetura e
// ganhos de desempenho"); routing stays on the device ("Olmo-core 3 escala el
// entrenamiento de mixture-of-experts a billones de parámetros", section "Cómo
// funciona"). The contraction is narrow (E columns) and long (K = d), so it is
// bound by reading x once; v_mfma_f32_16x16x32_bf16 keeps the arithmetic far
// below that, for any E up to 256.
//
// Forward: a workgroup takes 16 tokens; its 4 waves split K, each computes
// 16 x E16 partial logits (E16 = E rounded up to 16 x a power of two) from x
// rows and a transposed, zero-padded router weight W_r^T (written by
// router_wt_kernel into the workspace, fragment-major like the dl^T terms
// below: one contiguous kilobyte per 16 experts x 32 k step), then the partials are added in wave
// order in LDS, written out as fp32 logits, and each wave selects the top-k of
// its 4 tokens at once (16 lanes per token) with the rule of topk.h.
//
// Backward: dlogits (fp32, [T][E]) and its transpose split into two bf16
// terms, hi = bf16(dl) and lo = bf16(dl - hi), so the bf16 MFMA sees dl to
// about 16 bits. The two terms are stored fragment-major: the 16 x 32 block
// (16 experts, 32 tokens) one MFMA step reads is 1 KB, lane l's 16 bytes at
// 16 l, so each operand load is one contiguous kilobyte. dW_r^T's partial over a chunk of 256 tokens and 64 columns of
// d is one workgroup: the x tile [256 tok][64 col] is staged in LDS by DMA
// and read transposed (ds_read_b64_tr_b16) as the MFMA's row operand; the
// per-chunk partials are summed over chunks in order (deterministic).
#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {
namespace {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) v4s lds_v4s_t;

constexpr int kTokChunk = 256;  // tokens per dW_r partial

int pow2_blocks(int E) {
  int eb = 1;
  while (eb * 16 < E) eb <<= 1;
  return eb;  // E16 = 16 * eb
}

// W_r [d][E] -> W_r^T fragment-major, experts >= E zero: element i is
// expert 16 eb + (i / 8) % 16, row 32 s + 8 ((i / 128) % 4) + i % 8 of W_r,
// with eb, s = (i / 512) / (d / 32), (i / 512) % (d / 32): the MFMA operand
// of lane (i / 8) % 64 in k step s for experts 16 eb .. 16 eb + 15.
__global__ void router_wt_kernel(const bf16_t* __restrict__ w, int d, int E, int E16, bf16_t* __restrict__ wt) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(E16) * d) return;
  const int ln = static_cast<int>((i >> 3) & 63), ns = d >> 5;
  const int blk = static_cast<int>(i >> 9);
  const int e = (blk / ns) * 16 + (ln & 15);
  const int r = (blk % ns) * 32 + 8 * (ln >> 4) + static_cast<int>(i & 7);
  wt[i] = e < E ? w[static_cast<int64_t>(r) * E + e] : static_cast<bf16_t>(0);
}

template <int EB>
__global__ __launch_bounds__(256) void router_fwd_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wt,
                                                         int T, int d, int E, int k, float* __restrict__ logits,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_gate) {
  constexpr int E16 = EB * 16;
  // k steps in flight per wave: every load of a group is issued before its
  // first MFMA (the scheduler would otherwise interleave them and keep only
  // a third of the group in flight).
  constexpr int U = EB >= 16 ? 1 : (EB == 8 ? 4 : 16 / EB);
  __shared__ float buf[16][E16 + 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * 16;
  // MFMA operands: lane -> row (token) / column (expert) lane%16, k = 8 (lane/16) .. +7.
  const int row = min(t0 + (lane & 15), T - 1);  // rows past T are computed and dropped
  const bf16_t* xr = x + static_cast<int64_t>(row) * d + 8 * (lane >> 4);
  const bf16_t* wr = wt + 8 * lane;  // k step s of expert block eb: 512 (eb d / 32 + s) elements on
  const int64_t wstep = static_cast<int64_t>(d >> 5) * 512;
  floatx4 acc[EB];
#pragma unroll
  for (int eb = 0; eb < EB; ++eb) acc[eb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  // Wave w takes the w-th quarter of the k steps, so a row's consecutive
  // 64-byte pieces are read by one wave, back to back.
  const int nsteps = d / 32, s_hi = nsteps * (wave + 1) / 4;
  int s = nsteps * wave / 4;
  for (; s + U <= s_hi; s += U) {
    bf16x8 a[U], b[U][EB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      a[u] = *reinterpret_cast<const bf16x8*>(xr + (s + u) * 32);
#pragma unroll
      for (int eb = 0; eb < EB; ++eb)
        b[u][eb] = *reinterpret_cast<const bf16x8*>(wr + eb * wstep + (s + u) * 512);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int eb = 0; eb < EB; ++eb)
        acc[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[u][eb], acc[eb], 0, 0, 0);
  }
  for (; s < s_hi; ++s) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(xr + s * 32);
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(wr + eb * wstep + s * 512);
      acc[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[eb], 0, 0, 0);
    }
  }
  // Sum the four K quarters in wave order. Lane l holds tokens 4 (l/16) + r,
  // expert eb*16 + l%16.
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int eb = 0; eb < EB; ++eb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float& dst = buf[4 * (lane >> 4) + r][eb * 16 + (lane & 15)];
          dst = (w == 0) ? acc[eb][r] : dst + acc[eb][r];
        }
    }
    __syncthreads();
  }
  // Logits out, then top-k and gates: wave w takes tokens 4w .. 4w+3 in
  // parallel, 16 lanes each; lane l holds experts 16 q + l % 16.
  const int ti = wave * 4 + (lane >> 4), t = t0 + ti, sub = lane & 15;
  float v[EB];
  bool live[EB];
#pragma unroll
  for (int q = 0; q < EB; ++q) {
    const int e = 16 * q + sub;
    live[q] = e < E;  // tokens past T are selected for and not stored
    v[q] = live[q] ? buf[ti][e] : 0.0f;
    if (live[q] && t < T) logits[static_cast<int64_t>(t) * E + e] = v[q];
  }
  float sel_v[8], g[8];
  int sel_i[8];
  group16_topk(v, live, k, lane, sel_v, sel_i);
  topk_gates(sel_v, k, g);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < k && sub == j && t < T) {
      topk_idx[static_cast<int64_t>(t) * k + j] = sel_i[j];
      topk_gate[static_cast<int64_t>(t) * k + j] = g[j];
    }
}


// dlogits[t][e] = g_te (dgate_te - sum_j g_tj dgate_tj) on the chosen set,
// else 0; plus dl^T as two bf16 terms (zero for e >= E or t >= T). Element
// i of a term is expert e = 16 eb + (i / 8) % 16, token t = 32 ks + 8 ((i / 128) % 4) + i % 8,
// with eb, ks = (i / 512) / (Tp / 32), (i / 512) % (Tp / 32): the operand
// of lane (i / 8) % 64 in MFMA step ks for experts 16 eb .. 16 eb + 15.
__global__ void dlogits_split_kernel(const int32_t* __restrict__ idx, const float* __restrict__ gate,
                                     const float* __restrict__ dgate, int T, int Tp, int E, int E16, int k,
                                     float* __restrict__ dl, bf16_t* __restrict__ dlt_hi,
                                     bf16_t* __restrict__ dlt_lo) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(Tp) * E16) return;
  const int ln = static_cast<int>((i >> 3) & 63), nks = Tp >> 5;
  const int64_t blk = i >> 9;
  const int e = static_cast<int>(blk / nks) * 16 + (ln & 15);
  const int t = static_cast<int>(blk % nks) * 32 + 8 * (ln >> 4) + static_cast<int>(i & 7);
  float out = 0.0f;
  if (t < T && e < E) {
    const int32_t* it = idx + static_cast<int64_t>(t) * k;
    const float* gt = gate + static_cast<int64_t>(t) * k;
    const float* dt = dgate + static_cast<int64_t>(t) * k;
    float inner = 0.0f;
    for (int j = 0; j < k; ++j) inner = fmaf(gt[j], dt[j], inner);
    for (int j = 0; j < k; ++j)
      if (it[j] == e) out = gt[j] * (dt[j] - inner);
    dl[static_cast<int64_t>(t) * E + e] = out;
  }
  const bf16_t hi = f32_to_bf16(out);
  dlt_hi[i] = hi;
  dlt_lo[i] = f32_to_bf16(out - bf16_to_f32(hi));
}

// XOR applied to the 16-byte chunk index of x-tile row `row` (rows of 128 B):
// the transposing reads of a half-wave touch rows r..r+3 and r+8..r+11 (r a
// multiple of 4) at the same two chunks; this puts the 16 pieces on distinct
// banks.
__device__ __forceinline__ int xt_swz(int row) { return (((row >> 1) & 1) << 1) | (((row >> 3) & 1) << 2); }

// Buffer descriptor over [base, base + bytes) (out-of-range loads read 0),
// built from wave-uniform values so it lives in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
  const int n = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes < 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffffLL : bytes)));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo), 0, n,
                                           0x00020000);
}

// LDS DMA of 16 bytes per lane (lane i -> lds_wave + 16 i). The s_nop gives
// the wait states the compiler does not insert before inline assembly: 5
// after a VALU write of the descriptor SGPRs, 1 after the write of M0.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds_wave) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds" ::"v"(voff), "{m0}"(lds_wave), "s"(r)
               : "memory");
}

template <int EB>
__global__ __launch_bounds__(256) void router_wgrad_kernel(const bf16_t* __restrict__ x,
                                                           const bf16_t* __restrict__ dlt_hi,
                                                           const bf16_t* __restrict__ dlt_lo, int T, int Tp, int d,
                                                           int E, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) char xs[kTokChunk * 128];  // [256 tokens][64 columns] bf16
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int dc0 = blockIdx.x * 64, tc0 = blockIdx.y * kTokChunk;
  const int cw = wave * 16;                 // this wave's 16 columns of the tile
  const int g = lane >> 4, sl = lane & 15;  // 16-lane group, lane inside it
  // dl^T operands: step kk of expert block eb is the kilobyte at
  // 512 (eb Tp / 32 + tc0 / 32 + kk) elements; this lane's 8 at 8 lane.
  const int64_t fbase = (static_cast<int64_t>(tc0 >> 5) * 64 + lane) * 8;
  auto dl_off = [&](int eb, int kk) { return fbase + (static_cast<int64_t>(eb) * (Tp >> 5) + kk) * 512; };
  {
    const int valid = max(0, min(kTokChunk, T - tc0));  // rows past T read as zero
    const int64_t bytes = static_cast<int64_t>(valid) * d * 2;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(x + static_cast<int64_t>(tc0) * d + dc0, bytes);
    const uint32_t base = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(static_cast<void*>(xs))));
#pragma unroll
    for (int q = 0; q < kTokChunk * 128 / 4096; ++q) {
      const int byte0 = (q * 4 + wave) * 1024;
      const int kr = (byte0 >> 7) + (lane >> 3);
      const int ch = (lane & 7) ^ xt_swz(kr);
      load_lds16(rs, static_cast<uint32_t>(kr * d * 2 + ch * 16), base + byte0);
    }
  }
  // With few expert blocks, all of the chunk's dl^T operands (EB x 8 steps x
  // hi, lo: 16 bytes each) are requested while the x tile lands, so the
  // loop below does not wait on memory.
  constexpr bool kPrefetch = EB <= 2;
  constexpr int kSteps = kTokChunk / 32;
  bf16x8 pre_h[kPrefetch ? EB : 1][kPrefetch ? kSteps : 1], pre_l[kPrefetch ? EB : 1][kPrefetch ? kSteps : 1];
  if constexpr (kPrefetch) {
#pragma unroll
    for (int eb = 0; eb < EB; ++eb)
#pragma unroll
      for (int kk = 0; kk < kSteps; ++kk) {
        const int64_t o = dl_off(eb, kk);
        pre_h[eb][kk] = *reinterpret_cast<const bf16x8*>(dlt_hi + o);
        pre_l[eb][kk] = *reinterpret_cast<const bf16x8*>(dlt_lo + o);
      }
  }
  __builtin_amdgcn_s_waitcnt(0x0070 | (15 << 8));  // vmcnt(0): the x tile (and the dl^T operands)
  __syncthreads();

  floatx4 acc[EB];
#pragma unroll
  for (int eb = 0; eb < EB; ++eb) acc[eb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  // Without the prefetch, step kk + 1's dl^T operands are requested before
  // step kk's MFMAs, so each step waits on loads issued one step earlier.
  bf16x8 nx_h[kPrefetch ? 1 : EB], nx_l[kPrefetch ? 1 : EB];
  auto load_dl = [&](int kk) {
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) {
      const int64_t o = dl_off(eb, kk);
      nx_h[eb] = *reinterpret_cast<const bf16x8*>(dlt_hi + o);
      nx_l[eb] = *reinterpret_cast<const bf16x8*>(dlt_lo + o);
    }
  };
  if constexpr (!kPrefetch) load_dl(0);
#pragma unroll
  for (int kk = 0; kk < kSteps; ++kk) {
    bf16x8 cu_h[kPrefetch ? 1 : EB], cu_l[kPrefetch ? 1 : EB];
    if constexpr (!kPrefetch) {
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) {
        cu_h[eb] = nx_h[eb];
        cu_l[eb] = nx_l[eb];
      }
      if (kk + 1 < kSteps) load_dl(kk + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Row operand = x^T: lane -> column cw + lane%16, tokens 32 kk + 8 g .. +7.
    v4s h[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int kr = kk * 32 + 8 * g + 4 * half + (sl >> 2);
      const int col = cw + 4 * (sl & 3);
      const int off = kr * 128 + ((((col >> 3) ^ xt_swz(kr)) & 7) << 4) + ((col & 7) << 1);
      h[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(xs + off));
    }
    bf16x8 a;
    __builtin_memcpy(&a, h, 16);
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) {
      bf16x8 bh, bl;
      if constexpr (kPrefetch) {
        bh = pre_h[eb][kk];
        bl = pre_l[eb][kk];
      } else {
        bh = cu_h[eb];
        bl = cu_l[eb];
      }
      acc[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, acc[eb], 0, 0, 0);
      acc[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, acc[eb], 0, 0, 0);
    }
  }
  // Lane l holds columns 4 (l/16) + r of the wave's 16, expert eb*16 + l%16.
  float* out = part + (static_cast<int64_t>(blockIdx.y) * d + dc0 + cw) * E;
#pragma unroll
  for (int eb = 0; eb < EB; ++eb) {
    const int e = eb * 16 + sl;
    if (e < E)
#pragma unroll
      for (int r = 0; r < 4; ++r) out[static_cast<int64_t>(4 * g + r) * E + e] = acc[eb][r];
  }
}

// dW_r[i][e] = sum over token chunks c (in order) of part[c][i][e]. The
// loads of 8 chunks are issued before their in-order sum.
__global__ void reduce_router_chunks_kernel(const float* __restrict__ part, int nchunks, int64_t n,
                                            bf16_t* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  int c = 0;
  for (; c + 8 <= nchunks; c += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(c + u) * n + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; c < nchunks; ++c) s += part[c * n + i];
  out[i] = f32_to_bf16(s);
}

template <int EB>
hipError_t route_fwd_eb(const bf16_t* x, const bf16_t* wt, int T, int d, int E, int k, float* logits,
                        int32_t* idx, float* gate, hipStream_t s) {
  hipLaunchKernelGGL(router_fwd_kernel<EB>, dim3((T + 15) / 16), dim3(256), 0, s, x, wt, T, d, E, k, logits, idx,
                     gate);
  return hipGetLastError();
}

template <int EB>
hipError_t route_wgrad_eb(const bf16_t* x, const bf16_t* hi, const bf16_t* lo, int T, int Tp, int d, int E,
                          float* part, hipStream_t s) {
  hipLaunchKernelGGL(router_wgrad_kernel<EB>, dim3(d / 64, Tp / kTokChunk), dim3(256), 0, s, x, hi, lo, T, Tp, d, E,
                     part);
  return hipGetLastError();
}

}  // namespace

size_t route_bf16_workspace(int d, int E) { return static_cast<size_t>(16) * pow2_blocks(E) * d * 2; }

hipError_t launch_route_bf16(const void* x, const void* w_router, int T, int d, int E, int k, float* logits,
                             int32_t* topk_idx, float* topk_gate, void* ws, hipStream_t s) {
  const int eb = pow2_blocks(E), E16 = 16 * eb;
  bf16_t* wt = static_cast<bf16_t*>(ws);
  const int64_t n = static_cast<int64_t>(E16) * d;
  hipLaunchKernelGGL(router_wt_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                     static_cast<const bf16_t*>(w_router), d, E, E16, wt);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  switch (eb) {
    case 1: return route_fwd_eb<1>(xb, wt, T, d, E, k, logits, topk_idx, topk_gate, s);
    case 2: return route_fwd_eb<2>(xb, wt, T, d, E, k, logits, topk_idx, topk_gate, s);
    case 4: return route_fwd_eb<4>(xb, wt, T, d, E, k, logits, topk_idx, topk_gate, s);
    case 8: return route_fwd_eb<8>(xb, wt, T, d, E, k, logits, topk_idx, topk_gate, s);
    default: return route_fwd_eb<16>(xb, wt, T, d, E, k, logits, topk_idx, topk_gate, s);
  }
}

static size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

size_t route_bwd_bf16_workspace(int T, int d, int E) {
  const int Tp = (T + kTokChunk - 1) / kTokChunk * kTokChunk;
  const int E16 = 16 * pow2_blocks(E);
  const size_t part = static_cast<size_t>(Tp / kTokChunk) * d * E * sizeof(float);
  return align256(part) + 2 * align256(static_cast<size_t>(E16) * Tp * 2);
}

hipError_t launch_route_bwd_bf16(const void* x, const int32_t* topk_idx, const float* topk_gate, const float* dgate,
                                 int T, int d, int E, int k, float* dlogits, void* dw_router, void* ws,
                                 hipStream_t s) {
  const int Tp = (T + kTokChunk - 1) / kTokChunk * kTokChunk, nch = Tp / kTokChunk;
  const int eb = pow2_blocks(E), E16 = 16 * eb;
  char* w = static_cast<char*>(ws);
  float* part = reinterpret_cast<float*>(w);
  w += align256(static_cast<size_t>(nch) * d * E * sizeof(float));
  bf16_t* hi = reinterpret_cast<bf16_t*>(w);
  w += align256(static_cast<size_t>(E16) * Tp * 2);
  bf16_t* lo = reinterpret_cast<bf16_t*>(w);
  const int64_t n = static_cast<int64_t>(E16) * Tp;
  hipLaunchKernelGGL(dlogits_split_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, topk_idx,
                     topk_gate, dgate, T, Tp, E, E16, k, dlogits, hi, lo);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  switch (eb) {
    case 1: err = route_wgrad_eb<1>(xb, hi, lo, T, Tp, d, E, part, s); break;
    case 2: err = route_wgrad_eb<2>(xb, hi, lo, T, Tp, d, E, part, s); break;
    case 4: err = route_wgrad_eb<4>(xb, hi, lo, T, Tp, d, E, part, s); break;
    case 8: err = route_wgrad_eb<8>(xb, hi, lo, T, Tp, d, E, part, s); break;
    default: err = route_wgrad_eb<16>(xb, hi, lo, T, Tp, d, E, part, s); break;
  }
  if (err != hipSuccess) return err;
  const int64_t de = static_cast<int64_t>(d) * E;
  hipLaunchKernelGGL(reduce_router_chunks_kernel, dim3(static_cast<unsigned>((de + 255) / 256)), dim3(256), 0, s,
                     part, nch, de, static_cast<bf16_t*>(dw_router));
  return hipGetLastError();
}

}  // namespace moe
