// Dispatch (histogram, prefix scan, stable placement, row gather), combine,
// and their backward passes.
//
// The pages place routed rows straight into contiguous per-expert input
// buffers and keep the routing metadata on the GPU so the host enqueues work
// without waiting ("Olmo-core 3 escala el entrenamiento de mixture-of-experts
// a billones de parámetros", section "Cómo funciona"; "Ai2 rilascia Olmo-Core
// 3...", section "Parallelismo, precisione e tecniche di memoria"). On one GPU
// that placement is a local permute: a stable counting sort of the (token,
// slot) pairs by expert, followed by a token-major row copy that reads each
// token row once and writes it to its k destinations.
//
// Placement order inside an expert is increasing token index, which makes
// the permutation unique; it is computed without atomics on the slot order:
//   1. count:  per chunk of tokens, an LDS histogram of expert ids;
//   2. place:  per chunk, the workgroup first sums the [chunk][expert] counts
//              of all chunks (expert totals, offsets by a block scan) and of
//              the chunks before its own (its first row per expert); then
//              waves walk the slots in order, a ballot-based match gives each
//              slot its rank among equal experts of the wave, and per-wave
//              totals in LDS give the ranks across waves. Workgroup 0 also
//              writes counts, offsets and the status word.
// Chunks are 128 tokens while the [chunk][expert] table stays small (few
// tokens: more workgroups), else 512.
#include "common.h"
#include "kernels.h"

namespace moe {

// Tokens per histogram chunk.
static int chunk_tokens(int T, int E) {
  return static_cast<int64_t>((T + 127) / 128) * E <= 4096 ? 128 : 512;
}

struct DispatchWs {
  int32_t* status;       // 1 int (padded to 256 B)
  int32_t* chunk_counts; // [nch][E]
  int32_t* chunk_bad;    // [nch]
};

static size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

static DispatchWs carve(void* ws, int nch, int E) {
  char* p = static_cast<char*>(ws);
  DispatchWs w;
  w.status = reinterpret_cast<int32_t*>(p); p += 256;
  w.chunk_counts = reinterpret_cast<int32_t*>(p); p += align256(sizeof(int32_t) * nch * E);
  w.chunk_bad = reinterpret_cast<int32_t*>(p);
  return w;
}

size_t dispatch_workspace(int T, int E) {
  const int ct = chunk_tokens(T, E);
  const int nch = (T + ct - 1) / ct;
  return 256 + align256(sizeof(int32_t) * nch * E) + align256(sizeof(int32_t) * nch);
}

__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                             int ct, DispatchWs w) {
  __shared__ int hist[256];
  __shared__ int bad;
  const int c = blockIdx.x, tid = threadIdx.x;
  hist[tid] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  const int64_t s0 = static_cast<int64_t>(c) * ct * k;
  const int64_t s1 = min(static_cast<int64_t>(T), static_cast<int64_t>(c + 1) * ct) * k;
  int my_bad = 0;
  for (int64_t s = s0 + tid; s < s1; s += 256) {
    const int e = idx[s];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);  // integer counts: order-independent
    else my_bad = 1;
  }
  if (my_bad) bad = 1;
  __syncthreads();
  if (tid < E) w.chunk_counts[static_cast<int64_t>(c) * E + tid] = hist[tid];
  if (tid == 0) w.chunk_bad[c] = bad;
}

__global__ __launch_bounds__(256) void dispatch_place_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                             int bits, int ct, int nch, DispatchWs w,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ row_of_slot,
                                                             int32_t* __restrict__ token_of_row) {
  constexpr int kTab = 4096;  // ints of the [chunk][expert] table staged at a time
  __shared__ int tab[kTab];
  __shared__ int base[256];
  __shared__ int wcnt[4][256];
  __shared__ int wsum[4];
  const int c = blockIdx.x, tid = threadIdx.x, wave = tid >> 6;
  // Expert tid: total rows, and rows in the chunks before this one. The
  // table goes through LDS in pieces of whole chunk rows, read by all threads.
  int tot = 0, before = 0;
  const int rows_per = kTab / E;
  for (int c0 = 0; c0 < nch; c0 += rows_per) {
    const int nrow = min(rows_per, nch - c0);
    for (int i = tid; i < nrow * E; i += 256) tab[i] = w.chunk_counts[static_cast<int64_t>(c0) * E + i];
    __syncthreads();
    if (tid < E) {
      for (int r = 0; r < nrow; ++r) {
        const int n = tab[r * E + tid];
        tot += n;
        if (c0 + r < c) before += n;
      }
    }
    __syncthreads();
  }
  // Exclusive scan of the totals over experts: waves, then their sums.
  const int incl_w = wave_exclusive_scan(tot) + tot;
  if ((tid & 63) == 63) wsum[wave] = incl_w;
  __syncthreads();
  int off = incl_w - tot;
  for (int q = 0; q < wave; ++q) off += wsum[q];
  if (tid < E) {
    base[tid] = off + before;
#pragma unroll
    for (int q = 0; q < 4; ++q) wcnt[q][tid] = 0;
  }
  if (c == 0) {
    if (tid < E) {
      counts[tid] = tot;
      offsets[tid] = off;
    }
    if (tid == E - 1) offsets[E] = off + tot;
    if (tid == 0) {
      int bad = 0;
      for (int cc = 0; cc < nch; ++cc) bad |= w.chunk_bad[cc];
      w.status[0] = bad ? 1 : 0;
    }
  }
  __syncthreads();
  const int64_t s0 = static_cast<int64_t>(c) * ct * k;
  const int64_t s1 = min(static_cast<int64_t>(T), static_cast<int64_t>(c + 1) * ct) * k;
  for (int64_t sb = s0; sb < s1; sb += 256) {
    const int64_t s = sb + tid;
    const bool in = s < s1;
    const int e = in ? idx[s] : -1;
    const bool ok = in && e >= 0 && e < E;
    const uint64_t m = match_any(ok ? e : 0, ok, bits);
    const int rank = __popcll(m & lanemask_lt());
    if (ok && rank == 0) wcnt[wave][e] = __popcll(m);
    __syncthreads();
    if (ok) {
      int row = base[e] + rank;
      for (int q = 0; q < wave; ++q) row += wcnt[q][e];
      row_of_slot[s] = row;
      token_of_row[row] = static_cast<int32_t>(s / k);
    } else if (in) {
      row_of_slot[s] = -1;
    }
    __syncthreads();
    if (tid < E) {
      base[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
#pragma unroll
      for (int q = 0; q < 4; ++q) wcnt[q][tid] = 0;
    }
    __syncthreads();
  }
}

// Lanes per token for row kernels: enough 16-byte vectors to cover one row.
static int lanes_per_token(int nvec) {
  int l = 1;
  while (l < nvec && l < 256) l <<= 1;
  return l;
}

// xp[row_of_slot[t][j]] = x[t]: read the token row once, write it k times.
__global__ __launch_bounds__(256) void gather_rows_kernel(const char* __restrict__ x, const int32_t* __restrict__ row_of_slot,
                                                          int T, int k, int nvec, int lpt, char* __restrict__ xp) {
  const int tpw = 256 / lpt;
  const int t = blockIdx.x * tpw + threadIdx.x / lpt;
  const int sub = threadIdx.x % lpt;
  if (t >= T) return;
  const int64_t rb = static_cast<int64_t>(nvec) * 16;
  int rows[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) rows[j] = j < k ? row_of_slot[static_cast<int64_t>(t) * k + j] : -1;
  for (int v = sub; v < nvec; v += lpt) {
    const uint4 val = ld16(x + t * rb + v * 16);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (rows[j] >= 0) st16(xp + rows[j] * rb + v * 16, val);
  }
}

hipError_t launch_dispatch(const void* x, const int32_t* topk_idx, int elem_bytes, int T, int d, int E, int k,
                           int32_t* counts, int32_t* offsets, int32_t* row_of_slot, int32_t* token_of_row,
                           void* xp, void* ws, hipStream_t s) {
  const int ct = chunk_tokens(T, E);
  const int nch = (T + ct - 1) / ct;
  DispatchWs w = carve(ws, nch, E);
  int bits = 0;
  while ((1 << bits) < E) ++bits;
  hipLaunchKernelGGL(dispatch_count_kernel, dim3(nch), dim3(256), 0, s, topk_idx, T, E, k, ct, w);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_place_kernel, dim3(nch), dim3(256), 0, s, topk_idx, T, E, k, bits, ct, nch, w, counts,
                     offsets, row_of_slot, token_of_row);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int nvec = d * elem_bytes / 16;
  const int lpt = lanes_per_token(nvec);
  const int tpw = 256 / lpt;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((T + tpw - 1) / tpw), dim3(256), 0, s,
                     static_cast<const char*>(x), row_of_slot, T, k, nvec, lpt, static_cast<char*>(xp));
  return hipGetLastError();
}

// y[t] = sum_j gate[t][j] * o[row_of_slot[t][j]]  (fp32, slot order, one rounding).
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ o, const float* __restrict__ gate,
                                                      const int32_t* __restrict__ row_of_slot, int Tn, int k,
                                                      int nvec, int lpt, T* __restrict__ y) {
  constexpr int VE = Vec16<T>::N;
  const int tpw = 256 / lpt;
  const int t = blockIdx.x * tpw + threadIdx.x / lpt;
  const int sub = threadIdx.x % lpt;
  if (t >= Tn) return;
  const int64_t re = static_cast<int64_t>(nvec) * VE;  // elements per row
  int rows[8];
  float g[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    rows[j] = j < k ? row_of_slot[static_cast<int64_t>(t) * k + j] : -1;
    g[j] = j < k ? gate[static_cast<int64_t>(t) * k + j] : 0.0f;
  }
  for (int v = sub; v < nvec; v += lpt) {
    float acc[VE];
#pragma unroll
    for (int i = 0; i < VE; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (rows[j] < 0) continue;
      float ov[VE];
      unpack16(ld16(o + rows[j] * re + v * VE), ov);
#pragma unroll
      for (int i = 0; i < VE; ++i) acc[i] = fmaf(g[j], ov[i], acc[i]);
    }
    st16(y + t * re + v * VE, pack16(acc));
  }
}

// d_o[row(t,j)] = gate[t][j] * dy[t];  dgate[t][j] = <dy[t], o[row(t,j)]> (fp32,
// fixed reduction tree: per-thread partials, lane butterfly, then waves in order).
template <typename T>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const T* __restrict__ dy, const T* __restrict__ o,
                                                          const float* __restrict__ gate,
                                                          const int32_t* __restrict__ row_of_slot, int Tn, int k,
                                                          int nvec, int lpt, T* __restrict__ d_o,
                                                          float* __restrict__ dgate) {
  constexpr int VE = Vec16<T>::N;
  __shared__ float red[4][8];
  const int tpw = 256 / lpt;
  const int t = blockIdx.x * tpw + threadIdx.x / lpt;
  const int sub = threadIdx.x % lpt;
  const bool live = t < Tn;
  const int64_t re = static_cast<int64_t>(nvec) * VE;
  int rows[8];
  float g[8], part[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    rows[j] = (live && j < k) ? row_of_slot[static_cast<int64_t>(t) * k + j] : -1;
    g[j] = (live && j < k) ? gate[static_cast<int64_t>(t) * k + j] : 0.0f;
    part[j] = 0.0f;
  }
  if (live) {
    for (int v = sub; v < nvec; v += lpt) {
      float dv[VE];
      unpack16(ld16(dy + t * re + v * VE), dv);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (rows[j] < 0) continue;
        float ov[VE], sv[VE];
        unpack16(ld16(o + rows[j] * re + v * VE), ov);
#pragma unroll
        for (int i = 0; i < VE; ++i) {
          part[j] = fmaf(dv[i], ov[i], part[j]);
          sv[i] = g[j] * dv[i];
        }
        st16(d_o + rows[j] * re + v * VE, pack16(sv));
      }
    }
  }
  // Reduce part[j] over the lpt lanes of the token.
  const int width = lpt < 64 ? lpt : 64;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    for (int off = width >> 1; off > 0; off >>= 1) part[j] += __shfl_xor(part[j], off, kWave);
  if (lpt <= 64) {
    if (live && sub == 0)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < k) dgate[static_cast<int64_t>(t) * k + j] = rows[j] >= 0 ? part[j] : 0.0f;
  } else {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0)
#pragma unroll
      for (int j = 0; j < 8; ++j) red[wave][j] = part[j];
    __syncthreads();
    if (live && sub == 0) {
      const int w0 = (threadIdx.x / lpt) * (lpt / 64);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j >= k) break;
        float s = 0.0f;
        for (int q = 0; q < lpt / 64; ++q) s += red[w0 + q][j];
        dgate[static_cast<int64_t>(t) * k + j] = rows[j] >= 0 ? s : 0.0f;
      }
    }
  }
}

hipError_t launch_combine(const void* o, const float* gate, const int32_t* row_of_slot, bool is_f32, int T, int d,
                          int k, void* y, hipStream_t s) {
  const int nvec = d * (is_f32 ? 4 : 2) / 16;
  const int lpt = lanes_per_token(nvec), tpw = 256 / lpt;
  const dim3 grid((T + tpw - 1) / tpw);
  if (is_f32)
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(o), gate, row_of_slot,
                       T, k, nvec, lpt, static_cast<float*>(y));
  else
    hipLaunchKernelGGL(combine_kernel<bf16_t>, grid, dim3(256), 0, s, static_cast<const bf16_t*>(o), gate,
                       row_of_slot, T, k, nvec, lpt, static_cast<bf16_t*>(y));
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const void* dy, const void* o, const float* gate, const int32_t* row_of_slot,
                              bool is_f32, int T, int d, int k, void* d_o, float* dgate, hipStream_t s) {
  const int nvec = d * (is_f32 ? 4 : 2) / 16;
  const int lpt = lanes_per_token(nvec), tpw = 256 / lpt;
  const dim3 grid((T + tpw - 1) / tpw);
  if (is_f32)
    hipLaunchKernelGGL(combine_bwd_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(dy),
                       static_cast<const float*>(o), gate, row_of_slot, T, k, nvec, lpt, static_cast<float*>(d_o),
                       dgate);
  else
    hipLaunchKernelGGL(combine_bwd_kernel<bf16_t>, grid, dim3(256), 0, s, static_cast<const bf16_t*>(dy),
                       static_cast<const bf16_t*>(o), gate, row_of_slot, T, k, nvec, lpt,
                       static_cast<bf16_t*>(d_o), dgate);
  return hipGetLastError();
}

// W_r [d][E] -> W_rT [E][d] (same dtype), so the router term of dx reads rows.
template <typename T>
__global__ void transpose_router_kernel(const T* __restrict__ w, int d, int E, T* __restrict__ wt) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(d) * E) return;
  const int r = static_cast<int>(i / E), e = static_cast<int>(i % E);
  wt[static_cast<int64_t>(e) * d + r] = w[i];
}

// dx[t] = sum_j dxp[row(t,j)] (+ sum_{e: dl[t][e] != 0} dl[t][e] * W_rT[e]).
// dl is zero off the chosen set, so only those (at most k) columns are read.
// When a token has whole waves (lpt >= 64) each wave finds them with one
// ballot per 64 experts; narrower rows scan the E values per lane.
template <typename T>
__global__ __launch_bounds__(256) void dispatch_bwd_kernel(const T* __restrict__ dxp, const int32_t* __restrict__ row_of_slot,
                                                           const float* __restrict__ dl, const T* __restrict__ wt,
                                                           int Tn, int E, int k, int nvec, int lpt, T* __restrict__ dx) {
  constexpr int VE = Vec16<T>::N;
  const int tpw = 256 / lpt;
  const int t = blockIdx.x * tpw + threadIdx.x / lpt;
  const int sub = threadIdx.x % lpt;
  if (t >= Tn) return;
  const int64_t re = static_cast<int64_t>(nvec) * VE;
  int rows[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) rows[j] = j < k ? row_of_slot[static_cast<int64_t>(t) * k + j] : -1;
  // The token's router columns: (expert, dl) pairs, at most 8.
  int ce[8];
  float cv[8];
  int nr = 0;
  if (dl != nullptr) {
    const float* dlt = dl + static_cast<int64_t>(t) * E;
    if (lpt >= kWave) {
      const int lane = threadIdx.x & (kWave - 1);
      for (int c0 = 0; c0 < E; c0 += kWave) {
        const float c = (c0 + lane < E) ? dlt[c0 + lane] : 0.0f;
        uint64_t m = __ballot(c != 0.0f);
        while (m != 0 && nr < 8) {
          const int b = __ffsll(static_cast<long long>(m)) - 1;
          m &= m - 1;
          ce[nr] = c0 + b;
          cv[nr] = __shfl(c, b, kWave);
          ++nr;
        }
      }
    } else {
      for (int e = 0; e < E && nr < 8; ++e) {
        const float c = dlt[e];
        if (c != 0.0f) {
          ce[nr] = e;
          cv[nr] = c;
          ++nr;
        }
      }
    }
  }
  for (int v = sub; v < nvec; v += lpt) {
    float acc[VE];
#pragma unroll
    for (int i = 0; i < VE; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (rows[j] < 0) continue;
      float gv[VE];
      unpack16(ld16(dxp + rows[j] * re + v * VE), gv);
#pragma unroll
      for (int i = 0; i < VE; ++i) acc[i] += gv[i];
    }
    for (int r = 0; r < nr; ++r) {
      float wv[VE];
      unpack16(ld16(wt + ce[r] * re + v * VE), wv);
#pragma unroll
      for (int i = 0; i < VE; ++i) acc[i] = fmaf(cv[r], wv[i], acc[i]);
    }
    st16(dx + t * re + v * VE, pack16(acc));
  }
}

size_t dispatch_bwd_workspace(int d, int E, bool is_f32) {
  return static_cast<size_t>(d) * E * (is_f32 ? 4 : 2);
}

hipError_t launch_dispatch_bwd(const void* dxp, const int32_t* row_of_slot, const float* dlogits,
                               const void* w_router, bool is_f32, int T, int d, int E, int k, void* dx, void* ws,
                               hipStream_t s) {
  const bool router = dlogits != nullptr && w_router != nullptr;
  hipError_t err;
  if (router) {
    const int64_t n = static_cast<int64_t>(d) * E;
    const dim3 g(static_cast<unsigned>((n + 255) / 256));
    if (is_f32)
      hipLaunchKernelGGL(transpose_router_kernel<float>, g, dim3(256), 0, s, static_cast<const float*>(w_router), d,
                         E, static_cast<float*>(ws));
    else
      hipLaunchKernelGGL(transpose_router_kernel<bf16_t>, g, dim3(256), 0, s, static_cast<const bf16_t*>(w_router),
                         d, E, static_cast<bf16_t*>(ws));
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const int nvec = d * (is_f32 ? 4 : 2) / 16;
  const int lpt = lanes_per_token(nvec), tpw = 256 / lpt;
  const dim3 grid((T + tpw - 1) / tpw);
  const float* dl = router ? dlogits : nullptr;
  if (is_f32)
    hipLaunchKernelGGL(dispatch_bwd_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(dxp), row_of_slot,
                       dl, static_cast<const float*>(ws), T, E, k, nvec, lpt, static_cast<float*>(dx));
  else
    hipLaunchKernelGGL(dispatch_bwd_kernel<bf16_t>, grid, dim3(256), 0, s, static_cast<const bf16_t*>(dxp),
                       row_of_slot, dl, static_cast<const bf16_t*>(ws), T, E, k, nvec, lpt,
                       static_cast<bf16_t*>(dx));
  return hipGetLastError();
}

}  // namespace moe
