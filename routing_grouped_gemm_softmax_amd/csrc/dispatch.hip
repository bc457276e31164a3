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
#include "mx_encode.h"

#include <climits>
#include <mutex>
#include <type_traits>

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

// Per chunk: the LDS histogram of expert ids, and the chunk's fault bits
// (MOE_DEV_BAD_EXPERT: an id outside [0, E); MOE_DEV_DUP_EXPERT: one token
// names the same expert in two slots). One thread per token.
__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                             int ct, DispatchWs w) {
  __shared__ int hist[256];
  __shared__ int bad;
  const int c = blockIdx.x, tid = threadIdx.x;
  hist[tid] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  const int64_t t0 = static_cast<int64_t>(c) * ct;
  const int64_t t1 = min(static_cast<int64_t>(T), static_cast<int64_t>(c + 1) * ct);
  int my_bad = 0;
  for (int64_t t = t0 + tid; t < t1; t += 256) {
    int ids[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) ids[j] = j < k ? idx[t * k + j] : -1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= k) break;
      const int e = ids[j];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);  // integer counts: order-independent
      else my_bad |= 1;
#pragma unroll
      for (int i = 0; i < j; ++i) my_bad |= (ids[i] == e) ? 2 : 0;
    }
  }
  if (my_bad) atomicOr(&bad, my_bad);
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
      w.status[0] = bad;
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

// Writes the MXFP8 image of one piece of 8 values (vector v of a row of d =
// 8 * nvec values) to `rows`: E4M3 codes in q [S][d], E8M0 scales in sc
// [d/64][S][2]. The 4 lanes holding a 32-block (lanes aligned to 4) share its
// scale by two butterflies; the first lane of each 64-column piece (8 lanes)
// writes both of its scale bytes. Every lane of the 8-lane group must
// execute it. kExact: fp32 values, encoded with the exact encoder (bf16
// values may take the hardware conversion).
template <int NR, bool kExact>
__device__ __forceinline__ void mx_store_vals(const float (&f)[8], int v, int d, const int (&rows)[NR], int nr,
                                              uint8_t* __restrict__ q, uint8_t* __restrict__ sc, int S) {
  const int code = mx_group4_code(f);
  const uint2 codes = kExact ? mx_encode8_exact(f, code) : mx_encode8(f, code);
  const int lane = threadIdx.x & (kWave - 1);
  const int code_hi = __shfl(code, (lane & ~7) + 4, kWave);
  const uint16_t sv = static_cast<uint16_t>(code | (code_hi << 8));
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    if (j >= nr || rows[j] < 0) continue;
    *reinterpret_cast<uint2*>(q + static_cast<int64_t>(rows[j]) * d + v * 8) = codes;
    if ((v & 7) == 0)
      *reinterpret_cast<uint16_t*>(sc + (static_cast<int64_t>(v >> 3) * S + rows[j]) * 2) = sv;
  }
}
// Rows [p0, p0 + 128) of the padded row space (every expert's rows padded to
// a multiple of 64, experts in order): for each 64-row half h, the expert row
// its first padded row holds (src[h]) and how many of its 64 rows are real
// (valid[h]; 0 past the last expert). Wave 0 computes it (the padded offsets
// by a wave scan over the experts, 4 per lane); the caller syncs.
__device__ __forceinline__ void padded_halves(const int32_t* __restrict__ offsets, int E, int64_t p0, int* src_out,
                                              int* valid_out) {
  const int lane = threadIdx.x & (kWave - 1);
  int beg[4], n[4], pad[4], sum = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = lane * 4 + u;
    beg[u] = e < E ? offsets[e] : 0;
    n[u] = e < E ? offsets[e + 1] - beg[u] : 0;
    pad[u] = (n[u] + 63) & ~63;
    sum += pad[u];
  }
  const int excl = wave_exclusive_scan(sum);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t ph = p0 + 64 * h;
    int src = 0, valid = 0, found = 0, run = excl;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (ph >= run && ph < run + pad[u]) {
        found = 1;
        src = beg[u] + static_cast<int>(ph - run);
        valid = min(64, n[u] - static_cast<int>(ph - run));
      }
      run += pad[u];
    }
    const uint64_t who = __ballot(found);
    if (who) {
      const int l0 = __ffsll(static_cast<long long>(who)) - 1;
      src = __shfl(src, l0, kWave);
      valid = __shfl(valid, l0, kWave);
    } else {
      src = 0;
      valid = 0;
    }
    if (lane == 0) {
      src_out[h] = src;
      valid_out[h] = valid;
    }
  }
}

// MXFP8 images of an expert-ordered row matrix R [S][C] whose row r is
// gathered from a token-ordered bf16 matrix: R[r] = src[token_of_row[r]]
// (xp), or gate_of_row[r] * src[token_of_row[r]] in fp32 (GATE: dO, the
// product combine_bwd_kernel encodes and whose gates it wrote). Written:
// the image along each expert's tokens (codes tq [C][P] in e's rows padded
// to 64 from its padded offset, scales ts [P/64][C][2]: a weight gradient's
// operand); with KMAJOR also the image along C (codes kq [S][C], scales ks
// [C/64][S][2]: a row operand) and, where `rows` is not null, R's bf16 rows.
// Every code is decided on the fp32 value of R. The rows are made from src
// here instead of being stored and read back.
// One workgroup per (128 padded rows, kImgColBlocks blocks of 64 columns),
// column groups fastest in the (1-D) grid, so the workgroups running
// together read the same gathered rows. Wave 0 finds the experts of the two
// 64-row halves (padded_halves) and 128 threads resolve each row's token
// (and gate), once for all the column blocks. Per block, 8 lanes per row
// load its 128 bytes of src (the next block's loads go out before this
// block is encoded) into an fp32 LDS tile (zeros past an expert's end);
// from the tile each thread encodes one 32-block of a row (KMAJOR: 64 bytes
// of a K-major row per pair of threads) and one 32-row block of a column
// into an LDS output tile that leaves as full 128-byte rows of tq.
constexpr int kImgColBlocks = 8;
template <bool GATE, bool KMAJOR>
__global__ __launch_bounds__(256) void row_images_kernel(const bf16_t* __restrict__ src,
                                                         const float* __restrict__ gate_of_row,
                                                         const int32_t* __restrict__ token_of_row,
                                                         const int32_t* __restrict__ offsets, int E, int C, int S,
                                                         int64_t P, bf16_t* __restrict__ rows,
                                                         uint8_t* __restrict__ kq, uint8_t* __restrict__ ks,
                                                         uint8_t* __restrict__ tq, uint8_t* __restrict__ ts) {
  __shared__ __attribute__((aligned(16))) float tile[128][64 + 4];
  __shared__ __attribute__((aligned(16))) uint8_t qt[64][128 + 16];
  __shared__ int s_src[2], s_valid[2], s_tok[128], s_row[128];
  __shared__ float s_gate[128];
  const int tid = threadIdx.x, ncb = C / 64, ncg = (ncb + kImgColBlocks - 1) / kImgColBlocks;
  const int cb0 = static_cast<int>(blockIdx.x % ncg) * kImgColBlocks, cb1 = min(cb0 + kImgColBlocks, ncb);
  const int64_t p0 = static_cast<int64_t>(blockIdx.x / ncg) * 128;
  if (tid < 64) padded_halves(offsets, E, p0, s_src, s_valid);
  __syncthreads();
  if (tid < 128) {  // padded row tid: its expert row (-1 past an expert's end), token and gate
    const int h = tid >> 6, rr = tid & 63;
    const bool ok = rr < s_valid[h];
    const int rs = ok ? s_src[h] + rr : -1;
    s_row[tid] = rs;
    s_tok[tid] = ok ? token_of_row[rs] : 0;
    if constexpr (GATE) s_gate[tid] = ok ? gate_of_row[rs] : 0.0f;
  }
  __syncthreads();
  const int ch = tid & 7;
  const bf16_t* xr[4];  // this thread's 4 rows of src, at 16-byte piece ch
  int rrow[4];
  float rg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = i * 32 + (tid >> 3);
    xr[i] = src + static_cast<int64_t>(s_tok[r]) * C + ch * 8;
    rrow[i] = s_row[r];
    rg[i] = GATE ? s_gate[r] : 1.0f;
  }
  const int kr = tid >> 1, kb = tid & 1, krs = s_row[kr];  // along C: row, 32-block
  const int tcol = tid & 63, tblock = tid >> 6;             // along the tokens: column, 32-row block
  const int64_t pvalid = min(static_cast<int64_t>(128), P - p0);
  uint4 cur[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) cur[i] = ld16(xr[i] + cb0 * 64);
  for (int cb = cb0; cb < cb1; ++cb) {
    const int c0 = cb * 64;
    __syncthreads();  // the previous block's tile and qt are read out
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = i * 32 + (tid >> 3);
      float f[8];
      unpack16(cur[i], f);
#pragma unroll
      for (int u = 0; u < 8; ++u) f[u] = rrow[i] >= 0 ? (GATE ? rg[i] * f[u] : f[u]) : 0.0f;
      *reinterpret_cast<float4*>(&tile[r][ch * 8]) = make_float4(f[0], f[1], f[2], f[3]);
      *reinterpret_cast<float4*>(&tile[r][ch * 8 + 4]) = make_float4(f[4], f[5], f[6], f[7]);
      if (!GATE && rows != nullptr && rrow[i] >= 0)
        st16(rows + static_cast<int64_t>(rrow[i]) * C + c0 + ch * 8, cur[i]);
    }
    if (cb + 1 < cb1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) cur[i] = ld16(xr[i] + c0 + 64);
    }
    __syncthreads();
    if constexpr (KMAJOR) {
      float v[32];
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 t4 = *reinterpret_cast<const float4*>(&tile[kr][kb * 32 + 4 * i]);
        v[4 * i] = t4.x; v[4 * i + 1] = t4.y; v[4 * i + 2] = t4.z; v[4 * i + 3] = t4.w;
      }
      const int code = mx_encode_block(v, w);
      if (krs >= 0) {
        uint4* d = reinterpret_cast<uint4*>(kq + static_cast<int64_t>(krs) * C + c0 + kb * 32);
        d[0] = make_uint4(w[0], w[1], w[2], w[3]);
        d[1] = make_uint4(w[4], w[5], w[6], w[7]);
        ks[(static_cast<int64_t>(cb) * S + krs) * 2 + kb] = static_cast<uint8_t>(code);
      }
    }
    {
      float v[32];
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = tile[tblock * 32 + i][tcol];
      const int code = mx_encode_block(v, w);
      uint4* d = reinterpret_cast<uint4*>(&qt[tcol][tblock * 32]);
      d[0] = make_uint4(w[0], w[1], w[2], w[3]);
      d[1] = make_uint4(w[4], w[5], w[6], w[7]);
      if (p0 + tblock * 32 < P) {
        const int64_t sb = (p0 >> 6) + (tblock >> 1);
        ts[(sb * C + c0 + tcol) * 2 + (tblock & 1)] = static_cast<uint8_t>(code);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = i * 32 + (tid >> 3), c16 = tid & 7;
      if (c16 * 16 < pvalid)
        *reinterpret_cast<uint4*>(tq + static_cast<int64_t>(c0 + row) * P + p0 + c16 * 16) =
            *reinterpret_cast<const uint4*>(&qt[row][c16 * 16]);
    }
  }
}

static dim3 row_images_grid(int C, int64_t P) {
  const int ncg = (C / 64 + kImgColBlocks - 1) / kImgColBlocks;
  return dim3(static_cast<unsigned>(static_cast<int64_t>(ncg) * ((P + 127) / 128)));
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

static hipError_t dispatch_impl(const void* x, const int32_t* topk_idx, int elem_bytes, int T, int d, int E, int k,
                                int32_t* counts, int32_t* offsets, int32_t* row_of_slot, int32_t* token_of_row,
                                void* xp, const MxRowImages* mx, void* ws, hipStream_t s, int32_t* status = nullptr) {
  const int ct = chunk_tokens(T, E);
  const int nch = (T + ct - 1) / ct;
  DispatchWs w = carve(ws, nch, E);
  if (status != nullptr) w.status = status;  // the caller's status word instead of the workspace's
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
  const dim3 grid((T + tpw - 1) / tpw);
  if (mx != nullptr) {
    const int S = T * k;
    const int64_t P = mx_padded_rows(S, E);
    hipLaunchKernelGGL((row_images_kernel<false, true>), row_images_grid(d, P), dim3(256), 0, s,
                       static_cast<const bf16_t*>(x), nullptr, token_of_row, offsets, E, d, S, P,
                       static_cast<bf16_t*>(xp), mx->k.q, mx->k.s, mx->t.q, mx->t.s);
  } else
    hipLaunchKernelGGL(gather_rows_kernel, grid, dim3(256), 0, s, static_cast<const char*>(x), row_of_slot, T, k,
                       nvec, lpt, static_cast<char*>(xp));
  return hipGetLastError();
}

hipError_t launch_dispatch(const void* x, const int32_t* topk_idx, int elem_bytes, int T, int d, int E, int k,
                           int32_t* counts, int32_t* offsets, int32_t* row_of_slot, int32_t* token_of_row,
                           void* xp, void* ws, hipStream_t s) {
  return dispatch_impl(x, topk_idx, elem_bytes, T, d, E, k, counts, offsets, row_of_slot, token_of_row, xp, nullptr,
                       ws, s);
}

hipError_t launch_dispatch_mx(const void* x, const int32_t* topk_idx, int T, int d, int E, int k, int32_t* counts,
                              int32_t* offsets, int32_t* row_of_slot, int32_t* token_of_row, void* xp,
                              MxRowImages xp_mx, void* ws, hipStream_t s) {
  return dispatch_impl(x, topk_idx, 2, T, d, E, k, counts, offsets, row_of_slot, token_of_row, xp, &xp_mx, ws, s);
}

// The allocation-free dispatch's workspace: one array per GPU (each device
// holds its own copy of a __device__ variable), alive until the process
// ends. Host code never passes the array's name to a kernel: on the host the
// name is only a stand-in, so each device's address is looked up once with
// that device current and kept. Nothing in it must start at zero: the count
// pass writes every [chunk][expert] entry and every chunk's fault bits, and
// the placement pass writes the status word. Calls that overlap on one GPU
// (other streams, other host threads) share the array and race.
constexpr size_t kNoAllocBytes = size_t(1) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kNoAllocBytes];

size_t dispatch_noalloc_max() { return kNoAllocBytes; }

static hipError_t scratch_on_current_device(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_dispatch_noalloc(const void* x, const int32_t* topk_idx, int elem_bytes, int T, int d, int E,
                                   int k, int32_t* counts, int32_t* offsets, int32_t* row_of_slot,
                                   int32_t* token_of_row, void* xp, MxRowImages xp_mx, hipStream_t s) {
  if (dispatch_workspace(T, E) > kNoAllocBytes) return hipErrorInvalidValue;
  // The array's address is the current device's: a stream of another device
  // would run the kernels there with this device's address.
  if (s != nullptr) {
    int cur = -1, sdev = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess) e = hipStreamGetDevice(s, &sdev);
    if (e != hipSuccess) return e;
    if (sdev != cur) return hipErrorInvalidDevice;
  }
  void* ws = nullptr;
  const hipError_t err = scratch_on_current_device(&ws);
  if (err != hipSuccess) return err;
  return dispatch_impl(x, topk_idx, elem_bytes, T, d, E, k, counts, offsets, row_of_slot, token_of_row, xp,
                       xp_mx.k.q != nullptr ? &xp_mx : nullptr, ws, s);
}

// Row kernels take the slot count K as a template argument and issue the
// loads of all K rows of a piece before using any of them: with a runtime k
// and a branch per slot, each row's load waited for the one before it.
// A slot with row -1 (an expert id outside [0, E)) loads row 0 and leaves
// its contribution out by a select, which gives the same bits as skipping it.
template <typename F>
static hipError_t with_k(int k, F&& f) {
  switch (k) {
    case 1: return f(std::integral_constant<int, 1>{});
    case 2: return f(std::integral_constant<int, 2>{});
    case 3: return f(std::integral_constant<int, 3>{});
    case 4: return f(std::integral_constant<int, 4>{});
    case 5: return f(std::integral_constant<int, 5>{});
    case 6: return f(std::integral_constant<int, 6>{});
    case 7: return f(std::integral_constant<int, 7>{});
    case 8: return f(std::integral_constant<int, 8>{});
    default: return hipErrorInvalidValue;
  }
}

// y[t] = sum_j gate[t][j] * o[row_of_slot[t][j]]  (fp32, slot order, one rounding).
template <typename T, int K>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ o, const float* __restrict__ gate,
                                                      const int32_t* __restrict__ row_of_slot, int Tn, int nvec,
                                                      int lpt, T* __restrict__ y) {
  constexpr int VE = Vec16<T>::N;
  const int tpw = 256 / lpt;
  const int t = blockIdx.x * tpw + threadIdx.x / lpt;
  const int sub = threadIdx.x % lpt;
  if (t >= Tn) return;
  const int64_t re = static_cast<int64_t>(nvec) * VE;  // elements per row
  int rows[K];
  float g[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    rows[j] = row_of_slot[static_cast<int64_t>(t) * K + j];
    g[j] = gate[static_cast<int64_t>(t) * K + j];
  }
  for (int v = sub; v < nvec; v += lpt) {
    uint4 raw[K];
#pragma unroll
    for (int j = 0; j < K; ++j) raw[j] = ld16(o + max(rows[j], 0) * re + v * VE);
    float acc[VE];
#pragma unroll
    for (int i = 0; i < VE; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      float ov[VE];
      unpack16(raw[j], ov);
      const bool ok = rows[j] >= 0;
#pragma unroll
      for (int i = 0; i < VE; ++i) {
        const float a = fmaf(g[j], ov[i], acc[i]);
        acc[i] = ok ? a : acc[i];
      }
    }
    st16(y + t * re + v * VE, pack16(acc));
  }
}

// d_o[row(t,j)] = gate[t][j] * dy[t];  dgate[t][j] = <dy[t], o[row(t,j)]> (fp32,
// fixed reduction tree: per-thread partials, lane butterfly, then waves in order).
// DO is the type of d_o: T, or float for MXFP8 layers (bf16 T), whose d_o
// keeps the fp32 products. MX (DO = float only): the same pass writes d_o's
// K-major MXFP8 image (q, sc; S rows), each code decided on the fp32 product,
// the gate of every row (gate_of_row, for the token-major pass), and the fp32
// d_o rows only if d_o is not null.
template <typename T, typename DO, bool MX, int K>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const T* __restrict__ dy, const T* __restrict__ o,
                                                          const float* __restrict__ gate,
                                                          const int32_t* __restrict__ row_of_slot, int Tn, int nvec,
                                                          int lpt, DO* __restrict__ d_o, float* __restrict__ dgate,
                                                          uint8_t* __restrict__ q, uint8_t* __restrict__ sc, int S,
                                                          float* __restrict__ gate_of_row) {
  constexpr int VE = Vec16<T>::N;
  static_assert(!MX || (sizeof(DO) == 4 && VE == 8), "MXFP8 images come from fp32 d_o of bf16 layers");
  __shared__ float red[4][K];
  const int tpw = 256 / lpt;
  const int t = blockIdx.x * tpw + threadIdx.x / lpt;
  const int sub = threadIdx.x % lpt;
  const bool live = t < Tn;
  const int64_t re = static_cast<int64_t>(nvec) * VE;
  int rows[K];
  float g[K], part[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    rows[j] = live ? row_of_slot[static_cast<int64_t>(t) * K + j] : -1;
    g[j] = live ? gate[static_cast<int64_t>(t) * K + j] : 0.0f;
    part[j] = 0.0f;
  }
  if constexpr (MX) {
    if (live && sub == 0)
#pragma unroll
      for (int j = 0; j < K; ++j)
        if (rows[j] >= 0) gate_of_row[rows[j]] = g[j];
  }
  if (live) {
    for (int v = sub; v < nvec; v += lpt) {
      const uint4 draw = ld16(dy + t * re + v * VE);
      uint4 raw[K];
#pragma unroll
      for (int j = 0; j < K; ++j) raw[j] = ld16(o + max(rows[j], 0) * re + v * VE);
      float dv[VE];
      unpack16(draw, dv);
#pragma unroll
      for (int j = 0; j < K; ++j) {
        // Every row's value is used outside the branch below, so no load is
        // sunk into it (part[j] of a row -1 is never written out).
        float ov[VE], sv[VE];
        unpack16(raw[j], ov);
#pragma unroll
        for (int i = 0; i < VE; ++i) {
          part[j] = fmaf(dv[i], ov[i], part[j]);
          sv[i] = g[j] * dv[i];
        }
        if (rows[j] < 0) continue;  // the same for every lane of the token
        if constexpr (sizeof(DO) == sizeof(T)) {
          st16(d_o + rows[j] * re + v * VE, pack16(sv));
        } else {  // bf16 dy, fp32 d_o: the 8 products as two 16-byte pieces
          if (!MX || d_o != nullptr) {
            DO* dst = d_o + rows[j] * re + v * VE;
            const float lo[4] = {sv[0], sv[1], sv[2], sv[3]}, hi[4] = {sv[4], sv[5], sv[6], sv[7]};
            st16(dst, pack16(lo));
            st16(dst + 4, pack16(hi));
          }
          if constexpr (MX) {
            const int one[1] = {rows[j]};
            mx_store_vals<1, false>(sv, v, nvec * VE, one, 1, q, sc, S);
          }
        }
      }
    }
  }
  // Reduce part[j] over the lpt lanes of the token.
  const int width = lpt < 64 ? lpt : 64;
#pragma unroll
  for (int j = 0; j < K; ++j)
    for (int off = width >> 1; off > 0; off >>= 1) part[j] += __shfl_xor(part[j], off, kWave);
  if (lpt <= 64) {
    if (live && sub == 0)
#pragma unroll
      for (int j = 0; j < K; ++j) dgate[static_cast<int64_t>(t) * K + j] = rows[j] >= 0 ? part[j] : 0.0f;
  } else {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0)
#pragma unroll
      for (int j = 0; j < K; ++j) red[wave][j] = part[j];
    __syncthreads();
    if (live && sub == 0) {
      const int w0 = (threadIdx.x / lpt) * (lpt / 64);
#pragma unroll
      for (int j = 0; j < K; ++j) {
        float s = 0.0f;
        for (int w = 0; w < lpt / 64; ++w) s += red[w0 + w][j];
        dgate[static_cast<int64_t>(t) * K + j] = rows[j] >= 0 ? s : 0.0f;
      }
    }
  }
}

hipError_t launch_combine(const void* o, const float* gate, const int32_t* row_of_slot, bool is_f32, int T, int d,
                          int k, void* y, hipStream_t s) {
  const int nvec = d * (is_f32 ? 4 : 2) / 16;
  const int lpt = lanes_per_token(nvec), tpw = 256 / lpt;
  const dim3 grid((T + tpw - 1) / tpw);
  return with_k(k, [&](auto KC) {
    constexpr int K = decltype(KC)::value;
    if (is_f32)
      hipLaunchKernelGGL((combine_kernel<float, K>), grid, dim3(256), 0, s, static_cast<const float*>(o), gate,
                         row_of_slot, T, nvec, lpt, static_cast<float*>(y));
    else
      hipLaunchKernelGGL((combine_kernel<bf16_t, K>), grid, dim3(256), 0, s, static_cast<const bf16_t*>(o), gate,
                         row_of_slot, T, nvec, lpt, static_cast<bf16_t*>(y));
    return hipGetLastError();
  });
}

hipError_t launch_combine_bwd(const void* dy, const void* o, const float* gate, const int32_t* row_of_slot,
                              int kind, int T, int d, int k, void* d_o, float* dgate, hipStream_t s) {
  const int nvec = d * (kind == 0 ? 4 : 2) / 16;
  const int lpt = lanes_per_token(nvec), tpw = 256 / lpt;
  const dim3 grid((T + tpw - 1) / tpw);
  return with_k(k, [&](auto KC) {
    constexpr int K = decltype(KC)::value;
    if (kind == 0)
      hipLaunchKernelGGL((combine_bwd_kernel<float, float, false, K>), grid, dim3(256), 0, s,
                         static_cast<const float*>(dy), static_cast<const float*>(o), gate, row_of_slot, T, nvec, lpt,
                         static_cast<float*>(d_o), dgate, nullptr, nullptr, T * k, nullptr);
    else if (kind == 1)
      hipLaunchKernelGGL((combine_bwd_kernel<bf16_t, bf16_t, false, K>), grid, dim3(256), 0, s,
                         static_cast<const bf16_t*>(dy), static_cast<const bf16_t*>(o), gate, row_of_slot, T, nvec,
                         lpt, static_cast<bf16_t*>(d_o), dgate, nullptr, nullptr, T * k, nullptr);
    else
      hipLaunchKernelGGL((combine_bwd_kernel<bf16_t, float, false, K>), grid, dim3(256), 0, s,
                         static_cast<const bf16_t*>(dy), static_cast<const bf16_t*>(o), gate, row_of_slot, T, nvec,
                         lpt, static_cast<float*>(d_o), dgate, nullptr, nullptr, T * k, nullptr);
    return hipGetLastError();
  });
}

hipError_t launch_combine_bwd_mx(const void* dy, const void* o, const float* gate, const int32_t* row_of_slot,
                                 const int32_t* token_of_row, const int32_t* offsets, int T, int d, int E, int k,
                                 void* d_o, MxDoutImage d_o_mx, float* dgate, hipStream_t s) {
  const int nvec = d * 2 / 16;
  const int lpt = lanes_per_token(nvec), tpw = 256 / lpt;
  const dim3 grid((T + tpw - 1) / tpw);
  const int64_t S = static_cast<int64_t>(T) * k, P = mx_padded_rows(S, E);
  const hipError_t err = with_k(k, [&](auto KC) {
    constexpr int K = decltype(KC)::value;
    hipLaunchKernelGGL((combine_bwd_kernel<bf16_t, float, true, K>), grid, dim3(256), 0, s,
                       static_cast<const bf16_t*>(dy), static_cast<const bf16_t*>(o), gate, row_of_slot, T, nvec, lpt,
                       static_cast<float*>(d_o), dgate, d_o_mx.k.q, d_o_mx.k.s, T * k, d_o_mx.gate_of_row);
    return hipGetLastError();
  });
  if (err != hipSuccess) return err;
  // dO along each expert's tokens, rebuilt from dy and the gates the pass
  // above wrote.
  hipLaunchKernelGGL((row_images_kernel<true, false>), row_images_grid(d, P), dim3(256), 0, s,
                     static_cast<const bf16_t*>(dy), d_o_mx.gate_of_row, token_of_row, offsets, E, d,
                     static_cast<int>(S), P, nullptr, nullptr, nullptr, d_o_mx.t.q, d_o_mx.t.s);
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
// The router backward leaves dl zero off the token's chosen set, so a token
// has at most K non-zero columns: those are found once (when a token has
// whole waves, lpt >= 64, with one ballot per 64 experts; narrower rows scan
// the E values per lane) and their W_rT rows loaded beside the dxp rows. A
// token with more non-zero columns (a caller's dense dlogits, e.g. from an
// added loss term) takes every non-zero column in increasing expert order,
// which is also the order of the first path, so both give the same bits.
template <typename T, int K>
__global__ __launch_bounds__(256) void dispatch_bwd_kernel(const T* __restrict__ dxp, const int32_t* __restrict__ row_of_slot,
                                                           const float* __restrict__ dl, const T* __restrict__ wt,
                                                           int Tn, int E, int nvec, int lpt, T* __restrict__ dx) {
  constexpr int VE = Vec16<T>::N;
  const int tpw = 256 / lpt;
  const int t = blockIdx.x * tpw + threadIdx.x / lpt;
  const int sub = threadIdx.x % lpt;
  if (t >= Tn) return;
  const int64_t re = static_cast<int64_t>(nvec) * VE;
  int rows[K];
#pragma unroll
  for (int j = 0; j < K; ++j) rows[j] = row_of_slot[static_cast<int64_t>(t) * K + j];
  // The token's router columns: (expert, dl) pairs, the first K of them, and
  // how many there are in all.
  int ce[K];
  float cv[K];
  int nr = 0, nnz = 0;
  const float* dlt = dl != nullptr ? dl + static_cast<int64_t>(t) * E : nullptr;
  if (dl != nullptr) {
    if (lpt >= kWave) {
      const int lane = threadIdx.x & (kWave - 1);
      for (int c0 = 0; c0 < E; c0 += kWave) {
        const float c = (c0 + lane < E) ? dlt[c0 + lane] : 0.0f;
        uint64_t m = __ballot(c != 0.0f);
        nnz += __popcll(m);
        while (m != 0 && nr < K) {
          const int b = __ffsll(static_cast<long long>(m)) - 1;
          m &= m - 1;
          ce[nr] = c0 + b;
          cv[nr] = __shfl(c, b, kWave);
          ++nr;
        }
      }
    } else {
      for (int e = 0; e < E; ++e) {
        const float c = dlt[e];
        if (c != 0.0f) {
          if (nr < K) {
            ce[nr] = e;
            cv[nr] = c;
            ++nr;
          }
          ++nnz;
        }
      }
    }
  }
  const bool dense = nnz > K;  // the same for every lane of the token
  for (int v = sub; v < nvec; v += lpt) {
    // Slots past nr load row 0 and are selected out.
    uint4 raw[K], wraw[K];
#pragma unroll
    for (int j = 0; j < K; ++j) raw[j] = ld16(dxp + max(rows[j], 0) * re + v * VE);
    if (dl != nullptr && !dense) {
#pragma unroll
      for (int r = 0; r < K; ++r) wraw[r] = ld16(wt + (r < nr ? ce[r] : 0) * re + v * VE);
    }
    float acc[VE];
#pragma unroll
    for (int i = 0; i < VE; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      float gv[VE];
      unpack16(raw[j], gv);
      const bool ok = rows[j] >= 0;
#pragma unroll
      for (int i = 0; i < VE; ++i) acc[i] = ok ? acc[i] + gv[i] : acc[i];
    }
    if (dl != nullptr && !dense) {
#pragma unroll
      for (int r = 0; r < K; ++r) {
        float wv[VE];
        unpack16(wraw[r], wv);
        const bool ok = r < nr;
#pragma unroll
        for (int i = 0; i < VE; ++i) {
          const float a = fmaf(cv[r], wv[i], acc[i]);
          acc[i] = ok ? a : acc[i];
        }
      }
    } else if (dense) {
      for (int e = 0; e < E; ++e) {
        const float c = dlt[e];
        if (c == 0.0f) continue;
        float wv[VE];
        unpack16(ld16(wt + e * re + v * VE), wv);
#pragma unroll
        for (int i = 0; i < VE; ++i) acc[i] = fmaf(c, wv[i], acc[i]);
      }
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
  return with_k(k, [&](auto KC) {
    constexpr int K = decltype(KC)::value;
    if (is_f32)
      hipLaunchKernelGGL((dispatch_bwd_kernel<float, K>), grid, dim3(256), 0, s, static_cast<const float*>(dxp),
                         row_of_slot, dl, static_cast<const float*>(ws), T, E, nvec, lpt, static_cast<float*>(dx));
    else
      hipLaunchKernelGGL((dispatch_bwd_kernel<bf16_t, K>), grid, dim3(256), 0, s, static_cast<const bf16_t*>(dxp),
                         row_of_slot, dl, static_cast<const bf16_t*>(ws), T, E, nvec, lpt, static_cast<bf16_t*>(dx));
    return hipGetLastError();
  });
}

}  // namespace moe

namespace moe {

// Expert-load diagnostics from the routed counts (the real load, which a
// routing score meant to favour balance need not track: "Olmo-core 3 escala
// el entrenamiento...", section "Detalles clave"; "Ai2 rilascia Olmo-Core
// 3...", section "Risultati Documentati"). One workgroup, one thread per
// expert. Integer figures are exact; the two fp64 sums (entropy terms
// -p ln p with p = n/S, squared deviations from the mean) use a fixed LDS
// tree, so reruns are bit-identical. out: max, min, mean, max/mean, entropy
// (nats), entropy / ln E, empty experts, std/mean; the S = 0 and E = 1 cases
// as documented in moe.h.
__global__ __launch_bounds__(256) void load_stats_kernel(const int32_t* __restrict__ counts, int E,
                                                         double* __restrict__ out) {
  __shared__ long long s_sum[256];
  __shared__ int s_max[256], s_min[256], s_empty[256];
  __shared__ double s_ent[256], s_var[256];
  const int t = threadIdx.x;
  const int n = t < E ? counts[t] : 0;
  s_sum[t] = n;
  s_max[t] = t < E ? n : INT_MIN;
  s_min[t] = t < E ? n : INT_MAX;
  s_empty[t] = (t < E && n == 0) ? 1 : 0;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (t < h) {
      s_sum[t] += s_sum[t + h];
      s_max[t] = max(s_max[t], s_max[t + h]);
      s_min[t] = min(s_min[t], s_min[t + h]);
      s_empty[t] += s_empty[t + h];
    }
    __syncthreads();
  }
  const long long S = s_sum[0];
  const double mean = static_cast<double>(S) / E;
  double ent = 0.0, var = 0.0;
  if (t < E && S > 0) {
    const double p = static_cast<double>(n) / static_cast<double>(S);
    ent = n > 0 ? -p * log(p) : 0.0;
    const double dv = static_cast<double>(n) - mean;
    var = dv * dv;
  }
  s_ent[t] = ent;
  s_var[t] = var;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (t < h) {
      s_ent[t] += s_ent[t + h];
      s_var[t] += s_var[t + h];
    }
    __syncthreads();
  }
  if (t == 0) {
    const bool any = S > 0;
    out[0] = s_max[0];
    out[1] = s_min[0];
    out[2] = mean;
    out[3] = any ? s_max[0] / mean : 0.0;
    out[4] = any ? s_ent[0] : 0.0;
    out[5] = any ? (E > 1 ? s_ent[0] / log(static_cast<double>(E)) : 1.0) : 0.0;
    out[6] = s_empty[0];
    out[7] = any ? sqrt(s_var[0] / E) / mean : 0.0;
  }
}

hipError_t launch_load_stats(const int32_t* counts, int E, double* out, hipStream_t s) {
  hipLaunchKernelGGL(load_stats_kernel, dim3(1), dim3(256), 0, s, counts, E, out);
  return hipGetLastError();
}

}  // namespace moe
