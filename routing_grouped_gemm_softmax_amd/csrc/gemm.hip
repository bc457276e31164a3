// Device-scheduled grouped GEMMs of the expert SwiGLU FFN (forward, dgrad,
// wgrad) for gfx950.
//
// The pages run the experts' matmuls as one grouped GEMM whose schedule is
// read on the device, so that the host never waits for routing metadata
// ("Olmo-core 3 escala el entrenamiento de mixture-of-experts a billones de
// parámetros", section "Cómo funciona"; "Ai2 rilascia Olmo-Core 3...",
// section "Parallelismo, precisione e tecniche di memoria"). Here every
// workgroup reads the per-expert row offsets (E+1 ints written by the
// dispatch), derives the per-expert tile counts with a wave scan, and maps its
// own id to (expert, row tile, column tile). The grid is sized on the host
// from a bound that needs no counts: ceil(S/BM) + E row tiles.
//
// This file holds the kernel of fp32 layers (v_mfma_f32_32x32x2f32) and the
// host side of every FFN call; bf16 layers run the kernels of gemm_bf16.hip,
// MXFP8 layers those of gemm_mx.hip. Tiles: 256 threads (4 waves, 2x2), BM x
// BN output tile, each wave owns a (BM/2) x (BN/2) sub-tile of 32x32 MFMA
// blocks. K advances in slabs of 128 bytes (32 fp32). LDS holds both operands
// as [row][128 B] with the 16-byte chunks XOR-swizzled by the row,
// double-buffered through registers. Operands whose contiguous dimension in
// HBM is not K (the weights in the forward, both operands of the weight
// gradients) are transposed in registers on their way into LDS, so every
// MFMA fragment comes from 16-byte LDS reads.
#include "common.h"
#include "grouped_gemm.h"
#include "kernels.h"

#include <type_traits>

namespace moe {

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// Byte offset of element k of LDS row `row` (rows of 128 bytes, 16-byte chunks
// XOR-swizzled so both the row-wise fragment reads and the transposed writes
// spread over the banks).
template <int EB>
__device__ __forceinline__ int lds_off(int row, int k) {
  const int byte = k * EB;
  return row * 128 + (((byte >> 4) ^ swz(row)) << 4) + (byte & 15);
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// Pack element `nn` of KR 16-byte vectors of fp32 into KR*4 contiguous bytes.
template <int EB, int KR>
__device__ __forceinline__ void store_transposed(char* dst, const uint4 (&v)[KR], int nn) {
  static_assert(EB == 4, "fp32 layers only");
  uint32_t h[KR];
#pragma unroll
  for (int r = 0; r < KR; ++r)
    h[r] = nn == 0 ? v[r].x : nn == 1 ? v[r].y : nn == 2 ? v[r].z : v[r].w;
  if constexpr (KR == 4) {
    *reinterpret_cast<uint4*>(dst) = make_uint4(h[0], h[1], h[2], h[3]);
  } else {
    *reinterpret_cast<uint2*>(dst) = make_uint2(h[0], h[1]);
  }
}

template <typename T, int MODE, int BM, int BN>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(GemmParams p) {
  static_assert(std::is_same<T, float>::value, "fp32 layers only: bf16 and MXFP8 layers have their own kernels");
  constexpr int EB = sizeof(T);
  constexpr int BK = 128 / EB;      // K elements per slab
  constexpr int VE = 16 / EB;       // elements per 16-byte vector
  constexpr int MB = BM / 64;       // 32x32 blocks per wave along M
  constexpr int NB = BN / 64;       // ... along N
  constexpr bool A_T = (MODE == WGRAD);                                   // A stored [K][M]
  constexpr bool B_T = (MODE == FWD_GU || MODE == FWD_DOWN || MODE == WGRAD);  // B stored [K][N]
  constexpr int A_LD = A_T ? 1 : BM / 32;                 // K-contiguous: 16-byte chunks per thread
  constexpr int B_LD = B_T ? 1 : BN / 32;
  constexpr int KRA = BM * BK / (256 * VE);               // transposed: k-rows per thread
  constexpr int KRB = BN * BK / (256 * VE);
  static_assert(MODE != FWD_GU || BN == 128, "SwiGLU pairing needs two 32-column blocks per wave");

  extern __shared__ __attribute__((aligned(16))) char smem[];
  // Buffer b (0/1) holds the A tile then the B tile.
  auto a_lds = [&](int b) { return smem + b * (BM + BN) * 128; };
  auto b_lds = [&](int b) { return smem + b * (BM + BN) * 128 + BM * 128; };
  int* const s_info = reinterpret_cast<int*>(b_lds(1));

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int bid = blockIdx.x;
  const int NT = p.N / BN;

  // ---- device-side tile schedule ----------------------------------------------
  if (wave == 0) {
    int e_sel = -1, row0 = 0, row_end = 0, nt = 0, m0 = 0;
    if constexpr (MODE == WGRAD) {
      const int MT = p.M / BM;
      const int R = p.E * MT * NT;
      if (bid < R) {
        // Consecutive tiles of one expert share its K rows: keep them together.
        const int q = R / 8, rmd = R % 8, x = bid % 8, i = bid / 8;
        const int logical = x * q + min(x, rmd) + i;
        e_sel = logical / (MT * NT);
        const int rest = logical % (MT * NT);
        const int mt = rest / NT;
        nt = rest % NT;
        m0 = mt * BM;
        row0 = p.offsets[e_sel];
        row_end = p.offsets[e_sel + 1];
      }
    } else {
      int tq[4], tsum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = lane * 4 + q;
        const int n = (e < p.E) ? (p.offsets[e + 1] - p.offsets[e]) : 0;
        tq[q] = (n + BM - 1) / BM;
        tsum += tq[q];
      }
      const int excl = wave_exclusive_scan(tsum);
      const int RM = __shfl(excl + tsum, 63, kWave);
      const int R = RM * NT;
      if (bid < R) {
        // Bijection bid -> logical tile so that each XCD (bid % 8) works on a
        // contiguous range of tiles; inside it, groups of GM row tiles sweep
        // the column tiles so concurrently running tiles share operands in L2.
        const int q = R / 8, rmd = R % 8, x = bid % 8, i = bid / 8;
        const int logical = x * q + min(x, rmd) + i;
        constexpr int GM = 8;
        const int g = logical / (GM * NT);
        const int gm = min(GM, RM - g * GM);
        const int local = logical - g * GM * NT;
        const int mt = g * GM + local % gm;
        nt = local / gm;
        int run = excl;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int e = lane * 4 + q;
          if (mt >= run && mt < run + tq[q]) {
            e_sel = e;
            row0 = p.offsets[e] + (mt - run) * BM;
            row_end = p.offsets[e + 1];
          }
          run += tq[q];
        }
        // Exactly one lane found the expert; broadcast it.
        const uint64_t who = __ballot(e_sel >= 0);
        const int src = who ? __ffsll((long long)who) - 1 : 0;
        e_sel = __shfl(e_sel, src, kWave);
        row0 = __shfl(row0, src, kWave);
        row_end = __shfl(row_end, src, kWave);
        if (!who) e_sel = -1;
      }
    }
    if (lane == 0) {
      s_info[0] = e_sel; s_info[1] = row0; s_info[2] = row_end; s_info[3] = nt; s_info[4] = m0;
    }
  }
  __syncthreads();
  const int e = s_info[0];
  if (e < 0) return;
  const int row0 = s_info[1], row_end = s_info[2], nt = s_info[3], m0 = s_info[4];
  const int n0 = nt * BN;
  const int K = (MODE == WGRAD) ? (row_end - row0) : p.K;
  const int nk = (K + BK - 1) / BK;

  const char* const a_base = static_cast<const char*>(p.a);
  const int64_t bexp = static_cast<int64_t>(e) * p.bstride;

  uint4 ra[A_T ? KRA : A_LD];
  uint4 rb[B_T ? KRB : B_LD];

  // ---- global -> registers for K-slab kt --------------------------------------
  auto load_a = [&](int kt) {
    if constexpr (!A_T) {
#pragma unroll
      for (int i = 0; i < A_LD; ++i) {
        const int r = tid / 8 + 32 * i;
        const int grow = min(row0 + r, p.S - 1);  // rows past the expert are masked at the store
        ra[i] = ld16(a_base + (static_cast<int64_t>(grow) * p.lda + kt * BK + (tid % 8) * VE) * EB);
      }
    } else {
      const int ng = tid % (BM / VE), kg = tid / (BM / VE);
#pragma unroll
      for (int r = 0; r < KRA; ++r) {
        const int grow = row0 + kt * BK + kg * KRA + r;
        ra[r] = (grow < row_end)
                    ? ld16(a_base + (static_cast<int64_t>(grow) * p.lda + m0 + ng * VE) * EB)
                    : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto load_b = [&](int kt) {
    if constexpr (!B_T) {
      const char* src = static_cast<const char*>(p.b0);
      int kcol = kt * BK;
      if constexpr (MODE == BWD_GU) {
        if (kcol >= p.f) { src = static_cast<const char*>(p.b1); kcol -= p.f; }
      }
#pragma unroll
      for (int i = 0; i < B_LD; ++i) {
        const int n = tid / 8 + 32 * i;
        rb[i] = ld16(src + (bexp + static_cast<int64_t>(n0 + n) * p.ldb + kcol + (tid % 8) * VE) * EB);
      }
    } else {
      const int ng = tid % (BN / VE), kg = tid / (BN / VE);
      const char* src = static_cast<const char*>(p.b0);
      int col = n0 + ng * VE;
      if constexpr (MODE == FWD_GU) {
        // LDS row n of the B tile -> (gate or up, f column): wave column wn
        // holds 32 gate columns then the same 32 up columns.
        const int n = ng * VE;
        const int wcol = n / (BN / 2), nb = (n % (BN / 2)) / 32, c = n % 32;
        src = static_cast<const char*>(nb ? p.b1 : p.b0);
        col = nt * (BN / 2) + wcol * 32 + c;
      }
#pragma unroll
      for (int r = 0; r < KRB; ++r) {
        const int krow = kt * BK + kg * KRB + r;
        if constexpr (MODE == WGRAD) {
          const int grow = row0 + krow;
          rb[r] = (grow < row_end) ? ld16(src + (static_cast<int64_t>(grow) * p.ldb + col) * EB)
                                   : make_uint4(0, 0, 0, 0);
        } else {
          rb[r] = ld16(src + (bexp + static_cast<int64_t>(krow) * p.ldb + col) * EB);
        }
      }
    }
  };
  // ---- registers -> LDS -------------------------------------------------------------
  auto store_a = [&](char* dst) {
    if constexpr (!A_T) {
#pragma unroll
      for (int i = 0; i < A_LD; ++i)
        st16(dst + lds_off<EB>(tid / 8 + 32 * i, (tid % 8) * VE), ra[i]);
    } else {
      const int ng = tid % (BM / VE), kg = tid / (BM / VE);
#pragma unroll
      for (int nn = 0; nn < VE; ++nn)
        store_transposed<EB, KRA>(dst + lds_off<EB>(ng * VE + nn, kg * KRA), ra, nn);
    }
  };
  auto store_b = [&](char* dst) {
    if constexpr (!B_T) {
#pragma unroll
      for (int i = 0; i < B_LD; ++i)
        st16(dst + lds_off<EB>(tid / 8 + 32 * i, (tid % 8) * VE), rb[i]);
    } else {
      const int ng = tid % (BN / VE), kg = tid / (BN / VE);
#pragma unroll
      for (int nn = 0; nn < VE; ++nn)
        store_transposed<EB, KRB>(dst + lds_off<EB>(ng * VE + nn, kg * KRB), rb, nn);
    }
  };

  floatx16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto compute = [&](const char* al, const char* bl) {
    const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int k = kk * 16 + h * 8;
      {
        floatx4 fa[MB][2], fb[NB][2];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const int row = wm * (BM / 2) + i * 32 + l32;
          fa[i][0] = *reinterpret_cast<const floatx4*>(al + lds_off<EB>(row, k));
          fa[i][1] = *reinterpret_cast<const floatx4*>(al + lds_off<EB>(row, k + 4));
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int row = wn * (BN / 2) + j * 32 + l32;
          fb[j][0] = *reinterpret_cast<const floatx4*>(bl + lds_off<EB>(row, k));
          fb[j][1] = *reinterpret_cast<const floatx4*>(bl + lds_off<EB>(row, k + 4));
        }
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int q = 0; q < 8; ++q)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][q >> 2][q & 3], fb[j][q >> 2][q & 3],
                                                               acc[i][j], 0, 0, 0);
      }
    }
  };

  // ---- main loop: prefetch slab kt+1 into registers while computing slab kt ----
  if (nk > 0) {
    load_a(0);
    load_b(0);
    store_a(a_lds(0));
    store_b(b_lds(0));
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      load_a(kt + 1);
      load_b(kt + 1);
    }
    compute(a_lds(cur), b_lds(cur));
    if (kt + 1 < nk) {
      store_a(a_lds(cur ^ 1));
      store_b(b_lds(cur ^ 1));
    }
    __syncthreads();
  }

  // ---- epilogue -----------------------------------------------------------------
  // Accumulator element r of a 32x32 block in lane l: row 8*(r/4) + 4*(l/32) + r%4,
  // column l%32.
  const int h = lane >> 5, l32 = lane & 31;
  T* c0 = static_cast<T*>(p.c0);
  if constexpr (MODE == FWD_GU) {
    T* c1 = static_cast<T*>(p.c1);
    T* c2 = static_cast<T*>(p.c2);
    const int col = nt * (BN / 2) + wn * 32 + l32;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + wm * (BM / 2) + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < row_end) {
          const float g = acc[i][0][r], u = acc[i][1][r];
          const int64_t o = static_cast<int64_t>(row) * p.ldc + col;
          c0[o] = Elem<T>::from_f32(g);
          c1[o] = Elem<T>::from_f32(u);
          c2[o] = Elem<T>::from_f32(silu_f(g) * u);
        }
      }
  } else if constexpr (MODE == FWD_DOWN || MODE == BWD_GU) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + wm * (BM / 2) + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          const int col = n0 + wn * (BN / 2) + j * 32 + l32;
          if (row < row_end) c0[static_cast<int64_t>(row) * p.ldc + col] = Elem<T>::from_f32(acc[i][j][r]);
        }
  } else if constexpr (MODE == BWD_DOWN) {
    // dH -> (dG, dU) with the saved G and U; dGU row = [dG (f) | dU (f)].
    const T* sg = static_cast<const T*>(p.e0);
    const T* su = static_cast<const T*>(p.e1);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + wm * (BM / 2) + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          const int col = n0 + wn * (BN / 2) + j * 32 + l32;
          if (row < row_end) {
            const int64_t so = static_cast<int64_t>(row) * p.f + col;
            const float g = Elem<T>::to_f32(sg[so]), u = Elem<T>::to_f32(su[so]);
            const float dh = acc[i][j][r];
            const float s = 1.0f / (1.0f + __expf(-g));
            const float du = dh * g * s;
            const float dg = dh * u * s * (1.0f + g * (1.0f - s));
            const int64_t o = static_cast<int64_t>(row) * p.ldc + col;
            c0[o] = Elem<T>::from_f32(dg);
            c0[o + p.f] = Elem<T>::from_f32(du);
          }
        }
  } else {  // WGRAD: C[e][m][n], columns >= f go to the second output (dw_up).
    T* out = c0;
    int cn0 = n0;
    if (p.c1 != nullptr && n0 >= p.f) { out = static_cast<T*>(p.c1); cn0 = n0 - p.f; }
    const int ldc = p.ldc;
    T* base = out + static_cast<int64_t>(e) * p.cstride;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * (BM / 2) + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          const int col = cn0 + wn * (BN / 2) + j * 32 + l32;
          base[static_cast<int64_t>(row) * ldc + col] = Elem<T>::from_f32(acc[i][j][r]);
        }
  }
}

// ---------------------------------------------------------------------------------
// Host-side launchers.
// ---------------------------------------------------------------------------------

template <typename T, int MODE, int BM, int BN>
static hipError_t launch_mode(const GemmParams& p, int grid, hipStream_t s) {
  constexpr int lds = 2 * (BM + BN) * 128;
  auto kern = grouped_gemm_kernel<T, MODE, BM, BN>;
  static std::atomic<bool> attr_set{false};  // the attribute write is idempotent
  if (!attr_set.load(std::memory_order_acquire)) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (err != hipSuccess) return err;
    attr_set.store(true, std::memory_order_release);
  }
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, s, p);
  return hipGetLastError();
}

static int round8(int64_t g) { return static_cast<int>((g + 7) / 8 * 8); }

// Grid bound for row-ragged modes: sum_e ceil(n_e/BM) <= ceil(S/BM) + E.
static int ragged_grid(int S, int E, int BM, int NT) {
  return round8((static_cast<int64_t>((S + BM - 1) / BM) + E) * NT);
}

template <typename T, int MODE>
static hipError_t launch_ragged(const GemmParams& p, hipStream_t s) {
  // Column tile: 128 unless N is only a multiple of 64.
  if (MODE == FWD_GU || p.N % 128 == 0)
    return launch_mode<T, MODE, 128, 128>(p, ragged_grid(p.S, p.E, 128, p.N / 128), s);
  if constexpr (MODE != FWD_GU)
    return launch_mode<T, MODE, 128, 64>(p, ragged_grid(p.S, p.E, 128, p.N / 64), s);
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_wgrad(const GemmParams& p, hipStream_t s) {
  // A column tile must not straddle the gate|up split at column f.
  const int nsplit = p.c1 ? p.f : p.N;
  const int bm = (p.M % 128 == 0) ? 128 : 64;
  const int bn = (p.N % 128 == 0 && nsplit % 128 == 0) ? 128 : 64;
  const int grid = round8(static_cast<int64_t>(p.E) * (p.M / bm) * (p.N / bn));
  if (bm == 128 && bn == 128) return launch_mode<T, WGRAD, 128, 128>(p, grid, s);
  if (bm == 128) return launch_mode<T, WGRAD, 128, 64>(p, grid, s);
  if (bn == 128) return launch_mode<T, WGRAD, 64, 128>(p, grid, s);
  return launch_mode<T, WGRAD, 64, 64>(p, grid, s);
}

// fp32 layers use the kernel above; bf16 layers the kernel of gemm_bf16.hip.
template <typename T>
static hipError_t ragged_launch(int mode, const GemmParams& p, hipStream_t s) {
  if constexpr (std::is_same<T, float>::value) {
    switch (mode) {
      case FWD_GU: return launch_ragged<T, FWD_GU>(p, s);
      case FWD_DOWN: return launch_ragged<T, FWD_DOWN>(p, s);
      case BWD_DOWN: return launch_ragged<T, BWD_DOWN>(p, s);
      case BWD_GU: return launch_ragged<T, BWD_GU>(p, s);
      default: return hipErrorInvalidValue;
    }
  } else {
    return launch_bf16_ragged(mode, p, s);
  }
}

template <typename T>
static hipError_t ragged(int mode, const GemmParams& p, hipStream_t s) {
  ktimer_begin(mode, s);
  const hipError_t err = ragged_launch<T>(mode, p, s);
  ktimer_end(mode, s);
  return err;
}

template <typename T>
static hipError_t wgrad(const GemmParams& p, hipStream_t s) {
  ktimer_begin(WGRAD, s);
  hipError_t err;
  if constexpr (std::is_same<T, float>::value) err = launch_wgrad<T>(p, s);
  else err = launch_bf16_wgrad(p, s);
  ktimer_end(WGRAD, s);
  return err;
}

// G, U, H = SwiGLU(xp W_gate, xp W_up): the forward's first GEMM, and the
// backward's recomputation of its activations.
template <typename T>
static hipError_t gate_up_t(const FfnArgs& a, hipStream_t s) {
  const int d = a.d, f = a.f;
  GemmParams p{};
  p.offsets = a.offsets; p.E = a.E; p.S = a.S; p.f = f;
  p.a = a.xp; p.lda = d; p.b0 = a.w_gate; p.b1 = a.w_up; p.ldb = f;
  p.bstride = static_cast<int64_t>(d) * f;
  p.c0 = a.G; p.c1 = a.U; p.c2 = a.H; p.ldc = f; p.N = 2 * f; p.K = d;
  return ragged<T>(FWD_GU, p, s);
}

template <typename T>
static hipError_t ffn_fwd_t(const FfnArgs& a, hipStream_t s) {
  const int S = a.S, d = a.d, f = a.f;
  hipError_t err = gate_up_t<T>(a, s);
  if (err != hipSuccess) return err;
  // O = H W_down
  GemmParams q{};
  q.offsets = a.offsets; q.E = a.E; q.S = S; q.f = f;
  q.a = a.H; q.lda = f; q.b0 = a.w_down; q.ldb = d; q.bstride = static_cast<int64_t>(f) * d;
  q.c0 = a.o; q.ldc = d; q.N = d; q.K = f;
  return ragged<T>(FWD_DOWN, q, s);
}

template <typename T>
static hipError_t ffn_bwd_t(const FfnArgs& a, hipStream_t s) {
  const int S = a.S, d = a.d, f = a.f;
  hipError_t err;
  // Activation recompute: G, U, H come back from the gate/up GEMM, bit for
  // bit what the forward computed (same kernel, same operands).
  if (a.recompute && (err = gate_up_t<T>(a, s)) != hipSuccess) return err;
  {  // dGU = SwiGLU'(dO W_down^T)
    GemmParams p{};
    p.offsets = a.offsets; p.E = a.E; p.S = S; p.f = f;
    p.a = a.d_o; p.lda = d; p.b0 = a.w_down; p.ldb = d; p.bstride = static_cast<int64_t>(f) * d;
    p.c0 = a.dgu; p.ldc = 2 * f; p.e0 = a.G; p.e1 = a.U; p.N = f; p.K = d;
    if ((err = ragged<T>(BWD_DOWN, p, s)) != hipSuccess) return err;
  }
  {  // dXp = dG W_gate^T + dU W_up^T   (K = 2f)
    GemmParams p{};
    p.offsets = a.offsets; p.E = a.E; p.S = S; p.f = f;
    p.a = a.dgu; p.lda = 2 * f; p.b0 = a.w_gate; p.b1 = a.w_up; p.ldb = f;
    p.bstride = static_cast<int64_t>(d) * f;
    p.c0 = a.dxp; p.ldc = d; p.N = d; p.K = 2 * f;
    if ((err = ragged<T>(BWD_GU, p, s)) != hipSuccess) return err;
  }
  {  // dW_down[e] = H_e^T dO_e   ([f][d], K = n_e)
    GemmParams p{};
    p.offsets = a.offsets; p.E = a.E; p.S = S;
    p.a = a.H; p.lda = f; p.b0 = a.d_o; p.ldb = d;
    p.c0 = a.dw_down; p.c1 = nullptr; p.ldc = d; p.cstride = static_cast<int64_t>(f) * d; p.M = f; p.N = d; p.f = d;
    if ((err = wgrad<T>(p, s)) != hipSuccess) return err;
  }
  {  // [dW_gate | dW_up][e] = Xp_e^T [dG | dU]_e   ([d][2f] split at column f)
    GemmParams p{};
    p.offsets = a.offsets; p.E = a.E; p.S = S;
    p.a = a.xp; p.lda = d; p.b0 = a.dgu; p.ldb = 2 * f;
    p.c0 = a.dw_gate; p.c1 = a.dw_up; p.ldc = f; p.cstride = static_cast<int64_t>(d) * f; p.M = d; p.N = 2 * f; p.f = f;
    if ((err = wgrad<T>(p, s)) != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_ffn_fwd(const FfnArgs& a, bool is_f32, hipStream_t s) {
  return is_f32 ? ffn_fwd_t<float>(a, s) : ffn_fwd_t<bf16_t>(a, s);
}
hipError_t launch_ffn_bwd(const FfnArgs& a, bool is_f32, hipStream_t s) {
  return is_f32 ? ffn_bwd_t<float>(a, s) : ffn_bwd_t<bf16_t>(a, s);
}

}  // namespace moe
