// MXFP8 grouped GEMMs of the expert SwiGLU FFN for gfx950: E4M3 operands with
// one E8M0 scale per 32 elements along K, fp32 accumulation, bf16 outputs.
//
// The pages train the experts in MXFP8 and credit it with most of the gain of
// the expert computation and of the data moved for it ("Olmo-core 3 é
// lançado com infraestrutura para treinar modelos MoE", section "Otimizações e
// testes em escala de trilhões"; "Ai2 rilascia Olmo-Core 3...", section
// "Parallelismo, precisione e tecniche di memoria"). The grouped GEMM is the
// same device-scheduled one as the bf16 path (tile schedule and epilogues are
// shared, gemm_device.h); what changes is the main loop:
//  - both operands are K-major E4M3 (the quantisers write every operand that
//    way, transposing where the bf16 tensor is row-contiguous), so a slab of
//    64 k is a [rows][64 bytes] tile, loaded by LDS DMA exactly like the
//    bf16 kernel's 32-k slabs;
//  - each slab also carries the E8M0 scale tiles (2 bytes per row: the two
//    32-blocks of the slab), one 1 KB DMA per wave;
//  - v_mfma_scale_f32_32x32x64_f8f6f4 multiplies a 32 x 64 by a 64 x 32 block
//    with the block scales applied in the matrix core. Lane l supplies row
//    l%32 with k = 16 (l/32) .. +15 and 32 + 16 (l/32) .. +15 (two 16-byte
//    LDS reads) and the scale of (row l%32, 32-block l/32).
// Ring: 4 slots of one slab each. Iteration kt: wait for slab kt+1, barrier
// (slot kt's fragments are in registers), refill slot kt with slab kt+4, then
// read slab kt+1's fragments while slab kt's MFMAs run.
#include "common.h"
#include "gemm_device.h"
#include "grouped_gemm.h"
#include "kernels.h"

namespace moe {
namespace {

using namespace gemm;

constexpr int kStagesX = 4;
constexpr int kEpiWorkX = 4;    // a tile's epilogue costs about as much as this many slabs
constexpr int kScaleArea = 1024;  // LDS bytes per wave for the scale DMA

typedef int v8i __attribute__((ext_vector_type(8)));

// 32 bytes of fragment (32 rows x 64 k of E4M3) from a [rows][64 B] tile.
__device__ __forceinline__ v8i frag_mx(const char* t, int rb, int lane) {
  const bf16x8 lo = frag_kmajor(t, rb, 0, lane);
  const bf16x8 hi = frag_kmajor(t, rb, 1, lane);
  v8i v;
  __builtin_memcpy(&v, &lo, 16);
  __builtin_memcpy(reinterpret_cast<char*>(&v) + 16, &hi, 16);
  return v;
}

template <int MODE, int BM, int BN>
__global__ __launch_bounds__(256) void gg_mx_kernel(GemmParams p) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int TILE_M = BM * 64, TILE_N = BN * 64;
  constexpr int SCALES = 4 * kScaleArea;             // per slot: [M scales | N scales | up scales | spare]
  constexpr int STAGE = TILE_M + TILE_N + SCALES;
  static_assert(MODE != FWD_GU || NB % 2 == 0, "SwiGLU pairing needs gate and up blocks in every wave");

  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int s_info[8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  auto run_tile = [&](const TileCoord& tc) {
    const int e = tc.e, row0 = tc.row0, row_end = tc.row_end, nt = tc.nt, m0 = tc.m0;
    const int n0 = nt * BN;
    // WGRAD: [row0, row_end) is the expert's padded K range (a multiple of 64).
    const int nk = (MODE == WGRAD) ? (row_end - row0) / 64 : p.K / 64;
    const int64_t bexp = static_cast<int64_t>(e) * p.bstride;
    const int64_t bsexp = static_cast<int64_t>(e) * p.bs_estride;
    const uint8_t* A = static_cast<const uint8_t*>(p.a);
    const uint8_t* B0 = static_cast<const uint8_t*>(p.b0);
    const uint8_t* B1 = static_cast<const uint8_t*>(p.b1);

    // ---- HBM -> LDS for slab kt (empty descriptors at or past the end) -------------------
    // Each wave issues kLoads loads per slab: [0, LM) the M tile, [LM, LM + LN)
    // the N tile, then one 1 KB scale load: wave 0 the M side's scales, wave 1
    // the N side's (the gate half for FWD_GU), wave 2 the up half's for FWD_GU;
    // the remaining waves load nothing into their own area, so every wave
    // issues the same count (the vmcnt waits count them).
    constexpr int LM = BM / 64, LN = BN / 64, kLoads = LM + LN + 1;
    // W: wait states of the loads (load_lds16): 4 where a descriptor may have
    // just been written by a VALU instruction, 0 in the steady-state loop.
    auto issue = [&](int kt, uint32_t slot, auto L, auto w) {
      constexpr int l = decltype(L)::value, W = decltype(w)::value;
      const bool live = kt < nk;
      if constexpr (l < LM) {
        if constexpr (MODE == WGRAD) {
          const int64_t k0 = row0 + static_cast<int64_t>(kt) * 64;
          load_rows64<BM, W>(make_rsrc(A + m0 * p.lda + k0, live ? BM * p.lda : 0), p.lda, slot, wave, lane, l);
        } else {
          const int valid = live ? min(BM, row_end - row0) : 0;
          load_rows64<BM, W>(make_rsrc(A + static_cast<int64_t>(row0) * p.lda + kt * 64,
                                       static_cast<int64_t>(valid) * p.lda),
                             p.lda, slot, wave, lane, l);
        }
      } else if constexpr (l < LM + LN) {
        constexpr int q = l - LM;
        const uint32_t tn = slot + TILE_M;
        if constexpr (MODE == FWD_GU) {
          constexpr int half = q / (LN / 2), qq = q % (LN / 2);
          const int64_t off = bexp + static_cast<int64_t>(nt * (BN / 2)) * p.ldb + kt * 64;
          const int64_t bytes = live ? static_cast<int64_t>(BN / 2) * p.ldb : 0;
          load_rows64<BN / 2, W>(make_rsrc((half ? B1 : B0) + off, bytes), p.ldb, tn + half * (TILE_N / 2), wave,
                                 lane, qq);
        } else if constexpr (MODE == WGRAD) {
          const int64_t k0 = row0 + static_cast<int64_t>(kt) * 64;
          load_rows64<BN, W>(make_rsrc(B0 + n0 * p.ldb + k0, live ? BN * p.ldb : 0), p.ldb, tn, wave, lane, q);
        } else {  // FWD_DOWN, BWD_DOWN, BWD_GU: B stored [n][k] per expert
          const uint8_t* src = B0;
          int ks = kt;
          if constexpr (MODE == BWD_GU) {
            if (kt * 64 >= p.f) { src = B1; ks = kt - p.f / 64; }
          }
          load_rows64<BN, W>(make_rsrc(src + bexp + static_cast<int64_t>(n0) * p.ldb + ks * 64,
                                       live ? static_cast<int64_t>(BN) * p.ldb : 0),
                             p.ldb, tn, wave, lane, q);
        }
      } else {
        const uint32_t sc = slot + TILE_M + TILE_N + wave * kScaleArea;
        const uint32_t voff = static_cast<uint32_t>(lane * 16);
        if (wave == 0) {
          if constexpr (MODE == WGRAD) {
            const int64_t k0 = row0 + static_cast<int64_t>(kt) * 64;
            load_lds16<W>(make_rsrc(p.as + (k0 / 64) * p.as_slab + m0 * 2, live ? BM * 2 : 0), voff, sc);
          } else {
            // Buffer range checks are per dword: round the range up to whole
            // dwords or an odd row count loses its last row's scales. The extra
            // bytes are the scales of a row whose data reads as zero (it is
            // never written).
            const int valid = live ? min(BM, row_end - row0) : 0;
            load_lds16<W>(make_rsrc(p.as + static_cast<int64_t>(kt) * p.as_slab + row0 * 2, (valid * 2 + 3) & ~3),
                          voff, sc);
          }
        } else if (wave == 1 || (wave == 2 && MODE == FWD_GU)) {
          if constexpr (MODE == FWD_GU) {
            const int64_t so = bsexp + static_cast<int64_t>(kt) * p.bs_slab + nt * (BN / 2) * 2;
            load_lds16<W>(make_rsrc((wave == 1 ? p.bs0 : p.bs1) + so, live ? BN : 0), voff, sc);
          } else if constexpr (MODE == WGRAD) {
            const int64_t k0 = row0 + static_cast<int64_t>(kt) * 64;
            load_lds16<W>(make_rsrc(p.bs0 + (k0 / 64) * p.bs_slab + n0 * 2, live ? BN * 2 : 0), voff, sc);
          } else {
            const uint8_t* ssrc = p.bs0;
            int ks = kt;
            if constexpr (MODE == BWD_GU) {
              if (kt * 64 >= p.f) { ssrc = p.bs1; ks = kt - p.f / 64; }
            }
            load_lds16<W>(make_rsrc(ssrc + bsexp + static_cast<int64_t>(ks) * p.bs_slab + n0 * 2, live ? BN * 2 : 0),
                          voff, sc);
          }
        } else {
          load_lds16<W>(make_rsrc(p.as, 0), voff, sc);
        }
      }
    };

    floatx16 acc[NB][MB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

    struct Frags {
      v8i m[MB], n[NB];
      int sm[MB], sn[NB];
    };
    // Fragment FI (compile time) and its scale: [0, MB) M side, [MB, MB + NB) N side.
    auto read_frag = [&](const char* slotp, Frags& F, auto FI) {
      constexpr int fi = decltype(FI)::value;
      const char* tm = slotp;
      const char* tn = slotp + TILE_M;
      const uint8_t* sc = reinterpret_cast<const uint8_t*>(slotp + TILE_M + TILE_N);
      const int r32 = lane & 31, kb = lane >> 5;
      if constexpr (fi < MB) {
        const int row = wm * WM + fi * 32;
        F.m[fi] = frag_mx(tm, row, lane);
        F.sm[fi] = sc[(row + r32) * 2 + kb];
      } else {
        constexpr int j = fi - MB;
        if constexpr (MODE == FWD_GU) {
          constexpr int half = j / (NB / 2), jj = j % (NB / 2);
          const int row = wn * (WN / 2) + jj * 32;
          F.n[j] = frag_mx(tn + half * (TILE_N / 2), row, lane);
          F.sn[j] = sc[(1 + half) * kScaleArea + (row + r32) * 2 + kb];
        } else {
          const int row = wn * WN + j * 32;
          F.n[j] = frag_mx(tn, row, lane);
          F.sn[j] = sc[kScaleArea + (row + r32) * 2 + kb];
        }
      }
    };
    auto mfma_one = [&](const Frags& F, auto MI) {
      constexpr int mi = decltype(MI)::value, j = mi / MB, i = mi % MB;
      acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.n[j], F.m[i], acc[j][i], 0, 0, 0, F.sn[j], 0,
                                                                 F.sm[i]);
    };
    constexpr int kMfma = MB * NB, kFrags = MB + NB;

    const uint32_t ring = __builtin_amdgcn_readfirstlane(lds_addr(smem));
#pragma unroll
    for (int s0 = 0; s0 < kStagesX; ++s0)
      static_for<kLoads>([&](auto L) { issue(s0, ring + s0 * STAGE, L, std::integral_constant<int, 4>{}); });
    // One slab: wait for slab kt+1, barrier, then slab kt's MFMAs on `cur`
    // with the reads of slab kt+1 into `nxt` and the loads of slab kt+4 into
    // slot kt spread between them (a burst of LDS-DMA loads would back up the
    // texture-address unit into the issue of the MFMAs behind it). Two
    // register sets with fixed names (the loop is unrolled by two: a runtime
    // index would put them in scratch memory).
    auto step = [&](int kt, const Frags& cur, Frags& nxt) {
      wait_vmcnt<kLoads * (kStagesX - 2)>();   // slab kt+1 has landed
      __syncthreads();                          // slot kt is read out; slab kt+1 is visible
      const char* nslot = smem + ((kt + 1) % kStagesX) * STAGE;
      const uint32_t slot = ring + (kt % kStagesX) * STAGE;
      static_for<kLoads>([&](auto S) {
        constexpr int sg = decltype(S)::value;
        constexpr int m_lo = sg * kMfma / kLoads, m_hi = (sg + 1) * kMfma / kLoads;
        constexpr int f_lo = sg * kFrags / kLoads, f_hi = (sg + 1) * kFrags / kLoads;
        static_for<m_hi - m_lo>([&](auto D) { mfma_one(cur, std::integral_constant<int, m_lo + decltype(D)::value>{}); });
        static_for<f_hi - f_lo>([&](auto D) { read_frag(nslot, nxt, std::integral_constant<int, f_lo + decltype(D)::value>{}); });
        issue(kt + kStagesX, slot, S, std::integral_constant<int, 0>{});
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    Frags f0, f1;
    wait_vmcnt<kLoads * (kStagesX - 1)>();
    __syncthreads();
    static_for<kFrags>([&](auto FI) { read_frag(smem, f0, FI); });
    for (int kt = 0; kt < nk; kt += 2) {
      step(kt, f0, f1);
      if (kt + 1 < nk) step(kt + 1, f1, f0);
    }
    wait_vmcnt<0>();
    __syncthreads();  // every wave is done with the ring
    epilogue<MODE, BM, BN, true>(p, acc, smem, wave, lane, tc);
  };
  if constexpr (MODE == WGRAD) {
    wgrad_sched<BM, BN, 64, kEpiWorkX>(p, s_info, wave, lane);
    const int t_first = __builtin_amdgcn_readfirstlane(s_info[0]);
    const int t_end = __builtin_amdgcn_readfirstlane(s_info[1]);
    const int t_stride = __builtin_amdgcn_readfirstlane(s_info[2]);
    for (int t = t_first; t < t_end; t += t_stride) {
      run_tile(wgrad_tile<BM, BN>(p, t));
      __syncthreads();  // the staging area is the next tile's ring
    }
  } else {
    const TileCoord tc = ragged_tile<BM, BN>(p, s_info, wave, lane);
    if (tc.e < 0) return;
    run_tile(tc);
  }
}

int round8(int64_t g) { return static_cast<int>((g + 7) / 8 * 8); }

template <int MODE, int BM, int BN>
hipError_t launch_tile(const GemmParams& p, int tiles, hipStream_t s) {
  constexpr int ring = kStagesX * (BM * 64 + BN * 64 + 4 * kScaleArea), stage = 4 * 2 * (BM / 2) * 128;
  constexpr int lds = ring > stage ? ring : stage;
  auto kern = gg_mx_kernel<MODE, BM, BN>;
  static std::atomic<int> per_cu{0};  // resident workgroups per CU (idempotent)
  if (per_cu.load() == 0) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (err != hipSuccess) return err;
    int n = 0;
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(kern), 256, lds);
    if (err != hipSuccess) return err;
    per_cu.store(n > 0 ? n : 1);
  }
  if (tiles <= 0) return hipSuccess;
  // One workgroup per tile for the row-ragged modes, a persistent grid for
  // the weight gradients (as in the bf16 kernel).
  const int cap = max(8, device_cu_count() * per_cu.load() / 8 * 8);
  const int grid = MODE == WGRAD ? min(cap, round8(tiles)) : round8(tiles);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, s, p);
  return hipGetLastError();
}

int ragged_grid(int S, int E, int BM, int NT) {
  return round8((static_cast<int64_t>((S + BM - 1) / BM) + E) * NT);
}

// 256 x 256 tiles where N allows: a slab then moves 36 KB (data and scales)
// per 1024 MFMA cycles of each SIMD, against 28 KB per 512 cycles for
// 256 x 128 tiles, which saturates the LDS and the texture path.
template <int MODE>
hipError_t ragged_mode(const GemmParams& p, hipStream_t s) {
  // N is a multiple of 128 (MXFP8 layers need d, f multiples of 128).
  if (static_cast<int64_t>(p.S) >= 1024LL * p.E) {
    if (p.N % 256 == 0) return launch_tile<MODE, 256, 256>(p, ragged_grid(p.S, p.E, 256, p.N / 256), s);
    return launch_tile<MODE, 256, 128>(p, ragged_grid(p.S, p.E, 256, p.N / 128), s);
  }
  return launch_tile<MODE, 128, 128>(p, ragged_grid(p.S, p.E, 128, p.N / 128), s);
}

}  // namespace

hipError_t launch_mx_ragged(int mode, const GemmParams& p, hipStream_t s) {
  ktimer_begin(mode, s);
  hipError_t err;
  switch (mode) {
    case FWD_GU: err = ragged_mode<FWD_GU>(p, s); break;
    case FWD_DOWN: err = ragged_mode<FWD_DOWN>(p, s); break;
    case BWD_DOWN: err = ragged_mode<BWD_DOWN>(p, s); break;
    case BWD_GU: err = ragged_mode<BWD_GU>(p, s); break;
    default: err = hipErrorInvalidValue;
  }
  ktimer_end(mode, s);
  return err;
}

static hipError_t mx_wgrad(const GemmParams& p, hipStream_t s) {
  auto grid = [&](int bm, int bn) { return round8(static_cast<int64_t>(p.E) * (p.M / bm) * (p.N / bn)); };
  // A column tile must not straddle the gate|up split at column f.
  const int nsplit = p.c1 ? p.f : p.N;
  if (p.M % 256 == 0 && p.N % 256 == 0 && nsplit % 256 == 0) return launch_tile<WGRAD, 256, 256>(p, grid(256, 256), s);
  if (p.M % 256 == 0) return launch_tile<WGRAD, 256, 128>(p, grid(256, 128), s);
  return launch_tile<WGRAD, 128, 128>(p, grid(128, 128), s);
}

hipError_t launch_mx_wgrad(const GemmParams& p, hipStream_t s) {
  ktimer_begin(WGRAD, s);
  const hipError_t err = mx_wgrad(p, s);
  ktimer_end(WGRAD, s);
  return err;
}

}  // namespace moe
