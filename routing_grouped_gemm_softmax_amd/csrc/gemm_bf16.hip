// bf16 grouped GEMMs of the expert SwiGLU FFN for gfx950 (forward, dgrad,
// wgrad), scheduled on the device from the per-expert row offsets.
//
// The pages run the experts' matmuls as one grouped GEMM whose schedule lives
// on the device, so the host never waits for routing metadata ("Olmo-core 3
// escala el entrenamiento de mixture-of-experts a billones de parámetros",
// section "Cómo funciona"; "Ai2 rilascia Olmo-Core 3...", section
// "Parallelismo, precisione e tecniche di memoria"). Every workgroup reads the
// E+1 offsets and maps its id to (expert, row tile, column tile) with a wave
// scan over the per-expert tile counts (RowTileMap); the grid is sized on the
// host from the count-free bound ceil(S/BM) + E row tiles. The weight
// gradients, whose tiles cost as much as their expert has rows, run on a
// persistent grid with XCD ranges cut by cost when the load is skewed
// (gemm_device.h). FWD_DOWN, and the weight gradients of small experts, run
// as persistent grids that stream slabs across tiles (gg_bf16_stream_kernel).
//
// Tile: 256 threads = 4 waves in 2 x 2; a BM x BN output tile, each wave a
// (BM/2) x (BN/2) block of 32x32 MFMA tiles (v_mfma_f32_32x32x16_bf16) with
// the accumulators in AGPRs. K advances in slabs of 32 elements (64 bytes).
//
// Operands move HBM -> LDS with buffer_load ... lds (16 bytes per lane, no
// VGPR staging) into a ring of 4 slab slots: the loads of slabs kt+1..kt+3
// fly while slab kt is multiplied. The buffer range check zero-fills rows
// past an expert's end, which both masks ragged row tiles and gives the
// weight gradients their ragged K for free. LDS layouts:
//  - K-contiguous operand: [row][32 k] rows of 64 B, 16-byte chunks
//    XOR-swizzled by the row; fragments are one ds_read_b128 per lane.
//  - row-contiguous operand ([k][rows] in HBM: the weights in the forward and
//    both operands of the weight gradients): [32 k][rows] as stored, chunks
//    XOR-swizzled by k; fragments are two ds_read_b64_tr_b16 per lane, which
//    transpose 16 x 4 blocks on the way out of LDS.
// The N-side fragment is the MFMA's first operand, so every lane ends up with
// four consecutive output columns of one row: the epilogue stores 8 bytes per
// lane and reads the saved G, U the same way.
#include "common.h"
#include "grouped_gemm.h"
#include "gemm_device.h"
#include "kernels.h"

namespace moe {
namespace {

using namespace gemm;

constexpr int kBK = 32;     // K elements per slab (64 bytes of bf16)
constexpr int kStages = 4;  // LDS ring depth: slabs kt+1..kt+3 fly while kt is multiplied
constexpr int kEpiWork = 8; // a tile's epilogue costs about as much as this many slabs

template <int MODE, int BM, int BN>
__global__ __launch_bounds__(256) void gg_bf16_kernel(GemmParams p) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr bool M_MN = (MODE == WGRAD);                                      // A stored [k][m]
  constexpr bool N_MN = (MODE == FWD_GU || MODE == FWD_DOWN || MODE == WGRAD);  // B stored [k][n]
  constexpr int TILE_M = BM * kBK * 2, TILE_N = BN * kBK * 2;
  constexpr int STAGE = TILE_M + TILE_N;  // bytes of one ring slot
  static_assert(MODE != FWD_GU || NB % 2 == 0, "SwiGLU pairing needs gate and up blocks in every wave");

  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int s_info[8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  auto run_tile = [&](const TileCoord& tc) {
    const int e = tc.e, row0 = tc.row0, row_end = tc.row_end, nt = tc.nt, m0 = tc.m0;
    const int n0 = nt * BN;
    const int nk = (MODE == WGRAD) ? (row_end - row0 + kBK - 1) / kBK : p.K / kBK;

    const char* const A = static_cast<const char*>(p.a);
    const int64_t bexp = static_cast<int64_t>(e) * p.bstride;

    // ---- HBM -> LDS ------------------------------------------------------------------------
    // Descriptors of slab kt. A slab at or past the end (kt >= nk) gets empty
    // descriptors: its loads read nothing and only zero-fill a ring slot that
    // nobody reads again.
    auto rsrc_m = [&](int kt) {
      const bool live = kt < nk;
      if constexpr (!M_MN) {
        const char* base = A + (static_cast<int64_t>(row0) * p.lda + kt * kBK) * 2;
        const int valid = live ? min(BM, row_end - row0) : 0;
        return make_rsrc(base, static_cast<int64_t>(valid) * p.lda * 2);
      } else {
        const int k0 = row0 + kt * kBK;
        const char* base = A + (static_cast<int64_t>(k0) * p.lda + m0) * 2;
        const int valid = live ? min(kBK, row_end - k0) : 0;
        return make_rsrc(base, static_cast<int64_t>(valid) * p.lda * 2);
      }
    };
    auto rsrc_n = [&](int kt, int half) {
      const bool live = kt < nk;
      if constexpr (MODE == FWD_GU) {
        // Two sub-tiles [32 k][BN/2]: gate columns (half 0), the same up columns (half 1).
        const int64_t off = (bexp + static_cast<int64_t>(kt) * kBK * p.ldb + nt * (BN / 2)) * 2;
        const char* src = static_cast<const char*>(half ? p.b1 : p.b0);
        return make_rsrc(src + off, live ? static_cast<int64_t>(kBK) * p.ldb * 2 : 0);
      } else if constexpr (MODE == FWD_DOWN) {
        const int64_t off = (bexp + static_cast<int64_t>(kt) * kBK * p.ldb + n0) * 2;
        return make_rsrc(static_cast<const char*>(p.b0) + off, live ? static_cast<int64_t>(kBK) * p.ldb * 2 : 0);
      } else if constexpr (MODE == WGRAD) {
        const int k0 = row0 + kt * kBK;
        const int valid = live ? min(kBK, row_end - k0) : 0;
        return make_rsrc(static_cast<const char*>(p.b0) + (static_cast<int64_t>(k0) * p.ldb + n0) * 2,
                         static_cast<int64_t>(valid) * p.ldb * 2);
      } else {  // BWD_DOWN, BWD_GU: B stored [n][k]
        const char* src = static_cast<const char*>(p.b0);
        int kcol = kt * kBK;
        if constexpr (MODE == BWD_GU) {
          if (kcol >= p.f) { src = static_cast<const char*>(p.b1); kcol -= p.f; }
        }
        const char* base = src + (bexp + static_cast<int64_t>(n0) * p.ldb + kcol) * 2;
        return make_rsrc(base, live ? static_cast<int64_t>(BN) * p.ldb * 2 : 0);
      }
    };
    // Load L of a slab (each wave issues kLoads per slab): [0, LM) fill the M
    // tile, [LM, kLoads) the N tile. W: wait states (load_lds16).
    constexpr int LM = BM / 64, LN = BN / 64, kLoads = LM + LN;
    auto issue = [&](int kt, uint32_t slot, auto L, auto w) {
      constexpr int l = decltype(L)::value, W = decltype(w)::value;
      if constexpr (l < LM) {
        if constexpr (M_MN) load_mnmajor<BM, W>(rsrc_m(kt), p.lda, slot, wave, lane, l);
        else load_rows64<BM, W>(rsrc_m(kt), p.lda * 2, slot, wave, lane, l);
      } else {
        constexpr int q = l - LM;
        if constexpr (MODE == FWD_GU) {
          constexpr int half = q / (LN / 2), qq = q % (LN / 2);
          load_mnmajor<BN / 2, W>(rsrc_n(kt, half), p.ldb, slot + TILE_M + half * (TILE_N / 2), wave, lane, qq);
        } else if constexpr (N_MN) {
          load_mnmajor<BN, W>(rsrc_n(kt, 0), p.ldb, slot + TILE_M, wave, lane, q);
        } else {
          load_rows64<BN, W>(rsrc_n(kt, 0), p.ldb * 2, slot + TILE_M, wave, lane, q);
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

    // Fragments of one 16-deep k step: MB from the M side, NB from the N side.
    struct Frags {
      bf16x8 m[MB], n[NB];
    };
    // Fragment FI (compile time): [0, MB) M side, [MB, MB + NB) N side.
    auto read_frag = [&](const char* slotp, int kk, Frags& F, auto FI) {
      constexpr int fi = decltype(FI)::value;
      const char* tm = slotp;
      const char* tn = slotp + TILE_M;
      if constexpr (fi < MB) {
        if constexpr (M_MN) F.m[fi] = frag_mnmajor<BM>(tm, wm * WM + fi * 32, kk, lane);
        else F.m[fi] = frag_kmajor(tm, wm * WM + fi * 32, kk, lane);
      } else {
        constexpr int j = fi - MB;
        if constexpr (MODE == FWD_GU) {
          // Blocks [0, NB/2) are gate columns, [NB/2, NB) the same up columns.
          constexpr int half = j / (NB / 2), jj = j % (NB / 2);
          F.n[j] = frag_mnmajor<BN / 2>(tn + half * (TILE_N / 2), wn * (WN / 2) + jj * 32, kk, lane);
        } else if constexpr (N_MN) {
          F.n[j] = frag_mnmajor<BN>(tn, wn * WN + j * 32, kk, lane);
        } else {
          F.n[j] = frag_kmajor(tn, wn * WN + j * 32, kk, lane);
        }
      }
    };
    auto read_frags = [&](const char* slotp, int kk, Frags& F) {
      static_for<MB + NB>([&](auto FI) { read_frag(slotp, kk, F, FI); });
    };
    auto mfma_one = [&](const Frags& F, auto MI) {
      constexpr int mi = decltype(MI)::value, j = mi / MB, i = mi % MB;
      acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.n[j], F.m[i], acc[j][i], 0, 0, 0);
    };
    // LDS reads per k step, for the schedule hints.
    constexpr int kReads = MB * (M_MN ? 2 : 1) + NB * (N_MN ? 2 : 1);
    constexpr int kMfma = MB * NB;
    constexpr int kFrags = MB + NB;

    // ---- main loop -------------------------------------------------------------------------
    // Ring of kStages = 4 slots, one slab (32 k) each; each slab is two 16-deep
    // k steps. Iteration kt:
    //   A: MFMAs of step 0 of slab kt, interleaved with the LDS reads of step 1;
    //   wait until slab kt+1 has landed (slabs kt+2, kt+3 may still fly) and
    //   barrier: everyone is done reading slot kt, and slab kt+1 is visible;
    //   B: MFMAs of step 1 of slab kt, with the reads of step 0 of slab kt+1
    //   and the kLoads loads of slab kt+4 into slot kt spread between them.
    // A load has three slabs of MFMAs to land in. Spreading the loads keeps the
    // texture-address unit, which takes a 1 KB LDS-DMA load in many cycles,
    // from backing up into the issue of the MFMAs behind a burst of loads.
    static_assert(kStages == 4 && kBK == 32, "schedule written for a 4-slot ring of 2-step slabs");
    auto interleave = [&]() {
      constexpr int inter = kReads < kMfma ? kReads : kMfma;
#pragma unroll
      for (int r = 0; r < inter; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if constexpr (kReads > kMfma) __builtin_amdgcn_sched_group_barrier(0x100, kReads - kMfma, 0);
      if constexpr (kMfma > kReads) __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kReads, 0);
    };
    const uint32_t ring = __builtin_amdgcn_readfirstlane(lds_addr(smem));
#pragma unroll
    for (int s0 = 0; s0 < kStages; ++s0)
      static_for<kLoads>([&](auto L) { issue(s0, ring + s0 * STAGE, L, std::integral_constant<int, 4>{}); });
    Frags F[2];
    wait_vmcnt<kLoads * (kStages - 1)>();
    __syncthreads();
    read_frags(smem, 0, F[0]);
    for (int kt = 0; kt < nk; ++kt) {
      const char* cur = smem + (kt % kStages) * STAGE;
      const char* nxt = smem + ((kt + 1) % kStages) * STAGE;
      read_frags(cur, 1, F[1]);
      static_for<kMfma>([&](auto MI) { mfma_one(F[0], MI); });
      interleave();
      wait_vmcnt<kLoads * (kStages - 2)>();
      __syncthreads();
      const uint32_t slot = ring + (kt % kStages) * STAGE;
      static_for<kLoads>([&](auto S) {
        constexpr int sg = decltype(S)::value;
        constexpr int m_lo = sg * kMfma / kLoads, m_hi = (sg + 1) * kMfma / kLoads;
        constexpr int f_lo = sg * kFrags / kLoads, f_hi = (sg + 1) * kFrags / kLoads;
        static_for<m_hi - m_lo>([&](auto D) { mfma_one(F[1], std::integral_constant<int, m_lo + decltype(D)::value>{}); });
        static_for<f_hi - f_lo>([&](auto D) { read_frag(nxt, 0, F[0], std::integral_constant<int, f_lo + decltype(D)::value>{}); });
        issue(kt + kStages, slot, S, std::integral_constant<int, 0>{});
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    // Drain the (empty) loads still in flight before the LDS is reused or the
    // wave ends.
    wait_vmcnt<0>();

    __syncthreads();  // every wave is done with the ring
    epilogue<MODE, BM, BN>(p, acc, smem, wave, lane, tc);
  };
  if constexpr (MODE == WGRAD) {
    wgrad_sched<BM, BN, kBK, kEpiWork>(p, s_info, wave, lane);
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

// FWD_DOWN and the weight gradients with 256 x 256 tiles, as a persistent
// grid that streams slabs across tiles: each workgroup owns a strided share
// of its XCD's tile range (FWD_DOWN: lo, lo + wpx, ...; WGRAD: the range
// wgrad_sched gives it), and the ring never drains between tiles. The loads
// of the next tile's first slabs go out during the current tile's last
// slabs, and the epilogue (staged through a per-wave LDS area beside the
// ring, written with buffer stores) runs while they fly. Both modes have few
// slabs per tile: FWD_DOWN has K = d_ff; a weight gradient has K = its
// expert's rows, often under 16 slabs, and an empty expert has none (its
// tile is all epilogue, writing zeros). Measured at T = 8192, d = 2048, E =
// 8, k = 4, d_ff = 1024, FWD_DOWN runs in 156 us against 176 us with one tile
// per workgroup; with E = 128 (256 rows per expert) the two weight
// gradients take 229 + 441 us against 254 + 490 us. The same scheme gained
// nothing for the dgrad of the gate/up projection (64 slabs per tile), and
// the SwiGLU epilogue of the gate/up forward does not fit its registers
// beside the stream state.
//
// Epilogue stores are non-temporal (cache policy nt): the outputs are written
// once and read by a later kernel, and the stores complete sooner without
// allocating in the L2, which matters because the next slabs' waits count
// them.
constexpr int kStoreNT = 2;

// Wait counts: vmcnt counts loads and stores together, in issue order. The
// wait for slab g+1 must allow exactly the operations issued after that
// slab's loads: the loads of slabs g+2 and g+3, and kEpiStores stores for
// each epilogue since (every epilogue issues exactly that many: buffer
// stores, whose range check, not a branch, drops rows past the end). The
// kernel counts those epilogues per slab in flight; past two it waits for
// 63, which only waits longer.
template <int MODE>
__global__ __launch_bounds__(256) void gg_bf16_stream_kernel(GemmParams p) {
  constexpr int BM = 256, BN = 256, WM = 128, WN = 128, MB = 4, NB = 4;
  static_assert(MODE == FWD_DOWN || MODE == WGRAD, "streaming modes");
  constexpr bool M_MN = (MODE == WGRAD);  // A stored [k][m]
  constexpr int TILE_M = BM * kBK * 2, TILE_N = BN * kBK * 2;
  constexpr int STAGE = TILE_M + TILE_N;
  constexpr int RING = kStages * STAGE;
  constexpr int kStg = 64 * 128;  // per-wave staging tile: 64 rows x 64 bf16
  constexpr int kEpiStores = 4 * 8;
  constexpr int LM = BM / 64, LN = BN / 64, kLoads = LM + LN;
  constexpr int kWait0 = kLoads * (kStages - 2);
  constexpr int kWait1 = kWait0 + kEpiStores < 63 ? kWait0 + kEpiStores : 63;
  static_assert(kStages == 4, "epilogue accounting written for slabs g+1..g+3 in flight");

  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // ---- this workgroup's tiles ------------------------------------------------------------
  RowTileMap map;
  int lo, step, ntiles;
  if constexpr (MODE == FWD_DOWN) {
    map.init(p, BM, BN, lane);
    const int rmain = map.main_tiles(p.cus);
    const int x = blockIdx.x % 8, wpx = gridDim.x / 8;
    lo = xcd_cut(rmain, x) + blockIdx.x / 8;
    const int hi = xcd_cut(rmain, x + 1);
    step = wpx;
    ntiles = lo < hi ? (hi - lo + wpx - 1) / wpx : 0;
  } else {
    int* s_info = reinterpret_cast<int*>(smem + RING);  // the staging area, free until the first epilogue
    wgrad_sched<BM, BN, kBK, kEpiWork>(p, s_info, wave, lane);
    lo = __builtin_amdgcn_readfirstlane(s_info[0]);
    const int hi = __builtin_amdgcn_readfirstlane(s_info[1]);
    step = __builtin_amdgcn_readfirstlane(s_info[2]);
    ntiles = lo < hi ? (hi - lo + step - 1) / step : 0;
    __syncthreads();  // s_info is read out before any wave's epilogue stages there
  }
  if (ntiles == 0) return;
  auto tile_at = [&](int j) -> TileCoord {
    if constexpr (MODE == FWD_DOWN) return map.at(lo + j * step, lane);
    else return wgrad_tile<BM, BN>(p, lo + j * step);
  };
  auto slabs_of = [&](const TileCoord& tc) -> int {
    if constexpr (MODE == FWD_DOWN) return p.K / kBK;
    else return (tc.row_end - tc.row0 + kBK - 1) / kBK;
  };
  const char* const A = static_cast<const char*>(p.a);

  // ---- HBM -> LDS: load L of slab kt of tile tc (empty descriptors if !live) --------------
  auto issue = [&](const TileCoord& tc, int kt, bool live, uint32_t slot, auto L, auto w) {
    constexpr int l = decltype(L)::value, W = decltype(w)::value;
    if constexpr (MODE == FWD_DOWN) {
      if constexpr (l < LM) {
        const char* base = A + (static_cast<int64_t>(tc.row0) * p.lda + kt * kBK) * 2;
        const int valid = live ? min(BM, tc.row_end - tc.row0) : 0;
        load_rows64<BM, W>(make_rsrc(base, static_cast<int64_t>(valid) * p.lda * 2), p.lda * 2, slot, wave, lane, l);
      } else {
        // W_down [f][d] of the tile's expert: rows k, columns n.
        constexpr int q = l - LM;
        const int64_t off =
            (static_cast<int64_t>(tc.e) * p.bstride + static_cast<int64_t>(kt) * kBK * p.ldb + tc.nt * BN) * 2;
        load_mnmajor<BN, W>(
            make_rsrc(static_cast<const char*>(p.b0) + off, live ? static_cast<int64_t>(kBK) * p.ldb * 2 : 0),
            p.ldb, slot + TILE_M, wave, lane, q);
      }
    } else {
      // Both operands [k][m] / [k][n] over the expert's rows; rows past its
      // end read as zero.
      const int k0 = tc.row0 + kt * kBK;
      const int valid = live ? min(kBK, tc.row_end - k0) : 0;
      if constexpr (l < LM) {
        const char* base = A + (static_cast<int64_t>(k0) * p.lda + tc.m0) * 2;
        load_mnmajor<BM, W>(make_rsrc(base, static_cast<int64_t>(valid) * p.lda * 2), p.lda, slot, wave, lane, l);
      } else {
        constexpr int q = l - LM;
        const char* base = static_cast<const char*>(p.b0) + (static_cast<int64_t>(k0) * p.ldb + tc.nt * BN) * 2;
        load_mnmajor<BN, W>(make_rsrc(base, static_cast<int64_t>(valid) * p.ldb * 2), p.ldb, slot + TILE_M, wave,
                            lane, q);
      }
    }
  };

  floatx16 acc[NB][MB];
  struct Frags {
    bf16x8 m[MB], n[NB];
  };
  auto read_frag = [&](const char* slotp, int kk, Frags& F, auto FI) {
    constexpr int fi = decltype(FI)::value;
    const char* tm = slotp;
    const char* tn = slotp + TILE_M;
    if constexpr (fi < MB) {
      if constexpr (M_MN) F.m[fi] = frag_mnmajor<BM>(tm, wm * WM + fi * 32, kk, lane);
      else F.m[fi] = frag_kmajor(tm, wm * WM + fi * 32, kk, lane);
    } else {
      F.n[fi - MB] = frag_mnmajor<BN>(tn, wn * WN + (fi - MB) * 32, kk, lane);
    }
  };
  auto read_frags = [&](const char* slotp, int kk, Frags& F) {
    static_for<MB + NB>([&](auto FI) { read_frag(slotp, kk, F, FI); });
  };
  auto mfma_one = [&](const Frags& F, auto MI) {
    constexpr int mi = decltype(MI)::value, j = mi / MB, i = mi % MB;
    acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.n[j], F.m[i], acc[j][i], 0, 0, 0);
  };
  constexpr int kReads = MB * (M_MN ? 2 : 1) + NB * 2;
  constexpr int kMfma = MB * NB;
  constexpr int kFrags = MB + NB;
  auto interleave = [&]() {
    constexpr int inter = kReads < kMfma ? kReads : kMfma;
#pragma unroll
    for (int r = 0; r < inter; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (kReads > kMfma) __builtin_amdgcn_sched_group_barrier(0x100, kReads - kMfma, 0);
    if constexpr (kMfma > kReads) __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kReads, 0);
  };

  // ---- epilogue: this wave's 128 x 128 block through its 8 KB staging tile ----------------
  char* const wa = smem + RING + wave * kStg;
  const int hl = lane >> 5, l32 = lane & 31;
  auto st_off = [](int r, int col) { return r * 128 + ((((col >> 3) ^ (r >> 1)) & 7) << 4) + ((col & 4) << 1); };
  auto put4 = [&](int r, int col, uint2 v) { *reinterpret_cast<uint2*>(wa + st_off(r, col)) = v; };
  auto wave_sync = [&]() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
  };
  // Staging rows [0, 64) -> global rows g + r * ld for r < rows (8 buffer stores).
  auto flush = [&](const char* g, int64_t ld, int rows) {
    __builtin_amdgcn_sched_barrier(0);
    wave_sync();
    const auto rs = make_rsrc(g, static_cast<int64_t>(max(0, min(64, rows))) * ld);
    const int c = lane & 7;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int r = t * 8 + (lane >> 3);
      typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 v = *reinterpret_cast<const u32x4*>(wa + r * 128 + ((c ^ (r >> 1)) & 7) * 16);
      __builtin_amdgcn_raw_buffer_store_b128(v, rs, static_cast<uint32_t>(r * ld + c * 16), 0, kStoreNT);
    }
    wave_sync();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto acc4 = [&](int j, int i, int q) {
    return pack4(acc[j][i][4 * q], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2], acc[j][i][4 * q + 3]);
  };
  auto epilogue = [&](const TileCoord& tc) {
    const int64_t ld = p.ldc * 2;
    const char* out;
    int rows;
    if constexpr (MODE == FWD_DOWN) {
      const int mrow = tc.row0 + wm * WM;
      rows = tc.row_end - mrow;  // may be <= 0 or > WM: flush clamps
      out = static_cast<const char*>(p.c0) + (static_cast<int64_t>(mrow) * p.ldc + tc.nt * BN + wn * WN) * 2;
    } else {
      // dW[e] rows m0.., columns n0..; columns >= f of the gate|up gradient
      // go to the second output (dw_up).
      const char* base = static_cast<const char*>(p.c0);
      int cn0 = tc.nt * BN;
      if (p.c1 != nullptr && cn0 >= p.f) { base = static_cast<const char*>(p.c1); cn0 -= p.f; }
      rows = WM;
      out = base + (static_cast<int64_t>(tc.e) * p.cstride +
                    static_cast<int64_t>(tc.m0 + wm * WM) * p.ldc + cn0 + wn * WN) * 2;
    }
    static_for<2>([&](auto JP) {
      static_for<2>([&](auto HH) {
        constexpr int h = decltype(HH)::value;
        static_for<2>([&](auto II) {
          static_for<2>([&](auto JJ) {
            static_for<4>([&](auto Q) {
              put4(II * 32 + l32, JJ * 32 + 8 * Q + 4 * hl, acc4(JP * 2 + JJ, 2 * h + II, Q));
            });
          });
        });
        flush(out + static_cast<int64_t>(h) * 64 * ld + JP * 128, ld, rows - 64 * h);
      });
    });
  };

  // ---- the slab stream ------------------------------------------------------------------
  // Load side: tile index lj, its slab lkt and slab count lnk (tiles without
  // slabs are skipped here; they still get their epilogue below).
  int lj = 0, lkt = 0;
  TileCoord ltc = tile_at(0);
  int lnk = slabs_of(ltc);
  auto skip_empty = [&]() {
    while (lkt >= lnk && lj < ntiles) {
      lkt = 0;
      if (++lj < ntiles) {
        ltc = tile_at(lj);
        lnk = slabs_of(ltc);
      }
    }
  };
  skip_empty();
  auto advance = [&]() {
    ++lkt;
    skip_empty();
  };
  // Epilogues issued after the loads of slabs g+1, g+2, g+3 (g: the slab
  // being multiplied).
  int ep1 = 0, ep2 = 0, ep3 = 0;
  const uint32_t ring = __builtin_amdgcn_readfirstlane(lds_addr(smem));
#pragma unroll
  for (int s0 = 0; s0 < kStages; ++s0) {
    static_for<kLoads>([&](auto L) { issue(ltc, lkt, lj < ntiles, ring + s0 * STAGE, L, std::integral_constant<int, 4>{}); });
    advance();
  }
  Frags F[2];
  wait_vmcnt<kLoads * (kStages - 1)>();
  __syncthreads();
  read_frags(smem, 0, F[0]);
  int gk = 0;  // slabs consumed: slab gk sits in slot gk % kStages
  for (int j = 0; j < ntiles; ++j) {
    const TileCoord cur = tile_at(j);
    const int nk = slabs_of(cur);
#pragma unroll
    for (int jj = 0; jj < NB; ++jj)
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[jj][i][r] = 0.0f;
    for (int kt = 0; kt < nk; ++kt, ++gk) {
      const int sc = gk % kStages;
      const char* curp = smem + sc * STAGE;
      const char* nxtp = smem + ((gk + 1) % kStages) * STAGE;
      read_frags(curp, 1, F[1]);
      static_for<kMfma>([&](auto MI) { mfma_one(F[0], MI); });
      interleave();
      if (ep1 == 0) wait_vmcnt<kWait0>();
      else if (ep1 == 1) wait_vmcnt<kWait1>();
      else wait_vmcnt<63>();
      __syncthreads();
      const uint32_t slot = ring + sc * STAGE;
      const bool live = lj < ntiles;
      static_for<kLoads>([&](auto S) {
        constexpr int sg = decltype(S)::value;
        constexpr int m_lo = sg * kMfma / kLoads, m_hi = (sg + 1) * kMfma / kLoads;
        constexpr int f_lo = sg * kFrags / kLoads, f_hi = (sg + 1) * kFrags / kLoads;
        static_for<m_hi - m_lo>([&](auto D) { mfma_one(F[1], std::integral_constant<int, m_lo + decltype(D)::value>{}); });
        static_for<f_hi - f_lo>([&](auto D) { read_frag(nxtp, 0, F[0], std::integral_constant<int, f_lo + decltype(D)::value>{}); });
        issue(ltc, lkt, live, slot, S, std::integral_constant<int, 0>{});
        __builtin_amdgcn_sched_barrier(0);
      });
      advance();
      ep1 = ep2; ep2 = ep3; ep3 = 0;  // slab gk+4 was just issued
    }
    // F[0] already holds the first fragments of the next tile with slabs
    // (read during the last slab), whose slot is not refilled before the next
    // barrier.
    epilogue(cur);
    ++ep1; ++ep2; ++ep3;
  }
  // Drain the (empty) loads and the stores still in flight before the wave ends.
  wait_vmcnt<0>();
}

int round8(int64_t g) { return static_cast<int>((g + 7) / 8 * 8); }

// The quarter tiles of a launch whose tile list ends in a short round
// (p.tail = 1): at most p.cus workgroups.
template <int MODE, int BM, int BN>
hipError_t launch_tail(const GemmParams& p, int grid, hipStream_t s) {
  constexpr int ring = kStages * (BM + BN) * kBK * 2, stage = 4 * 2 * (BM / 2) * 128;
  constexpr int lds = ring > stage ? ring : stage;
  auto kern = gg_bf16_kernel<MODE, BM, BN>;
  static std::atomic<int> attr{0};
  if (attr.load() == 0) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (err != hipSuccess) return err;
    attr.store(1);
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, s, p);
  return hipGetLastError();
}

// The streaming kernel on as many workgroups as run at once (WGRAD: at most
// one per tile); for FWD_DOWN then the quarter tiles of its short last round
// (both launches split the tile list with the same p.cus).
template <int MODE>
hipError_t launch_stream(GemmParams p, int tiles, hipStream_t s) {
  constexpr int lds = kStages * (256 + 256) * kBK * 2 + 4 * 64 * 128;
  auto kern = gg_bf16_stream_kernel<MODE>;
  static std::atomic<int> per_cu{0};
  if (per_cu.load() == 0) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (err != hipSuccess) return err;
    int n = 0;
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(kern), 256, lds);
    if (err != hipSuccess) return err;
    per_cu.store(n > 0 ? n : 1);
  }
  const int cap = max(8, device_cu_count() * per_cu.load() / 8 * 8);
  if constexpr (MODE == WGRAD) {
    hipLaunchKernelGGL(kern, dim3(min(cap, round8(tiles))), dim3(256), lds, s, p);
    return hipGetLastError();
  } else {
    p.cus = cap;
    p.tail = 0;
    hipLaunchKernelGGL(kern, dim3(cap), dim3(256), lds, s, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    p.tail = 1;
    return launch_tail<MODE, 128, 128>(p, cap, s);
  }
}

template <int MODE, int BM, int BN>
hipError_t launch_tile(const GemmParams& p0, int tiles, hipStream_t s) {
  // The ring, reused by the epilogue's per-wave staging (4 waves x 2 tiles of
  // (BM/2) x 64 bf16).
  constexpr int ring = kStages * (BM + BN) * kBK * 2, stage = 4 * 2 * (BM / 2) * 128;
  constexpr int lds = ring > stage ? ring : stage;
  auto kern = gg_bf16_kernel<MODE, BM, BN>;
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
  const int cap = max(8, device_cu_count() * per_cu.load() / 8 * 8);
  if constexpr (MODE == WGRAD) {
    // A persistent grid: as many workgroups as run at once (a multiple of 8:
    // one share per XCD). 256 x 256 tiles stream their slabs when experts
    // average under 512 rows (16 slabs per tile); with longer tiles the
    // stream's bookkeeping costs more than the tile turnover it hides
    // (measured: -9% at 256 rows per expert, +5% at 4096 and on the Zipf
    // layer's hot experts).
    if constexpr (BM == 256 && BN == 256) {
      if (static_cast<int64_t>(p0.S) < 512LL * p0.E) return launch_stream<WGRAD>(p0, tiles, s);
    }
    hipLaunchKernelGGL(kern, dim3(min(cap, round8(tiles))), dim3(256), lds, s, p0);
    return hipGetLastError();
  } else {
    // One workgroup per tile of the count-free bound (the surplus exits at
    // once), or the streaming kernel. The full-size tiles leave a short last
    // round to quarter tiles (see RowTileMap): a second launch of the
    // half-size kernel.
    constexpr bool kQuarters = (BM == 256 && BN == 256);
    GemmParams p = p0;
    p.cus = kQuarters ? cap : 0;
    p.tail = 0;
    if constexpr (kQuarters && MODE == FWD_DOWN) {
      if (p.K / kBK >= kStages) return launch_stream<MODE>(p, 0, s);
    }
    hipLaunchKernelGGL(kern, dim3(round8(tiles)), dim3(256), lds, s, p);
    hipError_t err = hipGetLastError();
    if constexpr (kQuarters) {
      if (err == hipSuccess) {
        p.tail = 1;
        err = launch_tail<MODE, BM / 2, BN / 2>(p, cap, s);
      }
    }
    return err;
  }
}

// Grid bound for row-ragged modes: sum_e ceil(n_e/BM) <= ceil(S/BM) + E.
int ragged_grid(int S, int E, int BM, int NT) {
  return round8((static_cast<int64_t>((S + BM - 1) / BM) + E) * NT);
}

template <int MODE, int BM>
hipError_t ragged_bn(const GemmParams& p, hipStream_t s) {
  if (p.N % 256 == 0) return launch_tile<MODE, BM, 256>(p, ragged_grid(p.S, p.E, BM, p.N / 256), s);
  if (p.N % 128 == 0) return launch_tile<MODE, BM, 128>(p, ragged_grid(p.S, p.E, BM, p.N / 128), s);
  // N only a multiple of 64: narrow tiles (small shapes). FWD_GU has N = 2f,
  // always a multiple of 128.
  if constexpr (MODE != FWD_GU) return launch_tile<MODE, 128, 64>(p, ragged_grid(p.S, p.E, 128, p.N / 64), s);
  return hipErrorInvalidValue;
}

template <int MODE>
hipError_t ragged_mode(const GemmParams& p, hipStream_t s) {
  if (static_cast<int64_t>(p.S) >= 1024LL * p.E) return ragged_bn<MODE, 256>(p, s);
  // Under 512 rows per expert on average: 128-row tiles, which waste less on
  // short experts (measured: the split below costs 7% at 256 rows per expert).
  if (static_cast<int64_t>(p.S) < 512LL * p.E) return ragged_bn<MODE, 128>(p, s);
  // 512 to 1023 rows per expert on average, where loads are usually skewed:
  // the whole 256-row bands of the experts that have them in 256-row tiles,
  // the rest of every expert in 128-row tiles, which waste less on a short
  // remainder (measured on a Zipf-routed layer: row-ragged steps -12%).
  GemmParams q = p;
  q.band = 1;
  hipError_t err = ragged_bn<MODE, 256>(q, s);
  if (err != hipSuccess) return err;
  q.band = 2;
  return ragged_bn<MODE, 128>(q, s);
}

}  // namespace

hipError_t launch_bf16_ragged(int mode, const GemmParams& p, hipStream_t s) {
  switch (mode) {
    case FWD_GU: {
      // A 256-wide tile holds 128 gate + 128 up columns: needs f % 128 == 0.
      if (p.f % 128 == 0) return ragged_mode<FWD_GU>(p, s);
      if (static_cast<int64_t>(p.S) >= 1024LL * p.E)
        return launch_tile<FWD_GU, 256, 128>(p, ragged_grid(p.S, p.E, 256, p.N / 128), s);
      return launch_tile<FWD_GU, 128, 128>(p, ragged_grid(p.S, p.E, 128, p.N / 128), s);
    }
    case FWD_DOWN: return ragged_mode<FWD_DOWN>(p, s);
    case BWD_DOWN: return ragged_mode<BWD_DOWN>(p, s);
    case BWD_GU: return ragged_mode<BWD_GU>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bf16_wgrad(const GemmParams& p, hipStream_t s) {
  // A column tile must not straddle the gate|up split at column f.
  const int nsplit = p.c1 ? p.f : p.N;
  const bool m256 = p.M % 256 == 0, n256 = p.N % 256 == 0 && nsplit % 256 == 0;
  const bool m128 = p.M % 128 == 0, n128 = p.N % 128 == 0 && nsplit % 128 == 0;
  auto grid = [&](int bm, int bn) { return round8(static_cast<int64_t>(p.E) * (p.M / bm) * (p.N / bn)); };
  if (m256 && n256) return launch_tile<WGRAD, 256, 256>(p, grid(256, 256), s);
  if (m256 && n128) return launch_tile<WGRAD, 256, 128>(p, grid(256, 128), s);
  if (m128 && n256) return launch_tile<WGRAD, 128, 256>(p, grid(128, 256), s);
  if (m128 && n128) return launch_tile<WGRAD, 128, 128>(p, grid(128, 128), s);
  // Dimensions only multiples of 64: narrow tiles (small shapes).
  if (m128) return launch_tile<WGRAD, 128, 64>(p, grid(128, 64), s);
  if (n128) return launch_tile<WGRAD, 64, 128>(p, grid(64, 128), s);
  return launch_tile<WGRAD, 64, 64>(p, grid(64, 64), s);
}

}  // namespace moe
