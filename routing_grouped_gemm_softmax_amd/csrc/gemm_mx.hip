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
    const int nk = __builtin_amdgcn_readfirstlane((MODE == WGRAD) ? (row_end - row0) / 64 : p.K / 64);
    const int64_t bexp = static_cast<int64_t>(e) * p.bstride;
    const int64_t bsexp = static_cast<int64_t>(e) * p.bs_estride;
    const uint8_t* A = static_cast<const uint8_t*>(p.a);
    const uint8_t* B0 = static_cast<const uint8_t*>(p.b0);
    const uint8_t* B1 = static_cast<const uint8_t*>(p.b1);

    // ---- HBM -> LDS for slab kt ------------------------------------------------------------
    // Each wave issues kLoads loads per slab: [0, LM) the M tile, [LM, LM + LN)
    // the N tile, then one 1 KB scale load: wave 0 the M side's scales, wave 1
    // the N side's (the gate half for FWD_GU), wave 2 the up half's for FWD_GU;
    // the remaining waves load nothing into their own area, so every wave
    // issues the same count (the vmcnt waits count them).
    constexpr int LM = BM / 64, LN = BN / 64, kLoads = LM + LN + 1;
    // The tile's descriptors from its first k: the A rows, the B rows (FWD_GU
    // and BWD_GU: both sources, FWD_GU's as two half tiles) and the scale rows'
    // bases at slab 0. A slab only adds its k offset to each lane's offset
    // within the tile and moves the scale bases by whole slabs; slabs at or
    // past the end load from the empty descriptor.
    constexpr int BR = MODE == FWD_GU ? BN / 2 : BN;  // rows per B source
    constexpr int LB = BR / 64;                       // loads per B source
    const __amdgpu_buffer_rsrc_t r0 = make_rsrc(p.as, 0);
    __amdgpu_buffer_rsrc_t ra, rb, rb1 = r0;
    const uint8_t *sa, *sb, *sb1 = nullptr;
    int sa_n;
    if constexpr (MODE == WGRAD) {
      ra = make_rsrc(A + m0 * p.lda + row0, BM * p.lda);
      rb = make_rsrc(B0 + n0 * p.ldb + row0, BN * p.ldb);
      sa = p.as + static_cast<int64_t>(row0 / 64) * p.as_slab + m0 * 2;
      sb = p.bs0 + static_cast<int64_t>(row0 / 64) * p.bs_slab + n0 * 2;
      sa_n = BM * 2;
    } else {
      const int valid = min(BM, row_end - row0);
      ra = make_rsrc(A + static_cast<int64_t>(row0) * p.lda, static_cast<int64_t>(valid) * p.lda);
      sa = p.as + row0 * 2;
      // Whole dwords: an odd row count keeps its last row's scales (the extra
      // bytes are the scales of a row whose data reads as zero).
      sa_n = (valid * 2 + 3) & ~3;
      const int nb = MODE == FWD_GU ? nt * BR : n0;
      const int64_t boff = bexp + static_cast<int64_t>(nb) * p.ldb;
      rb = make_rsrc(B0 + boff, static_cast<int64_t>(BR) * p.ldb);
      sb = p.bs0 + bsexp + nb * 2;
      if constexpr (MODE == FWD_GU || MODE == BWD_GU) {
        rb1 = make_rsrc(B1 + boff, static_cast<int64_t>(BR) * p.ldb);
        sb1 = p.bs1 + bsexp + nb * 2;
      }
    }
    // Each lane's byte offset within a tile for load q: row (q * 4 + wave) *
    // 16 + lane / 4, its 16-byte chunk lane % 4 swizzled by the row.
    uint32_t voa[LM], vob[LB];
#pragma unroll
    for (int q = 0; q < LM; ++q) {
      const int row = (q * 4 + wave) * 16 + (lane >> 2);
      voa[q] = static_cast<uint32_t>(row * p.lda + (((lane & 3) ^ swz_row(row)) << 4));
    }
#pragma unroll
    for (int q = 0; q < LB; ++q) {
      const int row = (q * 4 + wave) * 16 + (lane >> 2);
      vob[q] = static_cast<uint32_t>(row * p.ldb + (((lane & 3) ^ swz_row(row)) << 4));
    }
    // W: wait states of the loads (load_lds16): 4 where a descriptor may have
    // just been written by a VALU instruction, 0 in the steady-state loop.
    // A slab at or past the end moves every lane's offset past any buffer's
    // range (descriptors hold at most 2^31 - 1 bytes), so it reads nothing.
    constexpr uint32_t kDead = 0x80000000u;
    auto issue = [&](int kt, uint32_t slot, auto L, auto w) {
      constexpr int l = decltype(L)::value, W = decltype(w)::value;
      const bool live = kt < nk;
      const uint32_t kofs = live ? static_cast<uint32_t>(kt * 64) : kDead;
      if constexpr (l < LM) {
        load_lds16<W>(ra, voa[l] + kofs, slot + (l * 4 + wave) * 16 * 64);
      } else if constexpr (l < LM + LN) {
        constexpr int q = l - LM;
        const uint32_t tn = slot + TILE_M;
        if constexpr (MODE == FWD_GU) {
          constexpr int half = q / LB, qq = q % LB;
          load_lds16<W>(half ? rb1 : rb, vob[qq] + kofs, tn + half * (TILE_N / 2) + (qq * 4 + wave) * 16 * 64);
        } else if constexpr (MODE == BWD_GU) {
          const bool second = kt * 64 >= p.f;
          const uint32_t bofs = live ? static_cast<uint32_t>((second ? kt - p.f / 64 : kt) * 64) : kDead;
          load_lds16<W>(second ? rb1 : rb, vob[q] + bofs, tn + (q * 4 + wave) * 16 * 64);
        } else {
          load_lds16<W>(rb, vob[q] + kofs, tn + (q * 4 + wave) * 16 * 64);
        }
      } else {
        const uint32_t sc = slot + TILE_M + TILE_N + wave * kScaleArea;
        const uint32_t voff = static_cast<uint32_t>(lane * 16);
        if (wave == 0) {
          load_lds16<W>(make_rsrc(sa + static_cast<int64_t>(kt) * p.as_slab, live ? sa_n : 0), voff, sc);
        } else if (wave == 1 || (wave == 2 && MODE == FWD_GU)) {
          const uint8_t* ssrc = sb + static_cast<int64_t>(kt) * p.bs_slab;
          if constexpr (MODE == FWD_GU) {
            if (wave == 2) ssrc = sb1 + static_cast<int64_t>(kt) * p.bs_slab;
          } else if constexpr (MODE == BWD_GU) {
            if (kt * 64 >= p.f) ssrc = sb1 + static_cast<int64_t>(kt - p.f / 64) * p.bs_slab;
          }
          load_lds16<W>(make_rsrc(ssrc, live ? BR * 2 : 0), voff, sc);
        } else {
          load_lds16<W>(r0, voff, sc);
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


// FWD_DOWN, BWD_GU and the weight gradients with 256 x 256 tiles as a
// persistent grid that streams slabs across tiles (one workgroup per CU):
// each workgroup owns a strided share of its XCD's tile range (the ragged
// modes: lo, lo + wpx, ...; WGRAD: the range wgrad_sched gives it) and its
// ring never drains between tiles. The loads of the next tile's first slabs
// go out during the current tile's last slabs, and the epilogue (bf16
// outputs, staged through a per-wave 4 KB LDS area beside the ring and
// written with range-checked buffer stores) runs while they fly. With one
// tile per workgroup every CU reached its epilogue at the same moment, so the
// stores of all of them ran as one burst with the matrix cores idle.
//
// LDS: 4 ring slots of [A 256 x 64 B | B 256 x 64 B | A scales 1 KB | B
// scales 1 KB] (scale loads: wave 0 the A side, wave 1 the B side; waves 2
// and 3 issue a zero-range load into a shared dump area, so that every wave
// issues the same count), then the staging areas, then the dump area.
//
// Wait counts: vmcnt counts loads and stores together, in issue order. The
// wait for slab g+1 must allow exactly the operations issued after that
// slab's loads: the loads of slabs g+2 and g+3, and kEpiStores stores for
// each epilogue since (every epilogue issues exactly that many). Past one
// epilogue the count exceeds 63 and the wait asks for 63, which only waits
// longer.
constexpr int kStreamStages = 4;
constexpr int kStoreNT = 2;  // buffer store cache policy bits: nt (non-temporal)
constexpr int kStreamStage = 256 * 64 * 2 + 2 * kScaleArea;
constexpr int kStreamStg = 32 * 128;  // per-wave staging: 32 rows x 64 bf16
constexpr int kStreamLds = kStreamStages * kStreamStage + 4 * kStreamStg + kScaleArea;

template <int MODE>
__global__ __launch_bounds__(256) void gg_mx_stream_kernel(GemmParams p) {
  constexpr int BM = 256, BN = 256, WM = 128, WN = 128, MB = 4, NB = 4;
  static_assert(MODE == FWD_DOWN || MODE == BWD_GU || MODE == WGRAD, "streaming modes");
  constexpr int TILE_M = BM * 64, TILE_N = BN * 64;
  constexpr int STAGE = kStreamStage;
  constexpr int RING = kStreamStages * STAGE;
  constexpr int kEpiStores = 8 * 4;  // 8 flushes of 4 stores
  constexpr int LM = BM / 64, LN = BN / 64, kLoads = LM + LN + 1;
  constexpr int kWait0 = kLoads * (kStreamStages - 2);
  constexpr int kWait1 = kWait0 + kEpiStores < 63 ? kWait0 + kEpiStores : 63;
  static_assert(kStreamStages == 4, "epilogue accounting written for slabs g+1..g+3 in flight");
  static_assert(kStreamLds <= 160 * 1024, "LDS");

  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // ---- this workgroup's tiles ------------------------------------------------------------
  RowTileMap map;
  int lo, step, ntiles;
  if constexpr (MODE != WGRAD) {
    map.init(p, BM, BN, lane);
    const int R = map.tiles();
    const int x = blockIdx.x % 8, wpx = gridDim.x / 8;
    lo = xcd_cut(R, x) + blockIdx.x / 8;
    const int hi = xcd_cut(R, x + 1);
    step = wpx;
    ntiles = lo < hi ? (hi - lo + wpx - 1) / wpx : 0;
  } else {
    int* s_info = reinterpret_cast<int*>(smem + RING);  // a staging area, free until the first epilogue
    wgrad_sched<BM, BN, 64, kEpiWorkX>(p, s_info, wave, lane);
    lo = __builtin_amdgcn_readfirstlane(s_info[0]);
    const int hi = __builtin_amdgcn_readfirstlane(s_info[1]);
    step = __builtin_amdgcn_readfirstlane(s_info[2]);
    ntiles = lo < hi ? (hi - lo + step - 1) / step : 0;
    __syncthreads();  // s_info is read out before any wave stages there
  }
  if (ntiles == 0) return;
  auto tile_at = [&](int j) -> TileCoord {
    if constexpr (MODE != WGRAD) return map.at(lo + j * step, lane);
    else return wgrad_tile<BM, BN>(p, lo + j * step);
  };
  // WGRAD: [row0, row_end) is the expert's padded K range (a multiple of 64).
  auto slabs_of = [&](const TileCoord& tc) -> int {
    if constexpr (MODE == WGRAD) return (tc.row_end - tc.row0) / 64;
    else return p.K / 64;
  };
  const uint8_t* A = static_cast<const uint8_t*>(p.a);
  const uint32_t dump = __builtin_amdgcn_readfirstlane(lds_addr(smem + RING + 4 * kStreamStg));

  // ---- HBM -> LDS ------------------------------------------------------------------------
  // The load side's tile keeps its buffer descriptors from the tile's first k
  // (empty once past the last tile): the A rows, the B rows (BWD_GU: both
  // sources), and the scale rows' bases at slab 0. A slab then only adds its
  // k offset to each lane's offset within the tile (row * ld + 16-byte chunk,
  // fixed for the kernel) and moves the scale bases by whole slabs, instead
  // of rebuilding every descriptor for every load.
  struct LoadTile {
    __amdgpu_buffer_rsrc_t ra, rb, rb1;  // rb1: BWD_GU's second source only
    const uint8_t* sa;   // A scales at slab 0
    const uint8_t* sb;   // B scales at slab 0 (BWD_GU: the first source's)
    const uint8_t* sb1;  // BWD_GU: the second source's at its slab 0
    int sa_n, sb_n;
  };
  auto load_tile = [&](const TileCoord& tc, bool live) -> LoadTile {
    LoadTile t{};
    const int n0 = tc.nt * BN;
    const uint8_t* B0 = static_cast<const uint8_t*>(p.b0);
    if constexpr (MODE == WGRAD) {
      t.ra = make_rsrc(A + tc.m0 * p.lda + tc.row0, live ? BM * p.lda : 0);
      t.rb = make_rsrc(B0 + n0 * p.ldb + tc.row0, live ? BN * p.ldb : 0);
      t.sa = p.as + static_cast<int64_t>(tc.row0 / 64) * p.as_slab + tc.m0 * 2;
      t.sb = p.bs0 + static_cast<int64_t>(tc.row0 / 64) * p.bs_slab + n0 * 2;
      t.sa_n = live ? BM * 2 : 0;
      t.sb_n = live ? BN * 2 : 0;
    } else {
      const int valid = live ? min(BM, tc.row_end - tc.row0) : 0;
      t.ra = make_rsrc(A + static_cast<int64_t>(tc.row0) * p.lda, static_cast<int64_t>(valid) * p.lda);
      const int64_t boff = static_cast<int64_t>(tc.e) * p.bstride + static_cast<int64_t>(n0) * p.ldb;
      t.rb = make_rsrc(B0 + boff, live ? static_cast<int64_t>(BN) * p.ldb : 0);
      t.sa = p.as + tc.row0 * 2;
      t.sb = p.bs0 + static_cast<int64_t>(tc.e) * p.bs_estride + n0 * 2;
      if constexpr (MODE == BWD_GU) {
        t.rb1 = make_rsrc(static_cast<const uint8_t*>(p.b1) + boff, live ? static_cast<int64_t>(BN) * p.ldb : 0);
        t.sb1 = p.bs1 + static_cast<int64_t>(tc.e) * p.bs_estride + n0 * 2;
      }
      // Whole dwords: an odd row count keeps its last row's scales.
      t.sa_n = (valid * 2 + 3) & ~3;
      t.sb_n = live ? BN * 2 : 0;
    }
    return t;
  };
  // Rows are interleaved inside each wave's 128-row block: LDS row L (the
  // rows fragment (L / 32) % 4 reads, lane L % 32) holds tile row
  // inter_row(L), so fragment f of a wave covers rows f, f + 4, f + 8, ...
  // of its block and a lane's four fragments are four consecutive rows. Their
  // eight scale bytes (two 32-blocks each) are then adjacent in the scale
  // tile, one 8-byte LDS read per side, and each MFMA picks its byte with
  // the scale operand's byte select. The epilogue writes accumulator row
  // (column) c of fragment f to row (column) 4 c + f.
  auto inter_row = [](int L) { return (L & ~127) + 4 * (L & 31) + ((L >> 5) & 3); };
  // Each lane's byte offset within a tile for A and B load q: LDS row (q * 4
  // + wave) * 16 + lane / 4, its 16-byte chunk lane % 4 swizzled by that LDS
  // row, taken from tile row inter_row of it.
  uint32_t voa[LM], vob[LN];
#pragma unroll
  for (int q = 0; q < LM; ++q) {
    const int row = (q * 4 + wave) * 16 + (lane >> 2);
    voa[q] = static_cast<uint32_t>(inter_row(row) * p.lda + (((lane & 3) ^ swz_row(row)) << 4));
  }
#pragma unroll
  for (int q = 0; q < LN; ++q) {
    const int row = (q * 4 + wave) * 16 + (lane >> 2);
    vob[q] = static_cast<uint32_t>(inter_row(row) * p.ldb + (((lane & 3) ^ swz_row(row)) << 4));
  }

  // Load L of slab kt of the load tile lt.
  auto issue = [&](const LoadTile& lt, int kt, uint32_t slot, auto L, auto w) {
    constexpr int l = decltype(L)::value, W = decltype(w)::value;
    if constexpr (l < LM) {
      load_lds16<W>(lt.ra, voa[l] + static_cast<uint32_t>(kt * 64), slot + (l * 4 + wave) * 16 * 64);
    } else if constexpr (l < LM + LN) {
      constexpr int q = l - LM;
      const uint32_t dst = slot + TILE_M + (q * 4 + wave) * 16 * 64;
      if constexpr (MODE == BWD_GU) {
        const bool second = kt * 64 >= p.f;
        load_lds16<W>(second ? lt.rb1 : lt.rb, vob[q] + static_cast<uint32_t>((second ? kt - p.f / 64 : kt) * 64),
                      dst);
      } else {
        load_lds16<W>(lt.rb, vob[q] + static_cast<uint32_t>(kt * 64), dst);
      }
    } else {
      const uint32_t voff = static_cast<uint32_t>(lane * 16);
      if (wave == 0) {
        load_lds16<W>(make_rsrc(lt.sa + static_cast<int64_t>(kt) * p.as_slab, lt.sa_n), voff,
                      slot + TILE_M + TILE_N);
      } else if (wave == 1) {
        const uint8_t* sb = lt.sb + static_cast<int64_t>(kt) * p.bs_slab;
        if constexpr (MODE == BWD_GU) {
          if (kt * 64 >= p.f) sb = lt.sb1 + static_cast<int64_t>(kt - p.f / 64) * p.bs_slab;
        }
        load_lds16<W>(make_rsrc(sb, lt.sb_n), voff, slot + TILE_M + TILE_N + kScaleArea);
      } else {
        load_lds16<W>(make_rsrc(p.as, 0), voff, dump);
      }
    }
  };

  floatx16 acc[NB][MB];
  struct Frags {
    v8i m[MB], n[NB];
    int sm[2], sn[2];  // fragment f's scale: byte 2 (f % 2) of word f / 2
  };
  // Fragment FI; with the first fragment of a side also that side's scales:
  // the 8 bytes of the lane's four interleaved rows, shifted so that the
  // lane's 32-block (lane / 32) sits in the even bytes.
  auto read_frag = [&](const char* slotp, Frags& F, auto FI) {
    constexpr int fi = decltype(FI)::value;
    const uint8_t* sc = reinterpret_cast<const uint8_t*>(slotp + TILE_M + TILE_N);
    const int r32 = lane & 31;
    const uint32_t kb8 = static_cast<uint32_t>(lane >> 5) * 8;
    if constexpr (fi < MB) {
      F.m[fi] = frag_mx(slotp, wm * WM + fi * 32, lane);
      if constexpr (fi == 0) {
        const uint64_t v = *reinterpret_cast<const uint64_t*>(sc + (wm * WM + 4 * r32) * 2) >> kb8;
        F.sm[0] = static_cast<int>(v);
        F.sm[1] = static_cast<int>(v >> 32);
      }
    } else {
      constexpr int j = fi - MB;
      F.n[j] = frag_mx(slotp + TILE_M, wn * WN + j * 32, lane);
      if constexpr (j == 0) {
        const uint64_t v = *reinterpret_cast<const uint64_t*>(sc + kScaleArea + (wn * WN + 4 * r32) * 2) >> kb8;
        F.sn[0] = static_cast<int>(v);
        F.sn[1] = static_cast<int>(v >> 32);
      }
    }
  };
  auto mfma_one = [&](const Frags& F, auto MI) {
    constexpr int mi = decltype(MI)::value, j = mi / MB, i = mi % MB;
    acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.n[j], F.m[i], acc[j][i], 0, 0, 2 * (j % 2),
                                                               F.sn[j / 2], 2 * (i % 2), F.sm[i / 2]);
  };
  constexpr int kMfma = MB * NB, kFrags = MB + NB;

  // ---- epilogue: this wave's 128 x 128 block through its 4 KB staging tile ----------------
  char* const wa = smem + RING + wave * kStreamStg;
  const int hl = lane >> 5, l32 = lane & 31;
  auto st_off = [](int r, int col) { return r * 128 + ((((col >> 3) ^ (r >> 1)) & 7) << 4) + ((col & 4) << 1); };
  auto put4 = [&](int r, int col, uint2 v) { *reinterpret_cast<uint2*>(wa + st_off(r, col)) = v; };
  auto wave_sync = [&]() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
  };
  // Staging rows [0, 32) -> rows 4 r + I of the wave's block, whose first
  // row (at this column half) is g, for rows below `rows` (4 buffer stores,
  // non-temporal: the outputs are written once and read by a later kernel,
  // and the stores complete sooner without allocating in the L2, which
  // matters because the next slabs' waits count them).
  auto flush = [&](const char* g, int64_t ld, int I, int rows) {
    __builtin_amdgcn_sched_barrier(0);
    wave_sync();
    const auto rs = make_rsrc(g, static_cast<int64_t>(max(0, min(WM, rows))) * ld);
    const int c = lane & 7;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = t * 8 + (lane >> 3);
      typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 v = *reinterpret_cast<const u32x4*>(wa + r * 128 + ((c ^ (r >> 1)) & 7) * 16);
      __builtin_amdgcn_raw_buffer_store_b128(v, rs, static_cast<uint32_t>((4 * r + I) * ld + c * 16), 0, kStoreNT);
    }
    wave_sync();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto epilogue = [&](const TileCoord& tc) {
    const int64_t ld = p.ldc * 2;
    const char* out;
    int rows;
    if constexpr (MODE != WGRAD) {
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
      out = base + (static_cast<int64_t>(tc.e) * p.cstride + static_cast<int64_t>(tc.m0 + wm * WM) * p.ldc + cn0 +
                    wn * WN) * 2;
    }
    // Column half H of the wave's block: accumulator columns c (element r
    // of lane l: c = 8 (r / 4) + 4 (l / 32) + r % 4) in [16 H, 16 H + 16),
    // i.e. r in [8 H, 8 H + 8); the four fragments' values of one c are
    // the four adjacent columns 4 c .. 4 c + 3.
    static_for<2>([&](auto H) {
      static_for<MB>([&](auto I) {
        static_for<8>([&](auto R) {
          constexpr int r = 8 * H + R;
          const int c = 8 * (r / 4) + 4 * hl + r % 4;
          put4(l32, 4 * c - 64 * H, pack4(acc[0][I][r], acc[1][I][r], acc[2][I][r], acc[3][I][r]));
        });
        flush(out + H * 128, ld, I, rows);
      });
    });
  };

  // ---- the slab stream ------------------------------------------------------------------
  // Load side: tile index lj, its slab lkt and slab count lnk (tiles without
  // slabs are skipped here; they still get their epilogue below).
  int lj = 0, lkt = 0;
  TileCoord ltc = tile_at(0);
  int lnk = slabs_of(ltc);
  LoadTile lt = load_tile(ltc, true);
  auto skip_empty = [&]() {
    while (lkt >= lnk && lj < ntiles) {
      lkt = 0;
      if (++lj < ntiles) {
        ltc = tile_at(lj);
        lnk = slabs_of(ltc);
      }
      lt = load_tile(ltc, lj < ntiles);
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
  for (int s0 = 0; s0 < kStreamStages; ++s0) {
    static_for<kLoads>([&](auto L) { issue(lt, lkt, ring + s0 * STAGE, L, std::integral_constant<int, 4>{}); });
    advance();
  }
  // One slab: wait for slab gk+1, barrier, then slab gk's MFMAs on `cur` with
  // the reads of slab gk+1 into `nxt` and the loads of the stream's next slab
  // into slot gk spread between them.
  int gk = 0;  // slabs consumed: slab gk sits in slot gk % kStreamStages
  auto slab = [&](const Frags& cur, Frags& nxt) {
    if (ep1 == 0) wait_vmcnt<kWait0>();
    else if (ep1 == 1) wait_vmcnt<kWait1>();
    else wait_vmcnt<63>();
    __syncthreads();  // slot gk is read out; slab gk+1 is visible
    const int sc = gk % kStreamStages;
    const char* nxtp = smem + ((gk + 1) % kStreamStages) * STAGE;
    const uint32_t slot = ring + sc * STAGE;
    static_for<kLoads>([&](auto S) {
      constexpr int sg = decltype(S)::value;
      constexpr int m_lo = sg * kMfma / kLoads, m_hi = (sg + 1) * kMfma / kLoads;
      constexpr int f_lo = sg * kFrags / kLoads, f_hi = (sg + 1) * kFrags / kLoads;
      static_for<m_hi - m_lo>([&](auto D) { mfma_one(cur, std::integral_constant<int, m_lo + decltype(D)::value>{}); });
      static_for<f_hi - f_lo>([&](auto D) {
        read_frag(nxtp, nxt, std::integral_constant<int, f_lo + decltype(D)::value>{});
      });
      issue(lt, lkt, slot, S, std::integral_constant<int, 0>{});
      __builtin_amdgcn_sched_barrier(0);
    });
    advance();
    ep1 = ep2; ep2 = ep3; ep3 = 0;  // the stream's next slab was just issued
    ++gk;
  };
  Frags f0, f1;
  wait_vmcnt<kLoads * (kStreamStages - 1)>();
  __syncthreads();
  static_for<kFrags>([&](auto FI) { read_frag(smem, f0, FI); });
  for (int j = 0; j < ntiles; ++j) {
    const TileCoord cur = tile_at(j);
    const int nk = slabs_of(cur);
#pragma unroll
    for (int jj = 0; jj < NB; ++jj)
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[jj][i][r] = 0.0f;
    // Two register sets with fixed names (a runtime index would put them in
    // scratch memory): slab kt multiplies f0 for even kt, f1 for odd kt.
    for (int kt = 0; kt < nk; kt += 2) {
      slab(f0, f1);
      if (kt + 1 < nk) slab(f1, f0);
    }
    // The next slab's fragments (the next tile with slabs) are in f1 after an
    // odd slab count; its slot is not refilled before the next barrier.
    if (nk & 1) f0 = f1;
    epilogue(cur);
    ++ep1; ++ep2; ++ep3;
  }
  // Drain the (empty) loads and the stores still in flight before the wave ends.
  wait_vmcnt<0>();
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

template <int MODE>
hipError_t launch_stream(const GemmParams& p, hipStream_t s) {
  auto kern = gg_mx_stream_kernel<MODE>;
  static std::atomic<int> set{0};
  if (set.load() == 0) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, kStreamLds);
    if (err != hipSuccess) return err;
    set.store(1);
  }
  const int grid = max(8, device_cu_count() / 8 * 8);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), kStreamLds, s, p);
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
    if constexpr (MODE == FWD_DOWN || MODE == BWD_GU) {
      if (p.N % 256 == 0) return launch_stream<MODE>(p, s);
    }
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
  if (p.M % 256 == 0 && p.N % 256 == 0 && nsplit % 256 == 0) return launch_stream<WGRAD>(p, s);
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
