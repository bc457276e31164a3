// Parameters of the device-scheduled grouped GEMMs of the expert SwiGLU FFN,
// shared by the fp32 kernel (gemm.hip) and the bf16 kernel (gemm_bf16.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// FWD_GU   [G|U|H] = SwiGLU(xp W_gate, xp W_up)       rows ragged by expert
// FWD_DOWN o = H W_down                                rows ragged
// BWD_DOWN dGU = SwiGLU'(dO W_down^T; saved G, U)      rows ragged
// BWD_GU   dxp = [dG|dU] [W_gate|W_up]^T  (K = 2f)     rows ragged
// WGRAD    dW[e] = X_e^T Y_e                           K = rows of expert e
enum GemmMode { FWD_GU = 0, FWD_DOWN = 1, BWD_DOWN = 2, BWD_GU = 3, WGRAD = 4 };

struct GemmParams {
  const void* a;      // A operand
  int64_t lda;
  const void* b0;     // B operand (first source)
  const void* b1;     // second source (w_up for FWD_GU / BWD_GU)
  int64_t ldb;
  int64_t bstride;    // elements between experts in b0/b1 (0 for WGRAD)
  void* c0;           // outputs
  void* c1;
  void* c2;
  int64_t ldc;
  const void* e0;     // epilogue inputs (BWD_DOWN: saved G, U)
  const void* e1;
  const int32_t* offsets;
  int E, S;
  int M;              // WGRAD: rows of each weight gradient
  int N, K;           // logical N (FWD_GU: 2f) and K (ragged modes)
  int f;              // split point: FWD_GU/BWD_GU/WGRAD(gate|up)
  int64_t cstride;    // WGRAD: elements between experts in c0/c1
  // MXFP8 operands: a, b0, b1 hold E4M3 bytes (row strides lda, ldb in
  // bytes); their E8M0 scales are slab-major, 2 bytes (two blocks of 32) per
  // row per 64-k slab: scale(row, k) = s[(k / 64) * slab + row * 2 + (k / 32) % 2].
  const uint8_t* as;  // scales of a
  const uint8_t* bs0; // scales of b0
  const uint8_t* bs1; // scales of b1
  int64_t as_slab;    // bytes between slabs of as
  int64_t bs_slab;    // bytes between slabs of bs0/bs1
  int64_t bs_estride; // bytes between experts in bs0/bs1
  // Row-ragged modes: with cus > 0 (workgroups that run at once) the tiles
  // past the last full round are left to a second launch (tail = 1) of
  // half-height, half-width tiles; see RowTileMap.
  int cus;
  int tail;
  // Row-ragged modes: the rows of each expert a launch covers. 0: all of
  // them; 1: only its whole 256-row bands; 2: only the rows after those bands
  // (so a 256-row-tile launch with band 1 and a 128-row-tile launch with
  // band 2 together cover every row once).
  int band;
  // MXFP8 kernels, FWD_GU and BWD_DOWN: the epilogue also writes its bf16
  // output rows (H; dG | dU) as the next GEMM's K-major E4M3 operand, q [S][ld]
  // and slab-major scales (as p.as above, slab = mxs_slab bytes).
  uint8_t* mxq;
  uint8_t* mxs;
  int64_t mxq_ld;
  int64_t mxs_slab;
  // MXFP8 BWD_DOWN: the epilogue also writes dG | dU as the weight
  // gradient's token-major operand: codes tq [2f][tq_ld] (tq_ld = P, every
  // expert's rows padded to a multiple of 64 starting at poff[e]) and
  // slab-major scales ts (ts_slab bytes per 64 tokens: 2 per channel).
  uint8_t* tq;
  uint8_t* ts;
  int64_t tq_ld;
  int64_t ts_slab;
  const int32_t* poff;
};

// bf16 grouped GEMMs (gemm_bf16.hip).
hipError_t launch_bf16_ragged(int mode, const GemmParams& p, hipStream_t s);
hipError_t launch_bf16_wgrad(const GemmParams& p, hipStream_t s);

// MXFP8 grouped GEMMs (gemm_mx.hip): both operands K-major E4M3 with slab-major
// E8M0 scales; WGRAD takes p.offsets = per-expert K ranges padded to 64.
hipError_t launch_mx_ragged(int mode, const GemmParams& p, hipStream_t s);
hipError_t launch_mx_wgrad(const GemmParams& p, hipStream_t s);

}  // namespace moe
