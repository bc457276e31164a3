// Device-side building blocks shared by the bf16 and MXFP8 grouped GEMMs:
// buffer descriptors and LDS DMA, LDS layouts and fragment reads, the
// device-side tile schedule, and the LDS-staged epilogues of every mode.
#pragma once

#include "common.h"
#include "grouped_gemm.h"
#include "mx_encode.h"

#include <type_traits>

namespace moe {
namespace gemm {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) v4s lds_v4s_t;

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

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// One 16-byte load per lane into LDS: lane i writes lds_wave + 16 i (lds_wave
// is wave-uniform and goes to M0). Issued as inline assembly so the compiler,
// which cannot tell the ring slots apart, does not add a full vmcnt(0) wait in
// front of every LDS read; the kernel waits for these loads itself
// (wait_vmcnt before the barrier that publishes a slab).
// The compiler does not look inside the assembly for hazards either, so the
// load carries its own wait states (s_nop W gives W + 1): a vector memory
// instruction must not read an SGPR (here the descriptor) within 5 wait states
// of a VALU write to it (v_readfirstlane, or v_readlane restoring a spilled
// SGPR), nor M0 within 1 of the SALU write that sets it. W = 4 covers both and
// is the default; W = 0 is only for loads whose descriptors are known to come
// from SALU arithmetic (the steady-state main loops), which a test checks on
// the built code object.
template <int W = 4>
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds_wave) {
  static_assert(W == 0 || W == 4, "wait states: 1 (M0 only) or 5 (M0 and descriptor)");
  if constexpr (W == 4)
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds" ::"v"(voff), "{m0}"(lds_wave), "s"(r)
                 : "memory");
  else
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds" ::"v"(voff), "{m0}"(lds_wave), "s"(r)
                 : "memory");
}

// K-contiguous tiles: rows of 64 bytes (4 chunks of 16); a 16-lane quarter of
// a ds_read_b128 reads one chunk column of 16 consecutive rows, so XOR-ing the
// chunk with (row / 4) % 4 spreads those rows over all 64 banks.
__device__ __forceinline__ int swz_row(int row) { return (row >> 2) & 3; }
// Row-contiguous tiles: a transposing read touches 4 consecutive k-rows x 32
// bytes per 16-lane group; XOR-ing the chunk index with 4 (k % 4) puts the 16
// (row, chunk) pairs of a half-wave on distinct banks (64 banks of 4 bytes).
// Rows of only 8 chunks (R = 64) use 2 (k % 4).
template <int R>
__device__ __forceinline__ int swz_k(int k) { return R >= 128 ? (k & 3) << 2 : (k & 3) << 1; }

// K-contiguous tile of R rows x 64 bytes (32 bf16 or 64 fp8 of k): rows
// [0, R) of a descriptor whose base is the tile's first row at the slab's
// first k. Load q (of R / 64) of a wave fills 16 rows. *_kmajor take the row
// stride in bf16 elements, *_rows64 in bytes; load_* issue one load, stage_*
// all of them.
template <int R, int W = 4>
__device__ __forceinline__ void load_rows64(__amdgpu_buffer_rsrc_t r, int64_t ld_bytes, uint32_t dst, int wave,
                                            int lane, int q) {
  const int rbase = (q * 4 + wave) * 16;
  const int row = rbase + (lane >> 2);
  const int g = (lane & 3) ^ swz_row(row);
  load_lds16<W>(r, static_cast<uint32_t>(row * ld_bytes + g * 16), dst + rbase * 64);
}
template <int R, int W = 4>
__device__ __forceinline__ void stage_rows64(__amdgpu_buffer_rsrc_t r, int64_t ld_bytes, uint32_t dst, int wave,
                                             int lane) {
#pragma unroll
  for (int q = 0; q < R / 64; ++q) load_rows64<R, W>(r, ld_bytes, dst, wave, lane, q);
}
template <int R, int W = 4>
__device__ __forceinline__ void stage_kmajor(__amdgpu_buffer_rsrc_t r, int64_t ld, uint32_t dst, int wave, int lane) {
  stage_rows64<R, W>(r, ld * 2, dst, wave, lane);
}

// Row-contiguous tile: 32 k-rows of R elements; descriptor base at (slab's
// first k, tile's first column). Load q (of R / 64) of a wave fills 1 KB.
template <int R, int W = 4>
__device__ __forceinline__ void load_mnmajor(__amdgpu_buffer_rsrc_t r, int64_t ld, uint32_t dst, int wave, int lane,
                                             int q) {
  constexpr int RB = R * 2;
  const int byte0 = (q * 4 + wave) * 1024;
  const int byte = byte0 + lane * 16;
  const int k = byte / RB;
  const int g = ((byte % RB) >> 4) ^ swz_k<R>(k);
  load_lds16<W>(r, static_cast<uint32_t>(k * ld * 2 + g * 16), dst + byte0);
}
template <int R, int W = 4>
__device__ __forceinline__ void stage_mnmajor(__amdgpu_buffer_rsrc_t r, int64_t ld, uint32_t dst, int wave, int lane) {
#pragma unroll
  for (int q = 0; q < R / 64; ++q) load_mnmajor<R, W>(r, ld, dst, wave, lane, q);
}

// Fragment (32 rows x 16 k) of a K-contiguous tile: lane -> row rb + lane%32,
// k = 16 kk + 8 (lane/32) .. +7.
__device__ __forceinline__ bf16x8 frag_kmajor(const char* t, int rb, int kk, int lane) {
  const int row = rb + (lane & 31);
  const int chunk = (kk * 2 + (lane >> 5)) ^ swz_row(row);
  return *reinterpret_cast<const bf16x8*>(t + row * 64 + chunk * 16);
}

// Same fragment from a row-contiguous tile of R columns, via two transposing
// reads: within each 16-lane group, source lane s points at (k0 + s/4, c0 +
// 4 (s%4)) and result lane i receives k0..k0+3 of column c0 + i.
template <int R>
__device__ __forceinline__ bf16x8 frag_mnmajor(const char* t, int cb, int kk, int lane) {
  constexpr int RB = R * 2;
  const int g = lane >> 4, s = lane & 15;
  const int c = cb + 16 * (g & 1) + 4 * (s & 3);
  const int kb = kk * 16 + 8 * (g >> 1) + (s >> 2);
  v4s h[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int k = kb + 4 * half;
    const int byte = c * 2;
    const int off = k * RB + ((((byte >> 4) ^ swz_k<R>(k))) << 4) + (byte & 15);
    h[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(const_cast<char*>(t) + off));
  }
  bf16x8 v;
  __builtin_memcpy(&v, h, 16);
  return v;
}

// Four fp32 -> four bf16 (round to nearest even) with gfx950's packed convert.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const bf16x2_t r = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
  uint32_t u;
  __builtin_memcpy(&u, &r, 4);
  return u;
}
__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  return make_uint2(pack2(a, b), pack2(c, d));
}
__device__ __forceinline__ void unpack4(uint2 v, float (&o)[4]) {
  o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
  o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding:
// vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1, fully unrolled, so
// accumulator indices stay compile-time constants (a runtime index would put
// the accumulators in scratch memory).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_impl(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) { static_for_impl<0, N>(f); }

__device__ __forceinline__ float sigmoid_f(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// The saved G, U of the MXFP8 layers: fp32 with the low 8 of the 23 mantissa
// bits rounded off (to nearest, ties away from zero; relative error at most
// 2^-17, below the fp32 accumulation error of the GEMM that produced them),
// four values in three dwords. fp24_round gives the fp32 value that is kept.
// Its inputs are MFMA results, whose NaNs carry the quiet bit, which the
// rounding keeps (only a NaN with nothing but the low 8 payload bits would
// turn into an infinity).
typedef unsigned int u32x3_t __attribute__((ext_vector_type(3)));
__device__ __forceinline__ float fp24_round(float x) {
  return __uint_as_float((__float_as_uint(x) + 0x80u) & 0xffffff00u);
}
// Packs four values already rounded by fp24_round.
__device__ __forceinline__ u32x3_t fp24_pack4(float a, float b, float c, float d) {
  const uint32_t t0 = __float_as_uint(a) >> 8, t1 = __float_as_uint(b) >> 8;
  const uint32_t t2 = __float_as_uint(c) >> 8, t3 = __float_as_uint(d) >> 8;
  return u32x3_t{t0 | (t1 << 24), (t1 >> 8) | (t2 << 16), (t2 >> 16) | (t3 << 8)};
}
__device__ __forceinline__ void fp24_unpack4(u32x3_t w, float (&o)[4]) {
  o[0] = __uint_as_float(w.x << 8);
  o[1] = __uint_as_float(((w.x >> 16) & 0xff00u) | (w.y << 16));
  o[2] = __uint_as_float(((w.y >> 8) & 0xffff00u) | (w.z << 24));
  o[3] = __uint_as_float(w.z & 0xffffff00u);
}


struct TileCoord {
  int e;        // expert (-1: no tile)
  int row0;     // ragged modes: first row of the tile; WGRAD: first K row of the expert
  int row_end;  // end of the expert's row range (K range for WGRAD)
  int nt;       // column tile
  int m0;       // WGRAD: first row of the weight-gradient tile
};

// Row tiles of the ragged modes, held per wave: lane l keeps experts 4l..4l+3
// (row ranges and tile counts of `tbm` rows) and the exclusive prefix of the
// tile counts, so any wave maps a tile index to its coordinates with
// lane-local compares and one ballot (no LDS, no barrier).
//
// Tiles are numbered by a logical index L so that tiles close in L share
// operands in L2: groups of 8 row tiles sweep the column tiles. With tiles of
// 256 rows the groups run on across expert boundaries; with shorter tiles an
// expert's few row tiles form a group of their own, so that a group does not
// read the weight panels of several experts (by measurement: the first order
// is as fast as the second at 256-row tiles and slower at 128). With R tiles
// and `cus` workgroups running at once, the rem = R % cus tiles past the last full
// round would keep the chip mostly idle for a whole tile time; when 4 rem <=
// cus they are left to a second launch (p.tail = 1) of a kernel with
// half-height, half-width tiles that takes each as 4 quarters, all in one
// round of a quarter of the time. Every launch derives the same tile list
// from the full-size tiles.
struct RowTileMap {
  int beg[4], end[4], tq[4], excl;  // per lane
  int RM, NT, tbm;                  // wave-uniform
  __device__ __forceinline__ void init(const GemmParams& p, int tbm_, int tbn, int lane) {
    tbm = tbm_;
    NT = p.N / tbn;
    int tsum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      beg[q] = e < p.E ? p.offsets[e] : 0;
      end[q] = e < p.E ? p.offsets[e + 1] : 0;
      const int bands = (end[q] - beg[q]) & ~255;
      if (p.band == 1) end[q] = beg[q] + bands;
      if (p.band == 2) beg[q] += bands;
      tq[q] = (end[q] - beg[q] + tbm - 1) / tbm;
      tsum += tq[q];
    }
    excl = wave_exclusive_scan(tsum);
    RM = __builtin_amdgcn_readfirstlane(__shfl(excl + tsum, 63, kWave));
  }
  __device__ __forceinline__ int tiles() const { return RM * NT; }
  // Tiles [0, main(cus)) go to full-size tiles; the rest, if any, to quarters.
  __device__ __forceinline__ int main_tiles(int cus) const {
    const int R = RM * NT;
    if (cus <= 0 || R <= 0) return R;
    const int rem = R >= cus ? R % cus : R;
    return 4 * rem > cus ? R : R - rem;
  }
  // Groups of 8 row tiles taken across the expert boundaries.
  __device__ __forceinline__ TileCoord at_across(int L, int lane) const {
    constexpr int GM = 8;
    const int g = L / (GM * NT);
    const int gm = min(GM, RM - g * GM);
    const int local = L - g * GM * NT;
    const int mt = g * GM + local % gm;
    int e_sel = -1, row0 = 0, row_end = 0, run = excl;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (mt >= run && mt < run + tq[q]) {
        e_sel = lane * 4 + q;
        row0 = beg[q] + (mt - run) * tbm;
        row_end = end[q];
      }
      run += tq[q];
    }
    const uint64_t who = __ballot(e_sel >= 0);
    const int src = who ? __ffsll(static_cast<long long>(who)) - 1 : 0;
    TileCoord t;
    t.e = who ? __builtin_amdgcn_readfirstlane(__shfl(e_sel, src, kWave)) : -1;
    t.row0 = __builtin_amdgcn_readfirstlane(__shfl(row0, src, kWave));
    t.row_end = __builtin_amdgcn_readfirstlane(__shfl(row_end, src, kWave));
    t.nt = __builtin_amdgcn_readfirstlane(local / gm);
    t.m0 = 0;
    return t;
  }
  // Coordinates of tile L (wave-uniform; e = -1 if L is past the end).
  __device__ __forceinline__ TileCoord at(int L, int lane) const {
    constexpr int GM = 8;
    if (tbm >= 256) return at_across(L, lane);
    // The lane holding L's expert finds it; the rest is wave-uniform.
    int e_sel = -1, t0_sel = 0, tq_sel = 0, beg_sel = 0, end_sel = 0, run = excl;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t0 = run * NT;
      if (L >= t0 && L < t0 + tq[q] * NT) {
        e_sel = lane * 4 + q;
        t0_sel = t0;
        tq_sel = tq[q];
        beg_sel = beg[q];
        end_sel = end[q];
      }
      run += tq[q];
    }
    const uint64_t who = __ballot(e_sel >= 0);
    TileCoord t{-1, 0, 0, 0, 0};
    if (!who) return t;
    const int src = __ffsll(static_cast<long long>(who)) - 1;
    t.e = __builtin_amdgcn_readfirstlane(__shfl(e_sel, src, kWave));
    const int local = L - __builtin_amdgcn_readfirstlane(__shfl(t0_sel, src, kWave));
    const int tqe = __builtin_amdgcn_readfirstlane(__shfl(tq_sel, src, kWave));
    const int g = local / (GM * NT), gm = min(GM, tqe - g * GM), in_g = local - g * GM * NT;
    t.row0 = __builtin_amdgcn_readfirstlane(__shfl(beg_sel, src, kWave)) + (g * GM + in_g % gm) * tbm;
    t.row_end = __builtin_amdgcn_readfirstlane(__shfl(end_sel, src, kWave));
    t.nt = in_g / gm;
    t.m0 = 0;
    return t;
  }
};

// First tile of XCD x's contiguous range when R tiles are cut into 8.
__device__ __forceinline__ int xcd_cut(int R, int x) { return x * (R / 8) + min(x, R % 8); }

// Row-ragged modes, one tile per workgroup: workgroup b runs on XCD b % 8,
// and each XCD takes a contiguous range of the main tiles. In the quarter
// launch (p.tail), workgroup b takes quarter b % 4 of tail tile b / 4.
// Wave 0 maps the id; the result is broadcast through LDS and kept
// wave-uniform (e < 0: no tile).
template <int BM, int BN>
__device__ __forceinline__ TileCoord ragged_tile(const GemmParams& p, int* s_info, int wave, int lane) {
  const int bid = blockIdx.x;
  if (wave == 0) {
    RowTileMap map;
    map.init(p, p.tail ? 2 * BM : BM, p.tail ? 2 * BN : BN, lane);
    const int rmain = map.main_tiles(p.cus);
    int L = -1, quarter = 0;
    if (!p.tail) {
      if (bid < rmain) L = xcd_cut(rmain, bid % 8) + bid / 8;
    } else if (bid < 4 * (map.tiles() - rmain)) {
      L = rmain + bid / 4;
      quarter = bid % 4;
    }
    TileCoord t{-1, 0, 0, 0, 0};
    if (L >= 0) {
      t = map.at(L, lane);
      if (p.tail && t.e >= 0) {  // quarter (row half, column half) of the full-size tile
        t.row0 += (quarter >> 1) * BM;
        t.nt = t.nt * 2 + (quarter & 1);
        if (t.row0 >= t.row_end) t.e = -1;
      }
    }
    if (lane == 0) {
      s_info[0] = t.e; s_info[1] = t.row0; s_info[2] = t.row_end; s_info[3] = t.nt;
    }
  }
  __syncthreads();
  TileCoord t;
  t.e = __builtin_amdgcn_readfirstlane(s_info[0]);
  t.row0 = __builtin_amdgcn_readfirstlane(s_info[1]);
  t.row_end = __builtin_amdgcn_readfirstlane(s_info[2]);
  t.nt = __builtin_amdgcn_readfirstlane(s_info[3]);
  t.m0 = 0;
  return t;
}

// Weight gradients: persistent workgroups (a multiple of 8; workgroup b runs
// on XCD b % 8). Tiles are (expert, M tile, N tile), numbered expert by
// expert, with K = the expert's rows, so their cost follows the load. Each XCD
// owns a contiguous range of the tile list (tiles sharing operands stay in
// one L2) and its workgroups take the range's tiles in turn. Ranges are cut at
// equal tile counts, unless that leaves some XCD more than 5/4 of the mean
// cost (K slabs + kEpiWork per tile): then they are cut at equal shares of the
// cost, so a hot expert's tiles spread over several XCDs. s_info receives
// {first tile, end, stride}.
template <int BM, int BN, int KB, int kEpiWork>
__device__ __forceinline__ void wgrad_sched(const GemmParams& p, int* s_info, int wave, int lane) {
  const int bid = blockIdx.x, x = bid % 8, i = bid / 8, wpx = gridDim.x / 8;
  if (wave == 0) {
    const int TE = (p.M / BM) * (p.N / BN);
    const int R = p.E * TE;
    int w[4], wsum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      w[q] = e < p.E ? (p.offsets[e + 1] - p.offsets[e] + KB - 1) / KB + kEpiWork : 0;
      wsum += w[q];
    }
    const int excl = wave_exclusive_scan(wsum);
    const int total = __shfl(excl + wsum, 63, kWave);
    // Count cuts and the cost of the XCD that gets the most.
    auto count_cut = [&](int xx) { return xx * (R / 8) + min(xx, R % 8); };
    int64_t worst = 0;
    for (int xx = 0; xx < 8; ++xx) {
      const int a = count_cut(xx), b = count_cut(xx + 1);
      int64_t c = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = lane * 4 + q;
        const int lo = max(a, e * TE), hi = min(b, (e + 1) * TE);
        if (w[q] > 0 && hi > lo) c += static_cast<int64_t>(hi - lo) * w[q];
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, kWave);
      worst = max(worst, c);
    }
    int first, end;
    if (worst * 32 <= static_cast<int64_t>(TE) * total * 5) {  // worst <= 5/4 of the mean (TE * total / 8)
      first = count_cut(x);
      end = count_cut(x + 1);
    } else {
      // First tile whose cost-start is at or past xx/8 of the summed cost.
      auto bound = [&](int xx) -> int {
        if (xx >= 8) return R;
        const int64_t B = static_cast<int64_t>(TE) * total * xx / 8;
        int t = -1, run = excl;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t P = static_cast<int64_t>(TE) * run;
          if (w[q] > 0 && B >= P && B < P + static_cast<int64_t>(TE) * w[q])
            t = (lane * 4 + q) * TE + static_cast<int>((B - P + w[q] - 1) / w[q]);
          run += w[q];
        }
        const uint64_t who = __ballot(t >= 0);
        return who ? __shfl(t, __ffsll(static_cast<long long>(who)) - 1, kWave) : R;
      };
      first = bound(x);
      end = bound(x + 1);
    }
    if (lane == 0) {
      s_info[0] = first + i; s_info[1] = end; s_info[2] = wpx;
    }
  }
  __syncthreads();
}

// Coordinates of weight-gradient tile t (wave-uniform).
template <int BM, int BN>
__device__ __forceinline__ TileCoord wgrad_tile(const GemmParams& p, int t) {
  const int NT = p.N / BN, TE = (p.M / BM) * NT;
  const int e = t / TE, j = t % TE;
  TileCoord tc;
  tc.e = __builtin_amdgcn_readfirstlane(e);
  tc.m0 = __builtin_amdgcn_readfirstlane((j / NT) * BM);
  tc.nt = __builtin_amdgcn_readfirstlane(j % NT);
  tc.row0 = __builtin_amdgcn_readfirstlane(p.offsets[e]);
  tc.row_end = __builtin_amdgcn_readfirstlane(p.offsets[e + 1]);
  return tc;
}

// Writes the accumulators of one BM x BN tile (and, for BWD_DOWN, reads the
// saved G, U it needs) through a per-wave LDS area of smem, which must hold
// 4 x 2 x (BM/2) x 128 bytes and be free of other use.
// With QUANT (the MXFP8 kernels), FWD_GU writes G, U (24-bit, fp24_pack4)
// in a blocked layout and H, and BWD_DOWN dG | dU, only as the next GEMMs'
// E4M3 operands (K-major p.mxq, p.mxs; token-major p.tq, p.ts), every code
// decided on the fp32 value in registers; BWD_DOWN reads the blocked G, U.
template <int MODE, int BM, int BN, bool QUANT = false>
__device__ __forceinline__ void epilogue(const GemmParams& p, floatx16 (&acc)[BN / 64][BM / 64], char* smem,
                                         int wave, int lane, const TileCoord& tc) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MB = WM / 32, NB = WN / 32;
  const int wm = wave >> 1, wn = wave & 1;
  const int e = tc.e, row0 = tc.row0, row_end = tc.row_end, nt = tc.nt, m0 = tc.m0;
  const int n0 = nt * BN;
  // acc[j][i] element r of lane l: n = wn*WN + 32 j + 8 (r/4) + 4 (l/32) + r%4,
  // m = wm*WM + 32 i + l%32; four consecutive r are four consecutive columns.
  // Outputs go through a per-wave LDS area in column groups of up to 64: the
  // lanes put their 8-byte pieces into a [WM rows][64 cols] bf16 staging
  // tile, then every store writes 128 contiguous bytes of a row. Saved inputs
  // of the epilogue (G, U for BWD_DOWN) come in the same way by LDS DMA.
  const int hl = lane >> 5, l32 = lane & 31;
  constexpr int kSlot = WM * 128;  // one staging tile: WM rows x 64 columns of bf16
  char* const wa = smem + wave * 2 * kSlot;
  // Chunk c (16 bytes) of staging row r lives at chunk c ^ ((r / 2) % 8).
  auto st_off = [](int r, int col) {
    return r * 128 + ((((col >> 3) ^ (r >> 1)) & 7) << 4) + ((col & 4) << 1);
  };
  auto put4 = [&](int slot, int r, int col, uint2 v) {
    *reinterpret_cast<uint2*>(wa + slot * kSlot + st_off(r, col)) = v;
  };
  auto get4 = [&](int slot, int r, int col) -> uint2 {
    return *reinterpret_cast<const uint2*>(wa + slot * kSlot + st_off(r, col));
  };
  auto wave_sync = [&]() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
  };
  const int mrow = (MODE == WGRAD ? m0 : row0) + wm * WM;   // first row of this wave's block
  // Rows [0, rows) and columns [0, cols) of staging tile `slot` -> global
  // rows g + r*ld (bytes), 16 bytes per lane, 8 lanes per 128-byte row.
  auto flush = [&](int slot, char* g, int64_t ld, int rows, int cols) {
    wave_sync();
    const int c = lane & 7;
#pragma unroll 4
    for (int t = 0; t < WM / 8; ++t) {
      const int r = t * 8 + (lane >> 3);
      const uint4 v = *reinterpret_cast<const uint4*>(wa + slot * kSlot + r * 128 + ((c ^ (r >> 1)) & 7) * 16);
      // Non-temporal: written once, read by a later kernel.
      typedef unsigned int u32x4nt __attribute__((ext_vector_type(4)));
      if (r < rows && c * 8 < cols)
        __builtin_nontemporal_store(u32x4nt{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4nt*>(g + r * ld + c * 16));
    }
    wave_sync();
  };
  const int rows = (MODE == WGRAD) ? WM : max(0, min(WM, row_end - mrow));
  auto acc4 = [&](int j, int i, int q) {
    return pack4(acc[j][i][4 * q], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2], acc[j][i][4 * q + 3]);
  };

  if constexpr (MODE == FWD_GU && QUANT) {
    // G, U (rounded to the 24 bits they are kept in) and H = G sig(G) U in
    // fp32 from those values, one 32 x 32 block (gate block JJ and up block
    // JJ + NB/2 cover the same 32 f-columns, row block I) at a time, straight
    // from the accumulators:
    //  - G and U to the save buffer in the blocked layout the down-dgrad
    //    epilogue reads back: block (padded row / 32, column / 32), 3 KB, in
    //    lane order (lane l: row l % 32, columns 8 Q + 4 (l / 32) .. +3 as one
    //    12-byte piece at 768 Q + 12 l), so every store and every later load
    //    is 768 contiguous bytes. Padded rows are poff[e] + row inside e.
    //  - H only as E4M3 operands, each code decided on the fp32 value:
    //    K-major along f (the down GEMM's A operand; a row's 32-block sits in
    //    lanes l and l ^ 32), and token-major [f][P] for the weight gradient
    //    of W_down (the block goes through LDS column-major; lane c < 32
    //    encodes column c, 32 tokens).
    // Blocks past the expert's rows padded to 64 are left alone (they are
    // the next expert's); rows past its end inside them are zeros (the A
    // operand reads 0 there).
    const int e_first = p.offsets[e];
    const int rel0 = mrow - e_first;
    const int n64 = (row_end - e_first + 63) & ~63;
    const int64_t pt0 = static_cast<int64_t>(p.poff[e]) + rel0;  // a multiple of 32
    const int fb = p.f / 32;
    const auto rQ = make_rsrc(p.mxq + static_cast<int64_t>(mrow) * p.mxq_ld, static_cast<int64_t>(rows) * p.mxq_ld);
    constexpr int kTgFloats = 32 * 36;
    float* const tgw = reinterpret_cast<float*>(smem + wave * (2 * kTgFloats * 4));
    typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
    // 256 x 256 tiles: the blocks go row group by row group, and a group's two
    // H column blocks (the wave's 64 columns of each K-major row) are staged
    // in LDS (two buffers of [32 rows][80 bytes] per wave, after the transpose
    // buffers) and leave 16 rows x 64 bytes per store instead of 32 bytes of
    // 32 rows. Other tiles store each block's pieces directly.
    constexpr bool kStageH = (BM == 256 && BN == 256);
    constexpr int kHst = 2 * 32 * 80;
    char* const hst = smem + 4 * (2 * kTgFloats * 4) + wave * kHst;
    static_assert(!kStageH || 4 * (2 * kTgFloats * 4 + kHst) <= 4 * (BM * 64 + BN * 64 + 4 * 1024),
                  "epilogue LDS fits in the ring");
    static_for<(NB / 2) * MB>([&](auto BI) {
      constexpr int bi = decltype(BI)::value;
      constexpr int JJ = kStageH ? bi % (NB / 2) : bi / MB, I = kStageH ? bi / (NB / 2) : bi % MB;
      const int col0 = nt * (BN / 2) + wn * (WN / 2) + JJ * 32;
      const bool live = rel0 + I * 32 < n64;
      float gk[16], uk[16], h[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        gk[r] = fp24_round(acc[JJ][I][r]);
        uk[r] = fp24_round(acc[JJ + NB / 2][I][r]);
        h[r] = gk[r] * sigmoid_f(gk[r]) * uk[r];
      }
      if (live) {
        const int64_t blk = ((pt0 / 32 + I) * fb + col0 / 32) * 3072;  // bytes
        const auto rGb = make_rsrc(static_cast<char*>(p.c0) + blk, 3072);
        const auto rUb = make_rsrc(static_cast<char*>(p.c1) + blk, 3072);
#pragma unroll
        for (int Q = 0; Q < 4; ++Q) {
          const uint32_t off = static_cast<uint32_t>(Q * 768 + lane * 12);
          __builtin_amdgcn_raw_buffer_store_b96(fp24_pack4(gk[4 * Q], gk[4 * Q + 1], gk[4 * Q + 2], gk[4 * Q + 3]), rGb,
                                                off, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b96(fp24_pack4(uk[4 * Q], uk[4 * Q + 1], uk[4 * Q + 2], uk[4 * Q + 3]), rUb,
                                                off, 0, 0);
        }
      }
      // Token-major: stage column-major.
      float* const tg = tgw + (bi & 1) * kTgFloats;
#pragma unroll
      for (int r = 0; r < 16; ++r) tg[(8 * (r / 4) + 4 * hl + r % 4) * 36 + l32] = h[r];
      // K-major along f.
      {
        float m = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(h[r]));
        const auto mm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
        const int code = mx_scale_code(fmaxf(__uint_as_float(mm[0]), __uint_as_float(mm[1])));
        uint32_t w[4];
#pragma unroll
        for (int Q = 0; Q < 4; ++Q)
          w[Q] = e4m3_encode4(ldexpf(h[4 * Q], 127 - code), ldexpf(h[4 * Q + 1], 127 - code),
                              ldexpf(h[4 * Q + 2], 127 - code), ldexpf(h[4 * Q + 3], 127 - code));
        const auto a = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
        const auto c = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
        if constexpr (kStageH) {
          char* const hb = hst + (I & 1) * (kHst / 2);
          *reinterpret_cast<u32x4_t*>(hb + l32 * 80 + JJ * 32 + 16 * hl) = u32x4_t{a[0], a[1], c[0], c[1]};
          if constexpr (JJ == NB / 2 - 1) {
            wave_sync();
            const int c16 = lane & 3;
            const int cbase = nt * (BN / 2) + wn * (WN / 2);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const int r = t * 16 + (lane >> 2);
              __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4_t*>(hb + r * 80 + c16 * 16), rQ,
                                                     static_cast<uint32_t>((I * 32 + r) * p.mxq_ld + cbase + c16 * 16),
                                                     0, 0);
            }
          }
        } else {
          __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{a[0], a[1], c[0], c[1]}, rQ,
                                                 static_cast<uint32_t>((I * 32 + l32) * p.mxq_ld + col0 + 16 * hl), 0,
                                                 0);
        }
        const auto rS = make_rsrc(p.mxs + static_cast<int64_t>(col0 / 64) * p.mxs_slab +
                                      static_cast<int64_t>(mrow) * 2,
                                  static_cast<int64_t>(rows) * 2);
        if (hl == 0)
          __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(code), rS,
                                               static_cast<uint32_t>((I * 32 + l32) * 2 + (col0 / 32) % 2), 0, 0);
      }
      // Token-major: lane c < 32 encodes column c of the block.
      if (live && lane < 32) {
        const float* col = tg + lane * 36;
        float v[32];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float4 x = *reinterpret_cast<const float4*>(col + 4 * t);
          v[4 * t] = x.x; v[4 * t + 1] = x.y; v[4 * t + 2] = x.z; v[4 * t + 3] = x.w;
        }
        float m = 0.0f;
#pragma unroll
        for (int t = 0; t < 32; ++t) m = fmaxf(m, fabsf(v[t]));
        const int code = mx_scale_code(m);
        uint32_t w[8];
#pragma unroll
        for (int t = 0; t < 8; ++t)
          w[t] = e4m3_encode4(ldexpf(v[4 * t], 127 - code), ldexpf(v[4 * t + 1], 127 - code),
                              ldexpf(v[4 * t + 2], 127 - code), ldexpf(v[4 * t + 3], 127 - code));
        const int64_t ch = col0 + lane, pt = pt0 + I * 32;
        uint8_t* dst = p.tq + ch * p.tq_ld + pt;
        *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{w[0], w[1], w[2], w[3]};
        *reinterpret_cast<u32x4_t*>(dst + 16) = u32x4_t{w[4], w[5], w[6], w[7]};
        p.ts[(pt / 64) * p.ts_slab + ch * 2 + (pt / 32) % 2] = static_cast<uint8_t>(code);
      }
    });
  } else if constexpr (MODE == BWD_DOWN && QUANT) {
    // dH -> dG = dH U sig(G) (1 + G (1 - sig(G))), dU = dH G sig(G) in fp32
    // from the saved G, U, one 32 x 32 block (J, I) at a time. The saved G, U
    // of a block come straight into registers in the accumulator layout
    // (lane: row 32 I + l%32, columns 8 Q + 4 (l/32) .. +3), as four
    // contiguous 768-byte pieces each from the blocked layout the gate/up
    // epilogue wrote, two blocks ahead of their use; rows past the expert's
    // end hold 0, so dG, dU are 0 there.
    // dG and dU leave only as the next GEMMs' E4M3 operands, each code
    // decided on the fp32 value:
    //  - K-major along 2f (dG in columns [0, f), dU in [f, 2f)): a row's
    //    32-block sits in lanes l and l ^ 32; one exchange gives its scale,
    //    a second gives each lane 16 consecutive codes;
    //  - token-major [2f][P] for the weight gradient: the block goes through
    //    LDS column-major (dG then dU, 36-dword columns: conflict-free 16-byte
    //    reads; two buffers, alternating by block, so a block's transpose
    //    overlaps the next block's arithmetic), and lane L encodes column
    //    L % 32 of tensor L / 32: 32 tokens, the 32-row block of that channel
    //    inside the expert's padded range.
    // Lane-half exchanges use v_permlane32_swap (a VALU op, no LDS round trip):
    // swap(x, y) leaves lanes 0..31 of x and lanes 32..63 of y in place and
    // exchanges lanes 32..63 of x with lanes 0..31 of y.
    const int e_first = p.offsets[e];
    const int rel0 = mrow - e_first;                       // first row of the block, inside the expert
    const int n64 = (row_end - e_first + 63) & ~63;        // the expert's rows padded to 64
    const int64_t pt0 = static_cast<int64_t>(p.poff[e]) + rel0;
    // G, U in the blocked layout the gate/up epilogue writes (3 KB per 32 x
    // 32 block, lane order): blocks past the expert's padded rows read 0.
    const int fb = p.f / 32;
    // The range covers this wave's row blocks only (at most WM rows), so it
    // stays far below the 2^31 bytes a descriptor holds however long the expert.
    const int64_t gb0 = (pt0 / 32) * fb * 3072;
    const int64_t gbytes = static_cast<int64_t>(min(WM, max(0, n64 - rel0)) / 32) * fb * 3072;
    const auto rG = make_rsrc(static_cast<const char*>(p.e0) + gb0, gbytes);
    const auto rU = make_rsrc(static_cast<const char*>(p.e1) + gb0, gbytes);
    const auto rQ = make_rsrc(p.mxq + static_cast<int64_t>(mrow) * p.mxq_ld, rows * p.mxq_ld);
    constexpr int kAhead = 2;       // blocks of G, U in flight ahead of the one in use
    u32x3_t gu[kAhead + 1][2][4];   // [buffer][G, U][Q]
    auto load_block = [&](auto B, int J, int I) {
      constexpr int b = decltype(B)::value;
      const int col0 = n0 + wn * WN + J * 32;
#pragma unroll
      for (int Q = 0; Q < 4; ++Q) {
        const uint32_t off = static_cast<uint32_t>((I * fb + col0 / 32) * 3072 + Q * 768 + lane * 12);
        gu[b][0][Q] = __builtin_amdgcn_raw_buffer_load_b96(rG, off, 0, 0);
        gu[b][1][Q] = __builtin_amdgcn_raw_buffer_load_b96(rU, off, 0, 0);
      }
    };
    // Per-wave LDS: two transpose buffers [2 tensors][32 columns][36].
    constexpr int kTgFloats = 2 * 32 * 36;
    float* const tgw = reinterpret_cast<float*>(smem + wave * (2 * kTgFloats * 4));
    // 256 x 256 tiles (a wave's 128 columns are one 128-byte line of each
    // K-major row): the blocks go row group by row group, and a group's four
    // column blocks are staged in LDS (two buffers of [2 tensors][32 rows][144
    // bytes] per wave, after the transpose buffers) and leave as whole lines,
    // 8 rows per store, instead of 32 bytes of 32 rows per store. Other tiles
    // store each block's 16-byte pieces directly, column block by column block.
    constexpr bool kStageK = (BM == 256 && BN == 256);
    constexpr int kKst = 2 * 2 * 32 * 144;
    char* const kst = smem + 4 * (2 * kTgFloats * 4) + wave * kKst;
    static_assert(!kStageK || 4 * (2 * kTgFloats * 4 + kKst) <= 4 * (BM * 64 + BN * 64 + 4 * 1024),
                  "epilogue LDS fits in the ring");
    constexpr auto blk_j = [](int bi) { return kStageK ? bi % NB : bi / MB; };
    constexpr auto blk_i = [](int bi) { return kStageK ? bi / NB : bi % MB; };
    static_for<kAhead>([&](auto B0) {
      constexpr int b0 = decltype(B0)::value;
      if constexpr (b0 < NB * MB) load_block(B0, blk_j(b0), blk_i(b0));
    });
    static_for<NB * MB>([&](auto BI) {
      constexpr int bi = decltype(BI)::value, J = blk_j(bi), I = blk_i(bi), b = bi % (kAhead + 1);
      if constexpr (bi + kAhead < NB * MB)
        load_block(std::integral_constant<int, (bi + kAhead) % (kAhead + 1)>{}, blk_j(bi + kAhead),
                   blk_i(bi + kAhead));
      float* const tg = tgw + (bi & 1) * kTgFloats;
      const int col0 = n0 + wn * WN + J * 32;
      float dg[16], du[16], gq[16], uq[16];
#pragma unroll
      for (int Q = 0; Q < 4; ++Q) {
        float g4[4], u4[4];
        fp24_unpack4(gu[b][0][Q], g4);
        fp24_unpack4(gu[b][1][Q], u4);
#pragma unroll
        for (int c = 0; c < 4; ++c) { gq[4 * Q + c] = g4[c]; uq[4 * Q + c] = u4[c]; }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float g = gq[r], u = uq[r];
        const float dh = acc[J][I][r];
        const float sg = sigmoid_f(g);
        du[r] = dh * g * sg;
        dg[r] = dh * u * sg * (1.0f + g * (1.0f - sg));
      }
      // Token-major: stage column-major, then one column per lane.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 8 * (r / 4) + 4 * hl + r % 4;
        tg[c * 36 + l32] = dg[r];
        tg[32 * 36 + c * 36 + l32] = du[r];
      }
      // K-major: the row's 32-block is in lanes l32 and l32 + 32.
      {
        float mg = 0.0f, mu = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          mg = fmaxf(mg, fabsf(dg[r]));
          mu = fmaxf(mu, fabsf(du[r]));
        }
        auto half_max = [](float m) {  // max over lanes l and l ^ 32
          const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
          return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
        };
        mg = half_max(mg);
        mu = half_max(mu);
        const int cg = mx_scale_code(mg), cu = mx_scale_code(mu);
        uint32_t wg[4], wu[4];
#pragma unroll
        for (int Q = 0; Q < 4; ++Q) {
          wg[Q] = e4m3_encode4(ldexpf(dg[4 * Q], 127 - cg), ldexpf(dg[4 * Q + 1], 127 - cg),
                               ldexpf(dg[4 * Q + 2], 127 - cg), ldexpf(dg[4 * Q + 3], 127 - cg));
          wu[Q] = e4m3_encode4(ldexpf(du[4 * Q], 127 - cu), ldexpf(du[4 * Q + 1], 127 - cu),
                               ldexpf(du[4 * Q + 2], 127 - cu), ldexpf(du[4 * Q + 3], 127 - cu));
        }
        // Lane half 0 holds columns 8Q..8Q+3, half 1 columns 8Q+4..8Q+7: two
        // swaps give half 0 columns 0..15 and half 1 columns 16..31 (swap(w0,
        // w2): half 0 keeps its w0 and receives half 1's w0, half 1 receives
        // half 0's w2 and keeps its own; likewise w1, w3).
        typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
        auto pack16 = [&](const uint32_t (&w)[4]) -> u32x4_t {
          const auto a = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
          const auto c = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
          return u32x4_t{a[0], a[1], c[0], c[1]};
        };
        const u32x4_t vg = pack16(wg), vu = pack16(wu);
        if constexpr (kStageK) {
          char* const kb = kst + (I & 1) * (kKst / 2);
          *reinterpret_cast<u32x4_t*>(kb + l32 * 144 + J * 32 + 16 * hl) = vg;
          *reinterpret_cast<u32x4_t*>(kb + 32 * 144 + l32 * 144 + J * 32 + 16 * hl) = vu;
          if constexpr (J == NB - 1) {
            wave_sync();
            const int c16 = lane & 7;
            const int cbase = n0 + wn * WN;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int r = t * 8 + (lane >> 3);
              const u32x4_t g = *reinterpret_cast<const u32x4_t*>(kb + r * 144 + c16 * 16);
              const u32x4_t u = *reinterpret_cast<const u32x4_t*>(kb + 32 * 144 + r * 144 + c16 * 16);
              const uint32_t off = static_cast<uint32_t>((I * 32 + r) * p.mxq_ld + cbase + c16 * 16);
              __builtin_amdgcn_raw_buffer_store_b128(g, rQ, off, 0, 0);
              __builtin_amdgcn_raw_buffer_store_b128(u, rQ, off + static_cast<uint32_t>(p.f), 0, 0);
            }
          }
        } else {
          const uint32_t qoff = static_cast<uint32_t>((I * 32 + l32) * p.mxq_ld + col0 + 16 * hl);
          __builtin_amdgcn_raw_buffer_store_b128(vg, rQ, qoff, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b128(vu, rQ, qoff + static_cast<uint32_t>(p.f), 0, 0);
        }
        // Scales: row r's byte of 32-block col / 32 (rows past the end dropped).
        const auto rS = make_rsrc(p.mxs + static_cast<int64_t>(col0 / 64) * p.mxs_slab + static_cast<int64_t>(mrow) * 2,
                                  static_cast<int64_t>(rows) * 2);
        const auto rS2 = make_rsrc(p.mxs + static_cast<int64_t>((p.f + col0) / 64) * p.mxs_slab +
                                       static_cast<int64_t>(mrow) * 2,
                                   static_cast<int64_t>(rows) * 2);
        if (hl == 0) {
          const uint32_t so = static_cast<uint32_t>((I * 32 + l32) * 2 + (col0 / 32) % 2);
          __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(cg), rS, so, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(cu), rS2,
                                               static_cast<uint32_t>((I * 32 + l32) * 2 + ((p.f + col0) / 32) % 2), 0, 0);
        }
      }
      // Token-major: lane L takes column L % 32 of dG (L < 32) or dU.
      if (rel0 + I * 32 < n64) {
        const float* col = tg + (lane >> 5) * 32 * 36 + (lane & 31) * 36;
        float v[32];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float4 x = *reinterpret_cast<const float4*>(col + 4 * t);
          v[4 * t] = x.x; v[4 * t + 1] = x.y; v[4 * t + 2] = x.z; v[4 * t + 3] = x.w;
        }
        float m = 0.0f;
#pragma unroll
        for (int t = 0; t < 32; ++t) m = fmaxf(m, fabsf(v[t]));
        const int code = mx_scale_code(m);
        uint32_t w[8];
#pragma unroll
        for (int t = 0; t < 8; ++t)
          w[t] = e4m3_encode4(ldexpf(v[4 * t], 127 - code), ldexpf(v[4 * t + 1], 127 - code),
                              ldexpf(v[4 * t + 2], 127 - code), ldexpf(v[4 * t + 3], 127 - code));
        const int64_t ch = (lane >> 5) * static_cast<int64_t>(p.f) + col0 + (lane & 31);
        const int64_t pt = pt0 + I * 32;
        typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
        uint8_t* dst = p.tq + ch * p.tq_ld + pt;
        *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{w[0], w[1], w[2], w[3]};
        *reinterpret_cast<u32x4_t*>(dst + 16) = u32x4_t{w[4], w[5], w[6], w[7]};
        p.ts[(pt / 64) * p.ts_slab + ch * 2 + (pt / 32) % 2] = static_cast<uint8_t>(code);
      }
    });
  } else if constexpr (MODE == FWD_GU) {
    // Gate blocks [0, NB/2) and up blocks [NB/2, NB) cover the same NB*16 f-columns.
    constexpr int GC = NB * 16;
    const int col0 = nt * (BN / 2) + wn * (WN / 2);
    const int64_t ld = p.ldc * 2;
    char* G = static_cast<char*>(p.c0) + (static_cast<int64_t>(mrow) * p.ldc + col0) * 2;
    char* U = static_cast<char*>(p.c1) + (static_cast<int64_t>(mrow) * p.ldc + col0) * 2;
    char* H = static_cast<char*>(p.c2) + (static_cast<int64_t>(mrow) * p.ldc + col0) * 2;
    // Pass 1: G and H (= silu(G) U) from the gate and up accumulators; pass 2: U.
    static_for<MB>([&](auto I) {
      static_for<NB / 2>([&](auto JJ) {
        static_for<4>([&](auto Q) {
          const int r = I * 32 + l32, col = JJ * 32 + 8 * Q + 4 * hl;
          float h[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float g = acc[JJ][I][4 * Q + c], u = acc[JJ + NB / 2][I][4 * Q + c];
            h[c] = g * sigmoid_f(g) * u;
          }
          put4(0, r, col, acc4(JJ, I, Q));
          put4(1, r, col, pack4(h[0], h[1], h[2], h[3]));
        });
      });
    });
    flush(0, G, ld, rows, GC);
    flush(1, H, ld, rows, GC);
    static_for<MB>([&](auto I) {
      static_for<NB / 2>([&](auto JJ) {
        static_for<4>([&](auto Q) { put4(0, I * 32 + l32, JJ * 32 + 8 * Q + 4 * hl, acc4(JJ + NB / 2, I, Q)); });
      });
    });
    flush(0, U, ld, rows, GC);
  } else if constexpr (MODE == BWD_DOWN && !QUANT && NB % 2 == 0 && MB % 2 == 0) {
    // dH -> dG = dH U sig(G) (1 + G (1 - sig(G))), dU = dH G sig(G); a row of
    // dGU is [dG (f) | dU (f)]. Pipelined over units (column group jp of 64,
    // row half h): the saved G, U of a unit come in by LDS DMA into rows
    // [h WM/2, (h+1) WM/2) of staging tiles 0, 1 while the unit before it is
    // computed and written; a unit's results leave as range-checked buffer
    // stores before the next unit's loads overwrite its rows. Every load and
    // store is issued whatever
    // the row count (the descriptors drop rows past the end), so the vmcnt
    // waits below count exactly: unit u waits for every operation issued
    // before the one issued after its loads.
    constexpr int HR = WM / 2, TL = HR / 8, L = 2 * TL;  // L: loads (or stores) per unit
    static_assert(2 * L < 64, "vmcnt range");
    const int64_t ld = p.ldc * 2, lds_ = static_cast<int64_t>(p.f) * 2;
    auto load_unit = [&](auto JP, auto H) {
      constexpr int jp = decltype(JP)::value, h = decltype(H)::value;
      const int col0 = n0 + wn * WN + jp * 64;
      const int64_t sbase = (static_cast<int64_t>(mrow) * p.f + col0) * 2;
      const int64_t sbytes = static_cast<int64_t>(rows) * p.f * 2;
      // Offsets are rebuilt from an opaque copy of the lane id in every unit:
      // kept live across units they cost registers the accumulators need.
      int ln = lane;
      asm volatile("" : "+v"(ln));
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        const auto rs = make_rsrc(static_cast<const char*>(sl ? p.e1 : p.e0) + sbase, sbytes);
        const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(wa + sl * kSlot));
#pragma unroll
        for (int tt = 0; tt < TL; ++tt) {
          const int t = h * TL + tt, r = t * 8 + (ln >> 3);
          const int cc = (ln & 7) ^ ((r >> 1) & 7);  // logical chunk held by this lane's slot
          load_lds16(rs, static_cast<uint32_t>(r * lds_ + cc * 16), dst + t * 1024);
        }
      }
    };
    auto compute_unit = [&](auto JP, auto H) {
      constexpr int jp = decltype(JP)::value, h = decltype(H)::value;
      static_for<MB / 2>([&](auto II) {
        constexpr int I = h * (MB / 2) + decltype(II)::value;
        static_for<2>([&](auto JJ) {
          static_for<4>([&](auto Q) {
            constexpr int j = jp * 2 + JJ;
            const int r = I * 32 + l32, col = JJ * 32 + 8 * Q + 4 * hl;
            float g[4], u[4], dg[4], du[4];
            unpack4(get4(0, r, col), g);
            unpack4(get4(1, r, col), u);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float dh = acc[j][I][4 * Q + q];
              const float sg = sigmoid_f(g[q]);
              du[q] = dh * g[q] * sg;
              dg[q] = dh * u[q] * sg * (1.0f + g[q] * (1.0f - sg));
            }
            put4(0, r, col, pack4(dg[0], dg[1], dg[2], dg[3]));
            put4(1, r, col, pack4(du[0], du[1], du[2], du[3]));
          });
        });
      });
    };
    typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
    // Store unit (jp, h): dG and dU rows out of staging as L range-checked
    // buffer stores; each store consumes its LDS read, so once they are
    // issued the rows of half h are free and `next` may issue the loads of
    // the unit that reuses them.
    auto drain_unit = [&](auto JP, auto H, auto next) {
      constexpr int jp = decltype(JP)::value, h = decltype(H)::value;
      wave_sync();  // the unit's results are in staging
      const int col0 = n0 + wn * WN + jp * 64;
      const char* C = static_cast<const char*>(p.c0) + (static_cast<int64_t>(mrow) * p.ldc + col0) * 2;
      const auto rg = make_rsrc(C, static_cast<int64_t>(rows) * ld);
      const auto ru = make_rsrc(C + static_cast<int64_t>(p.f) * 2, static_cast<int64_t>(rows) * ld);
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int cl = ln & 7;
#pragma unroll
      for (int tt = 0; tt < TL; ++tt) {
        const int r = (h * TL + tt) * 8 + (ln >> 3);
        const int off = r * 128 + ((cl ^ (r >> 1)) & 7) * 16;
        const u32x4_t vg = *reinterpret_cast<const u32x4_t*>(wa + off);
        const u32x4_t vu = *reinterpret_cast<const u32x4_t*>(wa + kSlot + off);
        __builtin_amdgcn_raw_buffer_store_b128(vg, rg, static_cast<uint32_t>(r * ld + cl * 16), 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(vu, ru, static_cast<uint32_t>(r * ld + cl * 16), 0, 0);
      }
      next();
    };
    using Z = std::integral_constant<int, 0>;
    using O = std::integral_constant<int, 1>;
    auto none = [] {};
    static_assert(NB / 2 == 1 || NB / 2 == 2, "one or two column groups of 64 per wave");
    if constexpr (NB / 2 == 2) {
      // Issue order: L(0,0) L(0,1) | S(0,0) L(1,0) | S(0,1) L(1,1) | S(1,0) | S(1,1).
      load_unit(Z{}, Z{});
      load_unit(Z{}, O{});
      wait_vmcnt<L>();  // (0,0) landed
      wave_sync();
      compute_unit(Z{}, Z{});
      drain_unit(Z{}, Z{}, [&] { load_unit(O{}, Z{}); });
      wait_vmcnt<2 * L>();  // (0,1) landed: S(0,0), L(1,0) may fly
      wave_sync();
      compute_unit(Z{}, O{});
      drain_unit(Z{}, O{}, [&] { load_unit(O{}, O{}); });
      wait_vmcnt<2 * L>();  // (1,0) landed: S(0,1), L(1,1) may fly
      wave_sync();
      compute_unit(O{}, Z{});
      drain_unit(O{}, Z{}, none);
      wait_vmcnt<L>();  // (1,1) landed: S(1,0) may fly
      wave_sync();
      compute_unit(O{}, O{});
      drain_unit(O{}, O{}, none);
    } else {
      load_unit(Z{}, Z{});
      load_unit(Z{}, O{});
      wait_vmcnt<L>();
      wave_sync();
      compute_unit(Z{}, Z{});
      drain_unit(Z{}, Z{}, none);
      wait_vmcnt<L>();  // (0,1) landed: S(0,0) may fly
      wave_sync();
      compute_unit(Z{}, O{});
      drain_unit(Z{}, O{}, none);
    }
  } else if constexpr (MODE == BWD_DOWN) {
    // dH -> dG = dH U sig(G) (1 + G (1 - sig(G))), dU = dH G sig(G); a row of
    // dGU is [dG (f) | dU (f)]. Column groups of 64 (NB = 1: 32).
    constexpr int GC = NB >= 2 ? 64 : 32;
    constexpr int JG = NB >= 2 ? 2 : 1;  // 32-column blocks per group
    const int64_t ld = p.ldc * 2, lds_ = static_cast<int64_t>(p.f) * 2;
    static_for<NB / JG>([&](auto JP) {
      const int col0 = n0 + wn * WN + JP * 64;
      // Saved G, U of this group -> staging tiles 0, 1 (rows past the end read 0).
      const int64_t sbase = (static_cast<int64_t>(mrow) * p.f + col0) * 2;
      const int64_t sbytes = static_cast<int64_t>(rows) * p.f * 2;
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        const auto rs = make_rsrc(static_cast<const char*>(sl ? p.e1 : p.e0) + sbase, sbytes);
        const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(wa + sl * kSlot));
#pragma unroll
        for (int t = 0; t < WM / 8; ++t) {
          const int r = t * 8 + (lane >> 3);
          const int c = (lane & 7) ^ ((r >> 1) & 7);   // logical chunk held by this lane's slot
          const uint32_t voff = (c * 8 < GC) ? static_cast<uint32_t>(r * lds_ + c * 16) : 0x80000000u;
          load_lds16(rs, voff, dst + t * 1024);
        }
      }
      wait_vmcnt<0>();
      wave_sync();
      static_for<MB>([&](auto I) {
        static_for<JG>([&](auto JJ) {
          static_for<4>([&](auto Q) {
            constexpr int j = JP * JG + JJ;
            const int r = I * 32 + l32, col = JJ * 32 + 8 * Q + 4 * hl;
            float g[4], u[4], dg[4], du[4];
            unpack4(get4(0, r, col), g);
            unpack4(get4(1, r, col), u);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const float dh = acc[j][I][4 * Q + c];
              const float sg = sigmoid_f(g[c]);
              du[c] = dh * g[c] * sg;
              dg[c] = dh * u[c] * sg * (1.0f + g[c] * (1.0f - sg));
            }
            put4(0, r, col, pack4(dg[0], dg[1], dg[2], dg[3]));
            put4(1, r, col, pack4(du[0], du[1], du[2], du[3]));
          });
        });
      });
      char* C = static_cast<char*>(p.c0) + (static_cast<int64_t>(mrow) * p.ldc + col0) * 2;
      flush(0, C, ld, rows, GC);
      flush(1, C + static_cast<int64_t>(p.f) * 2, ld, rows, GC);
    });
  } else {
    // FWD_DOWN, BWD_GU: C[row][n]; WGRAD: C[e][m][n], columns >= f of the
    // gate|up weight gradient go to the second output (dw_up).
    char* out = static_cast<char*>(p.c0);
    int cn0 = n0;
    if constexpr (MODE == WGRAD) {
      if (p.c1 != nullptr && n0 >= p.f) { out = static_cast<char*>(p.c1); cn0 = n0 - p.f; }
      out += static_cast<int64_t>(e) * p.cstride * 2;
    }
    constexpr int GC = NB >= 2 ? 64 : 32;
    constexpr int JG = NB >= 2 ? 2 : 1;
    const int64_t ld = p.ldc * 2;
    static_for<NB / JG>([&](auto JP) {
      static_for<MB>([&](auto I) {
        static_for<JG>([&](auto JJ) {
          static_for<4>([&](auto Q) {
            put4(JP & 1, I * 32 + l32, JJ * 32 + 8 * Q + 4 * hl, acc4(JP * JG + JJ, I, Q));
          });
        });
      });
      const int col0 = cn0 + wn * WN + JP * 64;
      flush(JP & 1, out + (static_cast<int64_t>(mrow) * p.ldc + col0) * 2, ld, rows, GC);
    });
  }
}

}  // namespace gemm
}  // namespace moe
