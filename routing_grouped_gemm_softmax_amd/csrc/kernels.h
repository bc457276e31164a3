// Internal launcher declarations shared by the kernel files and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct FfnArgs {
  int S, d, f, E;
  const int32_t* offsets;
  const void* xp;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  // forward outputs / saved activations
  void* G;
  void* U;
  void* H;
  void* o;
  // backward
  const void* d_o;
  void* dgu;      // [S][2f] workspace
  void* dxp;
  void* dw_gate;
  void* dw_up;
  void* dw_down;
  // MXFP8: the save-buffer region after the blocked G, U planes that the
  // forward fills with the backward's quantised weight copies and H's
  // token-major operand (ffn_mx_save_extra bytes). G, U are then the blocked
  // planes (ffn_mx_gu_plane bytes each) and H is unused.
  void* mx_save;
  // MXFP8, optional: the operand images of xp (mx_row_images layout) and d_o
  // (mx_dout_image layout) that moe_dispatch / moe_combine_bwd already wrote;
  // NULL = quantise here. With xp_mx, xp is not read (and may be null).
  const void* xp_mx;
  const void* d_o_mx;
  // Activation recompute: the forward keeps G, U, H (MXFP8: G, U and H's
  // images) in its workspace; the backward recomputes them (into the G, U, H
  // pointers) first.
  bool recompute;
};

// Kernel timing hook (moe_kernel_timer): the launcher of grouped-GEMM step
// `mode` calls ktimer_begin before its launch(es) and ktimer_end after.
void ktimer_begin(int mode, hipStream_t s);
void ktimer_end(int mode, hipStream_t s);

hipError_t launch_ffn_fwd(const FfnArgs& a, bool is_f32, hipStream_t s);
hipError_t launch_ffn_bwd(const FfnArgs& a, bool is_f32, hipStream_t s);

// Router (route.hip)
hipError_t launch_route(const void* x, const void* w_router, bool is_f32, int T, int d, int E, int k,
                        float* logits, int32_t* topk_idx, float* topk_gate, hipStream_t s);
size_t route_bwd_workspace(int T, int d, int E);
hipError_t launch_route_bwd(const void* x, const int32_t* topk_idx, const float* topk_gate,
                            const float* dgate, bool is_f32, int T, int d, int E, int k,
                            float* dlogits, void* dw_router, void* ws, hipStream_t s);

// bf16 router on the matrix cores (route_bf16.hip)
size_t route_bf16_workspace(int d, int E);
hipError_t launch_route_bf16(const void* x, const void* w_router, int T, int d, int E, int k, float* logits,
                             int32_t* topk_idx, float* topk_gate, void* ws, hipStream_t s);
size_t route_bwd_bf16_workspace(int T, int d, int E);
hipError_t launch_route_bwd_bf16(const void* x, const int32_t* topk_idx, const float* topk_gate, const float* dgate,
                                 int T, int d, int E, int k, float* dlogits, void* dw_router, void* ws,
                                 hipStream_t s);

// Dispatch / combine (dispatch.hip)
size_t dispatch_workspace(int T, int E);
hipError_t launch_dispatch(const void* x, const int32_t* topk_idx, int elem_bytes, int T, int d,
                           int E, int k, int32_t* counts, int32_t* offsets, int32_t* row_of_slot,
                           int32_t* token_of_row, void* xp, void* ws, hipStream_t s);
hipError_t launch_combine(const void* o, const float* gate, const int32_t* row_of_slot, bool is_f32,
                          int T, int d, int k, void* y, hipStream_t s);
// kind: 0 fp32 layer, 1 bf16 layer, 2 MXFP8 layer (bf16 dy and o, fp32 d_o).
hipError_t launch_combine_bwd(const void* dy, const void* o, const float* gate,
                              const int32_t* row_of_slot, int kind, int T, int d, int k,
                              void* d_o, float* dgate, hipStream_t s);
size_t dispatch_bwd_workspace(int d, int E, bool is_f32);
hipError_t launch_dispatch_bwd(const void* dxp, const int32_t* row_of_slot, const float* dlogits,
                               const void* w_router, bool is_f32, int T, int d, int E, int k,
                               void* dx, void* ws, hipStream_t s);

// Expert-load diagnostics from the routed counts (dispatch.hip): 8 doubles.
hipError_t launch_load_stats(const int32_t* counts, int E, double* out, hipStream_t s);

// MXFP8 operand image of a bf16 [rows][cols] matrix quantised along cols, in
// the grouped GEMM's A-operand layout: E4M3 codes [rows][cols], then E8M0
// scales [cols/64][rows][2]. Each part starts 256-byte aligned and keeps 16
// bytes of slack (a scale tile of a ragged row range is read up to the next
// whole dword).
struct MxImage {
  uint8_t* q;
  uint8_t* s;
};
inline size_t mx_part_bytes(size_t n) { return (n + 16 + 255) & ~static_cast<size_t>(255); }
inline size_t mx_image_bytes(int64_t rows, int64_t cols) {
  const size_t n = static_cast<size_t>(rows) * static_cast<size_t>(cols);
  return mx_part_bytes(n) + mx_part_bytes(n / 32);
}
inline MxImage mx_image(const void* base, int64_t rows, int64_t cols) {
  uint8_t* p = static_cast<uint8_t*>(const_cast<void*>(base));
  return MxImage{p, p + mx_part_bytes(static_cast<size_t>(rows) * static_cast<size_t>(cols))};
}

// The two MXFP8 images of an MXFP8 layer's expert-ordered row matrix
// [S][d] (xp, dO), one per GEMM that reads it: the K-major image (mx_image
// layout, a row operand) followed by the token-major one (codes [d][P],
// scales [P/64][d][2], every expert's rows padded to a multiple of 64
// starting at its padded offset: a weight gradient's operand).
inline int64_t mx_padded_rows(int64_t S, int64_t E) { return (S + 63 * E + 63) / 64 * 64; }
struct MxRowImages {
  MxImage k;  // [S][d] along d
  MxImage t;  // [d][P] along each expert's tokens
};
inline size_t mx_row_images_bytes(int64_t S, int64_t d, int64_t E) {
  const size_t pd = static_cast<size_t>(mx_padded_rows(S, E)) * static_cast<size_t>(d);
  return mx_image_bytes(S, d) + mx_part_bytes(pd) + mx_part_bytes(pd / 32);
}
inline MxRowImages mx_row_images(const void* base, int64_t S, int64_t d, int64_t E) {
  uint8_t* t = static_cast<uint8_t*>(const_cast<void*>(base)) + mx_image_bytes(S, d);
  const size_t pd = static_cast<size_t>(mx_padded_rows(S, E)) * static_cast<size_t>(d);
  return MxRowImages{mx_image(base, S, d), MxImage{t, t + mx_part_bytes(pd)}};
}

// Dispatch that writes xp's two images (and xp's bf16 rows unless xp is
// null) from x directly; d = cols, S = T k rows.
hipError_t launch_dispatch_mx(const void* x, const int32_t* topk_idx, int T, int d, int E, int k,
                              int32_t* counts, int32_t* offsets, int32_t* row_of_slot,
                              int32_t* token_of_row, void* xp, MxRowImages xp_mx, void* ws, hipStream_t s);
// dO's images, then the gate of every expert row ([S] fp32), which the
// combine backward's first pass writes for its second.
inline size_t mx_dout_image_bytes(int64_t S, int64_t d, int64_t E) {
  return mx_row_images_bytes(S, d, E) + mx_part_bytes(static_cast<size_t>(S) * 4);
}
struct MxDoutImage {
  MxImage k;           // [S][d] along d
  MxImage t;           // [d][P] along each expert's tokens
  float* gate_of_row;  // [S]
};
inline MxDoutImage mx_dout_image(const void* base, int64_t S, int64_t d, int64_t E) {
  const MxRowImages r = mx_row_images(base, S, d, E);
  uint8_t* g = static_cast<uint8_t*>(const_cast<void*>(base)) + mx_row_images_bytes(S, d, E);
  return MxDoutImage{r.k, r.t, reinterpret_cast<float*>(g)};
}
// d_o (fp32) may be null: then only the images are written. dO = gate * dy
// in fp32 is decided once per element and both images encode that value.
hipError_t launch_combine_bwd_mx(const void* dy, const void* o, const float* gate,
                                 const int32_t* row_of_slot, const int32_t* token_of_row,
                                 const int32_t* offsets, int T, int d, int E, int k, void* d_o,
                                 MxDoutImage d_o_mx, float* dgate, hipStream_t s);

// Dispatch whose workspace is the library's own device array (one per GPU,
// dispatch_noalloc_max() bytes) instead of a caller buffer: no allocation.
// xp_mx.k.q == nullptr: no MXFP8 images. Returns hipErrorInvalidValue when the
// shape needs more than the array holds, or when hipGetSymbolAddress fails.
size_t dispatch_noalloc_max();
hipError_t launch_dispatch_noalloc(const void* x, const int32_t* topk_idx, int elem_bytes, int T, int d, int E,
                                   int k, int32_t* counts, int32_t* offsets, int32_t* row_of_slot,
                                   int32_t* token_of_row, void* xp, MxRowImages xp_mx, hipStream_t s);

// MXFP8 (mxfp8.hip)
hipError_t launch_mxfp8_quantize(const void* in, int64_t rows, int64_t cols, int axis, uint8_t* q,
                                 uint8_t* scale, hipStream_t s);
hipError_t launch_mxfp8_quantize_grouped(const void* in, int64_t rows, int64_t cols, const int32_t* off, int G,
                                         uint8_t* q, uint8_t* scale, hipStream_t s);
// Into the grouped GEMM's layout (E4M3 K-major, scales [K/64][rows][2]):
// K along the columns of in [R][C] (batched)...
hipError_t launch_mx_kmajor(const void* in, int R, int C, int batches, int64_t in_bstride, uint8_t* q,
                            int64_t q_bstride, uint8_t* s, int64_t s_bstride, hipStream_t st);
// ... or K along the rows, transposed to q [C][P], blocked inside the row
// groups of offsets (padded to 64 rows as poff says), or one group if NULL.
// blk: the block table of launch_mx_blocks (nullptr: one group of R rows).
// qk, sk (optional, one group only): also write the columns-blocked copy in
// launch_mx_kmajor's layout from the same read.
hipError_t launch_mx_tgroup(const void* in, int R, int C, const void* blk, int batches, int64_t in_bstride,
                            uint8_t* q, int64_t P, int64_t q_bstride, uint8_t* s, int64_t s_bstride, hipStream_t st,
                            uint8_t* qk = nullptr, uint8_t* sk = nullptr);
// The fp32 forms (an MXFP8 layer's fp32 operands H, dO, dG | dU): K along the
// columns of in [R][C] (one batch), and K along the rows inside the row
// groups of blk (one batch), each encoded exactly from the fp32 values.
hipError_t launch_mx_kmajor_f32(const void* in, int R, int C, uint8_t* q, uint8_t* s, hipStream_t st);
hipError_t launch_mx_tgroup_f32(const void* in, int R, int C, const void* blk, uint8_t* q, int64_t P, uint8_t* s,
                                hipStream_t st);
// Block table of the grouped transposing quantiser (P/64 entries of 8 bytes).
hipError_t launch_mx_blocks(const int32_t* offsets, const int32_t* poff, int E, int64_t P, void* blk, hipStream_t st);
hipError_t launch_mx_poff(const int32_t* offsets, int E, int32_t* poff, hipStream_t st);

// MXFP8 expert FFN (ffn_mx.hip): workspace bytes and launch.
size_t ffn_mx_fwd_workspace(int S, int d, int f, int E, bool recompute);
// Extra save-buffer bytes of an MXFP8 layer (the backward's weight copies).
size_t ffn_mx_save_extra(int S, int d, int f, int E, bool recompute);
// Bytes of one blocked G or U plane of an MXFP8 layer (24-bit words: fp32
// with 16 mantissa bits): rows padded to 64 per expert, 32 x 32 blocks of
// 3 KB in accumulator lane order.
size_t ffn_mx_gu_plane(int S, int f, int E);
size_t ffn_mx_bwd_workspace(int S, int d, int f, int E, bool recompute);
hipError_t launch_ffn_mx_fwd(const FfnArgs& a, void* ws, hipStream_t s);
hipError_t launch_ffn_mx_bwd(const FfnArgs& a, void* ws, hipStream_t s);

}  // namespace moe
