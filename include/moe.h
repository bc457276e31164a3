/*
 * moe.h — C ABI of the MI355X (gfx950) MoE expert-layer library, libmoe.so.
 *
 * The layer, on one GPU's share of T tokens (forward, then backward):
 *   route     logits = x W_r; softmax; top-k experts per token; gates
 *             renormalised over the chosen k            [moe_route]
 *   dispatch  per-expert histogram and prefix scan on the device, then a
 *             stable placement of every routed token row into one contiguous
 *             per-expert input buffer xp                 [moe_dispatch]
 *   experts   grouped SwiGLU FFN over the per-expert row ranges, scheduled on
 *             the device from the offsets array          [moe_grouped_ffn_fwd]
 *   combine   y[t] = sum_j gate[t,j] * o[row_of_slot[t,j]] [moe_combine]
 *   backward  moe_combine_bwd, moe_grouped_ffn_bwd, moe_route_bwd,
 *             moe_dispatch_bwd; MXFP8 operands via mxfp8_quantize, or
 *             written by dispatch and combine backward as MXFP8 images.
 *
 * Sources. The pages that describe the method say, in words only:
 *  - each token activates 4 of the E experts — "Olmo-core 3 é lançado com
 *    infraestrutura para treinar modelos MoE" (noticiarioia.com), section
 *    "Mudança de arquitetura e ganhos de desempenho"; "Ai2 rilascia
 *    Olmo-Core 3, stack di addestramento aperto per MoE da trilioni di
 *    parametri" (unite.ai), introduction;
 *  - routed data is written straight into the experts' input buffers, the
 *    routing metadata stays on the GPU so the CPU enqueues work without
 *    waiting for copies back, and the expert matmuls run as a grouped GEMM
 *    scheduled on the device — "Olmo-core 3 escala el entrenamiento de
 *    mixture-of-experts a billones de parámetros" (bytechap.com), section
 *    "Cómo funciona"; unite.ai page, section "Parallelismo, precisione e
 *    tecniche di memoria";
 *  - MXFP8 is supported — noticiarioia.com page, section "Otimizações e testes
 *    em escala de trilhões"; unite.ai page, section "Parallelismo, precisione
 *    e tecniche di memoria".
 * The layer specification fixes what the pages leave open: softmax routing,
 * top-k gates renormalised to sum to 1 (ties in the logits go to the lower
 * expert index), SwiGLU experts silu(x W_gate) * (x W_up) then W_down, no
 * biases, no capacity limit, no dropped tokens, gates applied after the FFN.
 *
 * Conventions (all entry points):
 *  - Every pointer argument is DEVICE memory owned by the caller unless
 *    stated otherwise; the library never allocates, frees or keeps it.
 *  - `stream` is a hipStream_t (NULL = the default stream). Calls only
 *    enqueue work: no host synchronisation, no device-to-host copy. Counts,
 *    offsets and the permutation never leave the device.
 *  - Tensors are dense row-major. Sizes are int64_t. Floating tensors are in
 *    the layer dtype `shape->dtype` (MOE_F32 or MOE_BF16; MXFP8 layers keep
 *    bf16 inputs and outputs) unless the argument says fp32. MXFP8 layers
 *    decide every E4M3 code of a computed GEMM operand on its fp32 value
 *    rather than on a bf16 rounding of it: d_o is fp32, G and U (save
 *    buffer) are fp32 rounded to 16 mantissa bits, and H and dG | dU exist
 *    only as the E4M3 operands the GEMM epilogues write from fp32 values in
 *    registers. Weights:
 *    w_router [d][E]; w_gate, w_up [E][d][f]; w_down [E][f][d].
 *  - Row counts: S = T*k routed rows. Index tensors are int32.
 *  - Validation is host-side only and never reads device memory. Errors:
 *    MOE_ERR_INVALID_ARG (null pointer, bad sizes, k > E), MOE_ERR_UNSUPPORTED
 *    (d or f not a multiple of 64, E > 256, k > 8, dtype not available for
 *    the call, T*k above 2^30, d or f above 65536; MXFP8 layers: T*k + 63 E
 *    + 63 of 2^23 or more), MOE_ERR_MISALIGNED (a tensor pointer not 16-byte
 *    aligned),
 *    MOE_ERR_WORKSPACE (workspace/save buffer smaller than the query says),
 *    MOE_ERR_HIP (a launch failed; the message names the HIP error).
 *    On error nothing is enqueued. moe_last_error_message() gives a
 *    thread-local description of the last failure.
 *  - Results are deterministic: no floating-point atomics; reruns on the same
 *    inputs are bit-identical.
 *  - Calls that share a workspace or save buffer must be ordered on one
 *    stream (or otherwise serialised) by the caller.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 8

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,
  MOE_ERR_UNSUPPORTED = -2,
  MOE_ERR_MISALIGNED = -3,
  MOE_ERR_WORKSPACE = -4,
  MOE_ERR_HIP = -5
};

enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP8 = 2 };

/* Operation ids for moe_workspace_size. */
enum moe_op {
  MOE_OP_ROUTE = 0,
  MOE_OP_DISPATCH = 1,
  MOE_OP_FFN_FWD = 2,
  MOE_OP_FFN_BWD = 3,
  MOE_OP_ROUTE_BWD = 4,
  MOE_OP_DISPATCH_BWD = 5
};

/* Device-side status bits, read back with moe_read_device_status. */
enum moe_device_status { MOE_DEV_OK = 0, MOE_DEV_BAD_EXPERT = 1, MOE_DEV_DUP_EXPERT = 2 };

/* Layer options, bits of moe_shape.flags. */
enum moe_flags {
  /* Activation recompute. moe_grouped_ffn_fwd keeps G, U, H in its
   * workspace only (MXFP8 layers: G, U and H's token-major operand) and saves
   * no activations (moe_save_size is 0 for fp32 and bf16 layers; MXFP8 layers
   * keep only the dgrad weight copies there); moe_grouped_ffn_bwd runs the
   * gate/up grouped GEMM again from xp into its own workspace before the
   * backward GEMMs (MXFP8 layers first quantise w_gate, w_up in that GEMM's
   * layout again, and xp along d unless xp_mx holds its image). This trades
   * one extra 4*S*d*f-flop GEMM per step for the activations that otherwise
   * stay live between forward and backward. Results are bit-identical to the
   * layer without the flag. Passage: unite.ai page, "Parallelismo,
   * precisione e tecniche di memoria" (recomputing activations cuts
   * activation memory at some cost in throughput). */
  MOE_FLAG_RECOMPUTE = 1
};

typedef struct moe_shape {
  int64_t T;     /* tokens on this GPU (>= 1) */
  int64_t d;     /* model width (multiple of 64) */
  int64_t E;     /* experts (1..256) */
  int64_t k;     /* experts per token (1..min(E, 8)) */
  int64_t f;     /* expert FFN width d_ff (multiple of 64) */
  int32_t dtype; /* enum moe_dtype */
  int32_t flags; /* enum moe_flags bits (0: none); other bits must be 0 */
} moe_shape;

int moe_abi_version(void);
const char* moe_status_string(int status);
const char* moe_last_error_message(void);

/* Bytes of scratch workspace `op` needs for `shape` (0 if none). Never fails;
 * returns (size_t)-1 for an invalid shape. Workspaces carry no state between
 * calls except the device status word written by moe_dispatch. */
size_t moe_workspace_size(int op, const moe_shape* shape);

/* Bytes of the buffer that moe_grouped_ffn_fwd fills with what the backward
 * needs. fp32 and bf16 layers: G, U, H (three [S][f] tensors in the layer
 * dtype). MXFP8 layers: G and U as fp32 rounded to 16 mantissa bits (to
 * nearest, ties away from zero) and kept as 24-bit words, each in a blocked
 * layout (every expert's rows padded to a multiple of 64; 32 x 32 blocks of
 * 3 KB), H only
 * as the W_down weight gradient's E4M3 operand (blocked along each expert's
 * tokens), and the E4M3 copies (with their E8M0 scales) of w_gate, w_up and
 * w_down in the layouts of the backward's dgrad GEMMs, which the forward
 * writes from the same read that quantises its own copies. The layout of
 * the MXFP8 buffer is internal to the library.
 * 0 with MOE_FLAG_RECOMPUTE (then `save` may be NULL in the FFN calls). */
size_t moe_save_size(const moe_shape* shape);

/* Bytes of the MXFP8 image of a matrix [rows][cols] quantised along
 * cols (cols % 64 == 0), in the layout the MXFP8 grouped GEMMs read their
 * row operand in: rows*cols E4M3 codes, row-major; then the E8M0 scales as
 * [cols/64][rows][2] (the two 32-blocks of each 64-column piece of a row side
 * by side). Each part starts 256-byte aligned and is followed by at least 16
 * bytes of slack. Codes and scales are those of mxfp8_quantize with axis 0
 * (the OCP MX v1.0 conversion) of the values the image is made from.
 * moe_dispatch and moe_combine_bwd write images in this layout of xp and
 * d_o ([S][d]) for MXFP8 layers (as the first part of moe_mx_xp_image_size
 * and moe_mx_dout_image_size buffers), and the grouped FFN calls read them,
 * so neither row matrix is read again only to be quantised. Returns (size_t)-1 for
 * rows < 1 or cols not a positive multiple of 64. */
size_t moe_mx_image_size(int64_t rows, int64_t cols);

/* Router: logits[T][E] (fp32) = x[T][d] · w_router[d][E] with fp32
 * accumulation; then per token the k largest logits in decreasing order,
 * equal values to the lower expert index, written to topk_idx[T][k];
 * topk_gate[T][k] (fp32) = softmax over the k chosen logits, which equals the
 * full softmax renormalised over the chosen set.
 * ws: moe_workspace_size(MOE_OP_ROUTE) bytes (bf16 layers: a transposed copy
 * of w_router; 0 for fp32 layers, where ws may be NULL).
 * Passage: noticiarioia.com page, "Mudança de arquitetura e ganhos de
 * desempenho" (4 of E experts per token); bytechap.com page, "Cómo funciona"
 * (routing kept on the GPU). */
int moe_route(const void* x, const void* w_router, const moe_shape* shape,
              float* logits_out, int32_t* topk_idx_out, float* topk_gate_out,
              void* ws, size_t ws_bytes, void* stream);

/* Dispatch: counts[E] = rows per expert, offsets[E+1] = exclusive prefix sum
 * (offsets[E] = S), all computed on the device. Expert e's rows are
 * offsets[e]..offsets[e+1]-1 and hold its tokens in increasing token order;
 * row_of_slot[T][k] gives the row of every (token, slot); token_of_row[S] the
 * inverse; xp[S][d] (layer dtype) is x gathered into that order.
 * An expert id outside [0, E) is not routed (its row_of_slot is -1), and the
 * device status word in `ws` gets MOE_DEV_BAD_EXPERT. A token that names the
 * same expert in two slots sets MOE_DEV_DUP_EXPERT (both slots are routed,
 * to consecutive rows of that expert).
 * xp_mx_out (MXFP8 layers only; NULL to skip): receives the MXFP8 operands
 * of xp for the FFN calls, moe_mx_xp_image_size(shape) bytes, 256-byte
 * aligned: the image along d (moe_mx_image_size(S, d) bytes, the gate/up
 * GEMM's operand) followed by the image along each expert's tokens (the
 * dW_gate | dW_up weight gradient's operand, each expert's rows padded to a
 * multiple of 64), both made from x in one pass over the gathered rows. With
 * xp_mx_out, xp_out may be NULL: then xp's bf16 rows are not written (the
 * MXFP8 FFN calls need only the images). Must be NULL for fp32 and bf16
 * layers.
 * ws: at least moe_workspace_size(MOE_OP_DISPATCH) bytes, 256-byte aligned.
 * Passage: bytechap.com page, "Cómo funciona"; unite.ai page, "Parallelismo,
 * precisione e tecniche di memoria" (rows written straight into the experts'
 * input buffers; routing metadata stays on the GPU). */
int moe_dispatch(const void* x, const int32_t* topk_idx, const moe_shape* shape,
                 int32_t* counts_out, int32_t* offsets_out, int32_t* row_of_slot_out,
                 int32_t* token_of_row_out, void* xp_out, uint8_t* xp_mx_out, void* ws,
                 size_t ws_bytes, void* stream);

/* moe_dispatch for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, outputs and errors as moe_dispatch, minus ws / ws_bytes:
 * the workspace is a 1 MiB array inside the library, one per GPU, held until
 * the process ends. The call allocates and frees nothing. It fails with
 * MOE_ERR_WORKSPACE, enqueuing nothing, when moe_workspace_size(
 * MOE_OP_DISPATCH, shape) exceeds 1 MiB (above 2,064,384 tokens at E = 64,
 * 1,039,872 at E = 128, 521,728 at E = 256), and with MOE_ERR_HIP when
 * `stream` belongs to a device
 * other than the current one. Every call on one GPU shares that GPU's
 * array: calls that may overlap there (other streams, other host threads)
 * race, so the caller serialises them. The device status word lives in the
 * array and cannot be read back; callers that need it use moe_dispatch. */
int moe_dispatch_noalloc(const void* x, const int32_t* topk_idx, const moe_shape* shape,
                         int32_t* counts_out, int32_t* offsets_out, int32_t* row_of_slot_out,
                         int32_t* token_of_row_out, void* xp_out, uint8_t* xp_mx_out, void* stream);

/* Reads the device status word that the last moe_dispatch on `ws` wrote.
 * Synchronises `stream`. For debugging and tests; returns MOE_DEV_* bits
 * (0 when every token names k distinct experts in [0, E)), or a negative
 * moe_status on failure. */
int moe_read_device_status(const void* ws, void* stream);

/* Grouped SwiGLU FFN forward over the per-expert row ranges in `offsets`
 * (device array, E+1 entries; never read by the host). For expert e and each
 * of its rows r: G = xp[r] · w_gate[e], U = xp[r] · w_up[e],
 * H = silu(G) * U with silu(z) = z / (1 + exp(-z)), o[r] = H · w_down[e];
 * fp32 accumulation, one rounding to the layer dtype per stored value.
 * save (>= moe_save_size bytes) receives what the backward needs (see
 * moe_save_size).
 * ws: moe_workspace_size(MOE_OP_FFN_FWD) bytes (may be 0 -> NULL allowed).
 * xp_mx (MXFP8 layers only; NULL = quantise xp here): the MXFP8 operands of
 * xp that moe_dispatch wrote (moe_mx_xp_image_size bytes); it must hold the
 * current xp's codes, and with it xp is not read and may be NULL.
 * Passage: bytechap.com page, "Cómo funciona" (grouped GEMM combining many
 * small expert computations); unite.ai page, "Parallelismo, precisione e
 * tecniche di memoria" (matmuls scheduled on the device). */
int moe_grouped_ffn_fwd(const void* xp, const uint8_t* xp_mx, const void* w_gate, const void* w_up,
                        const void* w_down, const int32_t* offsets, const moe_shape* shape,
                        void* save, size_t save_bytes, void* o_out, void* ws, size_t ws_bytes,
                        void* stream);

/* Combine: y[t] = sum_j topk_gate[t,j] * o[row_of_slot[t,j]], summed in fp32
 * in slot order, one rounding. Slots with row -1 contribute nothing.
 * Passage: the gate-weighted combine of the layer specification. */
int moe_combine(const void* o, const float* topk_gate, const int32_t* row_of_slot,
                const moe_shape* shape, void* y_out, void* stream);

/* Combine backward: d_o[row_of_slot[t,j]] = topk_gate[t,j] * dy[t] (layer
 * dtype; fp32 for MXFP8 layers, the fp32 product) and dgate[t,j] (fp32) =
 * <dy[t], o[row_of_slot[t,j]]>, summed in fp32.
 * d_o_mx_out (MXFP8 layers only; NULL to skip): receives the MXFP8 operands
 * of d_o for the FFN backward, moe_mx_dout_image_size(shape) bytes, 256-byte
 * aligned: the image along d (moe_mx_image_size(S, d) bytes, the down-dgrad
 * GEMM's operand) followed by the image along each expert's tokens (the W_down
 * weight gradient's operand, each expert's rows padded to a multiple of 64).
 * Both encode the fp32 products. With d_o_mx_out, token_of_row and offsets
 * (moe_dispatch's outputs) are required, and d_o_out may be NULL: then no
 * fp32 d_o is written (the FFN backward needs only the image).
 * token_of_row, offsets: ignored (may be NULL) without d_o_mx_out.
 * Passage: the gate-weighted combine of the layer specification ("a
 * gate-weighted combine back to token order", forward and backward); the
 * MXFP8 image is the data moved to the experts in MXFP8 (unite.ai page,
 * "Parallelismo, precisione e tecniche di memoria"). */
int moe_combine_bwd(const void* dy, const void* o, const float* topk_gate,
                    const int32_t* row_of_slot, const int32_t* token_of_row,
                    const int32_t* offsets, const moe_shape* shape, void* d_o_out,
                    uint8_t* d_o_mx_out, float* dgate_out, void* stream);

/* Bytes of the d_o_mx buffer of an MXFP8 layer (moe_combine_bwd,
 * moe_grouped_ffn_bwd); (size_t)-1 for an invalid shape or a non-MXFP8 one. */
size_t moe_mx_dout_image_size(const moe_shape* shape);

/* Bytes of the xp_mx buffer of an MXFP8 layer (moe_dispatch,
 * moe_dispatch_noalloc, moe_grouped_ffn_fwd, moe_grouped_ffn_bwd); (size_t)-1
 * for an invalid shape or a non-MXFP8 one. */
size_t moe_mx_xp_image_size(const moe_shape* shape);

/* Grouped FFN backward, per expert e on its rows:
 *   dH = d_o · w_down[e]^T;  dU = dH * silu(G);
 *   dG = dH * U * sig(G) * (1 + G (1 - sig(G)))   (from the saved G, U, H)
 *   dxp = dG · w_gate[e]^T + dU · w_up[e]^T
 *   dw_down[e] = H^T · d_o;  dw_gate[e] = xp^T · dG;  dw_up[e] = xp^T · dU
 * Weight gradients of experts with no rows are written as zeros. All outputs
 * in the layer dtype (d_o is fp32 for MXFP8 layers, as moe_combine_bwd
 * writes it). ws: moe_workspace_size(MOE_OP_FFN_BWD) bytes; for fp32 and
 * bf16 layers it starts with the dG | dU rows ([S][2f], layer dtype).
 * MXFP8 layers quantise every operand along its GEMM's K (the weight
 * gradients along each expert's tokens, the range padded with zero rows).
 * d_o_mx (MXFP8 layers only; NULL = quantise d_o here): the MXFP8 operands
 * of d_o that moe_combine_bwd wrote (moe_mx_dout_image_size bytes); with it
 * d_o is not read and may be NULL.
 * xp_mx (MXFP8 layers only; NULL = quantise xp here): the MXFP8 operands of
 * xp that moe_dispatch wrote, as passed to the forward; with it xp is not
 * read and may be NULL (recompute reads the image along d).
 * Passage: the backward of the expert FFN (dgrad and wgrad grouped GEMMs) of
 * the layer specification; the grouped, device-scheduled GEMM of the
 * bytechap.com page, "Cómo funciona", and of the unite.ai page,
 * "Parallelismo, precisione e tecniche di memoria". */
int moe_grouped_ffn_bwd(const void* d_o, const uint8_t* d_o_mx, const void* xp, const uint8_t* xp_mx,
                        const void* w_gate, const void* w_up, const void* w_down,
                        const int32_t* offsets, const moe_shape* shape,
                        const void* save, void* dxp_out, void* dw_gate_out, void* dw_up_out,
                        void* dw_down_out, void* ws, size_t ws_bytes, void* stream);

/* Router backward through the renormalised top-k softmax:
 *   dlogits[t,i] = g_ti (dgate_ti - sum_j g_tj dgate_tj) for i in the chosen
 *   set of token t, 0 elsewhere (fp32 [T][E]);
 *   dw_router[d][E] (layer dtype) = x^T · dlogits, reduced over T in a fixed
 *   order (deterministic split over token blocks).
 * ws: moe_workspace_size(MOE_OP_ROUTE_BWD) bytes.
 * Passage: the router gradient of the layer specification (softmax over the
 * router logits with the top-k gates renormalised, differentiated); the
 * router itself: noticiarioia.com page, "Mudança de arquitetura e ganhos de
 * desempenho" (4 of E experts per token). */
int moe_route_bwd(const void* x, const void* w_router, const int32_t* topk_idx,
                  const float* topk_gate, const float* dgate, const moe_shape* shape,
                  float* dlogits_out, void* dw_router_out, void* ws, size_t ws_bytes,
                  void* stream);

/* Dispatch backward: dx[t] = sum_j dxp[row_of_slot[t,j]]
 * (+ sum_e dlogits[t,e] * w_router[:,e] over every non-zero dlogits[t,e]
 * when dlogits and w_router are both non-NULL), accumulated in fp32 (the k
 * rows in slot order, then the router columns in increasing expert order),
 * one rounding to the layer dtype. dlogits may be dense; rows with at most
 * k non-zeros (as moe_route_bwd writes them) take a faster path with the
 * same result. Slots with row -1 contribute nothing.
 * ws: moe_workspace_size(MOE_OP_DISPATCH_BWD) bytes (needed only with the
 * router term).
 * Passage: the adjoint of the placement of routed rows into the experts'
 * input buffers (bytechap.com page, "Cómo funciona"; unite.ai page,
 * "Parallelismo, precisione e tecniche di memoria"), plus the router term
 * of the layer specification's router gradient. */
int moe_dispatch_bwd(const void* dxp, const int32_t* row_of_slot, const float* dlogits,
                     const void* w_router, const moe_shape* shape, void* dx_out, void* ws,
                     size_t ws_bytes, void* stream);

/* Expert-load diagnostics of one step, computed on the device from the
 * counts[E] that moe_dispatch wrote (device int32; never read by the host).
 * stats_out (device, 8 doubles): [0] max n_e, [1] min n_e, [2] mean S/E,
 * [3] max/mean, [4] entropy -sum_e p_e ln p_e with p_e = n_e / S (nats,
 * 0 ln 0 = 0), [5] entropy / ln E (1 when E = 1), [6] experts with no rows,
 * [7] std/mean of the counts (population std). With S = 0, entries 3, 4, 5
 * and 7 are 0. Deterministic (fixed reduction order). Errors:
 * MOE_ERR_INVALID_ARG for a NULL pointer or E outside 1..256,
 * MOE_ERR_MISALIGNED for a pointer not 16-byte aligned.
 * Passage: bytechap.com page, "Detalles clave"; unite.ai page, "Risultati
 * Documentati" (a routing score meant to favour balance can improve while
 * the real per-expert load becomes less balanced: these figures measure the
 * real load). */
int moe_load_stats(const int32_t* counts, int64_t E, double* stats_out, void* stream);

/* MXFP8 quantisation of a bf16 matrix in_bf16[rows][cols]:
 * axis 0: blocks of 32 consecutive elements along a row (cols % 32 == 0);
 *         scale_out is [rows][cols/32].
 * axis 1: blocks of 32 consecutive rows within a column (rows % 32 == 0);
 *         scale_out is [rows/32][cols].
 * Per block: amax = max |v|; E8M0 scale code c = clamp(floor(log2 amax) - 8
 * + 127, 0, 254) (0 for an all-zero block); q_out = E4M3 ("FN": bias 7, max
 * 448) code of v / 2^(c-127), rounded to nearest even, saturated to +-448,
 * sign kept. q_out has the shape of the input. This is the OCP Microscaling
 * (MX) v1.0 conversion; the pages only say that MXFP8 is used —
 * noticiarioia.com page, "Otimizações e testes em escala de trilhões";
 * unite.ai page, "Parallelismo, precisione e tecniche di memoria".
 * Inputs must be finite. */
int mxfp8_quantize(const void* in_bf16, int64_t rows, int64_t cols, int axis, uint8_t* q_out,
                   uint8_t* scale_out, void* stream);

/* MXFP8 quantisation along rows inside row groups (the layout of a
 * weight-gradient operand, whose K runs over one expert's tokens): blocks of
 * 32 consecutive rows of one column within each group [group_offsets[g],
 * group_offsets[g+1]), a group's last block completed with zero rows, which
 * change no scale. Scale code and element rounding as in mxfp8_quantize.
 * in_bf16 [rows][cols]; q_out [rows][cols] (codes of every row of a group);
 * scale_out [rows/32 + groups][cols], block-major: the blocks of group 0 in
 * row order, then those of group 1, ...; rows past the last block are not
 * written. group_offsets: device int32 [groups + 1], nondecreasing from 0 to
 * rows (never read by the host; values are clamped into [0, rows], so a
 * malformed table gives wrong codes, not an access out of bounds).
 * Errors: MOE_ERR_INVALID_ARG (NULL pointer, rows or cols < 1, groups outside
 * 1..256), MOE_ERR_UNSUPPORTED (rows >= 2^31 or rows * cols > 2^40).
 * Passage: as for mxfp8_quantize; the grouping follows the experts' row
 * ranges of the grouped GEMM (bytechap.com page, "Cómo funciona"). */
int mxfp8_quantize_grouped(const void* in_bf16, int64_t rows, int64_t cols, const int32_t* group_offsets,
                           int64_t groups, uint8_t* q_out, uint8_t* scale_out, void* stream);

/* Grouped-GEMM steps of the expert FFN, for moe_kernel_timer. */
enum moe_gemm_mode {
  MOE_GEMM_FWD_GU = 0,   /* G, U = xp w_gate, xp w_up; H = silu(G) U   */
  MOE_GEMM_FWD_DOWN = 1, /* o = H w_down                                */
  MOE_GEMM_BWD_DOWN = 2, /* dG | dU from d_o w_down^T and the saved G, U */
  MOE_GEMM_BWD_GU = 3,   /* dxp = [dG | dU] [w_gate | w_up]^T           */
  MOE_GEMM_WGRAD = 4     /* dw_down, then [dw_gate | dw_up]: two launches per backward */
};

/* Kernel timing for benchmarks: brackets each of the next launches of one
 * grouped-GEMM step (gemm_mode, any layer dtype) with HIP events that the
 * caller created, recorded on the stream that step runs on, so that each
 * launch's duration can be read with hipEventElapsedTime. start and stop are
 * host arrays of `capacity` hipEvent_t handles; launches past `capacity` are
 * not recorded. Where a step runs as a main launch plus a short quarter-tile
 * launch (a small last round of tiles), one event pair brackets both.
 * capacity 0 (start and stop may then be NULL) disarms the timer. Returns
 * MOE_OK or MOE_ERR_INVALID_ARG (mode out of range, capacity < 0, NULL
 * arrays). Process-wide state: arm, run and read from one thread.
 * For the profiling of this library's own kernels; it is not part of the
 * layer's computation. */
int moe_kernel_timer(int gemm_mode, void* const* start, void* const* stop, int capacity);

/* Event pairs recorded since moe_kernel_timer last armed the timer. */
int moe_kernel_timer_count(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
