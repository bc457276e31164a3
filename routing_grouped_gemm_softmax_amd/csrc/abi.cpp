// C ABI of libmoe.so: host-side validation, workspace sizing and kernel launch.
// Validation never touches device memory; on any error nothing is enqueued.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/moe.h"
#include "kernels.h"

namespace {

thread_local char g_msg[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Bytes of an element of the layer's input and output tensors (MXFP8 layers:
// bf16) and of its stored computed activations G, U, H, dO, dG | dU (MXFP8
// layers keep G, U, H, dO in fp32, so every E4M3 code is decided on the fp32
// value; their dG | dU never leave the down-dgrad epilogue in fp32).
int elem_bytes(int dtype) { return dtype == MOE_F32 ? 4 : 2; }
int act_bytes(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }

// Shape checks shared by every layer entry point.
int check_shape(const moe_shape* s) {
  if (!s) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
  if (s->flags & ~MOE_FLAG_RECOMPUTE) return fail(MOE_ERR_INVALID_ARG, "unknown bits in shape.flags (%d)", s->flags);
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16 && s->dtype != MOE_MXFP8)
    return fail(MOE_ERR_INVALID_ARG, "unknown dtype %d", s->dtype);
  if (s->T < 1 || s->d < 1 || s->E < 1 || s->k < 1 || s->f < 1)
    return fail(MOE_ERR_INVALID_ARG, "T, d, E, k, f must be >= 1 (got %lld %lld %lld %lld %lld)",
                (long long)s->T, (long long)s->d, (long long)s->E, (long long)s->k, (long long)s->f);
  if (s->k > s->E) return fail(MOE_ERR_INVALID_ARG, "k (%lld) > E (%lld)", (long long)s->k, (long long)s->E);
  if (s->E > 256) return fail(MOE_ERR_UNSUPPORTED, "E > 256 is not supported");
  if (s->k > 8) return fail(MOE_ERR_UNSUPPORTED, "k > 8 is not supported");
  if (s->d % 64 || s->f % 64) return fail(MOE_ERR_UNSUPPORTED, "d and f must be multiples of 64");
  // Index arithmetic is 32-bit for row ids and 64-bit for element offsets.
  if (s->T * s->k > (int64_t)1 << 30 || s->d > 65536 || s->f > 65536 || s->T > (int64_t)1 << 28)
    return fail(MOE_ERR_UNSUPPORTED, "sizes beyond the supported range");
  // MXFP8 weight-gradient tiles address 256 rows of a token-major operand
  // (P bytes each, the routed rows padded per expert) through one buffer
  // descriptor and 32-bit offsets: P < 2^23.
  if (s->dtype == MOE_MXFP8 && moe::mx_padded_rows(s->T * s->k, s->E) >= (int64_t)1 << 23)
    return fail(MOE_ERR_UNSUPPORTED, "MXFP8 layers support T*k + 63*E + 63 below 2^23 (got T*k = %lld, E = %lld)",
                (long long)(s->T * s->k), (long long)s->E);
  return MOE_OK;
}

// MXFP8 layers run the grouped GEMMs on E4M3 operands whose slabs are 128
// bytes of K per 32-row block pair; the quantised layouts need d and f to be
// multiples of 128.
int check_ffn_dtype(const moe_shape* s, const char* who) {
  if (s->dtype == MOE_MXFP8 && (s->d % 128 || s->f % 128))
    return fail(MOE_ERR_UNSUPPORTED, "%s: MXFP8 layers need d and f to be multiples of 128", who);
  return MOE_OK;
}

#define CHECK(expr)              \
  do {                           \
    int _rc = (expr);            \
    if (_rc != MOE_OK) return _rc; \
  } while (0)

#define NEED(ptr)                                                                   \
  do {                                                                              \
    if (!(ptr)) return fail(MOE_ERR_INVALID_ARG, "%s: %s is NULL", __func__, #ptr); \
    if (!aligned16(ptr)) return fail(MOE_ERR_MISALIGNED, "%s: %s is not 16-byte aligned", __func__, #ptr); \
  } while (0)

// An optional MXFP8 image argument: MXFP8 layers only, 256-byte aligned.
#define MX_IMAGE_OK(ptr, s)                                                                      \
  do {                                                                                           \
    if ((ptr) != nullptr) {                                                                      \
      if ((s)->dtype != MOE_MXFP8)                                                               \
        return fail(MOE_ERR_INVALID_ARG, "%s: %s is only for MXFP8 layers", __func__, #ptr);     \
      if ((reinterpret_cast<uintptr_t>(ptr) & 255u) != 0)                                        \
        return fail(MOE_ERR_MISALIGNED, "%s: %s is not 256-byte aligned", __func__, #ptr);       \
    }                                                                                            \
  } while (0)

#define LAUNCH(call)                                          \
  do {                                                        \
    hipError_t _e = (call);                                   \
    if (_e != hipSuccess) return hip_fail(_e, __func__);      \
  } while (0)

bool recompute(const moe_shape* s) { return (s->flags & MOE_FLAG_RECOMPUTE) != 0; }

// G, U, H: three [S][f] planes (act_bytes each element); MXFP8 layers keep
// only G and U, as two blocked 24-bit planes over the rows padded per expert.
size_t gu_h_bytes(const moe_shape* s) {
  if (s->dtype == MOE_MXFP8) return 2 * moe::ffn_mx_gu_plane((int)(s->T * s->k), (int)s->f, (int)s->E);
  return ((size_t)3 * s->T * s->k * s->f * act_bytes(s->dtype) + 255) & ~(size_t)255;
}
// dG | dU rows of the backward workspace: [S][2f] (act_bytes each element).
size_t dgu_bytes_for(const moe_shape* s) {
  // MXFP8 layers keep dG | dU only as the E4M3 operands the down-dgrad
  // epilogue writes into their own workspace.
  if (s->dtype == MOE_MXFP8) return 0;
  return ((size_t)s->T * s->k * 2 * s->f * act_bytes(s->dtype) + 255) & ~(size_t)255;
}
// Saved G, U, H planes (none with recompute); MXFP8 layers add the backward's
// quantised weight copies.
size_t save_planes(const moe_shape* s) { return recompute(s) ? 0 : gu_h_bytes(s); }
size_t save_bytes_for(const moe_shape* s) {
  return save_planes(s) + (s->dtype == MOE_MXFP8 ? moe::ffn_mx_save_extra((int)(s->T * s->k), (int)s->d, (int)s->f,
                                                                          (int)s->E, recompute(s))
                                                 : 0);
}
// MXFP8 layers: bytes of the FFN workspaces' own pieces, before the G, U
// planes that recompute places after them.
size_t mx_fwd_bytes(const moe_shape* s) {
  return moe::ffn_mx_fwd_workspace((int)(s->T * s->k), (int)s->d, (int)s->f, (int)s->E, recompute(s));
}
size_t mx_bwd_bytes(const moe_shape* s) {
  return moe::ffn_mx_bwd_workspace((int)(s->T * s->k), (int)s->d, (int)s->f, (int)s->E, recompute(s));
}

// moe_kernel_timer's state: the armed mode (-1: none) and the caller's
// events. The mode is read without the lock on every GEMM launch.
struct KernelTimer {
  std::mutex mu;
  std::vector<hipEvent_t> start, stop;
  int n = 0;
};
KernelTimer& kernel_timer() {
  static KernelTimer t;
  return t;
}
std::atomic<int> g_timer_mode{-1};

}  // namespace

namespace moe {

void ktimer_begin(int mode, hipStream_t s) {
  if (g_timer_mode.load(std::memory_order_acquire) != mode) return;
  KernelTimer& t = kernel_timer();
  std::lock_guard<std::mutex> g(t.mu);
  if (t.n < static_cast<int>(t.start.size())) (void)hipEventRecord(t.start[t.n], s);
}

void ktimer_end(int mode, hipStream_t s) {
  if (g_timer_mode.load(std::memory_order_acquire) != mode) return;
  KernelTimer& t = kernel_timer();
  std::lock_guard<std::mutex> g(t.mu);
  if (t.n < static_cast<int>(t.stop.size())) (void)hipEventRecord(t.stop[t.n++], s);
}

}  // namespace moe

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_MISALIGNED: return "MOE_ERR_MISALIGNED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error_message(void) { return g_msg; }

size_t moe_workspace_size(int op, const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return (size_t)-1;
  const int T = (int)s->T, d = (int)s->d, E = (int)s->E, f = (int)s->f, k = (int)s->k;
  switch (op) {
    case MOE_OP_ROUTE: return s->dtype == MOE_F32 ? 0 : moe::route_bf16_workspace(d, E);
    case MOE_OP_DISPATCH: return moe::dispatch_workspace(T, E);
    case MOE_OP_FFN_FWD: {
      const size_t rec = recompute(s) ? gu_h_bytes(s) : 0;  // recompute: G, U, H live here
      return (s->dtype == MOE_MXFP8 ? mx_fwd_bytes(s) : 0) + rec;
    }
    case MOE_OP_FFN_BWD: {
      const size_t dgu = dgu_bytes_for(s);  // dG|dU rows
      const size_t rec = recompute(s) ? gu_h_bytes(s) : 0;  // recompute: G, U, H after the rest
      return dgu + (s->dtype == MOE_MXFP8 ? mx_bwd_bytes(s) : 0) + rec;
    }
    case MOE_OP_ROUTE_BWD:
      return s->dtype == MOE_F32 ? moe::route_bwd_workspace(T, d, E) : moe::route_bwd_bf16_workspace(T, d, E);
    case MOE_OP_DISPATCH_BWD: return moe::dispatch_bwd_workspace(d, E, s->dtype == MOE_F32);
    default: fail(MOE_ERR_INVALID_ARG, "unknown op %d", op); return (size_t)-1;
  }
}

size_t moe_mx_image_size(int64_t rows, int64_t cols) {
  if (rows < 1 || cols < 64 || cols % 64 || rows * cols > ((int64_t)1 << 40)) {
    fail(MOE_ERR_INVALID_ARG, "moe_mx_image_size: need rows >= 1 and cols a positive multiple of 64");
    return (size_t)-1;
  }
  return moe::mx_image_bytes(rows, cols);
}

size_t moe_save_size(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return (size_t)-1;
  return save_bytes_for(s);
}

int moe_route(const void* x, const void* w_router, const moe_shape* s, float* logits_out, int32_t* topk_idx_out,
              float* topk_gate_out, void* ws, size_t ws_bytes, void* stream) {
  CHECK(check_shape(s));
  NEED(x); NEED(w_router); NEED(logits_out); NEED(topk_idx_out); NEED(topk_gate_out);
  const size_t need = moe_workspace_size(MOE_OP_ROUTE, s);
  if (need) {
    NEED(ws);
    if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "moe_route: workspace %zu < %zu bytes", ws_bytes, need);
  }
  if (s->dtype == MOE_F32)
    LAUNCH(moe::launch_route(x, w_router, true, (int)s->T, (int)s->d, (int)s->E, (int)s->k, logits_out,
                             topk_idx_out, topk_gate_out, as_stream(stream)));
  else
    LAUNCH(moe::launch_route_bf16(x, w_router, (int)s->T, (int)s->d, (int)s->E, (int)s->k, logits_out, topk_idx_out,
                                  topk_gate_out, ws, as_stream(stream)));
  return MOE_OK;
}

int moe_dispatch(const void* x, const int32_t* topk_idx, const moe_shape* s, int32_t* counts_out,
                 int32_t* offsets_out, int32_t* row_of_slot_out, int32_t* token_of_row_out, void* xp_out,
                 uint8_t* xp_mx_out, void* ws, size_t ws_bytes, void* stream) {
  CHECK(check_shape(s));
  NEED(x); NEED(topk_idx); NEED(counts_out); NEED(offsets_out); NEED(row_of_slot_out); NEED(token_of_row_out);
  if (!xp_mx_out) NEED(xp_out);  // with xp's MXFP8 images, the bf16 rows are optional
  NEED(ws);
  MX_IMAGE_OK(xp_mx_out, s);
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(MOE_ERR_MISALIGNED, "moe_dispatch: ws must be 256-byte aligned");
  const size_t need = moe::dispatch_workspace((int)s->T, (int)s->E);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "moe_dispatch: workspace %zu < %zu bytes", ws_bytes, need);
  if (xp_mx_out)
    LAUNCH(moe::launch_dispatch_mx(x, topk_idx, (int)s->T, (int)s->d, (int)s->E, (int)s->k, counts_out, offsets_out,
                                   row_of_slot_out, token_of_row_out, xp_out,
                                   moe::mx_row_images(xp_mx_out, s->T * s->k, s->d, s->E), ws, as_stream(stream)));
  else
    LAUNCH(moe::launch_dispatch(x, topk_idx, elem_bytes(s->dtype), (int)s->T, (int)s->d, (int)s->E, (int)s->k,
                                counts_out, offsets_out, row_of_slot_out, token_of_row_out, xp_out, ws,
                                as_stream(stream)));
  return MOE_OK;
}

int moe_dispatch_noalloc(const void* x, const int32_t* topk_idx, const moe_shape* s, int32_t* counts_out,
                         int32_t* offsets_out, int32_t* row_of_slot_out, int32_t* token_of_row_out, void* xp_out,
                         uint8_t* xp_mx_out, void* stream) {
  CHECK(check_shape(s));
  NEED(x); NEED(topk_idx); NEED(counts_out); NEED(offsets_out); NEED(row_of_slot_out); NEED(token_of_row_out);
  if (!xp_mx_out) NEED(xp_out);
  MX_IMAGE_OK(xp_mx_out, s);
  const size_t need = moe::dispatch_workspace((int)s->T, (int)s->E), have = moe::dispatch_noalloc_max();
  if (need > have)
    return fail(MOE_ERR_WORKSPACE,
                "moe_dispatch_noalloc: this shape needs %zu bytes of scratch; the library's array holds %zu "
                "(use moe_dispatch with a workspace)", need, have);
  moe::MxRowImages im{{nullptr, nullptr}, {nullptr, nullptr}};
  if (xp_mx_out) im = moe::mx_row_images(xp_mx_out, s->T * s->k, s->d, s->E);
  LAUNCH(moe::launch_dispatch_noalloc(x, topk_idx, elem_bytes(s->dtype), (int)s->T, (int)s->d, (int)s->E,
                                      (int)s->k, counts_out, offsets_out, row_of_slot_out, token_of_row_out, xp_out,
                                      im, as_stream(stream)));
  return MOE_OK;
}

int moe_read_device_status(const void* ws, void* stream) {
  if (!ws) return fail(MOE_ERR_INVALID_ARG, "moe_read_device_status: ws is NULL");
  int32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, ws, sizeof(v), hipMemcpyDeviceToHost, as_stream(stream));
  if (e == hipSuccess) e = hipStreamSynchronize(as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "moe_read_device_status");
  return v;
}

int moe_grouped_ffn_fwd(const void* xp, const uint8_t* xp_mx, const void* w_gate, const void* w_up,
                        const void* w_down, const int32_t* offsets, const moe_shape* s, void* save, size_t save_bytes,
                        void* o_out, void* ws, size_t ws_bytes, void* stream) {
  CHECK(check_shape(s));
  CHECK(check_ffn_dtype(s, "moe_grouped_ffn_fwd"));
  if (!xp_mx) NEED(xp);  // with xp's MXFP8 images, xp itself is not read
  NEED(w_gate); NEED(w_up); NEED(w_down); NEED(offsets); NEED(o_out);
  if (save_bytes_for(s) > 0) NEED(save);
  MX_IMAGE_OK(xp_mx, s);
  const size_t need = moe_workspace_size(MOE_OP_FFN_FWD, s);
  if (need) {
    NEED(ws);
    if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "moe_grouped_ffn_fwd: workspace %zu < %zu bytes", ws_bytes, need);
  }
  if (save_bytes < save_bytes_for(s))
    return fail(MOE_ERR_WORKSPACE, "moe_grouped_ffn_fwd: save buffer %zu < %zu bytes", save_bytes, save_bytes_for(s));
  moe::FfnArgs a{};
  a.S = (int)(s->T * s->k); a.d = (int)s->d; a.f = (int)s->f; a.E = (int)s->E;
  a.offsets = offsets; a.xp = xp; a.w_gate = w_gate; a.w_up = w_up; a.w_down = w_down; a.xp_mx = xp_mx;
  const size_t plane = s->dtype == MOE_MXFP8 ? gu_h_bytes(s) / 2 : (size_t)a.S * a.f * act_bytes(s->dtype);
  // G, U, H (MXFP8: blocked G, U): the save buffer, or with recompute the
  // workspace (after the MXFP8 pieces).
  char* gu_h = recompute(s) ? static_cast<char*>(ws) + (s->dtype == MOE_MXFP8 ? mx_fwd_bytes(s) : 0)
                            : static_cast<char*>(save);
  a.G = gu_h; a.U = gu_h + plane; a.H = s->dtype == MOE_MXFP8 ? nullptr : gu_h + 2 * plane;
  a.recompute = recompute(s);
  a.mx_save = static_cast<char*>(save) + save_planes(s);
  a.o = o_out;
  if (s->dtype == MOE_MXFP8)
    LAUNCH(moe::launch_ffn_mx_fwd(a, ws, as_stream(stream)));
  else
    LAUNCH(moe::launch_ffn_fwd(a, s->dtype == MOE_F32, as_stream(stream)));
  return MOE_OK;
}

int moe_combine(const void* o, const float* topk_gate, const int32_t* row_of_slot, const moe_shape* s, void* y_out,
                void* stream) {
  CHECK(check_shape(s));
  NEED(o); NEED(topk_gate); NEED(row_of_slot); NEED(y_out);
  LAUNCH(moe::launch_combine(o, topk_gate, row_of_slot, s->dtype == MOE_F32, (int)s->T, (int)s->d, (int)s->k, y_out,
                             as_stream(stream)));
  return MOE_OK;
}

int moe_combine_bwd(const void* dy, const void* o, const float* topk_gate, const int32_t* row_of_slot,
                    const int32_t* token_of_row, const int32_t* offsets, const moe_shape* s, void* d_o_out,
                    uint8_t* d_o_mx_out, float* dgate_out, void* stream) {
  CHECK(check_shape(s));
  NEED(dy); NEED(o); NEED(topk_gate); NEED(row_of_slot); NEED(dgate_out);
  MX_IMAGE_OK(d_o_mx_out, s);
  if (d_o_mx_out) {
    NEED(token_of_row); NEED(offsets);
    if (d_o_out) NEED(d_o_out);
    LAUNCH(moe::launch_combine_bwd_mx(dy, o, topk_gate, row_of_slot, token_of_row, offsets, (int)s->T, (int)s->d,
                                      (int)s->E, (int)s->k, d_o_out,
                                      moe::mx_dout_image(d_o_mx_out, s->T * s->k, s->d, s->E), dgate_out,
                                      as_stream(stream)));
    return MOE_OK;
  }
  NEED(d_o_out);
  const int kind = s->dtype == MOE_F32 ? 0 : (s->dtype == MOE_BF16 ? 1 : 2);
  LAUNCH(moe::launch_combine_bwd(dy, o, topk_gate, row_of_slot, kind, (int)s->T, (int)s->d, (int)s->k,
                                 d_o_out, dgate_out, as_stream(stream)));
  return MOE_OK;
}

size_t moe_mx_xp_image_size(const moe_shape* s) {
  if (check_shape(s) != MOE_OK || s->dtype != MOE_MXFP8) return (size_t)-1;
  return moe::mx_row_images_bytes(s->T * s->k, s->d, s->E);
}

size_t moe_mx_dout_image_size(const moe_shape* s) {
  if (check_shape(s) != MOE_OK || s->dtype != MOE_MXFP8) return (size_t)-1;
  return moe::mx_dout_image_bytes(s->T * s->k, s->d, s->E);
}

int moe_grouped_ffn_bwd(const void* d_o, const uint8_t* d_o_mx, const void* xp, const uint8_t* xp_mx,
                        const void* w_gate, const void* w_up, const void* w_down, const int32_t* offsets,
                        const moe_shape* s, const void* save, void* dxp_out, void* dw_gate_out, void* dw_up_out,
                        void* dw_down_out, void* ws, size_t ws_bytes, void* stream) {
  CHECK(check_shape(s));
  CHECK(check_ffn_dtype(s, "moe_grouped_ffn_bwd"));
  if (!d_o_mx || d_o) NEED(d_o);  // with the MXFP8 operands of d_o, d_o itself is not read
  if (!xp_mx || xp) NEED(xp);     // likewise xp with its MXFP8 images
  NEED(w_gate); NEED(w_up); NEED(w_down); NEED(offsets); NEED(dxp_out);
  NEED(dw_gate_out); NEED(dw_up_out); NEED(dw_down_out); NEED(ws);
  if (save_bytes_for(s) > 0) NEED(save);
  MX_IMAGE_OK(d_o_mx, s);
  MX_IMAGE_OK(xp_mx, s);
  const size_t need = moe_workspace_size(MOE_OP_FFN_BWD, s);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "moe_grouped_ffn_bwd: workspace %zu < %zu bytes", ws_bytes, need);
  moe::FfnArgs a{};
  a.S = (int)(s->T * s->k); a.d = (int)s->d; a.f = (int)s->f; a.E = (int)s->E;
  a.offsets = offsets; a.xp = xp; a.xp_mx = xp_mx; a.w_gate = w_gate; a.w_up = w_up; a.w_down = w_down;
  const size_t plane = s->dtype == MOE_MXFP8 ? gu_h_bytes(s) / 2 : (size_t)a.S * a.f * act_bytes(s->dtype);
  const size_t dgu_bytes = dgu_bytes_for(s);
  char* sv = const_cast<char*>(static_cast<const char*>(save));
  // Recompute: G, U, H are rebuilt in the workspace, after the dG|dU rows
  // (MXFP8: after the backward's own pieces).
  char* gu_h = recompute(s) ? static_cast<char*>(ws) + dgu_bytes + (s->dtype == MOE_MXFP8 ? mx_bwd_bytes(s) : 0)
                            : sv;
  a.G = gu_h; a.U = gu_h + plane; a.H = s->dtype == MOE_MXFP8 ? nullptr : gu_h + 2 * plane;
  a.recompute = recompute(s);
  a.mx_save = sv + save_planes(s);
  a.d_o = d_o; a.d_o_mx = d_o_mx; a.dgu = ws; a.dxp = dxp_out; a.dw_gate = dw_gate_out; a.dw_up = dw_up_out; a.dw_down = dw_down_out;
  if (s->dtype == MOE_MXFP8) {
    LAUNCH(moe::launch_ffn_mx_bwd(a, static_cast<char*>(ws) + dgu_bytes, as_stream(stream)));
  } else {
    LAUNCH(moe::launch_ffn_bwd(a, s->dtype == MOE_F32, as_stream(stream)));
  }
  return MOE_OK;
}

int moe_route_bwd(const void* x, const void* w_router, const int32_t* topk_idx, const float* topk_gate,
                  const float* dgate, const moe_shape* s, float* dlogits_out, void* dw_router_out, void* ws,
                  size_t ws_bytes, void* stream) {
  (void)w_router;
  CHECK(check_shape(s));
  NEED(x); NEED(topk_idx); NEED(topk_gate); NEED(dgate); NEED(dlogits_out); NEED(dw_router_out); NEED(ws);
  const size_t need = moe_workspace_size(MOE_OP_ROUTE_BWD, s);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "moe_route_bwd: workspace %zu < %zu bytes", ws_bytes, need);
  if (s->dtype == MOE_F32)
    LAUNCH(moe::launch_route_bwd(x, topk_idx, topk_gate, dgate, true, (int)s->T, (int)s->d, (int)s->E, (int)s->k,
                                 dlogits_out, dw_router_out, ws, as_stream(stream)));
  else
    LAUNCH(moe::launch_route_bwd_bf16(x, topk_idx, topk_gate, dgate, (int)s->T, (int)s->d, (int)s->E, (int)s->k,
                                      dlogits_out, dw_router_out, ws, as_stream(stream)));
  return MOE_OK;
}

int moe_dispatch_bwd(const void* dxp, const int32_t* row_of_slot, const float* dlogits, const void* w_router,
                     const moe_shape* s, void* dx_out, void* ws, size_t ws_bytes, void* stream) {
  CHECK(check_shape(s));
  NEED(dxp); NEED(row_of_slot); NEED(dx_out);
  const bool router = dlogits != nullptr && w_router != nullptr;
  if ((dlogits == nullptr) != (w_router == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch_bwd: dlogits and w_router must be both set or both NULL");
  if (router) {
    NEED(dlogits); NEED(w_router); NEED(ws);
    const size_t need = moe::dispatch_bwd_workspace((int)s->d, (int)s->E, s->dtype == MOE_F32);
    if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "moe_dispatch_bwd: workspace %zu < %zu bytes", ws_bytes, need);
  }
  LAUNCH(moe::launch_dispatch_bwd(dxp, row_of_slot, dlogits, w_router, s->dtype == MOE_F32, (int)s->T, (int)s->d,
                                  (int)s->E, (int)s->k, dx_out, ws, as_stream(stream)));
  return MOE_OK;
}

int moe_kernel_timer(int gemm_mode, void* const* start, void* const* stop, int capacity) {
  if (gemm_mode < MOE_GEMM_FWD_GU || gemm_mode > MOE_GEMM_WGRAD)
    return fail(MOE_ERR_INVALID_ARG, "moe_kernel_timer: unknown gemm_mode %d", gemm_mode);
  if (capacity < 0 || (capacity > 0 && (!start || !stop)))
    return fail(MOE_ERR_INVALID_ARG, "moe_kernel_timer: need capacity >= 0 and, above 0, both event arrays");
  KernelTimer& t = kernel_timer();
  std::lock_guard<std::mutex> g(t.mu);
  g_timer_mode.store(-1, std::memory_order_release);
  t.start.clear();
  t.stop.clear();
  t.n = 0;
  for (int i = 0; i < capacity; ++i) {
    if (!start[i] || !stop[i]) return fail(MOE_ERR_INVALID_ARG, "moe_kernel_timer: NULL event %d", i);
    t.start.push_back(static_cast<hipEvent_t>(start[i]));
    t.stop.push_back(static_cast<hipEvent_t>(stop[i]));
  }
  if (capacity > 0) g_timer_mode.store(gemm_mode, std::memory_order_release);
  return MOE_OK;
}

int moe_kernel_timer_count(void) {
  KernelTimer& t = kernel_timer();
  std::lock_guard<std::mutex> g(t.mu);
  return t.n;
}

int moe_load_stats(const int32_t* counts, int64_t E, double* stats_out, void* stream) {
  NEED(counts); NEED(stats_out);
  if (E < 1 || E > 256) return fail(MOE_ERR_INVALID_ARG, "moe_load_stats: E must be in 1..256 (got %lld)", (long long)E);
  LAUNCH(moe::launch_load_stats(counts, (int)E, stats_out, as_stream(stream)));
  return MOE_OK;
}

int mxfp8_quantize(const void* in_bf16, int64_t rows, int64_t cols, int axis, uint8_t* q_out, uint8_t* scale_out,
                   void* stream) {
  if (!in_bf16 || !q_out || !scale_out) return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize: NULL pointer");
  if (rows < 1 || cols < 1) return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize: rows and cols must be >= 1");
  if (axis != 0 && axis != 1) return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize: axis must be 0 or 1");
  if ((axis == 0 && cols % 32) || (axis == 1 && rows % 32))
    return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize: the blocked axis must be a multiple of 32");
  if (axis == 0 && (!aligned16(in_bf16) || !aligned16(q_out)))
    return fail(MOE_ERR_MISALIGNED, "mxfp8_quantize: in and q must be 16-byte aligned");
  if (rows * cols > ((int64_t)1 << 40)) return fail(MOE_ERR_UNSUPPORTED, "mxfp8_quantize: too large");
  LAUNCH(moe::launch_mxfp8_quantize(in_bf16, rows, cols, axis, q_out, scale_out, as_stream(stream)));
  return MOE_OK;
}

int mxfp8_quantize_grouped(const void* in_bf16, int64_t rows, int64_t cols, const int32_t* group_offsets,
                           int64_t groups, uint8_t* q_out, uint8_t* scale_out, void* stream) {
  if (!in_bf16 || !group_offsets || !q_out || !scale_out)
    return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize_grouped: NULL pointer");
  if (rows < 1 || cols < 1) return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize_grouped: rows and cols must be >= 1");
  if (groups < 1 || groups > 256)
    return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize_grouped: groups must be in 1..256 (got %lld)", (long long)groups);
  if (rows >= ((int64_t)1 << 31) || rows * cols > ((int64_t)1 << 40))
    return fail(MOE_ERR_UNSUPPORTED, "mxfp8_quantize_grouped: too large");
  LAUNCH(moe::launch_mxfp8_quantize_grouped(in_bf16, rows, cols, group_offsets, (int)groups, q_out, scale_out,
                                            as_stream(stream)));
  return MOE_OK;
}

}  // extern "C"
