// Exercises the host-side validation of every C entry point of libmoe
// (abi.cpp built for the host only, linked against stubs.cpp): each bad
// argument gives its documented status and enqueues nothing; each good call
// reaches its launcher with the sizes it was given. Built and run under
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_abi_host.py.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "moe.h"
#include "stubs.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what, int line) {
  if (!ok) {
    std::fprintf(stderr, "FAILED line %d: %s (last message: %s)\n", line, what, moe_last_error_message());
    ++failures;
  }
}
#define EXPECT(x) expect((x), #x, __LINE__)

// The status of `call`, and whether it launched (exactly one launch on OK,
// none on an error).
#define RC(call, want)                                                        \
  do {                                                                        \
    const int before_ = stub::launches;                                       \
    const int rc_ = (call);                                                   \
    expect(rc_ == (want), #call " -> " #want, __LINE__);                      \
    if (rc_ != MOE_OK) expect(stub::launches == before_, "no launch on error", __LINE__); \
  } while (0)

// Fake device buffers: aligned host memory the stubs never touch.
alignas(256) char g_buf[1 << 16];
char* buf(size_t off) { return g_buf + off; }
float* fbuf(size_t off) { return reinterpret_cast<float*>(g_buf + off); }
int32_t* ibuf(size_t off) { return reinterpret_cast<int32_t*>(g_buf + off); }

moe_shape shape(int64_t T, int64_t d, int64_t E, int64_t k, int64_t f, int dtype, int flags = 0) {
  moe_shape s;
  s.T = T; s.d = d; s.E = E; s.k = k; s.f = f; s.dtype = dtype; s.flags = flags;
  return s;
}

}  // namespace

int main() {
  const size_t BAD = static_cast<size_t>(-1);
  EXPECT(moe_abi_version() == MOE_ABI_VERSION);
  EXPECT(std::strcmp(moe_status_string(MOE_ERR_WORKSPACE), "MOE_ERR_WORKSPACE") == 0);
  EXPECT(std::strcmp(moe_status_string(42), "MOE_ERR_UNKNOWN") == 0);

  // Shape checks through the size queries.
  const moe_shape ok = shape(256, 128, 8, 4, 128, MOE_BF16);
  EXPECT(moe_workspace_size(MOE_OP_DISPATCH, &ok) != BAD);
  EXPECT(moe_workspace_size(MOE_OP_DISPATCH, nullptr) == BAD);
  EXPECT(moe_workspace_size(99, &ok) == BAD);
  moe_shape bad = ok; bad.dtype = 7;
  EXPECT(moe_workspace_size(MOE_OP_FFN_FWD, &bad) == BAD);
  bad = ok; bad.flags = 4;
  EXPECT(moe_save_size(&bad) == BAD);
  bad = ok; bad.k = 9; bad.E = 16;
  EXPECT(moe_save_size(&bad) == BAD);
  bad = ok; bad.k = 9;
  EXPECT(moe_save_size(&bad) == BAD);
  bad = ok; bad.E = 300;
  EXPECT(moe_save_size(&bad) == BAD);
  bad = ok; bad.d = 96;
  EXPECT(moe_save_size(&bad) == BAD);
  bad = ok; bad.T = 0;
  EXPECT(moe_save_size(&bad) == BAD);
  bad = ok; bad.T = (int64_t)1 << 40;
  EXPECT(moe_save_size(&bad) == BAD);
  bad = ok; bad.flags = 2;  // an unknown flag bit
  EXPECT(moe_save_size(&bad) == BAD);
  const moe_shape rec = shape(256, 128, 8, 4, 128, MOE_BF16, MOE_FLAG_RECOMPUTE);
  EXPECT(moe_save_size(&rec) == 0);
  EXPECT(moe_save_size(&ok) == (size_t)3 * 256 * 4 * 128 * 2);
  const moe_shape mx = shape(256, 128, 8, 4, 128, MOE_MXFP8);
  EXPECT(moe_save_size(&mx) > (size_t)3 * 256 * 4 * 128 * 4);  // fp32 G, U, H plus the weight copies
  EXPECT(moe_mx_image_size(10, 96) == BAD);
  EXPECT(moe_mx_image_size(0, 64) == BAD);
  EXPECT(moe_mx_image_size(10, 64) >= 10 * 64 + 20);

  void* s = nullptr;  // stream
  const size_t big = sizeof(g_buf);

  // moe_route
  RC(moe_route(buf(0), buf(256), &ok, fbuf(512), ibuf(1024), fbuf(2048), buf(4096), big, s), MOE_OK);
  EXPECT(stub::last_T == 256 && stub::last_d == 128 && stub::last_E == 8 && stub::last_k == 4);
  RC(moe_route(nullptr, buf(256), &ok, fbuf(512), ibuf(1024), fbuf(2048), buf(4096), big, s), MOE_ERR_INVALID_ARG);
  RC(moe_route(buf(1), buf(256), &ok, fbuf(512), ibuf(1024), fbuf(2048), buf(4096), big, s), MOE_ERR_MISALIGNED);
  RC(moe_route(buf(0), buf(256), &ok, fbuf(512), ibuf(1024), fbuf(2048), buf(4096), 16, s), MOE_ERR_WORKSPACE);
  RC(moe_route(buf(0), buf(256), nullptr, fbuf(512), ibuf(1024), fbuf(2048), buf(4096), big, s), MOE_ERR_INVALID_ARG);

  // moe_dispatch: the workspace must be 256-byte aligned; images only for MXFP8.
  RC(moe_dispatch(buf(0), ibuf(256), &ok, ibuf(512), ibuf(768), ibuf(1024), ibuf(2048), buf(4096), nullptr,
                  buf(8192), big, s), MOE_OK);
  RC(moe_dispatch(buf(0), ibuf(256), &ok, ibuf(512), ibuf(768), ibuf(1024), ibuf(2048), buf(4096), nullptr,
                  buf(8192 + 16), big, s), MOE_ERR_MISALIGNED);
  RC(moe_dispatch(buf(0), ibuf(256), &ok, ibuf(512), ibuf(768), ibuf(1024), ibuf(2048), buf(4096),
                  reinterpret_cast<uint8_t*>(buf(12288)), buf(8192), big, s), MOE_ERR_INVALID_ARG);
  RC(moe_dispatch(buf(0), ibuf(256), &ok, ibuf(512), ibuf(768), ibuf(1024), ibuf(2048), buf(4096), nullptr,
                  buf(8192), 100, s), MOE_ERR_WORKSPACE);
  RC(moe_dispatch(buf(0), ibuf(256), &mx, ibuf(512), ibuf(768), ibuf(1024), ibuf(2048), buf(4096),
                  reinterpret_cast<uint8_t*>(buf(12288 + 16)), buf(8192), big, s), MOE_ERR_MISALIGNED);
  RC(moe_dispatch(buf(0), ibuf(256), &mx, ibuf(512), ibuf(768), ibuf(1024), ibuf(2048), buf(4096),
                  reinterpret_cast<uint8_t*>(buf(12288)), buf(8192), big, s), MOE_OK);
  // With xp's MXFP8 operands the bf16 rows are optional; without them not.
  RC(moe_dispatch(buf(0), ibuf(256), &mx, ibuf(512), ibuf(768), ibuf(1024), ibuf(2048), nullptr,
                  reinterpret_cast<uint8_t*>(buf(12288)), buf(8192), big, s), MOE_OK);
  RC(moe_dispatch(buf(0), ibuf(256), &mx, ibuf(512), ibuf(768), ibuf(1024), ibuf(2048), nullptr, nullptr,
                  buf(8192), big, s), MOE_ERR_INVALID_ARG);
  // moe_dispatch_noalloc: no workspace argument; shapes whose dispatch
  // workspace exceeds the library's 1 MiB array are refused on the host.
  RC(moe_dispatch_noalloc(buf(0), ibuf(256), &ok, ibuf(512), ibuf(768), ibuf(1024), ibuf(2048), buf(4096), nullptr,
                          s), MOE_OK);
  EXPECT(stub::last_T == 256 && stub::last_E == 8);
  RC(moe_dispatch_noalloc(buf(0), ibuf(256), &ok, ibuf(512), ibuf(768), ibuf(1024), ibuf(2048), buf(4096),
                          reinterpret_cast<uint8_t*>(buf(12288)), s), MOE_ERR_INVALID_ARG);
  RC(moe_dispatch_noalloc(buf(0), ibuf(256), &mx, ibuf(512), ibuf(768), ibuf(1024), ibuf(2048), buf(4096),
                          reinterpret_cast<uint8_t*>(buf(12288)), s), MOE_OK);
  RC(moe_dispatch_noalloc(buf(0), nullptr, &ok, ibuf(512), ibuf(768), ibuf(1024), ibuf(2048), buf(4096), nullptr, s),
     MOE_ERR_INVALID_ARG);
  const moe_shape huge = shape(int64_t(1) << 22, 128, 256, 4, 128, MOE_BF16);  // 8 MiB of chunk counts
  RC(moe_dispatch_noalloc(buf(0), ibuf(256), &huge, ibuf(512), ibuf(768), ibuf(1024), ibuf(2048), buf(4096), nullptr,
                          s), MOE_ERR_WORKSPACE);
  EXPECT(std::strstr(moe_last_error_message(), "1048576") != nullptr);
  EXPECT(moe_read_device_status(nullptr, s) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_read_device_status(buf(8192), s) == 0);

  // moe_grouped_ffn_fwd / _bwd: save and workspace sizes, MXFP8 widths.
  std::vector<char> save(moe_save_size(&ok) + 256);
  char* sv = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(save.data()) + 255) & ~uintptr_t(255));
  const size_t svn = moe_save_size(&ok);
  RC(moe_grouped_ffn_fwd(buf(0), nullptr, buf(256), buf(512), buf(768), ibuf(1024), &ok, sv, svn, buf(2048),
                         nullptr, 0, s), MOE_OK);
  EXPECT(stub::last_T == 256 * 4 && stub::last_f == 128);
  RC(moe_grouped_ffn_fwd(buf(0), nullptr, buf(256), buf(512), buf(768), ibuf(1024), &ok, sv, svn - 1, buf(2048),
                         nullptr, 0, s), MOE_ERR_WORKSPACE);
  RC(moe_grouped_ffn_fwd(buf(0), reinterpret_cast<uint8_t*>(buf(4096)), buf(256), buf(512), buf(768), ibuf(1024),
                         &ok, sv, svn, buf(2048), nullptr, 0, s), MOE_ERR_INVALID_ARG);
  const moe_shape mx64 = shape(256, 192, 8, 4, 128, MOE_MXFP8);
  RC(moe_grouped_ffn_fwd(buf(0), nullptr, buf(256), buf(512), buf(768), ibuf(1024), &mx64, sv, svn, buf(2048),
                         buf(4096), big, s), MOE_ERR_UNSUPPORTED);
  const size_t wsb = moe_workspace_size(MOE_OP_FFN_BWD, &ok);
  std::vector<char> wsv(wsb + 256);
  char* ws = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(wsv.data()) + 255) & ~uintptr_t(255));
  RC(moe_grouped_ffn_bwd(buf(0), nullptr, buf(256), nullptr, buf(512), buf(768), buf(1024), ibuf(1280), &ok, sv, buf(2048),
                         buf(2304), buf(2560), buf(2816), ws, wsb, s), MOE_OK);
  RC(moe_grouped_ffn_bwd(buf(0), nullptr, buf(256), nullptr, buf(512), buf(768), buf(1024), ibuf(1280), &ok, sv, buf(2048),
                         buf(2304), buf(2560), buf(2816), ws, wsb - 1, s), MOE_ERR_WORKSPACE);
  RC(moe_grouped_ffn_bwd(buf(0), nullptr, buf(256), nullptr, buf(512), buf(768), buf(1024), ibuf(1280), &ok, sv, nullptr,
                         buf(2304), buf(2560), buf(2816), ws, wsb, s), MOE_ERR_INVALID_ARG);
  // Recompute layers save nothing: the FFN calls accept a NULL save buffer.
  const size_t wsr = moe_workspace_size(MOE_OP_FFN_FWD, &rec);
  std::vector<char> wr(wsr + 256);
  char* wrp = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(wr.data()) + 255) & ~uintptr_t(255));
  RC(moe_grouped_ffn_fwd(buf(0), nullptr, buf(256), buf(512), buf(768), ibuf(1024), &rec, nullptr, 0, buf(2048),
                         wrp, wsr, s), MOE_OK);
  RC(moe_grouped_ffn_fwd(buf(0), nullptr, buf(256), buf(512), buf(768), ibuf(1024), &rec, nullptr, 0, buf(2048),
                         wrp, wsr - 1, s), MOE_ERR_WORKSPACE);

  // combine and its backward; the MXFP8 backward writes fp32 d_o (kind 2).
  RC(moe_combine(buf(0), fbuf(256), ibuf(512), &ok, buf(1024), s), MOE_OK);
  RC(moe_combine(buf(0), fbuf(256), nullptr, &ok, buf(1024), s), MOE_ERR_INVALID_ARG);
  // token_of_row and offsets are read only with the MXFP8 operands of d_o,
  // and then d_o itself may be NULL.
  uint8_t* img = reinterpret_cast<uint8_t*>(buf(4096));
  RC(moe_combine_bwd(buf(0), buf(256), fbuf(512), ibuf(768), nullptr, nullptr, &ok, buf(1024), nullptr, fbuf(2048),
                     s), MOE_OK);
  EXPECT(stub::last_kind == 1);
  RC(moe_combine_bwd(buf(0), buf(256), fbuf(512), ibuf(768), nullptr, nullptr, &ok, nullptr, nullptr, fbuf(2048), s),
     MOE_ERR_INVALID_ARG);
  RC(moe_combine_bwd(buf(0), buf(256), fbuf(512), ibuf(768), nullptr, nullptr, &mx, buf(1024), nullptr, fbuf(2048),
                     s), MOE_OK);
  EXPECT(stub::last_kind == 2);
  RC(moe_combine_bwd(buf(0), buf(256), fbuf(512), ibuf(768), ibuf(8192), ibuf(12288), &mx, buf(1024), img,
                     fbuf(2048), s), MOE_OK);
  EXPECT(stub::last_kind == 3 && stub::last_E == 8);
  RC(moe_combine_bwd(buf(0), buf(256), fbuf(512), ibuf(768), ibuf(8192), ibuf(12288), &mx, nullptr, img,
                     fbuf(2048), s), MOE_OK);
  EXPECT(stub::last_kind == 4);
  RC(moe_combine_bwd(buf(0), buf(256), fbuf(512), ibuf(768), nullptr, ibuf(12288), &mx, nullptr, img, fbuf(2048), s),
     MOE_ERR_INVALID_ARG);
  RC(moe_combine_bwd(buf(0), buf(256), fbuf(512), ibuf(768), ibuf(8192), ibuf(12288), &ok, buf(1024), img,
                     fbuf(2048), s), MOE_ERR_INVALID_ARG);
  EXPECT(moe_mx_dout_image_size(&mx) != BAD && moe_mx_dout_image_size(&mx) > moe_mx_image_size(mx.T * mx.k, mx.d));
  EXPECT(moe_mx_dout_image_size(&ok) == BAD);
  EXPECT(moe_mx_xp_image_size(&mx) != BAD && moe_mx_xp_image_size(&mx) < moe_mx_dout_image_size(&mx) &&
         moe_mx_xp_image_size(&mx) > moe_mx_image_size(mx.T * mx.k, mx.d));
  EXPECT(moe_mx_xp_image_size(&ok) == BAD);

  // router backward and dispatch backward
  RC(moe_route_bwd(buf(0), buf(256), ibuf(512), fbuf(768), fbuf(1024), &ok, fbuf(2048), buf(4096), buf(8192), big,
                   s), MOE_OK);
  RC(moe_route_bwd(buf(0), buf(256), ibuf(512), fbuf(768), fbuf(1024), &ok, fbuf(2048), buf(4096), buf(8192), 8, s),
     MOE_ERR_WORKSPACE);
  RC(moe_dispatch_bwd(buf(0), ibuf(256), nullptr, nullptr, &ok, buf(512), nullptr, 0, s), MOE_OK);
  RC(moe_dispatch_bwd(buf(0), ibuf(256), fbuf(512), nullptr, &ok, buf(1024), nullptr, 0, s), MOE_ERR_INVALID_ARG);
  RC(moe_dispatch_bwd(buf(0), ibuf(256), fbuf(512), buf(768), &ok, buf(1024), buf(4096), big, s), MOE_OK);
  RC(moe_dispatch_bwd(buf(0), ibuf(256), fbuf(512), buf(768), &ok, buf(1024), buf(4096), 64, s), MOE_ERR_WORKSPACE);

  // load statistics, quantisers
  RC(moe_load_stats(ibuf(0), 8, reinterpret_cast<double*>(buf(256)), s), MOE_OK);
  RC(moe_load_stats(ibuf(0), 0, reinterpret_cast<double*>(buf(256)), s), MOE_ERR_INVALID_ARG);
  RC(moe_load_stats(ibuf(0), 257, reinterpret_cast<double*>(buf(256)), s), MOE_ERR_INVALID_ARG);
  uint8_t* q = reinterpret_cast<uint8_t*>(buf(4096));
  uint8_t* sc = reinterpret_cast<uint8_t*>(buf(8192));
  RC(mxfp8_quantize(buf(0), 64, 96, 0, q, sc, s), MOE_OK);
  RC(mxfp8_quantize(buf(0), 64, 96, 2, q, sc, s), MOE_ERR_INVALID_ARG);
  RC(mxfp8_quantize(buf(0), 64, 100, 0, q, sc, s), MOE_ERR_INVALID_ARG);
  RC(mxfp8_quantize(buf(0), 60, 96, 1, q, sc, s), MOE_ERR_INVALID_ARG);
  RC(mxfp8_quantize(buf(2), 64, 96, 0, q, sc, s), MOE_ERR_MISALIGNED);
  RC(mxfp8_quantize(buf(0), (int64_t)1 << 30, (int64_t)1 << 20, 0, q, sc, s), MOE_ERR_UNSUPPORTED);
  RC(mxfp8_quantize_grouped(buf(0), 100, 64, ibuf(256), 3, q, sc, s), MOE_OK);
  RC(mxfp8_quantize_grouped(buf(0), 100, 64, ibuf(256), 0, q, sc, s), MOE_ERR_INVALID_ARG);
  RC(mxfp8_quantize_grouped(buf(0), 100, 64, nullptr, 3, q, sc, s), MOE_ERR_INVALID_ARG);

  // The kernel timer: arguments, arm and disarm (its events are recorded
  // only by the GEMM launchers, which are stubbed here).
  void* ev[2] = {buf(0), buf(256)};
  void* nul[2] = {nullptr, nullptr};
  EXPECT(moe_kernel_timer(7, ev, ev, 2) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_kernel_timer(MOE_GEMM_WGRAD, ev, ev, -1) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_kernel_timer(MOE_GEMM_WGRAD, nullptr, ev, 2) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_kernel_timer(MOE_GEMM_WGRAD, nul, nul, 2) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_kernel_timer(MOE_GEMM_WGRAD, ev, ev, 2) == MOE_OK);
  EXPECT(moe_kernel_timer_count() == 0);
  EXPECT(moe_kernel_timer(MOE_GEMM_WGRAD, nullptr, nullptr, 0) == MOE_OK);
  EXPECT(stub::events_recorded == 0);

  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("abi host checks passed\n");
  return 0;
}
