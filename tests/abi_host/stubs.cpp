// Host-only stand-ins for the library's kernel launchers and the four HIP
// runtime calls the C ABI layer makes, so that abi.cpp can be built with g++
// under AddressSanitizer and UndefinedBehaviorSanitizer and its validation
// exercised on a host without a GPU. Every launcher counts its calls and
// keeps the last shape it saw; none touches the pointers it is given.
#include <hip/hip_runtime.h>

#include "kernels.h"
#include "stubs.h"

namespace stub {
int launches = 0;
int last_T = 0, last_d = 0, last_E = 0, last_k = 0, last_f = 0;
int last_kind = -1;
int events_recorded = 0;
}  // namespace stub

namespace {
hipError_t hit(int T = 0, int d = 0, int E = 0, int k = 0, int f = 0) {
  ++stub::launches;
  stub::last_T = T; stub::last_d = d; stub::last_E = E; stub::last_k = k; stub::last_f = f;
  return hipSuccess;
}
}  // namespace

extern "C" {
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { ++stub::events_recorded; return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "stub error"; }
hipError_t hipMemcpyAsync(void* dst, const void*, size_t n, hipMemcpyKind, hipStream_t) {
  if (dst && n == sizeof(int32_t)) *static_cast<int32_t*>(dst) = 0;
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
}

namespace moe {
hipError_t launch_ffn_fwd(const FfnArgs& a, bool, hipStream_t) { return hit(a.S, a.d, a.E, 0, a.f); }
hipError_t launch_ffn_bwd(const FfnArgs& a, bool, hipStream_t) { return hit(a.S, a.d, a.E, 0, a.f); }
hipError_t launch_route(const void*, const void*, bool, int T, int d, int E, int k, float*, int32_t*, float*,
                        hipStream_t) { return hit(T, d, E, k); }
size_t route_bwd_workspace(int, int, int) { return 4096; }
hipError_t launch_route_bwd(const void*, const int32_t*, const float*, const float*, bool, int T, int d, int E, int k,
                            float*, void*, void*, hipStream_t) { return hit(T, d, E, k); }
size_t route_bf16_workspace(int, int) { return 2048; }
hipError_t launch_route_bf16(const void*, const void*, int T, int d, int E, int k, float*, int32_t*, float*, void*,
                             hipStream_t) { return hit(T, d, E, k); }
size_t route_bwd_bf16_workspace(int, int, int) { return 8192; }
hipError_t launch_route_bwd_bf16(const void*, const int32_t*, const float*, const float*, int T, int d, int E, int k,
                                 float*, void*, void*, hipStream_t) { return hit(T, d, E, k); }
// The dispatch workspace's real size: status word, [chunk][expert] counts and
// per-chunk flags, chunks of 128 tokens while that table stays small, else 512.
size_t dispatch_workspace(int T, int E) {
  auto a256 = [](size_t n) { return (n + 255) & ~size_t(255); };
  const int ct = static_cast<int64_t>((T + 127) / 128) * E <= 4096 ? 128 : 512;
  const size_t nch = (static_cast<size_t>(T) + ct - 1) / ct;
  return 256 + a256(4 * nch * E) + a256(4 * nch);
}
hipError_t launch_dispatch(const void*, const int32_t*, int, int T, int d, int E, int k, int32_t*, int32_t*, int32_t*,
                           int32_t*, void*, void*, hipStream_t) { return hit(T, d, E, k); }
hipError_t launch_combine(const void*, const float*, const int32_t*, bool, int T, int d, int k, void*, hipStream_t) {
  return hit(T, d, 0, k);
}
hipError_t launch_combine_bwd(const void*, const void*, const float*, const int32_t*, int kind, int T, int d, int k,
                              void*, float*, hipStream_t) {
  stub::last_kind = kind;
  return hit(T, d, 0, k);
}
size_t dispatch_bwd_workspace(int d, int E, bool is_f32) { return static_cast<size_t>(d) * E * (is_f32 ? 4 : 2); }
hipError_t launch_dispatch_bwd(const void*, const int32_t*, const float*, const void*, bool, int T, int d, int E,
                               int k, void*, void*, hipStream_t) { return hit(T, d, E, k); }
hipError_t launch_load_stats(const int32_t*, int E, double*, hipStream_t) { return hit(0, 0, E); }
hipError_t launch_dispatch_mx(const void*, const int32_t*, int T, int d, int E, int k, int32_t*, int32_t*, int32_t*,
                              int32_t*, void*, MxRowImages, void*, hipStream_t) { return hit(T, d, E, k); }
size_t dispatch_noalloc_max() { return size_t(1) << 20; }
hipError_t launch_dispatch_noalloc(const void*, const int32_t*, int, int T, int d, int E, int k, int32_t*, int32_t*,
                                   int32_t*, int32_t*, void*, MxRowImages, hipStream_t) { return hit(T, d, E, k); }
hipError_t launch_combine_bwd_mx(const void*, const void*, const float*, const int32_t*, const int32_t*,
                                 const int32_t*, int T, int d, int E, int k, void* d_o, MxDoutImage, float*,
                                 hipStream_t) {
  stub::last_kind = d_o ? 3 : 4;
  return hit(T, d, E, k);
}
hipError_t launch_mxfp8_quantize(const void*, int64_t rows, int64_t cols, int, uint8_t*, uint8_t*, hipStream_t) {
  return hit(static_cast<int>(rows), static_cast<int>(cols));
}
hipError_t launch_mxfp8_quantize_grouped(const void*, int64_t rows, int64_t cols, const int32_t*, int G, uint8_t*,
                                         uint8_t*, hipStream_t) {
  return hit(static_cast<int>(rows), static_cast<int>(cols), G);
}
size_t ffn_mx_fwd_workspace(int S, int d, int f, int, bool rec) {
  return static_cast<size_t>(S) * (d + f) + (rec ? static_cast<size_t>(S) * f : 0) + 4096;
}
size_t ffn_mx_save_extra(int S, int d, int f, int E, bool) {
  return static_cast<size_t>(E) * d * f * 3 + static_cast<size_t>(S + 64 * E) * f + 4096;
}
size_t ffn_mx_gu_plane(int S, int f, int E) { return static_cast<size_t>(S + 64 * E) * f * 4; }
size_t ffn_mx_bwd_workspace(int S, int d, int f, int, bool rec) {
  return static_cast<size_t>(S) * (2 * d + 4 * f) + (rec ? static_cast<size_t>(S) * (d + 2 * f) : 0) + 4096;
}
hipError_t launch_ffn_mx_fwd(const FfnArgs& a, void*, hipStream_t) { return hit(a.S, a.d, a.E, 0, a.f); }
hipError_t launch_ffn_mx_bwd(const FfnArgs& a, void*, hipStream_t) { return hit(a.S, a.d, a.E, 0, a.f); }
}  // namespace moe
