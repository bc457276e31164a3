// MXFP8 expert FFN, forward and backward: quantise every grouped-GEMM operand
// along that GEMM's K into the MX GEMM's layout, then run the grouped GEMMs.
//
// The pages use MXFP8 for the expert computation ("Olmo-core 3 é lançado com
// infraestrutura para treinar modelos MoE", section "Otimizações e testes em
// escala de trilhões"; "Ai2 rilascia Olmo-Core 3...", section "Parallelismo,
// precisione e tecniche di memoria"). Inputs, O, dXp and the weight
// gradients are bf16; every E4M3 code of a computed GEMM operand (H, dO,
// dG | dU) is decided on its fp32 value: dO is kept in fp32, G and U in
// fp32 rounded to 16 mantissa bits (24-bit words), H exists only inside the
// gate/up epilogue (from those G, U) and dG | dU only inside the down-dgrad
// epilogue, each of which writes both E4M3 operand layouts of its tensor.
// Each GEMM consumes
// E4M3 copies with one E8M0 scale per 32 elements along its K:
//   forward   G,U = q(Xp) q(W_gate), q(W_up)   K = d  (weights transposed)
//             O   = q(H) q(W_down)              K = f  (weight transposed)
//   dgrad     dGU = SwiGLU'(q(dO) q(W_down)^T)  K = d
//             dXp = q(dGU) q([W_gate|W_up])^T   K = 2f
//   wgrad     dW_down = q(H)^T q(dO), [dW_gate|dW_up] = q(Xp)^T q(dGU), K =
//             an expert's tokens, each expert's range padded to 64 rows.
// q(Xp) and q(dO) along d can arrive ready-made from the dispatch and
// combine-backward passes, which write them beside their rows; q(H) and
// q(dGU) along K, and q(dGU) along the tokens, come from the epilogues of the
// GEMMs that produce them.
#include "common.h"
#include "grouped_gemm.h"
#include "kernels.h"

namespace moe {

namespace {

size_t a256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

// Bump allocator over the caller's workspace: 256-byte aligned pieces, each
// with 16 bytes of slack (a scale tile of a ragged row range is read up to the
// next whole dword).
struct Carve {
  char* p;
  size_t used = 0;
  uint8_t* take(size_t n) {
    uint8_t* r = reinterpret_cast<uint8_t*>(p + used);
    used += a256(n + 16);
    return r;
  }
};

int64_t padded_rows(int S, int E) { return (static_cast<int64_t>(S) + 63LL * E + 63) / 64 * 64; }

struct FwdWs {
  uint8_t *xq, *xs, *wgq, *wgs, *wuq, *wus, *hq, *hs, *wdq, *wds;
  int32_t* poff;     // per-expert offsets of the rows padded to 64
  uint8_t *ht, *hts; // recompute only: H along the tokens (else in the save buffer)
};
FwdWs carve_fwd(char* base, int S, int d, int f, int E, bool rec, size_t* total) {
  Carve c{base};
  const size_t sd = static_cast<size_t>(S) * d, sf = static_cast<size_t>(S) * f;
  const size_t w = static_cast<size_t>(E) * d * f;
  const size_t P = static_cast<size_t>(padded_rows(S, E));
  FwdWs o;
  o.xq = c.take(sd); o.xs = c.take(sd / 32);
  o.wgq = c.take(w); o.wgs = c.take(w / 32);
  o.wuq = c.take(w); o.wus = c.take(w / 32);
  o.hq = c.take(sf); o.hs = c.take(sf / 32);
  o.wdq = c.take(w); o.wds = c.take(w / 32);
  o.poff = reinterpret_cast<int32_t*>(c.take(static_cast<size_t>(E + 1) * 4));
  o.ht = o.hts = nullptr;
  if (rec) {
    o.ht = c.take(P * f); o.hts = c.take(P * f / 32);
  }
  if (total) *total = c.used;
  return o;
}

// Save-buffer region of an MXFP8 layer after the blocked G, U planes: the
// columns-blocked weight copies the backward's dgrad GEMMs use, written by
// the forward's weight pass, and H as the W_down weight gradient's
// token-major operand, written by the gate/up epilogue (not with
// recompute: the backward rebuilds it).
struct SaveMx {
  uint8_t *wgq, *wgs, *wuq, *wus, *wdq, *wds, *ht, *hts;
};
SaveMx carve_save(char* base, int S, int d, int f, int E, bool rec, size_t* total) {
  Carve c{base};
  const size_t w = static_cast<size_t>(E) * d * f;
  const size_t P = static_cast<size_t>(padded_rows(S, E));
  SaveMx o;
  o.wgq = c.take(w); o.wgs = c.take(w / 32);
  o.wuq = c.take(w); o.wus = c.take(w / 32);
  o.wdq = c.take(w); o.wds = c.take(w / 32);
  o.ht = o.hts = nullptr;
  if (!rec) {
    o.ht = c.take(P * f); o.hts = c.take(P * f / 32);
  }
  if (total) *total = c.used;
  return o;
}

struct BwdWs {
  uint8_t *doq, *dos, *dguq, *dgus;
  int32_t* poff;
  uint8_t* blk;  // block table of the grouped transposing quantiser
  uint8_t *dot, *dots, *xt, *xts, *dgut, *dguts;
};
BwdWs carve_bwd(char* base, int S, int d, int f, int E, size_t* total) {
  Carve c{base};
  const size_t sd = static_cast<size_t>(S) * d, s2f = static_cast<size_t>(S) * 2 * f;
  const size_t w = static_cast<size_t>(E) * d * f;
  const size_t P = static_cast<size_t>(padded_rows(S, E));
  BwdWs o;
  o.doq = c.take(sd); o.dos = c.take(sd / 32);
  o.dguq = c.take(s2f); o.dgus = c.take(s2f / 32);
  o.poff = reinterpret_cast<int32_t*>(c.take(static_cast<size_t>(E + 1) * 4));
  o.blk = c.take(P / 64 * 8);
  o.dot = c.take(P * d); o.dots = c.take(P * d / 32);
  o.xt = c.take(P * d); o.xts = c.take(P * d / 32);
  o.dgut = c.take(P * 2 * f); o.dguts = c.take(P * 2 * f / 32);
  if (total) *total = c.used;
  return o;
}

// Recompute, after the backward's pieces: what the gate/up GEMM needs to run
// again (q(Xp) along d, q(W_gate)^T and q(W_up)^T along d) and writes (q(H)
// along f, unused, and along the tokens).
struct RecWs {
  uint8_t *xq, *xs, *wgq, *wgs, *wuq, *wus, *hq, *hs, *ht, *hts;
};
RecWs carve_rec(char* base, int S, int d, int f, int E, size_t* total) {
  Carve c{base};
  const size_t sd = static_cast<size_t>(S) * d, sf = static_cast<size_t>(S) * f;
  const size_t w = static_cast<size_t>(E) * d * f;
  const size_t P = static_cast<size_t>(padded_rows(S, E));
  RecWs o;
  o.xq = c.take(sd); o.xs = c.take(sd / 32);
  o.wgq = c.take(w); o.wgs = c.take(w / 32);
  o.wuq = c.take(w); o.wus = c.take(w / 32);
  o.hq = c.take(sf); o.hs = c.take(sf / 32);
  o.ht = c.take(P * f); o.hts = c.take(P * f / 32);
  if (total) *total = c.used;
  return o;
}

#define TRY(x)                                \
  do {                                        \
    hipError_t _e = (x);                      \
    if (_e != hipSuccess) return _e;          \
  } while (0)

}  // namespace

size_t ffn_mx_fwd_workspace(int S, int d, int f, int E, bool rec) {
  size_t n = 0;
  carve_fwd(nullptr, S, d, f, E, rec, &n);
  return n;
}

size_t ffn_mx_save_extra(int S, int d, int f, int E, bool rec) {
  size_t n = 0;
  carve_save(nullptr, S, d, f, E, rec, &n);
  return n;
}

size_t ffn_mx_gu_plane(int S, int f, int E) {
  return a256(static_cast<size_t>(padded_rows(S, E)) * f * 3);
}

size_t ffn_mx_bwd_workspace(int S, int d, int f, int E, bool rec) {
  size_t n = 0, r = 0;
  carve_bwd(nullptr, S, d, f, E, &n);
  if (rec) carve_rec(nullptr, S, d, f, E, &r);
  return n + r;
}

hipError_t launch_ffn_mx_fwd(const FfnArgs& a, void* ws, hipStream_t s) {
  const int S = a.S, d = a.d, f = a.f, E = a.E;
  const FwdWs w = carve_fwd(static_cast<char*>(ws), S, d, f, E, a.recompute, nullptr);
  const int64_t wsz = static_cast<int64_t>(d) * f;
  const SaveMx sv = carve_save(static_cast<char*>(a.mx_save), S, d, f, E, a.recompute, nullptr);
  const int64_t P = padded_rows(S, E);
  TRY(launch_mx_poff(a.offsets, E, w.poff, s));
  // Operands: Xp along d; W_gate, W_up along d, transposed to [f][d]. The same
  // read of each weight also writes its copy blocked along f ([d][f], in the
  // save buffer) for the backward's dXp GEMM.
  uint8_t *xq = w.xq, *xs = w.xs;
  if (a.xp_mx != nullptr) {  // written by the dispatch pass
    const MxImage im = mx_row_images(a.xp_mx, S, d, E).k;
    xq = im.q;
    xs = im.s;
  } else {
    TRY(launch_mx_kmajor(a.xp, S, d, 1, 0, xq, 0, xs, 0, s));
  }
  TRY(launch_mx_tgroup(a.w_gate, d, f, nullptr, E, wsz, w.wgq, d, wsz, w.wgs, wsz / 32, s, sv.wgq,
                       sv.wgs));
  TRY(launch_mx_tgroup(a.w_up, d, f, nullptr, E, wsz, w.wuq, d, wsz, w.wus, wsz / 32, s, sv.wuq,
                       sv.wus));
  {
    GemmParams p{};
    p.offsets = a.offsets; p.E = E; p.S = S; p.f = f;
    p.a = xq; p.lda = d; p.as = xs; p.as_slab = 2LL * S;
    p.b0 = w.wgq; p.b1 = w.wuq; p.ldb = d; p.bstride = wsz;
    p.bs0 = w.wgs; p.bs1 = w.wus; p.bs_slab = 2LL * f; p.bs_estride = wsz / 32;
    p.c0 = a.G; p.c1 = a.U; p.ldc = f; p.N = 2 * f; p.K = d;
    // G, U go to the save buffer in the blocked layout of the down-dgrad
    // epilogue; H leaves only as E4M3 operands: along f (the next GEMM's A
    // operand) and along the expert's tokens (the W_down weight gradient's).
    p.mxq = w.hq; p.mxs = w.hs; p.mxq_ld = f; p.mxs_slab = 2LL * S;
    p.tq = a.recompute ? w.ht : sv.ht; p.ts = a.recompute ? w.hts : sv.hts;
    p.tq_ld = P; p.ts_slab = 2LL * f; p.poff = w.poff;
    TRY(launch_mx_ragged(FWD_GU, p, s));
  }
  // Operands: H along f (above); W_down along f, transposed to [d][f] (and
  // its copy blocked along d, [f][d], for the backward's dH GEMM).
  TRY(launch_mx_tgroup(a.w_down, f, d, nullptr, E, wsz, w.wdq, f, wsz, w.wds, wsz / 32, s, sv.wdq,
                       sv.wds));
  GemmParams q{};
  q.offsets = a.offsets; q.E = E; q.S = S; q.f = f;
  q.a = w.hq; q.lda = f; q.as = w.hs; q.as_slab = 2LL * S;
  q.b0 = w.wdq; q.ldb = f; q.bstride = wsz; q.bs0 = w.wds; q.bs_slab = 2LL * d; q.bs_estride = wsz / 32;
  q.c0 = a.o; q.ldc = d; q.N = d; q.K = f;
  return launch_mx_ragged(FWD_DOWN, q, s);
}

hipError_t launch_ffn_mx_bwd(const FfnArgs& a, void* ws, hipStream_t s) {
  const int S = a.S, d = a.d, f = a.f, E = a.E;
  size_t bwd_bytes = 0;
  const BwdWs w = carve_bwd(static_cast<char*>(ws), S, d, f, E, &bwd_bytes);
  const SaveMx sv = carve_save(static_cast<char*>(a.mx_save), S, d, f, E, a.recompute, nullptr);
  const int64_t wsz = static_cast<int64_t>(d) * f;
  const int64_t P = padded_rows(S, E);
  // Per-expert padded offsets of the token-major (weight-gradient) layouts.
  TRY(launch_mx_poff(a.offsets, E, w.poff, s));
  TRY(launch_mx_blocks(a.offsets, w.poff, E, P, w.blk, s));
  uint8_t *ht = sv.ht, *hts = sv.hts;
  if (a.recompute) {
    // The gate/up GEMM again, from xp and the weights as the forward ran it:
    // the same operand bytes and the same kernel give bit-identical G, U and
    // H images. Only the layouts that GEMM reads are rebuilt (the dgrad weight
    // copies are in the save buffer).
    const RecWs r = carve_rec(static_cast<char*>(ws) + bwd_bytes, S, d, f, E, nullptr);
    uint8_t *xq = r.xq, *xs = r.xs;
    if (a.xp_mx != nullptr) {  // the dispatch pass's image, as the forward read it
      const MxImage im = mx_row_images(a.xp_mx, S, d, E).k;
      xq = im.q;
      xs = im.s;
    } else {
      TRY(launch_mx_kmajor(a.xp, S, d, 1, 0, r.xq, 0, r.xs, 0, s));
    }
    TRY(launch_mx_tgroup(a.w_gate, d, f, nullptr, E, wsz, r.wgq, d, wsz, r.wgs, wsz / 32, s, nullptr, nullptr));
    TRY(launch_mx_tgroup(a.w_up, d, f, nullptr, E, wsz, r.wuq, d, wsz, r.wus, wsz / 32, s, nullptr, nullptr));
    GemmParams p{};
    p.offsets = a.offsets; p.E = E; p.S = S; p.f = f;
    p.a = xq; p.lda = d; p.as = xs; p.as_slab = 2LL * S;
    p.b0 = r.wgq; p.b1 = r.wuq; p.ldb = d; p.bstride = wsz;
    p.bs0 = r.wgs; p.bs1 = r.wus; p.bs_slab = 2LL * f; p.bs_estride = wsz / 32;
    p.c0 = a.G; p.c1 = a.U; p.ldc = f; p.N = 2 * f; p.K = d;
    p.mxq = r.hq; p.mxs = r.hs; p.mxq_ld = f; p.mxs_slab = 2LL * S;
    p.tq = r.ht; p.ts = r.hts; p.tq_ld = P; p.ts_slab = 2LL * f; p.poff = w.poff;
    TRY(launch_mx_ragged(FWD_GU, p, s));
    ht = r.ht;
    hts = r.hts;
  }
  {  // dGU = SwiGLU'(q(dO) q(W_down)^T): dO along d; W_down [f][d] along d
     // was quantised by the forward.
    uint8_t *doq = w.doq, *dos = w.dos;
    if (a.d_o_mx != nullptr) {  // written by the combine backward pass
      const MxImage im = mx_dout_image(a.d_o_mx, S, d, E).k;
      doq = im.q;
      dos = im.s;
    } else {
      TRY(launch_mx_kmajor_f32(a.d_o, S, d, doq, dos, s));
    }
    GemmParams p{};
    p.offsets = a.offsets; p.E = E; p.S = S; p.f = f;
    p.a = doq; p.lda = d; p.as = dos; p.as_slab = 2LL * S;
    p.b0 = sv.wdq; p.ldb = d; p.bstride = wsz; p.bs0 = sv.wds; p.bs_slab = 2LL * f; p.bs_estride = wsz / 32;
    p.ldc = 2 * f; p.e0 = a.G; p.e1 = a.U; p.N = f; p.K = d;
    // dG | dU leave the epilogue only as E4M3 operands: along 2f (the dXp
    // GEMM's A operand) and along the expert's tokens (the weight gradient's).
    p.mxq = w.dguq; p.mxs = w.dgus; p.mxq_ld = 2LL * f; p.mxs_slab = 2LL * S;
    p.tq = w.dgut; p.ts = w.dguts; p.tq_ld = P; p.ts_slab = 4LL * f; p.poff = w.poff;
    TRY(launch_mx_ragged(BWD_DOWN, p, s));
  }
  {  // dXp = q(dGU) q([W_gate | W_up])^T: dGU along 2f (above); the weights
     // [d][f] along f were quantised by the forward.
    GemmParams p{};
    p.offsets = a.offsets; p.E = E; p.S = S; p.f = f;
    p.a = w.dguq; p.lda = 2 * f; p.as = w.dgus; p.as_slab = 2LL * S;
    p.b0 = sv.wgq; p.b1 = sv.wuq; p.ldb = f; p.bstride = wsz;
    p.bs0 = sv.wgs; p.bs1 = sv.wus; p.bs_slab = 2LL * d; p.bs_estride = wsz / 32;
    p.c0 = a.dxp; p.ldc = d; p.N = d; p.K = 2 * f;
    TRY(launch_mx_ragged(BWD_GU, p, s));
  }
  // Weight gradients: every operand along the expert's tokens, transposed.
  {  // dW_down[e] = q(H_e)^T q(dO_e); q(H) along the tokens came from the
     // forward's gate/up epilogue, q(dO) along the tokens from the combine
     // backward (else from d_o here).
    uint8_t *dot = w.dot, *dots = w.dots;
    if (a.d_o_mx != nullptr) {
      const MxImage im = mx_dout_image(a.d_o_mx, S, d, E).t;
      dot = im.q;
      dots = im.s;
    } else {
      TRY(launch_mx_tgroup_f32(a.d_o, S, d, w.blk, w.dot, P, w.dots, s));
    }
    GemmParams p{};
    p.offsets = w.poff; p.E = E; p.S = S;
    p.a = ht; p.lda = P; p.as = hts; p.as_slab = 2LL * f;
    p.b0 = dot; p.ldb = P; p.bs0 = dots; p.bs_slab = 2LL * d;
    p.c0 = a.dw_down; p.c1 = nullptr; p.ldc = d; p.cstride = static_cast<int64_t>(f) * d; p.M = f; p.N = d; p.f = d;
    TRY(launch_mx_wgrad(p, s));
  }
  {  // [dW_gate | dW_up][e] = q(Xp_e)^T q(dGU_e); q(Xp) along the tokens
     // came from the dispatch pass (else from xp here).
    uint8_t *xt = w.xt, *xts = w.xts;
    if (a.xp_mx != nullptr) {
      const MxImage im = mx_row_images(a.xp_mx, S, d, E).t;
      xt = im.q;
      xts = im.s;
    } else {
      TRY(launch_mx_tgroup(a.xp, S, d, w.blk, 1, 0, w.xt, P, 0, w.xts, 0, s));
    }
    GemmParams p{};
    p.offsets = w.poff; p.E = E; p.S = S;
    p.a = xt; p.lda = P; p.as = xts; p.as_slab = 2LL * d;
    p.b0 = w.dgut; p.ldb = P; p.bs0 = w.dguts; p.bs_slab = 4LL * f;
    p.c0 = a.dw_gate; p.c1 = a.dw_up; p.ldc = f; p.cstride = static_cast<int64_t>(d) * f; p.M = d; p.N = 2 * f; p.f = f;
    TRY(launch_mx_wgrad(p, s));
  }
  return hipSuccess;
}

}  // namespace moe
