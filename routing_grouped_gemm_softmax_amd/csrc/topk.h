// Top-k selection and gate renormalisation for one token, shared by the fp32
// and bf16 routers so both apply the same rule.
//
// Each token activates k of the E experts ("Olmo-core 3 é lançado com
// infraestrutura para treinar modelos MoE", section "Mudança de arquitetura e
// ganhos de desempenho"). Selection is on the logits (softmax is monotone):
// k rounds of a wave-wide arg-max, the larger value wins and equal values go
// to the lower expert index; the gates are the softmax over the k chosen
// logits, g_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) with l_0 the largest,
// which equals the full softmax renormalised over the chosen set.
#pragma once

#include "common.h"

namespace moe {

// v[q], live[q]: logit of expert q*64 + lane (E <= 256). On return sel_i[j],
// sel_v[j] (j < k <= 8) hold the chosen experts in selection order, in every
// lane.
__device__ __forceinline__ void wave_topk(float (&v)[4], bool (&live)[4], int k, int lane, float (&sel_v)[8],
                                          int (&sel_i)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {  // fully unrolled so sel_v/sel_i stay in registers
    if (j >= k) break;
    float bv = 0.0f;
    int bi = -1;
#pragma unroll
    for (int q = 0; q < 4; ++q)  // ascending index inside the lane; strict > keeps the lower index
      if (live[q] && (bi < 0 || v[q] > bv)) { bv = v[q]; bi = q * 64 + lane; }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      const bool take = (oi >= 0) && (bi < 0 || ov > bv || (ov == bv && oi < bi));
      if (take) { bv = ov; bi = oi; }
    }
    sel_v[j] = bv;
    sel_i[j] = bi;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (q == (bi >> 6) && (bi & 63) == lane) live[q] = false;
  }
}

// The same rule over 16-lane groups, one token per group: lane l holds
// v[q], live[q] of expert 16 q + l % 16 (E <= 16 NQ). Each lane first takes
// its best (ascending q, strict >), then four merges across the group. The
// order (larger value, then lower index) is total for non-NaN logits, so the
// choice equals wave_topk's.
template <int NQ>
__device__ __forceinline__ void group16_topk(const float (&v)[NQ], bool (&live)[NQ], int k, int lane,
                                             float (&sel_v)[8], int (&sel_i)[8]) {
  const int sub = lane & 15;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    float bv = 0.0f;
    int bi = -1;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      if (live[q] && (bi < 0 || v[q] > bv)) { bv = v[q]; bi = 16 * q + sub; }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 16);
      const int oi = __shfl_xor(bi, o, 16);
      const bool take = (oi >= 0) && (bi < 0 || ov > bv || (ov == bv && oi < bi));
      if (take) { bv = ov; bi = oi; }
    }
    sel_v[j] = bv;
    sel_i[j] = bi;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      if (bi == 16 * q + sub) live[q] = false;
  }
}

// Softmax over the chosen logits (sel_v[0] is the largest).
__device__ __forceinline__ void topk_gates(const float (&sel_v)[8], int k, float (&g)[8]) {
  float ex[8], sum = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < k) { ex[j] = expf(sel_v[j] - sel_v[0]); sum += ex[j]; }
#pragma unroll
  for (int j = 0; j < 8; ++j) g[j] = (j < k) ? ex[j] / sum : 0.0f;
}

}  // namespace moe
