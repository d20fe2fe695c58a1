// Router softmax + top-k for one token per wave, shared by the routing kernel
// and the fused routing + alignment kernel.
//
// Pages: "vLLM support for NVIDIA Vera Rubin NVL72" (hardware growth vs
// bottlenecks) ties FP32 exp throughput to softmax; the V100 vLLM fork article
// ("wall 5") names the MoE routing kernels. Ordering (logit descending, expert
// index ascending) and the optional renormalisation are this library's reading.
//
// Each lane keeps VPL = ceil(E/64) logits in registers (expert e = i*64 + lane).
// max and sum(exp) are wave butterflies; the k winners are found by k rounds of
// a wave arg-max under the total order (value desc, index asc). Selection works
// on the fp32 logits themselves, so it is exact and reproducible.
#pragma once

#include "moe_common.h"

namespace moe {

constexpr int kNoExpert = 0x7fffffff;

// One step of the wave arg-max: keep the better of (bv, be) and the partner's
// under (value desc, index asc); kNoExpert marks an empty candidate.
template <int STEP>
__device__ __forceinline__ void argmax_step(float& bv, int& be) {
  const float ov = wave_partner<STEP>(bv);
  const int oe = wave_partner<STEP>(be);
  const bool better = oe != kNoExpert && (be == kNoExpert || ov > bv || (ov == bv && oe < be));
  if (better) {
    bv = ov;
    be = oe;
  }
}

// This lane's logits of token t: expert i*64 + lane in v[i] (-inf past E).
template <int VPL>
__device__ __forceinline__ void load_logits(const float* __restrict__ logits, int t, int E,
                                            float (&v)[VPL]) {
  const int lane = threadIdx.x & 63;
  const float* row = logits + (size_t)t * E;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = i * kWave + lane;
    v[i] = (e < E) ? row[e] : -INFINITY;
  }
}

// Routes token t, whose logits the calling wave holds in v (load_logits);
// writes its k ids and weights (WT: with device-scope stores, for readers in
// the same kernel on other XCDs), and the ids also to ids_copy (e.g. LDS)
// when that is not null.
template <int VPL, bool WT = false>
__device__ __forceinline__ void route_token(const float (&v)[VPL], int t, int E, int k,
                                            int renorm, int32_t* __restrict__ ids,
                                            float* __restrict__ wts, int32_t* ids_copy) {
  const int lane = threadIdx.x & 63;
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < VPL; ++i) m = fmaxf(m, v[i]);
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i)
    if (i * kWave + lane < E) s += expf(v[i] - m);
  s = wave_sum(s);

  constexpr int kNone = kNoExpert;
  uint32_t taken = 0;
  int my_id[VPL];
  float my_p[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    my_id[i] = 0;
    my_p[i] = 0.f;
  }
  float psum = 0.f;
  for (int j = 0; j < k; ++j) {
    // best untaken expert of this lane; ascending i means ascending e, so a
    // strict '>' keeps the lower index on equal logits
    float bv = 0.f;
    int be = kNone;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = i * kWave + lane;
      if (e < E && !((taken >> i) & 1u) && (be == kNone || v[i] > bv)) {
        bv = v[i];
        be = e;
      }
    }
    // wave arg-max under (value desc, index asc); the order is total, so the
    // reduction leaves the same winner in every lane
    argmax_step<0>(bv, be);
    argmax_step<1>(bv, be);
    argmax_step<2>(bv, be);
    argmax_step<3>(bv, be);
    argmax_step<4>(bv, be);
    argmax_step<5>(bv, be);
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    const float p = expf(bv - m) / s;
    psum += p;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (i == (j >> 6) && lane == (j & 63)) {
        my_id[i] = be;
        my_p[i] = p;
      }
  }
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int j = i * kWave + lane;
    if (j < k) {
      const float wj = renorm ? my_p[i] / psum : my_p[i];
      if (WT) {
        st_dev(ids + (size_t)t * k + j, my_id[i]);
        st_dev(wts + (size_t)t * k + j, wj);
      } else {
        ids[(size_t)t * k + j] = my_id[i];
        wts[(size_t)t * k + j] = wj;
      }
      if (ids_copy) ids_copy[(size_t)t * k + j] = my_id[i];
    }
  }
}

}  // namespace moe
