// Router softmax + top-k: one wave64 per token.
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
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

template <int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int renorm,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  const float* row = logits + (size_t)t * E;

  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = i * kWave + lane;
    v[i] = (e < E) ? row[e] : -INFINITY;
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < VPL; ++i) m = fmaxf(m, v[i]);
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i)
    if (i * kWave + lane < E) s += expf(v[i] - m);
  s = wave_sum(s);

  constexpr int kNone = 0x7fffffff;
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
    // butterfly leaves the same winner in every lane
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      const bool better = oe != kNone && (be == kNone || ov > bv || (ov == bv && oe < be));
      if (better) {
        bv = ov;
        be = oe;
      }
    }
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
      ids[(size_t)t * k + j] = my_id[i];
      wts[(size_t)t * k + j] = renorm ? my_p[i] / psum : my_p[i];
    }
  }
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int renorm, int32_t* ids,
                             float* wts, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + 3) / 4), block(256);
  const int vpl = (E + kWave - 1) / kWave;
  if (vpl <= 1)
    route_topk_kernel<1><<<grid, block, 0, stream>>>(logits, T, E, k, renorm, ids, wts);
  else if (vpl <= 2)
    route_topk_kernel<2><<<grid, block, 0, stream>>>(logits, T, E, k, renorm, ids, wts);
  else if (vpl <= 4)
    route_topk_kernel<4><<<grid, block, 0, stream>>>(logits, T, E, k, renorm, ids, wts);
  else if (vpl <= 8)
    route_topk_kernel<8><<<grid, block, 0, stream>>>(logits, T, E, k, renorm, ids, wts);
  else
    route_topk_kernel<16><<<grid, block, 0, stream>>>(logits, T, E, k, renorm, ids, wts);
  return hipGetLastError();
}

}  // namespace moe
