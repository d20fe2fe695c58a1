// Router softmax + top-k: one wave64 per token (route_token, moe_route_dev.h).
#include "moe_common.h"
#include "moe_launch.h"
#include "moe_route_dev.h"

namespace moe {

template <int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int renorm,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ wts) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  float v[VPL];
  load_logits<VPL>(logits, t, E, v);
  route_token<VPL>(v, t, E, k, renorm, ids, wts, nullptr);
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
