// Token-to-expert alignment: a deterministic stable counting sort of the flat
// slots s = t*k + j by expert, each expert's run padded to a multiple of
// block_m with the sentinel S.
//
// Pages: "vLLM SM architecture adaptation", section 4.3 and the selection-flow
// figure of section 9, run the MoE layer as one fused kernel over all experts;
// the block-aligned index lists such a kernel walks are this library's reading.
//
// One workgroup of 8 waves. Wave w owns the contiguous slot range
// [w*per, (w+1)*per). (1) each wave histograms its range into its own LDS row
// (atomic increments: counts do not depend on order); (2) padded run lengths
// and their exclusive scan give each expert's offset; (3) a per-(wave, expert)
// base = offset + counts of lower waves; (4) each wave re-walks its range 64
// slots at a time: lanes holding the same expert are found with one ballot per
// expert-id bit, a lane's rank is the number of such lanes below it, and the
// group's leader advances the wave's running base. Every placement follows from
// slot order alone, so the output is identical on every run. Ids outside
// [0, E) mark slots of experts served by another shard and are left out.
#include "moe_common.h"
#include "moe_launch.h"
#include "moe_route_dev.h"

namespace moe {

constexpr int kAlignWaves = 8;
constexpr int kAlignThreads = kAlignWaves * kWave;
constexpr int kAlignMaxE = 1024;
constexpr int kAlignUnroll = 16;
constexpr int kFuseMaxTokens = kAlignWaves;  // fused routing + alignment: one token per wave
constexpr int kFuseMaxSlots = 4096;          // and ids that fit a 16 KB LDS table
constexpr int kAlignWideWaves = 16;          // align_kernel's width for large batches
constexpr int kAlignWideSlots = 16384;

// The whole alignment, run by one workgroup of NW waves. ids may live in
// global memory or in LDS; cnt and off are the workgroup's LDS tables.
template <int NW>
__device__ __forceinline__ void align_body(const int32_t* ids, int S, int E, int log2m, int cap,
                                           int32_t* __restrict__ sorted_ids,
                                           int32_t* __restrict__ block_expert,
                                           int32_t* __restrict__ num_padded,
                                           int (*cnt)[kAlignMaxE], int* off) {
  constexpr int kAlignWaves = NW, kAlignThreads = NW * kWave;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int M = 1 << log2m;

  for (int i = tid; i < kAlignWaves * E; i += kAlignThreads) cnt[i / E][i % E] = 0;
  for (int i = tid; i < cap; i += kAlignThreads) sorted_ids[i] = S;
  for (int i = tid; i < (cap >> log2m); i += kAlignThreads) block_expert[i] = -1;
  __syncthreads();

  const int per = (S + kAlignWaves - 1) / kAlignWaves;
  const int s0 = min(S, w * per), s1 = min(S, s0 + per);

  // (1) per-wave histogram
  for (int sb = s0; sb < s1; sb += kWave * kAlignUnroll) {
    int e[kAlignUnroll];
#pragma unroll
    for (int u = 0; u < kAlignUnroll; ++u) {
      const int s = sb + u * kWave + lane;
      e[u] = s < s1 ? ids[s] : -1;
    }
#pragma unroll
    for (int u = 0; u < kAlignUnroll; ++u)
      if ((unsigned)e[u] < (unsigned)E) atomicAdd(&cnt[w][e[u]], 1);  // else: remote or past s1
  }
  __syncthreads();

  // (2) padded run length per expert, then exclusive scan by wave 0
  for (int e = tid; e < E; e += kAlignThreads) {
    int c = 0;
#pragma unroll
    for (int q = 0; q < kAlignWaves; ++q) c += cnt[q][e];
    off[e] = ((c + M - 1) >> log2m) << log2m;
  }
  __syncthreads();
  if (w == 0) {
    const int chunk = (E + kWave - 1) / kWave;
    const int e0 = min(E, lane * chunk), e1 = min(E, e0 + chunk);
    int local = 0;
    for (int e = e0; e < e1; ++e) local += off[e];
    int incl = local;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    int run = incl - local;
    for (int e = e0; e < e1; ++e) {
      const int pe = off[e];
      off[e] = run;
      run += pe;
    }
    if (lane == kWave - 1) off[E] = incl;
  }
  __syncthreads();

  // (3) per-(wave, expert) bases and the block -> expert map
  for (int e = tid; e < E; e += kAlignThreads) {
    int run = off[e];
#pragma unroll
    for (int q = 0; q < kAlignWaves; ++q) {
      const int c = cnt[q][e];
      cnt[q][e] = run;
      run += c;
    }
    const int b1 = off[e + 1] >> log2m;
    for (int b = off[e] >> log2m; b < b1; ++b) block_expert[b] = e;
  }
  if (tid == 0) num_padded[0] = off[E];
  __syncthreads();

  // (4) stable scatter, 64 slots at a time in slot order
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  for (int sb = s0; sb < s1; sb += kWave * kAlignUnroll) {
    int ev[kAlignUnroll];
#pragma unroll
    for (int u = 0; u < kAlignUnroll; ++u) {
      const int s = sb + u * kWave + lane;
      ev[u] = s < s1 ? ids[s] : -1;
    }
#pragma unroll
    for (int u = 0; u < kAlignUnroll; ++u) {
      const int s = sb + u * kWave + lane;
      const bool valid = (unsigned)ev[u] < (unsigned)E;
      const int e = valid ? ev[u] : 0;
      uint64_t same = __ballot(valid);
      for (int bit = 0; bit < nbits; ++bit) {
        const bool one = (e >> bit) & 1;
        const uint64_t b = __ballot(valid && one);
        same &= one ? b : ~b;
      }
      const int rank = __popcll(same & below);
      const int tot = __popcll(same);
      int base = 0;
      if (valid) base = cnt[w][e];
      if (valid) sorted_ids[base + rank] = s;
      if (valid && rank == 0) cnt[w][e] = base + tot;
    }
  }
}

template <int NW>
__global__ __launch_bounds__(NW * kWave) void align_kernel(
    const int32_t* __restrict__ ids, int S, int E, int log2m, int cap,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ num_padded) {
  __shared__ int cnt[NW][kAlignMaxE];  // per-wave histograms, then per-wave bases
  __shared__ int off[kAlignMaxE + 1];  // padded exclusive offsets; off[E] = total
  align_body<NW>(ids, S, E, log2m, cap, sorted_ids, block_expert, num_padded, cnt, off);
}

// Alignment of a small batch (S <= NT slots, NT = 256, 512 or 1024 threads):
// one thread per slot. A slot's rank among its expert's slots is the number
// of equal ids before it in slot order (a pass over the ids in LDS), the
// expert counts come from LDS atomic increments (order-free), and one scan of
// the padded counts over the workgroup gives the offsets: the same placement
// as align_body, with three barriers instead of its per-wave tables. ids may
// live in global memory or in LDS; every thread of the workgroup (NT or more)
// calls this.
constexpr int kAlignSmallSlots = 1024;  // the largest NT

template <int NT>
struct AlignSmallLds {
  alignas(16) int ids[NT];
  int cnt[kAlignMaxE];
  int off[kAlignMaxE];
  int wsum[NT / kWave];
};

template <int NT>
__device__ __forceinline__ void align_small_body(const int32_t* ids, int S, int E, int log2m,
                                                 int cap, int32_t* __restrict__ sorted_ids,
                                                 int32_t* __restrict__ block_expert,
                                                 int32_t* __restrict__ num_padded,
                                                 AlignSmallLds<NT>& L) {
  static_assert(kAlignMaxE % NT == 0 && NT % kWave == 0, "small alignment width");
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, nt = blockDim.x;
  const int M = 1 << log2m;
  const int e = t < S ? ids[t] : -1;
  if (t < NT) L.ids[t] = e;
  for (int i = t; i < E; i += nt) L.cnt[i] = 0;
  for (int i = t; i < cap; i += nt) sorted_ids[i] = S;
  for (int i = t; i < (cap >> log2m); i += nt) block_expert[i] = -1;
  __syncthreads();
  const bool valid = (unsigned)e < (unsigned)E;  // else: remote slot or past S
  int rank = 0;
  if (valid) {
    // ids before this slot, four per LDS read; four reads per step, so that
    // a slot near the end of a large batch has several in flight instead of
    // waiting out one LDS round trip per four ids
    const int4* v4 = (const int4*)L.ids;
    int q = 0;
    for (; q + 16 <= t; q += 16) {
      const int4 v0 = v4[(q >> 2) + 0], v1 = v4[(q >> 2) + 1];
      const int4 v2 = v4[(q >> 2) + 2], v3 = v4[(q >> 2) + 3];
      rank += (v0.x == e) + (v0.y == e) + (v0.z == e) + (v0.w == e);
      rank += (v1.x == e) + (v1.y == e) + (v1.z == e) + (v1.w == e);
      rank += (v2.x == e) + (v2.y == e) + (v2.z == e) + (v2.w == e);
      rank += (v3.x == e) + (v3.y == e) + (v3.z == e) + (v3.w == e);
    }
    for (; q + 4 <= t; q += 4) {
      const int4 v = v4[q >> 2];
      rank += (v.x == e) + (v.y == e) + (v.z == e) + (v.w == e);
    }
    for (; q < t; ++q) rank += L.ids[q] == e;
    atomicAdd(&L.cnt[e], 1);
  }
  __syncthreads();
  // exclusive scan of the padded counts: thread t < NT owns experts
  // [kPer t, kPer t + kPer)
  constexpr int kPer = kAlignMaxE / NT;
  const bool scan = t < NT;
  int pc[kPer], local = 0, incl = 0;
  if (scan) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int x = kPer * t + i;
      pc[i] = x < E ? ((L.cnt[x] + M - 1) >> log2m) << log2m : 0;
      local += pc[i];
    }
    incl = local;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    if (lane == kWave - 1) L.wsum[w] = incl;
  }
  __syncthreads();
  if (scan) {
    int run = incl - local;
    for (int v = 0; v < w; ++v) run += L.wsum[v];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int x = kPer * t + i;
      if (x < E) {
        L.off[x] = run;
        for (int b = run >> log2m; b < (run + pc[i]) >> log2m; ++b) block_expert[b] = x;
      }
      run += pc[i];
    }
    if (t == NT - 1) num_padded[0] = run;
  }
  __syncthreads();
  if (valid) sorted_ids[L.off[e] + rank] = t;
}

template <int NT>
__global__ __launch_bounds__(NT) void align_small_kernel(
    const int32_t* __restrict__ ids, int S, int E, int log2m, int cap,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ num_padded) {
  __shared__ AlignSmallLds<NT> L;
  align_small_body<NT>(ids, S, E, log2m, cap, sorted_ids, block_expert, num_padded, L);
}

// Routing and alignment of a small batch in one launch: wave w routes token w
// (at most 8 tokens), keeping the ids in LDS as well, then the same workgroup
// aligns them from LDS: one launch and one memory round trip less than the
// two kernels. A wave that routes several tokens does them one after the
// other (about 5 us each on MI355X), which costs more than the launch it
// saves, so larger batches take the two kernels.
template <int VPL>
__global__ __launch_bounds__(kAlignThreads) void route_align_kernel(
    const float* __restrict__ logits, int T, int E, int k, int renorm,
    int32_t* __restrict__ ids, float* __restrict__ wts, int log2m, int cap,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ num_padded) {
  __shared__ union {
    struct {
      int cnt[kAlignWaves][kAlignMaxE];
      int off[kAlignMaxE + 1];
    } wide;
    AlignSmallLds<kAlignThreads> small;
  } lds;
  __shared__ int32_t ids_lds[kFuseMaxSlots];
  const int t = threadIdx.x >> 6;
  if (t < T) {  // uniform per wave
    float v[VPL];
    load_logits<VPL>(logits, t, E, v);
    route_token<VPL>(v, t, E, k, renorm, ids, wts, ids_lds);
  }
  __syncthreads();
  if (T * k <= kAlignThreads)
    align_small_body<kAlignThreads>(ids_lds, T * k, E, log2m, cap, sorted_ids, block_expert,
                                    num_padded, lds.small);
  else
    align_body<kAlignWaves>(ids_lds, T * k, E, log2m, cap, sorted_ids, block_expert, num_padded,
                            lds.wide.cnt, lds.wide.off);
}

static int ilog2_align(int block_m) {
  int log2m = 0;
  while ((1 << log2m) < block_m) ++log2m;
  return log2m;
}

bool route_align_fusable(int T, int E, int k) {
  (void)E;
  return T <= kFuseMaxTokens && (long)T * k <= kFuseMaxSlots;
}

hipError_t launch_route_align(const float* logits, int T, int E, int k, int renorm,
                              int32_t* ids, float* wts, int block_m, int cap,
                              int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                              hipStream_t stream) {
  const int log2m = ilog2_align(block_m);
  const int vpl = (E + kWave - 1) / kWave;
#define MOE_ROUTE_ALIGN(V)                                                               \
  route_align_kernel<V><<<1, kAlignThreads, 0, stream>>>(logits, T, E, k, renorm, ids, wts, \
                                                         log2m, cap, sorted_ids,            \
                                                         block_expert, num_padded)
  if (vpl <= 1)
    MOE_ROUTE_ALIGN(1);
  else if (vpl <= 2)
    MOE_ROUTE_ALIGN(2);
  else if (vpl <= 4)
    MOE_ROUTE_ALIGN(4);
  else if (vpl <= 8)
    MOE_ROUTE_ALIGN(8);
  else
    MOE_ROUTE_ALIGN(16);
#undef MOE_ROUTE_ALIGN
  return hipGetLastError();
}

hipError_t launch_align(const int32_t* ids, int S, int E, int block_m, int cap,
                        int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                        hipStream_t stream) {
  int log2m = 0;
  while ((1 << log2m) < block_m) ++log2m;
  if (S <= 256)
    align_small_kernel<256><<<1, 256, 0, stream>>>(ids, S, E, log2m, cap, sorted_ids,
                                                   block_expert, num_padded);
  else if (S <= kAlignSmallSlots)
    align_small_kernel<kAlignSmallSlots><<<1, kAlignSmallSlots, 0, stream>>>(
        ids, S, E, log2m, cap, sorted_ids, block_expert, num_padded);
  else if (S >= kAlignWideSlots)  // many slots: 16 waves share the two passes over them
    align_kernel<kAlignWideWaves><<<1, kAlignWideWaves * kWave, 0, stream>>>(
        ids, S, E, log2m, cap, sorted_ids, block_expert, num_padded);
  else
    align_kernel<kAlignWaves><<<1, kAlignThreads, 0, stream>>>(ids, S, E, log2m, cap, sorted_ids,
                                                               block_expert, num_padded);
  return hipGetLastError();
}

}  // namespace moe
