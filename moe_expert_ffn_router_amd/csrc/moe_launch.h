// Internal launchers (host side). Arguments are validated by the C ABI layer
// before any of these is called; each only enqueues kernels on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int renorm, int32_t* ids,
                             float* wts, hipStream_t stream);

hipError_t launch_align(const int32_t* ids, int S, int E, int block_m, int cap,
                        int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                        hipStream_t stream);

// Routing + alignment in one single-workgroup launch; only for batches with
// route_align_fusable(T, E, k).
bool route_align_fusable(int T, int E, int k);
hipError_t launch_route_align(const float* logits, int T, int E, int k, int renorm,
                              int32_t* ids, float* wts, int block_m, int cap,
                              int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                              hipStream_t stream);

// Workspace carve-up shared by the FFN launchers and moe_ffn_workspace_bytes.
struct FfnWorkspace {
  size_t h_off, h_bytes;    // h per slot: bf16 [S, I] (bf16), f32 [S, I] (fp8, f32)
  size_t hq_off, hq_bytes;  // fp8: e4m3 codes of h [S, I]
  size_t hs_off, hs_bytes;  // fp8: scales of h, per slot [S] (block FP8: [S, I/128])
  size_t xq_off, xq_bytes;  // fp8: e4m3 codes of x [T, H]
  size_t xs_off, xs_bytes;  // fp8: scales of x, per token [T] (block FP8: [T, H/128])
  size_t y_off, y_bytes;    // per-slot FC2 output [S, H]: bf16 (bf16), f32 (fp8, f32)
  size_t q_off, q_bytes;    // work counters of the dense kernels, int32 [16]
  size_t plan_off, plan_bytes;  // token-range plan of the grouped-GEMM tiles (E > 0)
  size_t total;
};
// E = 0 leaves out the plan region (the small-batch forward has no use for it).
FfnWorkspace ffn_workspace_layout(int T, int E, int H, int I, int k, int dtype);

// Grouped-GEMM tiles of prefill-sized batches (moe_gemm.hip): a one-workgroup
// plan kernel cuts every expert's run of the aligned list into token ranges of
// at most 256 and zeroes the 2 x 8 work counters; FC1 / FC2 then run
// (range, 256-row tile) units.
size_t gemm_plan_ints(int S, int E);
bool gemm_supported(int T, int k, int H, int I);
hipError_t launch_gemm_plan(const int32_t* sorted_ids, const int32_t* block_expert,
                            const int32_t* num_padded, int S, int E, int log2m, int* plan,
                            int* queues, hipStream_t stream);
hipError_t launch_gemm_fc1(const void* x, const void* w1, const int32_t* sorted_ids,
                           const int* plan, int* queue, int H, int I, int k, int S, int remap,
                           void* h, hipStream_t stream);
hipError_t launch_gemm_fc2(const void* h, const void* w2, const int32_t* sorted_ids,
                           const int* plan, int* queue, int H, int I, int S, int remap, void* y,
                           hipStream_t stream);

struct FfnProblem {
  const void* x;
  const void* w1;
  const float* w1_scale;
  const void* w2;
  const float* w2_scale;
  const int32_t* topk_ids;
  const float* topk_weights;
  const int32_t* sorted_ids;
  const int32_t* block_expert;
  const int32_t* num_padded;
  int T, E, H, I, k, block_m;
  unsigned flags;
  void* workspace;
  void* out;
};

hipError_t launch_ffn_bf16(const FfnProblem& p, hipStream_t stream);
hipError_t launch_ffn_fp8(const FfnProblem& p, hipStream_t stream);
hipError_t launch_ffn_w8a16(const FfnProblem& p, hipStream_t stream);
hipError_t launch_ffn_fp8_block(const FfnProblem& p, hipStream_t stream);

// Forward of a small batch (T <= kSmallTokens, T k <= kSmallSlots): up to
// kSmallKernelTokens tokens and kSmallKernelSlots slots the small kernels
// (no alignment; split launches or one cooperative kernel), beyond them
// routing, alignment at the default block size and the FFN launchers.
constexpr int kSmallTokens = 64;
constexpr int kSmallExperts = 1024;
constexpr int kSmallSlots = 512;
constexpr int kSmallKernelTokens = 16;
constexpr int kSmallKernelSlots = 256;
inline bool small_kernels(int T, int k) {
  return T <= kSmallKernelTokens && (long)T * k <= kSmallKernelSlots;
}
// The block size of the decode regime for this batch (moe_default_block_m).
inline int default_block_m(int T, int E, int k) { return (long)T * k >= 128L * E ? 256 : 64; }
// Entries of sorted_ids the alignment may write: round_up(S + min(E, S)(M - 1), M).
inline size_t align_capacity(long S, int E, int block_m) {
  const long active = S < E ? S : E;
  const long cap = S + active * (block_m - 1);
  return (size_t)((cap + block_m - 1) / block_m * block_m);
}
struct SmallProblem {
  const float* logits;
  const void* x;
  const void* w1;
  const float* w1_scale;
  const void* w2;
  const float* w2_scale;
  int T, E, H, I, k, renorm;
  unsigned flags;
  int dtype;  // MOE_DTYPE_BF16 or MOE_DTYPE_FP8
  int32_t* ids;
  float* wts;
  void* workspace;
  void* out;
};
// Small kernels: ffn_workspace_layout of the dtype, then the barrier words
// (the last 4 bytes: the status word). Beyond them: the alignment outputs,
// then the FFN workspace.
size_t small_workspace_bytes(int T, int E, int H, int I, int k, int dtype);
hipError_t launch_forward_small(const SmallProblem& p, hipStream_t stream);

// Device address (current device) of the static scratch array of the
// allocation-free small-batch forward, kStaticScratchBytes long; looked up
// once per device.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
hipError_t static_scratch(void** ptr);
hipError_t launch_ffn_f32(const FfnProblem& p, hipStream_t stream);

}  // namespace moe
