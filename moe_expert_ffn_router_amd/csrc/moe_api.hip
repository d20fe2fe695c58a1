// C ABI of libmoe.so: argument validation, then the launchers. Declared in
// include/moe.h; every export is listed there with its meaning and limits.
#include <hip/hip_runtime.h>

#include <limits.h>

#include "../../include/moe.h"
#include "moe_launch.h"

#define MOE_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kMaxE = 1024;
constexpr long kMaxSlots = 1L << 24;

bool is_pow2_le256(int v) { return v >= 1 && v <= 256 && (v & (v - 1)) == 0; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

moe_status check_common(int T, int E, int k) {
  if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > E) return MOE_ERR_SHAPE;
  if ((long)T * k >= kMaxSlots || (long)T * E > INT_MAX) return MOE_ERR_SHAPE;
  return MOE_OK;
}

size_t capacity(long S, int E, int block_m) { return moe::align_capacity(S, E, block_m); }

// Validation shared by the FFN entry points; H and I must be multiples of
// mult (f32: 4; bf16 and fp8: 8; weight-only and block-scaled fp8: 128).
moe_status check_ffn(const void* x, const void* w1, const void* w2, const int32_t* topk_ids,
                     const float* topk_weights, const int32_t* sorted_ids,
                     const int32_t* block_expert, const int32_t* num_padded, int T, int E, int H,
                     int I, int k, int block_m, unsigned flags, const void* workspace,
                     size_t workspace_bytes, const void* out, int dtype, int mult) {
  moe_status s = check_common(T, E, k);
  if (s != MOE_OK) return s;
  if (H < mult || I < mult || H % mult != 0 || I % mult != 0) return MOE_ERR_SHAPE;
  if (!is_pow2_le256(block_m)) return MOE_ERR_SHAPE;
  const unsigned known = MOE_FFN_STAGE_PREP | MOE_FFN_STAGE_FC1 | MOE_FFN_STAGE_FC2 |
                         MOE_FFN_STAGE_COMBINE | MOE_FFN_PREPARED | MOE_FFN_NO_XCD_REMAP |
                         MOE_FFN_RANGE_GEMM;
  if (flags & ~known) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w1 || !w2 || !topk_ids || !topk_weights || !sorted_ids || !block_expert ||
      !num_padded || !workspace || !out)
    return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w2, 16) || !aligned(out, 16) ||
      !aligned(workspace, 256) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4) ||
      !aligned(sorted_ids, 4) || !aligned(block_expert, 4) || !aligned(num_padded, 4))
    return MOE_ERR_ALIGN;
  if (workspace_bytes < moe::ffn_workspace_layout(T, E, H, I, k, dtype).total)
    return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

moe::FfnProblem problem(const void* x, const void* w1, const float* w1s, const void* w2,
                        const float* w2s, const int32_t* topk_ids, const float* topk_weights,
                        const int32_t* sorted_ids, const int32_t* block_expert,
                        const int32_t* num_padded, int T, int E, int H, int I, int k,
                        int block_m, unsigned flags, void* workspace, void* out) {
  return moe::FfnProblem{x, w1, w1s, w2, w2s, topk_ids, topk_weights, sorted_ids, block_expert,
                         num_padded, T, E, H, I, k, block_m, flags, workspace, out};
}

}  // namespace

MOE_EXPORT const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: a size is out of range or inconsistent";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: a pointer is not suitably aligned";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: request not served by this library";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP runtime call or kernel launch failed";
  }
  return "MOE_ERR_UNKNOWN: not a moe_status value";
}

MOE_EXPORT int moe_abi_version(void) { return MOE_ABI_VERSION; }

MOE_EXPORT moe_status moe_route_topk(const float* logits, int T, int E, int k, int renormalize,
                                     int32_t* topk_ids, float* topk_weights,
                                     moe_stream_t stream) {
  moe_status s = check_common(T, E, k);
  if (s != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_weights) return MOE_ERR_NULL;
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4))
    return MOE_ERR_ALIGN;
  return hip_status(moe::launch_route_topk(logits, T, E, k, renormalize ? 1 : 0, topk_ids,
                                           topk_weights, (hipStream_t)stream));
}

MOE_EXPORT size_t moe_align_capacity(int T, int k, int E, int block_m) {
  if (check_common(T, E, k) != MOE_OK || !is_pow2_le256(block_m)) return 0;
  return capacity((long)T * k, E, block_m);
}

MOE_EXPORT moe_status moe_align_block(const int32_t* topk_ids, int T, int k, int E, int block_m,
                                      int32_t* sorted_ids, int32_t* block_expert,
                                      int32_t* num_padded, moe_stream_t stream) {
  moe_status s = check_common(T, E, k);
  if (s != MOE_OK) return s;
  if (!is_pow2_le256(block_m)) return MOE_ERR_SHAPE;
  const long S = (long)T * k;
  const size_t cap = capacity(S, E, block_m);
  if (!num_padded) return MOE_ERR_NULL;
  if (S > 0 && !topk_ids) return MOE_ERR_NULL;
  if (cap > 0 && (!sorted_ids || !block_expert)) return MOE_ERR_NULL;
  if (!aligned(topk_ids, 4) || !aligned(sorted_ids, 4) || !aligned(block_expert, 4) ||
      !aligned(num_padded, 4))
    return MOE_ERR_ALIGN;
  return hip_status(moe::launch_align(topk_ids, (int)S, E, block_m, (int)cap, sorted_ids,
                                      block_expert, num_padded, (hipStream_t)stream));
}

MOE_EXPORT moe_status moe_route_align(const float* logits, int T, int E, int k, int renormalize,
                                      int block_m, int32_t* topk_ids, float* topk_weights,
                                      int32_t* sorted_ids, int32_t* block_expert,
                                      int32_t* num_padded, moe_stream_t stream) {
  moe_status s = check_common(T, E, k);
  if (s != MOE_OK) return s;
  if (!is_pow2_le256(block_m)) return MOE_ERR_SHAPE;
  const long S = (long)T * k;
  const size_t cap = capacity(S, E, block_m);
  if (!num_padded) return MOE_ERR_NULL;
  if (T > 0 && (!logits || !topk_ids || !topk_weights)) return MOE_ERR_NULL;
  if (cap > 0 && (!sorted_ids || !block_expert)) return MOE_ERR_NULL;
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4) ||
      !aligned(sorted_ids, 4) || !aligned(block_expert, 4) || !aligned(num_padded, 4))
    return MOE_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  if (moe::route_align_fusable(T, E, k))
    return hip_status(moe::launch_route_align(logits, T, E, k, renormalize ? 1 : 0, topk_ids,
                                              topk_weights, block_m, (int)cap, sorted_ids,
                                              block_expert, num_padded, st));
  if (T > 0) {
    const hipError_t e = moe::launch_route_topk(logits, T, E, k, renormalize ? 1 : 0, topk_ids,
                                                topk_weights, st);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return hip_status(moe::launch_align(topk_ids, (int)S, E, block_m, (int)cap, sorted_ids,
                                      block_expert, num_padded, st));
}

MOE_EXPORT int moe_small_max_tokens(void) { return moe::kSmallTokens; }

static moe_status check_small(int T, int E, int H, int I, int k, int dtype, unsigned flags) {
  moe_status s = check_common(T, E, k);
  if (s != MOE_OK) return s;
  if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_FP8) return MOE_ERR_UNSUPPORTED;
  if (T > moe::kSmallTokens || E > moe::kSmallExperts || (long)T * k > moe::kSmallSlots)
    return MOE_ERR_SHAPE;
  if (H < 128 || I < 128 || H % 128 != 0 || I % 128 != 0) return MOE_ERR_SHAPE;
  if (flags & ~(unsigned)(MOE_FFN_NO_XCD_REMAP | MOE_FORWARD_ONE_KERNEL)) return MOE_ERR_UNSUPPORTED;
  // the single cooperative kernel exists for the small kernels' batches only
  if ((flags & MOE_FORWARD_ONE_KERNEL) && !moe::small_kernels(T, k)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

MOE_EXPORT size_t moe_forward_small_workspace_bytes(int T, int E, int H, int I, int k,
                                                    int dtype) {
  if (check_small(T, E, H, I, k, dtype, 0) != MOE_OK) return 0;
  return moe::small_workspace_bytes(T, E, H, I, k, dtype);
}

MOE_EXPORT moe_status moe_forward_small(const float* logits, const uint16_t* x, const void* w1,
                                        const float* w1_scale, const void* w2,
                                        const float* w2_scale, int T, int E, int H, int I,
                                        int k, int renormalize, int dtype, unsigned flags,
                                        int32_t* topk_ids, float* topk_weights, void* workspace,
                                        size_t workspace_bytes, uint16_t* out,
                                        moe_stream_t stream) {
  moe_status s = check_small(T, E, H, I, k, dtype, flags);
  if (s != MOE_OK || T == 0) return s;
  const bool fp8 = dtype == MOE_DTYPE_FP8;
  if (!logits || !x || !w1 || !w2 || !topk_ids || !topk_weights || !workspace || !out)
    return MOE_ERR_NULL;
  if (fp8 && (!w1_scale || !w2_scale)) return MOE_ERR_NULL;
  if (!aligned(logits, 4) || !aligned(x, 16) || !aligned(w1, 16) || !aligned(w2, 16) ||
      !aligned(out, 16) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4) ||
      !aligned(workspace, 256) || (fp8 && (!aligned(w1_scale, 16) || !aligned(w2_scale, 16))))
    return MOE_ERR_ALIGN;
  if (workspace_bytes < moe::small_workspace_bytes(T, E, H, I, k, dtype)) return MOE_ERR_WORKSPACE;
  moe::SmallProblem p{logits, x, w1, fp8 ? w1_scale : nullptr, w2, fp8 ? w2_scale : nullptr,
                      T, E, H, I, k, renormalize ? 1 : 0, flags, dtype, topk_ids, topk_weights,
                      workspace, out};
  return hip_status(moe::launch_forward_small(p, (hipStream_t)stream));
}

MOE_EXPORT moe_status moe_forward_small_static(const float* logits, const uint16_t* x,
                                               const void* w1, const float* w1_scale,
                                               const void* w2, const float* w2_scale, int T,
                                               int E, int H, int I, int k, int renormalize,
                                               int dtype, unsigned flags, int32_t* topk_ids,
                                               float* topk_weights, uint16_t* out,
                                               moe_stream_t stream) {
  static_assert(moe::kStaticScratchBytes == MOE_STATIC_SCRATCH_BYTES, "scratch size");
  moe_status s = check_small(T, E, H, I, k, dtype, flags);
  if (s != MOE_OK || T == 0) return s;
  if (moe::small_workspace_bytes(T, E, H, I, k, dtype) > moe::kStaticScratchBytes)
    return MOE_ERR_WORKSPACE;
  const bool fp8 = dtype == MOE_DTYPE_FP8;
  if (!logits || !x || !w1 || !w2 || !topk_ids || !topk_weights || !out) return MOE_ERR_NULL;
  if (fp8 && (!w1_scale || !w2_scale)) return MOE_ERR_NULL;
  if (!aligned(logits, 4) || !aligned(x, 16) || !aligned(w1, 16) || !aligned(w2, 16) ||
      !aligned(out, 16) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4) ||
      (fp8 && (!aligned(w1_scale, 16) || !aligned(w2_scale, 16))))
    return MOE_ERR_ALIGN;
  void* ws = nullptr;
  if (moe::static_scratch(&ws) != hipSuccess) return MOE_ERR_HIP;
  moe::SmallProblem p{logits, x, w1, fp8 ? w1_scale : nullptr, w2, fp8 ? w2_scale : nullptr,
                      T, E, H, I, k, renormalize ? 1 : 0, flags, dtype, topk_ids, topk_weights,
                      ws, out};
  return hip_status(moe::launch_forward_small(p, (hipStream_t)stream));
}

MOE_EXPORT int moe_default_block_m(int T, int E, int k) {
  if (check_common(T, E, k) != MOE_OK) return 0;
  return moe::default_block_m(T, E, k);
}

MOE_EXPORT size_t moe_ffn_workspace_bytes(int T, int E, int H, int I, int k, int block_m,
                                          int dtype) {
  (void)block_m;
  if (dtype != MOE_DTYPE_F32 && dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_FP8 &&
      dtype != MOE_DTYPE_W8A16 && dtype != MOE_DTYPE_FP8_BLOCK)
    return 0;
  if (T < 0 || E < 1 || H < 1 || I < 1 || k < 1) return 0;
  // W8A16 keeps the bf16 path's intermediates
  return moe::ffn_workspace_layout(T, E, H, I, k,
                                   dtype == MOE_DTYPE_W8A16 ? MOE_DTYPE_BF16 : dtype)
      .total;
}

MOE_EXPORT moe_status moe_ffn_bf16(const uint16_t* x, const uint16_t* w1, const uint16_t* w2,
                                   const int32_t* topk_ids, const float* topk_weights,
                                   const int32_t* sorted_ids, const int32_t* block_expert,
                                   const int32_t* num_padded, int T, int E, int H, int I, int k,
                                   int block_m, unsigned flags, void* workspace,
                                   size_t workspace_bytes, uint16_t* out, moe_stream_t stream) {
  moe_status s = check_ffn(x, w1, w2, topk_ids, topk_weights, sorted_ids, block_expert,
                           num_padded, T, E, H, I, k, block_m, flags, workspace, workspace_bytes,
                           out, MOE_DTYPE_BF16, 8);
  if (s != MOE_OK || T == 0) return s;
  return hip_status(moe::launch_ffn_bf16(
      problem(x, w1, nullptr, w2, nullptr, topk_ids, topk_weights, sorted_ids, block_expert,
              num_padded, T, E, H, I, k, block_m, flags, workspace, out),
      (hipStream_t)stream));
}

MOE_EXPORT moe_status moe_ffn_fp8(const uint16_t* x, const uint8_t* w1, const float* w1_scale,
                                  const uint8_t* w2, const float* w2_scale,
                                  const int32_t* topk_ids, const float* topk_weights,
                                  const int32_t* sorted_ids, const int32_t* block_expert,
                                  const int32_t* num_padded, int T, int E, int H, int I, int k,
                                  int block_m, unsigned flags, void* workspace,
                                  size_t workspace_bytes, uint16_t* out, moe_stream_t stream) {
  moe_status s = check_ffn(x, w1, w2, topk_ids, topk_weights, sorted_ids, block_expert,
                           num_padded, T, E, H, I, k, block_m, flags, workspace, workspace_bytes,
                           out, MOE_DTYPE_FP8, 8);
  if (s != MOE_OK || T == 0) return s;
  if (!w1_scale || !w2_scale) return MOE_ERR_NULL;
  if (!aligned(w1_scale, 16) || !aligned(w2_scale, 16)) return MOE_ERR_ALIGN;
  return hip_status(moe::launch_ffn_fp8(
      problem(x, w1, w1_scale, w2, w2_scale, topk_ids, topk_weights, sorted_ids, block_expert,
              num_padded, T, E, H, I, k, block_m, flags, workspace, out),
      (hipStream_t)stream));
}

MOE_EXPORT moe_status moe_ffn_w8a16(const uint16_t* x, const uint8_t* w1, const float* w1_scale,
                                    const uint8_t* w2, const float* w2_scale,
                                    const int32_t* topk_ids, const float* topk_weights,
                                    const int32_t* sorted_ids, const int32_t* block_expert,
                                    const int32_t* num_padded, int T, int E, int H, int I, int k,
                                    int block_m, unsigned flags, void* workspace,
                                    size_t workspace_bytes, uint16_t* out, moe_stream_t stream) {
  // the bf16 path's shape rules (H, I multiples of 128: whole 128-byte lines of codes) and
  // its workspace
  moe_status s = check_ffn(x, w1, w2, topk_ids, topk_weights, sorted_ids, block_expert, num_padded, T, E,
                H, I, k, block_m, flags, workspace, workspace_bytes, out, MOE_DTYPE_BF16, 128);
  if (s != MOE_OK || T == 0) return s;
  if (!w1_scale || !w2_scale) return MOE_ERR_NULL;
  if (!aligned(w1_scale, 16) || !aligned(w2_scale, 16)) return MOE_ERR_ALIGN;
  return hip_status(moe::launch_ffn_w8a16(
      problem(x, w1, w1_scale, w2, w2_scale, topk_ids, topk_weights, sorted_ids, block_expert,
              num_padded, T, E, H, I, k, block_m, flags, workspace, out),
      (hipStream_t)stream));
}

MOE_EXPORT moe_status moe_ffn_fp8_block(const uint16_t* x, const uint8_t* w1,
                                        const float* w1_scale, const uint8_t* w2,
                                        const float* w2_scale, const int32_t* topk_ids,
                                        const float* topk_weights, const int32_t* sorted_ids,
                                        const int32_t* block_expert, const int32_t* num_padded,
                                        int T, int E, int H, int I, int k, int block_m,
                                        unsigned flags, void* workspace, size_t workspace_bytes,
                                        uint16_t* out, moe_stream_t stream) {
  moe_status s = check_ffn(x, w1, w2, topk_ids, topk_weights, sorted_ids, block_expert,
                           num_padded, T, E, H, I, k, block_m, flags, workspace, workspace_bytes,
                           out, MOE_DTYPE_FP8_BLOCK, 128);
  if (s != MOE_OK || T == 0) return s;
  if (!w1_scale || !w2_scale) return MOE_ERR_NULL;
  if (!aligned(w1_scale, 4) || !aligned(w2_scale, 4)) return MOE_ERR_ALIGN;
  return hip_status(moe::launch_ffn_fp8_block(
      problem(x, w1, w1_scale, w2, w2_scale, topk_ids, topk_weights, sorted_ids, block_expert,
              num_padded, T, E, H, I, k, block_m, flags, workspace, out),
      (hipStream_t)stream));
}

MOE_EXPORT moe_status moe_ffn_f32(const float* x, const float* w1, const float* w2,
                                  const int32_t* topk_ids, const float* topk_weights,
                                  const int32_t* sorted_ids, const int32_t* block_expert,
                                  const int32_t* num_padded, int T, int E, int H, int I, int k,
                                  int block_m, unsigned flags, void* workspace,
                                  size_t workspace_bytes, float* out, moe_stream_t stream) {
  moe_status s = check_ffn(x, w1, w2, topk_ids, topk_weights, sorted_ids, block_expert,
                           num_padded, T, E, H, I, k, block_m, flags, workspace, workspace_bytes,
                           out, MOE_DTYPE_F32, 4);
  if (s != MOE_OK || T == 0) return s;
  return hip_status(moe::launch_ffn_f32(
      problem(x, w1, nullptr, w2, nullptr, topk_ids, topk_weights, sorted_ids, block_expert,
              num_padded, T, E, H, I, k, block_m, flags, workspace, out),
      (hipStream_t)stream));
}
