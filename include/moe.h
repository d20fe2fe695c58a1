/*
 * moe.h -- C ABI of libmoe.so: the fused MoE expert feed-forward of LLM
 * serving on one AMD Instinct MI355X (gfx950).
 *
 * Path: router softmax + top-k  ->  token-to-expert alignment  ->
 *       FC1 (gate|up) + SiLU-and-mul  ->  FC2 (down)  ->  top-k weighted combine.
 *
 * Sources (web pages; cited by title and section):
 *  - "vLLM support for NVIDIA Vera Rubin NVL72" (Chinese summary), section
 *    "Locality domain": in small-token MoE decode the forward pass is dominated
 *    by reading the FC1/FC2 expert weights from HBM.
 *  - "vLLM SM architecture adaptation" (Chinese), section 4.3 and the selection
 *    flow figure of section 9: one fused kernel over all experts, FP8 dequant
 *    inside the GEMM loop; section 3.1: scaled GEMM with scales applied around
 *    an fp32 accumulator; section 1: FP8 is E4M3.
 *  - V100 vLLM fork article (Japanese), "wall 2": silu_and_mul between FC1 and
 *    FC2; "wall 5": MoE routing kernels and an FP8 activation quantiser.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never frees, keeps or reallocates them. Tensors are row-major, contiguous.
 *  - bf16 is passed as its uint16_t bit pattern; fp8 is OCP e4m3fn bytes
 *    (bias 7, max 448, no infinities).
 *  - Each call validates its arguments on the host, enqueues its kernels on
 *    `stream` (NULL = the null stream) and returns; it never synchronises the
 *    host, never allocates device memory and keeps no state between calls
 *    other than a per-device cache of launch geometry (CU count and resident
 *    workgroups per kernel) and, for moe_forward_small_static only, the
 *    device address of its static scratch array.
 *  - On a bad argument nothing is launched and the status says why. A launch
 *    failure returns MOE_ERR_HIP. Faults inside a kernel surface at the
 *    caller's next synchronisation, as usual in HIP. Device-resident values
 *    are not validated (e.g. an expert id outside [0, E) is undefined).
 *  - Inputs are never written. Calls are reentrant when their outputs and
 *    workspaces do not overlap.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t* moe_stream_t; /* identical to hipStream_t */

#define MOE_ABI_VERSION 1

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  MOE_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
  MOE_ERR_WORKSPACE = 4,   /* workspace too small */
  MOE_ERR_UNSUPPORTED = 5, /* a valid request this library does not serve */
  MOE_ERR_HIP = 6          /* a HIP runtime call or launch failed */
} moe_status;

/* Element types of the FFN (argument `dtype` of moe_ffn_workspace_bytes). */
enum {
  MOE_DTYPE_F32 = 0,
  MOE_DTYPE_BF16 = 1,
  MOE_DTYPE_FP8 = 2,
  MOE_DTYPE_W8A16 = 3,
  MOE_DTYPE_FP8_BLOCK = 4
};

/* `flags` bits of the moe_ffn_* calls.
 * Stage bits select which stages run; 0 (no stage bit) runs the whole FFN.
 *   PREP     : what FC1's kernel needs first: clearing the work counters of
 *              the dynamically scheduled launches [fp8: + per-token
 *              quantisation of x; block FP8: + x group quantisation]. A call
 *              that runs FC1 runs PREP too, unless it passes MOE_FFN_PREPARED:
 *              then an earlier call on the same workspace ran PREP for these
 *              inputs, and no FC1 ran since.
 * Running the stages in separate calls with the same workspace gives the same
 * result as one call (the workspace carries the intermediates). A call that
 * runs FC2 without FC1 continues from the last call on that workspace that
 * ran FC1 (with the same problem and buffers): it reads that call's h, and the
 * work counters its PREP cleared (each FC2 launch leaves them cleared again,
 * so FC2 may be run more than once).
 *   FC1      : FC1 gate|up + SiLU*up (with PREP unless MOE_FFN_PREPARED)
 *   FC2      : [fp8: per-slot quantisation of h +] FC2
 *   COMBINE  : top-k weighted combine into `out`
 * MOE_FFN_NO_XCD_REMAP turns off the placement of contiguous weight ranges
 * on one XCD (for A/B measurement); results are identical either way.
 * MOE_FFN_RANGE_GEMM (bf16, block_m >= 128, H and I multiples of 128 and at
 * least 256): run FC1 and FC2 as 256 x 256 tiles over balanced token ranges
 * of each expert (up to 256 of its tokens x 256 weight rows) instead of the
 * default 128-row tiles of the aligned blocks; results agree within the bf16
 * tolerance. Ignored where its conditions do not hold. */
#define MOE_FFN_STAGE_FC1 (1u << 0)
#define MOE_FFN_STAGE_FC2 (1u << 1)
#define MOE_FFN_STAGE_COMBINE (1u << 2)
#define MOE_FFN_STAGE_PREP (1u << 3)
#define MOE_FFN_PREPARED (1u << 11)
#define MOE_FFN_NO_XCD_REMAP (1u << 8)
#define MOE_FFN_RANGE_GEMM (1u << 10)
/* moe_forward_small only: run the whole layer as one cooperative kernel */
#define MOE_FORWARD_ONE_KERNEL (1u << 9)

/* Human-readable name of a status (static storage, never NULL). */
const char* moe_status_str(moe_status s);

/* MOE_ABI_VERSION of the loaded library. */
int moe_abi_version(void);

/*
 * Router softmax + top-k.
 * Passage: the Vera Rubin page ("hardware growth vs bottlenecks") links FP32
 * exp throughput to softmax; the V100 article ("wall 5") names the MoE routing
 * kernels. The ordering rule is this library's reading (the pages give none).
 *
 *  logits        [T, E] float32, device.
 *  topk_ids      [T, k] int32, device, written: for each token the k experts
 *                first in the order (logit descending, expert index ascending;
 *                -0.0 equals +0.0; -inf sorts last). Slot j is the j-th.
 *  topk_weights  [T, k] float32, device, written: p[e] = softmax(logits[t])[e]
 *                of each chosen expert, computed in fp32; divided by the sum
 *                of the k chosen p when renormalize != 0.
 *  Limits: 0 <= T, 1 <= E <= 1024, 1 <= k <= E. T == 0 launches nothing.
 *  NaN logits, or a row whose logits are all -inf, are outside the contract.
 */
moe_status moe_route_topk(const float* logits, int T, int E, int k, int renormalize,
                          int32_t* topk_ids, float* topk_weights, moe_stream_t stream);

/*
 * Token-to-expert alignment.
 * Passage: "vLLM SM architecture adaptation", section 4.3 and the section 9
 * figure run the MoE layer as one fused kernel over all experts; the index
 * structure such a kernel needs is this library's reading.
 *
 * moe_align_capacity returns the number of int32 elements `sorted_ids` must
 * hold: round_up(S + min(E, S) * (block_m - 1), block_m), S = T * k. The
 * number of blocks is capacity / block_m (the length of `block_expert`).
 *
 *  topk_ids      [T, k] int32, device: expert of flat slot s = t*k + j. An
 *                id outside [0, E) marks a slot whose expert another shard
 *                serves (expert parallelism, local expert numbering): the slot
 *                is left out of the lists.
 *  sorted_ids    [capacity] int32, device, written: for e = 0..E-1 the slots
 *                routed to e in ascending s, each expert's run padded to a
 *                multiple of block_m with the sentinel S. Entries at and past
 *                *num_padded also hold S.
 *  block_expert  [capacity / block_m] int32, device, written: the expert of
 *                each block; -1 for blocks at and past *num_padded / block_m.
 *  num_padded    [1] int32, device, written: total padded length (a multiple
 *                of block_m).
 *  Limits: 0 <= T, 1 <= E <= 1024, 1 <= k <= E, T * k < 2^24, block_m a power
 *  of two in [1, 256]. The result is deterministic (no order-dependent atomics).
 */
size_t moe_align_capacity(int T, int k, int E, int block_m);
moe_status moe_align_block(const int32_t* topk_ids, int T, int k, int E, int block_m,
                           int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                           moe_stream_t stream);

/*
 * Routing and alignment in one call: the same results as moe_route_topk
 * followed by moe_align_block on its topk_ids (same passages, same argument
 * meanings and limits). Batches of at most 8 tokens (and T * k <= 4096) run
 * as a single one-workgroup launch that keeps the ids on chip between the two
 * steps; larger batches run the two kernels. T == 0 still writes
 * *num_padded = 0.
 */
moe_status moe_route_align(const float* logits, int T, int E, int k, int renormalize,
                           int block_m, int32_t* topk_ids, float* topk_weights,
                           int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                           moe_stream_t stream);

/*
 * Block size suggested for a batch: 256 when the average number of slots per
 * expert, T*k/E, is at least 128 (prefill-sized blocks: the FFN then runs
 * grouped-GEMM tiles of 256 weight rows x 256 tokens), else 64 (decode: the
 * FFN streams weight tiles and shares up to 64 tokens of a block per tile).
 * Any power of two in [1, 256] is valid for every entry point; this one only
 * picks the fast regime. Returns 0 for invalid T, E or k.
 */
int moe_default_block_m(int T, int E, int k);

/*
 * Bytes of device workspace the FFN needs (dtype = MOE_DTYPE_*). Base must be
 * 256-byte aligned; its contents need no initialisation. Layout, S = T*k,
 * each region starting at the next 256-byte boundary after the previous one:
 *   bf16: h bf16 [S, I] | y bf16 [S, H]
 *   fp8 : h f32 [S, I] | hq e4m3 [S, I] | hs f32 [S] | xq e4m3 [T, H] |
 *         xs f32 [T] | y f32 [S, H]
 *   f32 : h f32 [S, I] | y f32 [S, H]
 *   w8a16: as bf16
 *   fp8_block: as fp8, with hs f32 [S, I/128] and xs f32 [T, H/128]
 * h = SiLU(gate) * up and y = FC2 output, both indexed by flat slot
 * s = t*k + j; hq/hs and xq/xs are the quantised h and x with their scales.
 */
size_t moe_ffn_workspace_bytes(int T, int E, int H, int I, int k, int block_m, int dtype);

/*
 * FFN, bf16 weights and activations, fp32 accumulation.
 * Passage: FC1/FC2 of the Vera Rubin page ("Locality domain"); silu_and_mul of
 * the V100 article ("wall 2"); the combine (sum over a token's k slots of
 * weight x expert output) is the plain reading of a top-k MoE layer.
 *
 *  x             [T, H] bf16.
 *  w1            [E, 2I, H] bf16: rows [0, I) gate, rows [I, 2I) up.
 *  w2            [E, H, I] bf16.
 *  topk_ids, topk_weights   from moe_route_topk (weights are read by COMBINE).
 *  sorted_ids, block_expert, num_padded   from moe_align_block with the same
 *                T, k, E and block_m.
 *  out           [T, H] bf16, written: out[t] = sum_j w[t,j] * y[t*k+j],
 *                accumulated in fp32 in j order, rounded once (RNE). Slots
 *                whose id lies outside [0, E) (served by another shard) add
 *                nothing, so out is this shard's partial sum.
 *  Intermediate h is rounded to bf16 before FC2.
 *  Limits: 0 <= T, 1 <= E <= 1024, 1 <= k <= E, T * k < 2^24, H and I
 *  multiples of 8, block_m a power of two in [1, 256]; x, w1, w2, out and
 *  workspace 16-byte aligned (workspace 256-byte aligned). H and I multiples
 *  of 128 run the tiled kernels (weight streaming, grouped-GEMM tiles); other
 *  multiples of 8 a plain path of one wave per output element, which reads
 *  the weights once per slot (correct for any such shape, not a fast path).
 */
moe_status moe_ffn_bf16(const uint16_t* x, const uint16_t* w1, const uint16_t* w2,
                        const int32_t* topk_ids, const float* topk_weights,
                        const int32_t* sorted_ids, const int32_t* block_expert,
                        const int32_t* num_padded, int T, int E, int H, int I, int k,
                        int block_m, unsigned flags, void* workspace, size_t workspace_bytes,
                        uint16_t* out, moe_stream_t stream);

/*
 * FFN, W8A8 OCP fp8 e4m3fn with fp32 accumulation (scaled-GEMM semantics of
 * "vLLM SM architecture adaptation" section 3.1; FP8 activation quantiser of
 * the V100 article, "wall 5").
 *
 *  x             [T, H] bf16; quantised inside per token: a_t = absmax/448
 *                (fp32; 1 for a zero row), code = e4m3fn_rne_sat(x / a_t).
 *  w1            [E, 2I, H] e4m3fn codes, w1_scale [E, 2I] fp32 per output row.
 *  w2            [E, H, I] e4m3fn codes, w2_scale [E, H] fp32 per output row.
 *  h = SiLU(g) * u is formed in fp32 with g = acc * w1_scale * a_t (likewise u)
 *  and quantised per (token, expert) slot row the same way before FC2;
 *  y = acc * w2_scale * b_s. Other arguments and limits as moe_ffn_bf16.
 */
moe_status moe_ffn_fp8(const uint16_t* x, const uint8_t* w1, const float* w1_scale,
                       const uint8_t* w2, const float* w2_scale, const int32_t* topk_ids,
                       const float* topk_weights, const int32_t* sorted_ids,
                       const int32_t* block_expert, const int32_t* num_padded, int T, int E,
                       int H, int I, int k, int block_m, unsigned flags, void* workspace,
                       size_t workspace_bytes, uint16_t* out, moe_stream_t stream);

/*
 * FFN, block-scaled OCP fp8 e4m3fn: 128 x 128 weight blocks and 1 x 128
 * activation groups, each with an fp32 scale, fp32 accumulation. Passage:
 * "vLLM SM architecture adaptation", sections 4.1 (block FP8 MoE backends),
 * 4.2 (block-wise FP8 grouped GEMM) and the runtime selection-flow figure of
 * section 9 (block-wise FP8 dequantisation inside the GEMM loop); the
 * 128-element block edge follows the 128-wide tiles named in that figure.
 *
 *  x             [T, H] bf16; quantised inside per (token, group of 128
 *                columns): a = absmax/448 (fp32; 1 for an all-zero group),
 *                code = e4m3fn_rne_sat(x / a).
 *  w1            [E, 2I, H] e4m3fn codes; w1_scale [E, 2I/128, H/128] fp32,
 *                one per 128 x 128 block (row block, column block).
 *  w2            [E, H, I] e4m3fn codes; w2_scale [E, H/128, I/128] fp32.
 *  For output row n and K-block c the partial sum over the block's 128 codes
 *  is multiplied by w_scale[e, n/128, c] * a[row, c] and added in fp32:
 *  g, u -> h = SiLU(g) * u in fp32, quantised per (slot, group of 128) the
 *  same way, -> y; combine as moe_ffn_fp8. Other arguments and limits as
 *  moe_ffn_bf16, but H and I multiples of 128; scale pointers non-null and
 *  4-byte aligned when T > 0. Workspace: moe_ffn_workspace_bytes(...,
 *  MOE_DTYPE_FP8_BLOCK). Every block runs the decode-regime streaming
 *  kernels (weights re-read once per 8 tokens of a block): meant for small T.
 */
moe_status moe_ffn_fp8_block(const uint16_t* x, const uint8_t* w1, const float* w1_scale,
                             const uint8_t* w2, const float* w2_scale, const int32_t* topk_ids,
                             const float* topk_weights, const int32_t* sorted_ids,
                             const int32_t* block_expert, const int32_t* num_padded, int T,
                             int E, int H, int I, int k, int block_m, unsigned flags,
                             void* workspace, size_t workspace_bytes, uint16_t* out,
                             moe_stream_t stream);

/*
 * FFN, weight-only fp8 (W8A16): e4m3fn weight codes with fp32 per-output-row
 * scales, bf16 activations, fp32 accumulation. The codes are widened on the
 * fly to bf16 (exact: every e4m3fn value is a bf16 value) and multiplied on
 * the bf16 matrix cores; no activation is quantised. Passage: "vLLM SM
 * architecture adaptation", sections 4.2 (weight-only fallback MoE backend)
 * and 5.2 (one FP8 weight format served either by FP8 matrix units or by
 * dequantising weights for 16-bit matrix units).
 *
 *  x             [T, H] bf16.
 *  w1            [E, 2I, H] e4m3fn codes, w1_scale [E, 2I] fp32 per output row.
 *  w2            [E, H, I] e4m3fn codes, w2_scale [E, H] fp32 per output row.
 *  g = w1_scale[e, n] * sum_c dec(w1[e, n, c]) * x[t, c] (likewise u);
 *  h = SiLU(g) * u rounded to bf16; y = w2_scale[e, n] * (dec(w2[e, n]) . h)
 *  rounded to bf16; combine and everything else as moe_ffn_bf16 (same limits
 *  but H and I multiples of 128, scale pointers non-null and 16-byte aligned
 *  when T > 0). Workspace:
 *  moe_ffn_workspace_bytes(..., MOE_DTYPE_W8A16). Every block runs the
 *  decode-regime streaming kernels (weights are re-read once per 8 tokens of a
 *  block), so the path is meant for small T.
 */
moe_status moe_ffn_w8a16(const uint16_t* x, const uint8_t* w1, const float* w1_scale,
                         const uint8_t* w2, const float* w2_scale, const int32_t* topk_ids,
                         const float* topk_weights, const int32_t* sorted_ids,
                         const int32_t* block_expert, const int32_t* num_padded, int T, int E,
                         int H, int I, int k, int block_m, unsigned flags, void* workspace,
                         size_t workspace_bytes, uint16_t* out, moe_stream_t stream);

/*
 * FFN, fp32 throughout (small problems; plain wave-per-output kernels, not a
 * performance path). Same semantics as moe_ffn_bf16 with float32 x, w1, w2,
 * h and out. Limits: H and I multiples of 4; otherwise as moe_ffn_bf16.
 */
moe_status moe_ffn_f32(const float* x, const float* w1, const float* w2,
                       const int32_t* topk_ids, const float* topk_weights,
                       const int32_t* sorted_ids, const int32_t* block_expert,
                       const int32_t* num_padded, int T, int E, int H, int I, int k,
                       int block_m, unsigned flags, void* workspace, size_t workspace_bytes,
                       float* out, moe_stream_t stream);

/*
 * Forward of a small batch in one call: router softmax + top-k, FC1 +
 * SiLU*up, FC2 and the combine. Passage: "vLLM SM architecture adaptation",
 * section 4.3: for a batch of at most 8 tokens the grouped-GEMM path's launch
 * overhead is what a single-kernel path avoids.
 * Up to 16 tokens and 256 slots it runs without an alignment step: by default
 * as separate launches (routing; fp8: x quantiser; FC1; fp8: h quantiser; FC2;
 * combine) in which FC1 and FC2 each group the slots by expert in LDS from the
 * routed ids; with MOE_FORWARD_ONE_KERNEL the whole layer is one cooperative
 * persistent kernel (plus a 256-thread kernel that clears its barrier words).
 * The results equal, bit for bit, moe_route_topk -> moe_align_block ->
 * moe_ffn_bf16 / moe_ffn_fp8 at the same T (any block_m): every expert's slots
 * are served by the same 8-token streaming passes.
 * From 17 to 64 tokens (or beyond 256 slots) it runs exactly those calls
 * (moe_route_topk, moe_align_block at moe_default_block_m, then the FFN) in
 * its own workspace: on MI355X the separate launches beat one cooperative
 * kernel, and the aligned FFN stages the tokens of a popular expert once
 * instead of once per 8 of them.
 *
 *  logits        [T, E] fp32; renormalize as in moe_route_topk.
 *  x             [T, H] bf16.
 *  w1, w2        dtype MOE_DTYPE_BF16: bf16 [E, 2I, H] and [E, H, I];
 *                MOE_DTYPE_FP8: e4m3fn codes with w1_scale [E, 2I] and
 *                w2_scale [E, H] fp32 (16-byte aligned), as moe_ffn_fp8.
 *  topk_ids, topk_weights   [T, k], written (as moe_route_topk).
 *  out           [T, H] bf16, written.
 *  workspace     moe_forward_small_workspace_bytes(T, E, H, I, k, dtype)
 *                bytes (or more), 256-byte aligned, no initialisation needed.
 *                With MOE_FORWARD_ONE_KERNEL the last 4 of those bytes are a
 *                status word:
 *                0 after the call has run, nonzero if a device-side barrier
 *                wait gave up (out is then undefined; not expected, the launch
 *                guarantees residency).
 *  flags         0 or MOE_FFN_NO_XCD_REMAP, optionally | MOE_FORWARD_ONE_KERNEL
 *                (T <= 16 and T * k <= 256 only).
 *  Limits: 0 <= T <= moe_small_max_tokens() (64), 1 <= E <= 1024,
 *  1 <= k <= E, T * k <= 512, H and I multiples of 128. Returns
 *  MOE_ERR_SHAPE beyond them, MOE_ERR_UNSUPPORTED for another dtype or flag
 *  (or MOE_FORWARD_ONE_KERNEL beyond its batches), MOE_ERR_HIP if a launch
 *  (the cooperative one) is refused. Calls that share a workspace must not
 *  overlap in time.
 */
int moe_small_max_tokens(void);
size_t moe_forward_small_workspace_bytes(int T, int E, int H, int I, int k, int dtype);
moe_status moe_forward_small(const float* logits, const uint16_t* x, const void* w1,
                             const float* w1_scale, const void* w2, const float* w2_scale, int T,
                             int E, int H, int I, int k, int renormalize, int dtype,
                             unsigned flags, int32_t* topk_ids, float* topk_weights,
                             void* workspace, size_t workspace_bytes, uint16_t* out,
                             moe_stream_t stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same
 * computation, arguments, limits, flags and results (bit for bit) as
 * moe_forward_small, without the workspace arguments: the intermediates live
 * in a static device array of MOE_STATIC_SCRATCH_BYTES owned by the library,
 * one per GPU, allocated when the library's device code is loaded on that
 * GPU and held until the process ends. The call allocates nothing.
 *
 *  Errors: as moe_forward_small; MOE_ERR_WORKSPACE when the layer needs more
 *  than MOE_STATIC_SCRATCH_BYTES, i.e. when
 *  moe_forward_small_workspace_bytes(T, E, H, I, k, dtype) exceeds it;
 *  MOE_ERR_HIP if the array's device address cannot be obtained.
 *  Every call on one GPU uses that GPU's single array and leaves its
 *  contents behind; calls that overlap in time on one GPU (two streams, two
 *  host threads) race and give undefined results. Calls in one stream are
 *  ordered and safe. The device is the current device, as for every entry
 *  point.
 */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
moe_status moe_forward_small_static(const float* logits, const uint16_t* x, const void* w1,
                                    const float* w1_scale, const void* w2, const float* w2_scale,
                                    int T, int E, int H, int I, int k, int renormalize,
                                    int dtype, unsigned flags, int32_t* topk_ids,
                                    float* topk_weights, uint16_t* out, moe_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
