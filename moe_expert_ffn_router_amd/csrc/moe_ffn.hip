// Expert FFN of the fused MoE layer: FC1 (gate|up) + SiLU-and-mul, FC2, and
// the top-k weighted combine, for bf16 and W8A8 fp8 (e4m3fn) on gfx950, plus
// a plain fp32 path for small problems.
//
// Pages: "vLLM support for NVIDIA Vera Rubin NVL72", section "Locality
// domain": in small-token MoE decode the forward is dominated by reading the
// FC1/FC2 expert weights from HBM, activations are small. "vLLM SM
// architecture adaptation", sections 4.3 and 9: one fused kernel covers all
// experts and FP8 scales are applied around the fp32 accumulator (section 3.1).
// V100 fork article, "wall 2": silu_and_mul sits between FC1 and FC2.
//
// Design (MI355X). FC1 and FC2 are weight streams; one persistent launch per
// projection. The work list is made of quads: 4 consecutive 16-row weight
// tiles of one aligned block (one tile per wave of a 256-thread workgroup).
// Its length comes from num_padded on the device, so the host never waits.
// Workgroups own contiguous equal shares of the list; with the XCD remap the
// workgroups of one XCD (id mod 8) own one contiguous eighth, so each XCD's L2
// serves a contiguous slice of (expert, rows). A quad never straddles blocks,
// so its mode is uniform across the workgroup:
//  * cold (block holds <= 8 tokens): each wave streams its 16 rows on its own
//    as two "half-split" 8-row MFMA tiles that read whole 128-byte lines with
//    non-temporal loads, and gathers the few token rows straight from L2;
//  * hot (> 8 tokens): the workgroup stages the block's token rows in LDS,
//    256 bytes of K at a time, double buffered; each wave streams its 16 rows
//    in the plain 16x16 MFMA layout, reading next chunk's weights while it
//    multiplies the current one, and takes B fragments from LDS, so the
//    activations cross L2 once per quad instead of once per wave.
// Batches of at most 16 tokens take launches without the hot path (more
// registers for deeper load groups); their FC1 splits each cold tile's K range
// over the 4 waves of a workgroup instead (bf16 up to 16 tokens, the other
// formats up to 8), with (block, tile) units. When units are fewer than
// workgroups, unit i goes to workgroup i, which spreads them over the CUs.
// Prefill-sized
// blocks (block_m >= 128) take grouped-GEMM tiles through LDS instead.
// FC1 pairs gate rows with the matching up rows inside each tile so that
// SiLU(gate) * up is formed in registers.
#include "moe_common.h"
#include "moe_launch.h"
#include "moe_route_dev.h"

#include <map>
#include <mutex>
#include <type_traits>

#include "../../include/moe.h"

namespace moe {

constexpr int kColdMax = 8;     // a block with at most this many tokens is cold
// Work counters of a launch's dynamic schedule: FC1 uses queue[0, kQueues),
// FC2 queue[kQueues, 2 kQueues); queue[2 kQueues] counts FC2's finished
// workgroups (finish_queue).
constexpr int kQueues = 8;
constexpr int kQueueInts = 2 * kQueues + 1;
constexpr int kHotTok = 64;     // tokens per pass of a hot quad (4 MFMA column tiles)
constexpr int kHotChunk = 256;  // bytes of K per staged chunk (both dtypes)
// LDS rows are 256 bytes, unpadded: 16-byte column c of row r sits at column
// c ^ (r & 7), so the staging stores and the MFMA fragment reads (rows
// r0..r0+15 at one column) hit distinct banks.
constexpr int kLdsRow = kHotChunk;
// LDS of a hot launch: two staging buffers, the queue's two pick words, then
// the hot-first block order (hot_first_order: kOrdMax + kOrdCnt ints)
constexpr int kHotLds = 2 * kHotTok * kLdsRow + 16;
constexpr int kHotLdsTotal = kHotLds + 4 * (2048 + 12);
__device__ __forceinline__ int hswz(int row, int col16) { return row * kLdsRow + ((col16 ^ (row & 7)) << 4); }

// ------------------------------------------------- work partitioning ---

struct Share {
  long q0, q1;
};

// Fewer units than workgroups: unit i goes to workgroup i, so consecutive
// units land on different XCDs and, within an XCD, on different CUs (equal
// contiguous shares would give the units to every other workgroup, which the
// dispatcher packs onto every other CU).
__device__ __forceinline__ Share wg_share(long total, int remap) {
  int wg = blockIdx.x;
  const int G = gridDim.x;
  if (total < G) return wg < total ? Share{wg, wg + 1} : Share{0, 0};
  if (remap && (G & 7) == 0) wg = (wg & 7) * (G >> 3) + (wg >> 3);
  return {total * wg / G, total * (wg + 1) / G};
}

// Dynamic scheduler of streaming launches that mix hot and cold blocks (their
// quads differ in cost, so equal static shares would leave workgroups idle
// while others still hold slow quads). Workgroup g starts with unit v(g), its
// XCD-remapped index; every later unit comes from one global counter (zero at
// launch), published to the workgroup through one of two LDS words,
// alternating, with one barrier. A short unit requests its successor as it
// starts, so the atomic's latency hides under its streaming; a long one
// (early()) requests it only when it ends: taken at its start, the successor
// would be tied to this workgroup for the whole long unit while others run
// dry (kernel timestamps at 64 tokens, top-8 of 128 experts: every
// workgroup holding a hot unit of ~170 us had taken a second unit at time
// zero, and the last workgroups ended 100 us after the first).
// Which workgroup computes a unit never changes the result.
struct QuadQueue {
  int* cnt;
  int total, nxt = -1, par = 0;  // nxt: thread 0's requested unit, -1 none yet
  __device__ QuadQueue(int* c, int n, int remap) : cnt(c), total(n) {}
  __device__ __forceinline__ int first(int remap) {
    int wg = blockIdx.x;
    const int G = gridDim.x;
    if (remap && (G & 7) == 0) wg = (wg & 7) * (G >> 3) + (wg >> 3);
    return wg < total ? wg : -1;
  }
  // Request the successor of a unit now (all threads call it; thread 0 acts).
  __device__ __forceinline__ void early() {
    if (threadIdx.x == 0) nxt = (int)gridDim.x + atomicAdd(cnt, 1);
  }
  // All threads call it after finishing a unit.
  __device__ __forceinline__ int next(volatile __attribute__((address_space(3))) int* slots) {
    if (threadIdx.x == 0) {
      slots[par] = nxt >= 0 ? nxt : (int)gridDim.x + atomicAdd(cnt, 1);
      nxt = -1;
    }
    __syncthreads();
    const int u = slots[par];
    par ^= 1;
    return u < total ? u : -1;
  }
};

// End of an FC2 launch's dynamic schedule (all threads call it once, after
// their last pick): the last workgroup to get here sets the launch's n
// counters and the finish counter q[kQueues] back to zero, so a later call
// that runs FC2 alone finds them as the FC1 call's zeroing left them. Every
// workgroup arrives only after its last atomic on the counters has
// returned, so nothing touches them after the reset; the stores reach the
// next kernel at the launch boundary.
__device__ __forceinline__ void finish_queue(int* __restrict__ q, int n) {
  if (threadIdx.x == 0) {
    int* done = q + kQueues;
    if (atomicAdd(done, 1) == (int)gridDim.x - 1) {
      for (int i = 0; i < n; ++i) q[i] = 0;
      *done = 0;
    }
  }
}

// Hot-first block order of the dynamic queue. ord[0, nb) receives the blocks
// holding more than M/2 tokens ("very hot") first, then the other blocks of
// more than kColdMax tokens, both in list order, then the rest (reverse list
// order): hot units cost more than cold ones (they stage the block's token
// rows as well) and more so the more tokens the block holds, so handing them
// out heaviest first lets the cheaper units fill the tail, like a
// longest-first schedule. Real entries of a block form a prefix, so a block
// holds more than n tokens iff its entry n is a real slot: a load or two per
// block. All threads of the workgroup call it; returns the number of hot
// blocks (very hot included), or -1 (ord untouched) when nb exceeds kOrdMax.
// `wcnt` is 12 ints of LDS, `tmp` kOrdMax ints of LDS (scratch). Every
// workgroup computes the same order (it only depends on the block lists).
constexpr int kOrdMax = 2048;
constexpr int kOrdCnt = 12;
static_assert(kHotLdsTotal == kHotLds + 4 * (kOrdMax + kOrdCnt), "hot LDS layout");
__device__ int hot_first_order(const int32_t* __restrict__ sorted_ids,
                               const int32_t* __restrict__ block_expert, int nb, int M, int S,
                               int E, int* ord, int* wcnt, int* tmp) {
  if (nb > kOrdMax) return -1;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const uint64_t below = (1ull << lane) - 1;
  const int kv = M / 2;  // more tokens than this: very hot
  int v_base = 0, h_base = 0, c_base = 0;
  for (int b0 = 0; b0 < nb; b0 += 256) {
    const int b = b0 + t;
    bool hot = false, vhot = false;
    if (b < nb && M > kColdMax) {
      const int e = block_expert[b];
      const int32_t* ids = sorted_ids + (size_t)b * M;
      hot = (unsigned)e < (unsigned)E && (unsigned)ids[kColdMax] < (unsigned)S;
      vhot = hot && kv > kColdMax && (unsigned)ids[kv] < (unsigned)S;
    }
    const uint64_t vb = __ballot(vhot), hb = __ballot(hot && !vhot), cb = __ballot(b < nb && !hot);
    if (lane == 0) {
      wcnt[w] = __popcll(vb);
      wcnt[4 + w] = __popcll(hb);
      wcnt[8 + w] = __popcll(cb);
    }
    __syncthreads();
    int vp = v_base, hp = h_base, cp = c_base, vt = 0, ht = 0, ct = 0;
    for (int i = 0; i < 4; ++i) {
      if (i < w) {
        vp += wcnt[i];
        hp += wcnt[4 + i];
        cp += wcnt[8 + i];
      }
      vt += wcnt[i];
      ht += wcnt[4 + i];
      ct += wcnt[8 + i];
    }
    if (b < nb) {
      if (vhot) ord[vp + __popcll(vb & below)] = b;
      else if (hot) tmp[hp + __popcll(hb & below)] = b;
      else ord[nb - 1 - (cp + __popcll(cb & below))] = b;
    }
    v_base += vt;
    h_base += ht;
    c_base += ct;
    __syncthreads();
  }
  for (int i = t; i < h_base; i += 256) ord[v_base + i] = tmp[i];
  __syncthreads();
  return v_base + h_base;
}

// Number of real (non-sentinel) entries of block b; they form a prefix.
__device__ __forceinline__ int block_valid(const int32_t* __restrict__ sorted_ids, int b, int M,
                                           int S) {
  const int lane = threadIdx.x & 63;
  int m = 0;
  for (int i0 = 0; i0 < M; i0 += kWave) {
    const int i = i0 + lane;
    const bool v = i < M && sorted_ids[(size_t)b * M + i] < S;
    m += __popcll(__ballot(v));
  }
  return m;
}

// Aligned blocks to run: *num_padded / M, clamped to the capacity the
// alignment buffers hold for this block size, round_up(S + min(E, S)(M - 1),
// M) / M, so that a num_padded written for another block size cannot make a
// launch index past sorted_ids or block_expert.
__device__ __forceinline__ int num_blocks(const int32_t* __restrict__ num_padded, int S, int E,
                                          int log2m) {
  const long M = 1L << log2m;
  const long cap = (S + (long)min(E, S) * (M - 1) + M - 1) >> log2m;
  const long nb = (long)max(num_padded[0], 0) >> log2m;
  return (int)min(nb, cap);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// -------------------------------------------------- operand fragments ---
// bf16: one 16-byte load feeds v_mfma_f32_16x16x32_bf16 (8 elements/lane).
// fp8 : 32 bytes per lane feed v_mfma_scale_f32_16x16x128_f8f6f4; the two
//       16-byte halves sit `step` bytes apart (the same placement in A and B,
//       so every product pairs equal k).

template <bool FP8>
struct Frag;
template <>
struct Frag<false> {
  bf16x8 v;
  __device__ __forceinline__ void load_nt(const uint8_t* p, int) {
    v = __builtin_nontemporal_load((const bf16x8*)p);
  }
  __device__ __forceinline__ void load(const uint8_t* p, int) { v = *(const bf16x8*)p; }
  __device__ __forceinline__ void load_lo(const uint8_t* p) { v = *(const bf16x8*)p; }
  __device__ __forceinline__ void lds(const uint8_t* p, int) { v = *(const bf16x8*)p; }
  __device__ __forceinline__ void zero() { v = bf16x8{}; }
};
template <>
struct Frag<true> {
  i32x8 v;
  __device__ __forceinline__ void set(const u32x4& lo, const u32x4& hi) {
    v = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  __device__ __forceinline__ void load_nt(const uint8_t* p, int step) {
    set(__builtin_nontemporal_load((const u32x4*)p), __builtin_nontemporal_load((const u32x4*)(p + step)));
  }
  __device__ __forceinline__ void load(const uint8_t* p, int step) {
    set(*(const u32x4*)p, *(const u32x4*)(p + step));
  }
  // the first half only; the second is absent (a trailing half chunk)
  __device__ __forceinline__ void load_lo(const uint8_t* p) { set(*(const u32x4*)p, u32x4{0, 0, 0, 0}); }
  __device__ __forceinline__ void lds(const uint8_t* p, int step) {
    set(*(const u32x4*)p, *(const u32x4*)(p + step));
  }
  __device__ __forceinline__ void zero() { v = i32x8{}; }
};

__device__ __forceinline__ f32x4 mfma(const Frag<false>& a, const Frag<false>& b, const f32x4& c) {
  return mfma_bf16(a.v, b.v, c);
}
__device__ __forceinline__ f32x4 mfma(const Frag<true>& a, const Frag<true>& b, const f32x4& c) {
  return mfma_fp8(a.v, b.v, c);
}

// ------------------------------------------------ cold: half-split tiles ---
// A tile of 8 weight rows in which MFMA A-rows i and i+8 hold the SAME weight
// row (i & 7): A-row i < 8 carries the first 64 bytes of each 128-byte line of
// that row, A-row i >= 8 the second 64 bytes; B-columns j < 8 / j >= 8 carry
// the first / second halves of token (j & 7). The diagonal 8x8 blocks of D
// are the two half-sums and D[i][j] + D[i+8][j+8] the full dot product, while
// every load instruction reads 8 rows x one whole 128-byte line (lane l: row
// l & 7, half (l & 15) >> 3, 16 bytes at k-group l >> 4), so the weights can
// be loaded non-temporally without fetching any line twice. A k-chunk is one
// line (bf16) or two lines (fp8, `step` = 128) of each row. After the sum lane
// l in 0..7 holds tile rows 0..3 and lane l in 16..23 tile rows 4..7 (D row
// 4*(l >> 4) + r), both for token (l & 7).

template <bool FP8>
struct Cold {
  static constexpr int kChunk = FP8 ? 256 : 128;
  static constexpr int kStep = 128;
};

// k-chunks per pipeline group: more bytes in flight per wave, paid in
// registers. In the cold-only launch 4 (bf16) means 3 waves per SIMD instead
// of 4 but twice the bytes in flight per wave (FC2 of 16-token decode: +4%,
// FC1 unchanged). A launch that also holds the LDS-staged hot path runs two
// waves per SIMD for the hot passes' sake, so 4 costs it nothing there (FC2
// at 64 tokens, top-8 of 128 experts: 123.7 -> 121.0 us against 2).
template <bool FP8, bool HOT>
constexpr int cold_u() {
  return FP8 ? 1 : 4;
}

__device__ __forceinline__ int half_split_off() {
  const int lane = threadIdx.x & 63;
  return ((lane & 15) >> 3) * 64 + (lane >> 4) * 16;
}

template <bool FP8, int U>
struct ColdGroup {
  Frag<FP8> p[U], q[U], b[U];
  __device__ __forceinline__ void issue(const uint8_t* __restrict__ ap,
                                        const uint8_t* __restrict__ aq,
                                        const uint8_t* __restrict__ bp, bool ok, int c) {
    constexpr int CH = Cold<FP8>::kChunk, ST = Cold<FP8>::kStep;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      p[u].load_nt(ap + (size_t)(c + u) * CH, ST);
      q[u].load_nt(aq + (size_t)(c + u) * CH, ST);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      b[u].zero();
      if (ok) b[u].load(bp + (size_t)(c + u) * CH, ST);
    }
  }
  __device__ __forceinline__ void compute(f32x4& accp, f32x4& accq) const {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      accp = mfma(p[u], b[u], accp);
      accq = mfma(q[u], b[u], accq);
    }
  }
};

// accp/accq += tiles P/Q (this lane: ap, aq) . the token tile (this lane: bp,
// loaded only if ok) over kbytes bytes of every row. Two register groups
// alternate: the next group's loads are issued before the current group's
// MFMAs, so with in-order load counters they stay in flight meanwhile.
//
// The groups are walked in rotated order, starting at group rot mod ngrp and
// wrapping around (the chunks past the last whole group, and an fp8 trailing
// half chunk, still come last). Callers rotate by cold_rot(tile index): the
// waves that start together then read their rows at different offsets instead
// of all starting at a row's first line and advancing in step (5 is odd, so
// with a power-of-two group count consecutive tiles start on distinct groups).
// Measured at 16 tokens, fp8 FC1 kernel traces of one box: 127.2 -> 123.4 us,
// and with the XCD placement off 143.0 -> 123.5 us: the unrotated stream's
// rate depended on placement (fp8 FC1 had also ranged over 126-149 us from
// box to box), the rotated one did not. The bf16 tiles (rows twice as long,
// four chunks per group) measured 0.5-1.5 % slower rotated, so only fp8
// rotates.
__host__ __device__ constexpr int cold_rot(int r) { return r * 5; }

// First chunk (of U) of the gi-th group walked when ngrp groups start at
// group s0 (< ngrp) and wrap around.
template <int U>
__device__ __forceinline__ int rot_chunk(int gi, int s0, int ngrp) {
  const int x = gi + s0;
  return (x >= ngrp ? x - ngrp : x) * U;
}

template <bool FP8, int U>
__device__ __forceinline__ void cold_kloop(const uint8_t* __restrict__ ap,
                                           const uint8_t* __restrict__ aq,
                                           const uint8_t* __restrict__ bp, bool ok, int kbytes,
                                           f32x4& accp, f32x4& accq, int rot) {
  constexpr int CH = Cold<FP8>::kChunk, ST = Cold<FP8>::kStep;
  const int nch = kbytes / CH;
  const int ngrp = nch / U;
  const int s0 = FP8 && ngrp > 0 ? rot % ngrp : 0;
  // first chunk of the gi-th group walked (bf16: in order, see above)
  auto chunk = [&](int gi) {
    if constexpr (!FP8) return gi * U;
    return rot_chunk<U>(gi, s0, ngrp);
  };
  ColdGroup<FP8, U> g0, g1;
  if (ngrp > 0) g0.issue(ap, aq, bp, ok, chunk(0));
  int g = 0;
  for (; g + 1 < ngrp; g += 2) {
    g1.issue(ap, aq, bp, ok, chunk(g + 1));
    g0.compute(accp, accq);
    if (g + 2 < ngrp) g0.issue(ap, aq, bp, ok, chunk(g + 2));
    g1.compute(accp, accq);
  }
  if (g < ngrp) g0.compute(accp, accq);
  for (int c = ngrp * U; c < nch; ++c) {
    Frag<FP8> fp, fq, fb;
    fp.load_nt(ap + (size_t)c * CH, ST);
    fq.load_nt(aq + (size_t)c * CH, ST);
    fb.zero();
    if (ok) fb.load(bp + (size_t)c * CH, ST);
    accp = mfma(fp, fb, accp);
    accq = mfma(fq, fb, accq);
  }
  if (FP8 && (kbytes % CH) != 0) {  // trailing 128 bytes: one line per row
    Frag<FP8> fp, fq, fb;
    fp.load_lo(ap + (size_t)nch * CH);
    fq.load_lo(aq + (size_t)nch * CH);
    fb.zero();
    if (ok) fb.load_lo(bp + (size_t)nch * CH);
    accp = mfma(fp, fb, accp);
    accq = mfma(fq, fb, accq);
  }
}

// Full dot products of a half-split tile: lanes 0..7 and 16..23 hold them.
__device__ __forceinline__ f32x4 diag_sum(const f32x4& a) {
  const int src = ((threadIdx.x & 63) + 40) & 63;
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = a[i] + __shfl(a[i], src);
  return r;
}

// ------------------------------------------- hot: LDS-staged activations ---
// Plain 16x16 layout: lane l holds A row (l & 15) and B column (l & 15), k-group
// l >> 4; D rows 4*(l >> 4) + i, column l & 15. A chunk of 256 bytes of K is
// 4 (bf16) or 2 (fp8) MFMA k-steps; within a k-step of `kstep` bytes a lane
// takes 16 bytes at 16*g (bf16: kstep = 64) or 16 bytes at 16*g and at
// 64 + 16*g (fp8: kstep = 128), in A, in B and in LDS alike.

template <bool FP8>
struct Hot {
  static constexpr int kKstep = FP8 ? 128 : 64;
  static constexpr int kSteps = kHotChunk / kKstep;  // MFMA k-steps per chunk
};

template <bool FP8>
struct HotA {
  Frag<FP8> f[Hot<FP8>::kSteps];
  __device__ __forceinline__ void load(const uint8_t* __restrict__ a, int chunk) {
#pragma unroll
    for (int s = 0; s < Hot<FP8>::kSteps; ++s)
      f[s].load(a + (size_t)chunk * kHotChunk + s * Hot<FP8>::kKstep, 64);
  }
  // trailing half chunk (fp8 only: 128 bytes = one k-step)
  __device__ __forceinline__ void load_tail(const uint8_t* __restrict__ a, int chunk) {
    f[0].load(a + (size_t)chunk * kHotChunk, 64);
#pragma unroll
    for (int s = 1; s < Hot<FP8>::kSteps; ++s) f[s].zero();
  }
};

// One chunk of MFMAs for this wave's NT tiles: A from registers, B fragments
// from the LDS buffer, each B fragment read once for all NT tiles. A B
// fragment of k-step s takes the 16-byte column s*kKstep/16 + g (and, for fp8,
// the column 4 further); fragment rows are 16-aligned bases + (lane & 15), so
// the swizzle term is lane & 7.
template <bool FP8, int MT, int NT>
__device__ __forceinline__ void hot_compute(const HotA<FP8> (&a)[NT],
                                            const uint8_t* __restrict__ buf,
                                            f32x4 (&acc)[NT][4]) {
  const int lane = threadIdx.x & 63;
  const uint8_t* base = buf + (lane & 15) * kLdsRow;
  const int x = lane & 7, g = lane >> 4;
#pragma unroll
  for (int s = 0; s < Hot<FP8>::kSteps; ++s) {
    const int c0 = ((s * Hot<FP8>::kKstep / 16 + g) ^ x) << 4;
    const int c1 = ((s * Hot<FP8>::kKstep / 16 + 4 + g) ^ x) << 4;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      Frag<FP8> b;
      b.lds(base + t * 16 * kLdsRow + c0, c1 - c0);
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n][t] = mfma(a[n].f[s], b, acc[n][t]);
    }
  }
}

// Staging: 256 threads move 64 token rows x 256 bytes (4 x 16 bytes each).
struct Stage {
  u32x4 v[4];
  const uint8_t* src[4];  // this thread's 4 source rows (+ its byte offset), or null
  __device__ __forceinline__ void load(int chunk, int kbytes) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = u32x4{0, 0, 0, 0};
      const int off = chunk * kHotChunk + (threadIdx.x & 15) * 16;
      if (src[i] && off < kbytes) v[i] = *(const u32x4*)(src[i] + off);
    }
  }
  __device__ __forceinline__ void store(uint8_t* __restrict__ buf) const {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(u32x4*)(buf + hswz((threadIdx.x >> 4) + 16 * i, threadIdx.x & 15)) = v[i];
  }
};

// A chunk of this wave's NT weight tiles into registers (the trailing half
// chunk of fp8 rows zero-padded).
template <bool FP8, int NT>
__device__ __forceinline__ void hot_load_a(HotA<FP8> (&f)[NT], const uint8_t* const (&a)[NT],
                                           int chunk, bool half) {
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    if (half) f[n].load_tail(a[n], chunk);
    else f[n].load(a[n], chunk);
  }
}

// acc[n][t] += A (16 rows of tile n: this lane's a[n]) . B (token tile t from
// the staged rows) over kbytes of K. `stage` holds this thread's source rows.
// All 256 threads of the workgroup call this together; the token rows are
// staged once for the NT tiles of every wave.
template <bool FP8, int MT, int NT>
__device__ __forceinline__ void hot_kloop(const uint8_t* const (&a)[NT], Stage& stage,
                                          int kbytes, uint8_t* __restrict__ lds,
                                          f32x4 (&acc)[NT][4]) {
  uint8_t* buf0 = lds;
  uint8_t* buf1 = lds + kHotTok * kLdsRow;
  const int nch = (kbytes + kHotChunk - 1) / kHotChunk;
  const bool tail = (kbytes % kHotChunk) != 0;  // fp8 only: last chunk is 128 bytes
  HotA<FP8> a0[NT], a1[NT];
  stage.load(0, kbytes);
  hot_load_a<FP8, NT>(a0, a, 0, tail && nch == 1);
  stage.store(buf0);
  __syncthreads();
  int c = 0;
  for (; c + 1 < nch; c += 2) {
    // chunk c from buf0 / a0 while chunk c+1 loads into buf1 / a1
    stage.load(c + 1, kbytes);
    hot_load_a<FP8, NT>(a1, a, c + 1, tail && c + 2 == nch);
    hot_compute<FP8, MT, NT>(a0, buf0, acc);
    stage.store(buf1);
    __syncthreads();
    if (c + 2 < nch) {
      stage.load(c + 2, kbytes);
      hot_load_a<FP8, NT>(a0, a, c + 2, tail && c + 3 == nch);
    }
    hot_compute<FP8, MT, NT>(a1, buf1, acc);
    if (c + 2 < nch) stage.store(buf0);
    __syncthreads();
  }
  if (c < nch) {
    hot_compute<FP8, MT, NT>(a0, buf0, acc);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- FC1 ---

struct Fc1Args {
  const void* x;       // bf16 [T,H] (bf16 path) or e4m3 codes [T,H] (fp8 path)
  const float* xs;     // fp8: per-token scale [T]
  const void* w1;      // [E, 2I, H]
  const float* w1s;    // fp8: [E, 2I]
  const int32_t* sorted_ids;
  const int32_t* block_expert;
  const int32_t* num_padded;
  int H, I, k, S, log2m, remap;
  void* h;             // bf16 [S, I] (bf16 path) or f32 [S, I] (fp8 path)
  int* queue;          // work counters, zero at launch (dense and hot launches)
  int E;               // experts: a block whose expert lies outside [0, E) is skipped
};

// Store SiLU(g)*u for 4 consecutive h columns of one slot (WT: device-scope
// stores, for a reader in the same kernel on another XCD).
template <bool FP8, bool WT = false>
__device__ __forceinline__ void store_h(const Fc1Args& p, int slot, int col, const f32x4& g,
                                        const f32x4& u) {
  if (FP8) {
    f32x4 hv;
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = silu_mul(g[i], u[i]);
    float* dst = (float*)p.h + (size_t)slot * p.I + col;
    if (WT) {
#pragma unroll
      for (int i = 0; i < 4; ++i) st_dev(dst + i, hv[i]);
    } else {
      *(f32x4*)dst = hv;
    }
  } else {
    uint32_t hb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hb[i] = f32_to_bf16_rne(silu_mul(g[i], u[i]));
    const u32x2 v{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
    uint32_t* dst = (uint32_t*)((uint16_t*)p.h + (size_t)slot * p.I + col);
    if (WT) {
      st_dev(dst, v.x);
      st_dev(dst + 1, v.y);
    } else {
      *(u32x2*)dst = v;
    }
  }
}

// Cold FC1 tile r (h columns [8r, 8r+8)): P = gate rows [8r, 8r+8), Q = the
// matching up rows [I+8r, I+8r+8). After the diagonal sums a lane holds g and
// u of the same (column, token).
template <bool FP8, int U, bool WT = false>
__device__ __forceinline__ void fc1_cold(const Fc1Args& p, int e, int r, int slot) {
  const int lane = threadIdx.x & 63;
  const size_t rowb = (size_t)p.H * (FP8 ? 1 : 2);
  const int off = half_split_off();
  const uint8_t* w = (const uint8_t*)p.w1 + (size_t)e * 2 * p.I * rowb;
  const uint8_t* ap = w + (size_t)(r * 8 + (lane & 7)) * rowb + off;
  const uint8_t* aq = w + (size_t)(p.I + r * 8 + (lane & 7)) * rowb + off;
  const bool ok = slot < p.S;
  const uint8_t* bp = (const uint8_t*)p.x + (size_t)(ok ? slot / p.k : 0) * rowb + off;
  const bool holder = (lane & 8) == 0 && lane < 32;  // lanes 0..7, 16..23
  const int col = r * 8 + 4 * (lane >> 4);
  // epilogue scales are fetched before the K loop so their latency is hidden
  float xs = 1.f;
  f32x4 sg = {1.f, 1.f, 1.f, 1.f}, su = sg;
  if (FP8 && holder && ok) {
    xs = p.xs[slot / p.k];
    sg = *(const f32x4*)(p.w1s + (size_t)e * 2 * p.I + col);
    su = *(const f32x4*)(p.w1s + (size_t)e * 2 * p.I + p.I + col);
  }
  f32x4 accp = {}, accq = {};
  cold_kloop<FP8, U>(ap, aq, bp, ok, (int)rowb, accp, accq, cold_rot(r));
  f32x4 g = diag_sum(accp), u = diag_sum(accq);
  if (holder && ok) {
    if (FP8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        g[i] *= sg[i] * xs;
        u[i] *= su[i] * xs;
      }
    }
    store_h<FP8, WT>(p, slot, col, g, u);
  }
}

// K slices of a cold tile shared by the 4 waves of a workgroup: wave w takes
// chunks [kslice(n, w), kslice(n, w + 1)) of the n chunks of a row (the last
// slice also takes a trailing half chunk).
__device__ __forceinline__ int kslice(int n, int w) { return (w * n) >> 2; }

// LDS of the sliced cold tiles: two buffers of [wave][P|Q][lane] partial
// accumulators, alternating from one tile to the next.
constexpr int kRedF4 = 4 * 2 * 64;

// The meeting of a sliced tile's 4 waves: every wave leaves its partial
// accumulators in buffer j & 1, and wave (j & 3) gets their sums in wave order
// back in accp/accq (true); the other waves get false. One barrier per tile:
// a buffer is written again two tiles later, after the next tile's barrier,
// which its reader has passed only after reading it.
__device__ __forceinline__ bool sliced_reduce(f32x4* __restrict__ red, int j, f32x4& accp,
                                              f32x4& accq) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  f32x4* buf = red + (j & 1) * kRedF4;
  buf[(2 * w) * 64 + lane] = accp;
  buf[(2 * w + 1) * 64 + lane] = accq;
  __syncthreads();
  if (w != (j & 3)) return false;
  accp = buf[lane];
  accq = buf[64 + lane];
#pragma unroll
  for (int v = 1; v < 4; ++v) {
    accp += buf[(2 * v) * 64 + lane];
    accq += buf[(2 * v + 1) * 64 + lane];
  }
  return true;
}

// Cold FC1 tile r (as fc1_cold) computed by all 4 waves of the workgroup,
// each over a quarter of K; the partial accumulators are summed in wave order
// by wave (j & 3), which finishes the tile. j counts the workgroup's sliced
// tiles (same on every wave); `slot` is this lane's token slot.
template <bool FP8, int U, bool WT = false>
__device__ __forceinline__ void fc1_cold_sliced(const Fc1Args& p, int e, int r, int slot,
                                                f32x4* __restrict__ red, int j) {
  constexpr int CH = Cold<FP8>::kChunk;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const size_t rowb = (size_t)p.H * (FP8 ? 1 : 2);
  const int nch = (int)(rowb / CH);
  const int c0 = kslice(nch, w), c1 = kslice(nch, w + 1);
  const int kb = (c1 - c0) * CH + (w == 3 ? (int)(rowb % CH) : 0);
  const int off = half_split_off() + c0 * CH;
  const uint8_t* wb = (const uint8_t*)p.w1 + (size_t)e * 2 * p.I * rowb;
  const uint8_t* ap = wb + (size_t)(r * 8 + (lane & 7)) * rowb + off;
  const uint8_t* aq = wb + (size_t)(p.I + r * 8 + (lane & 7)) * rowb + off;
  const bool ok = slot < p.S;
  const uint8_t* bp = (const uint8_t*)p.x + (size_t)(ok ? slot / p.k : 0) * rowb + off;
  const bool fin = w == (j & 3);
  const bool holder = (lane & 8) == 0 && lane < 32;
  const int col = r * 8 + 4 * (lane >> 4);
  float xs = 1.f;
  f32x4 sg = {1.f, 1.f, 1.f, 1.f}, su = sg;
  if (FP8 && fin && holder && ok) {
    xs = p.xs[slot / p.k];
    sg = *(const f32x4*)(p.w1s + (size_t)e * 2 * p.I + col);
    su = *(const f32x4*)(p.w1s + (size_t)e * 2 * p.I + p.I + col);
  }
  f32x4 accp = {}, accq = {};
  cold_kloop<FP8, U>(ap, aq, bp, ok, kb, accp, accq, cold_rot(r));
  if (!sliced_reduce(red, j, accp, accq)) return;
  f32x4 g = diag_sum(accp), u = diag_sum(accq);
  if (holder && ok) {
    if (FP8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        g[i] *= sg[i] * xs;
        u[i] *= su[i] * xs;
      }
    }
    store_h<FP8, WT>(p, slot, col, g, u);
  }
}

// Hot FC1 tiles r0 .. r0+NT-1 (NT per wave): rows 0..7 of a 16-row tile r are
// gate rows [8r, 8r+8), rows 8..15 the matching up rows; lanes l and l^32 hold
// g and u of the same (column, token) after the MFMAs.
template <bool FP8, int MT, int NT>
__device__ __forceinline__ void fc1_hot_pass(const Fc1Args& p, int e, int r0, int b, int M,
                                             int m, int t0, uint8_t* lds) {
  const int lane = threadIdx.x & 63, g = lane >> 4, rho = lane & 15;
  const size_t rowb = (size_t)p.H * (FP8 ? 1 : 2);
  const uint8_t* a[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int r = r0 + n;
    const int wrow = rho < 8 ? (r * 8 + rho) : (p.I + r * 8 + rho - 8);
    a[n] = (const uint8_t*)p.w1 + ((size_t)e * 2 * p.I + wrow) * rowb + 16 * g;
  }
  Stage st;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ti = t0 + (threadIdx.x >> 4) + 16 * i;
    const int slot = ti < m ? p.sorted_ids[(size_t)b * M + ti] : p.S;
    st.src[i] = slot < p.S ? (const uint8_t*)p.x + (size_t)(slot / p.k) * rowb : nullptr;
  }
  f32x4 acc[NT][4] = {};
  hot_kloop<FP8, MT, NT>(a, st, (int)rowb, lds, acc);
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int r = r0 + n;
    f32x4 sc = {1.f, 1.f, 1.f, 1.f};
    if (FP8) {
      const int srow = g < 2 ? (r * 8 + 4 * g) : (p.I + r * 8 + 4 * (g - 2));
      sc = *(const f32x4*)(p.w1s + (size_t)e * 2 * p.I + srow);
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int ti = t0 + 16 * t + rho;
      const int slot = ti < m ? p.sorted_ids[(size_t)b * M + ti] : p.S;
      const bool ok = slot < p.S;
      f32x4 v = acc[n][t];
      if (FP8) {
        const float xs = ok ? p.xs[slot / p.k] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] *= sc[i] * xs;
      }
      f32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = __shfl_xor(v[i], 32);
      if (lane < 32 && ok) store_h<FP8>(p, slot, r * 8 + 4 * g, v, o);
    }
  }
}

// Hot-pass policies of run_quads. kOcts: hot blocks run as octs (two tiles per
// wave); bf16 only, the fp8 passes would drop to one wave per SIMD. kOctsIfFull:
// only when the octs fill at least half of the grid; with fewer, an oct is
// long against the launch's whole work and the last ones set its time, so
// quads (more, shorter units) finish sooner. FC1 kernel traces at 64 tokens,
// top-8 of 128 experts: whole layer (384 octs, 512 workgroups) octs 214 against
// quads 238 us; its EP2 share 167.5 against 135.0 us, its TP2 share (192 octs)
// 167.0 against 127.7 us. FC2's units are shorter: octs won in all three.
template <bool FP8>
struct Fc1Hot {
  static constexpr bool kOcts = !FP8;
  static constexpr bool kOctsIfFull = true;
  static constexpr bool kOctsOneRound = false;
  static constexpr bool kResetQueue = false;  // FC1 calls zero the counters first
  template <int MT, int NT>
  static __device__ __forceinline__ void pass(const Fc1Args& p, int e, int r0, int b, int M,
                                              int m, int t0, uint8_t* lds) {
    fc1_hot_pass<FP8, MT, NT>(p, e, r0, b, M, m, t0, lds);
  }
};

// --------------------------------------------------------------- FC2 ---

struct Fc2Args {
  const void* h;       // bf16 [S, I] (bf16 path) or e4m3 codes [S, I] (fp8 path)
  const float* hs;     // fp8: per-slot scale [S]
  const void* w2;      // [E, H, I]
  const float* w2s;    // fp8: [E, H]
  const int32_t* sorted_ids;
  const int32_t* block_expert;
  const int32_t* num_padded;
  int H, I, S, log2m, remap;
  void* y;             // per-slot FC2 output [S, H]: bf16 (bf16 path) or f32
  int y_bf16;
  int* queue;          // work counters, zero at launch (dense and hot launches)
  int E;               // experts: a block whose expert lies outside [0, E) is skipped
};

// Store 4 consecutive FC2 outputs of one slot (WT as store_h).
template <bool WT = false>
__device__ __forceinline__ void store_y(const Fc2Args& p, int slot, int row, const f32x4& v) {
  if (p.y_bf16) {
    const u32x2 b{f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                  f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16)};
    uint32_t* dst = (uint32_t*)((uint16_t*)p.y + (size_t)slot * p.H + row);
    if (WT) {
      st_dev(dst, b.x);
      st_dev(dst + 1, b.y);
    } else {
      *(u32x2*)dst = b;
    }
  } else {
    float* dst = (float*)p.y + (size_t)slot * p.H + row;
    if (WT) {
#pragma unroll
      for (int i = 0; i < 4; ++i) st_dev(dst + i, v[i]);
    } else {
      *(f32x4*)dst = v;
    }
  }
}

// Cold FC2 tile r: P = output rows [16r, 16r+8), Q = [16r+8, 16r+16).
template <bool FP8, int U, bool WT = false>
__device__ __forceinline__ void fc2_cold(const Fc2Args& p, int e, int r, int slot) {
  const int lane = threadIdx.x & 63;
  const size_t rowb = (size_t)p.I * (FP8 ? 1 : 2);
  const int off = half_split_off();
  const uint8_t* w = (const uint8_t*)p.w2 + (size_t)e * p.H * rowb;
  const uint8_t* ap = w + (size_t)(r * 16 + (lane & 7)) * rowb + off;
  const uint8_t* aq = w + (size_t)(r * 16 + 8 + (lane & 7)) * rowb + off;
  const bool ok = slot < p.S;
  const uint8_t* bp = (const uint8_t*)p.h + (size_t)(ok ? slot : 0) * rowb + off;
  const bool holder = (lane & 8) == 0 && lane < 32;
  const int row = r * 16 + 4 * (lane >> 4);
  // epilogue scales are fetched before the K loop so their latency is hidden
  float hs = 1.f;
  f32x4 sp = {1.f, 1.f, 1.f, 1.f}, sq = sp;
  if (FP8 && holder && ok) {
    hs = p.hs[slot];
    sp = *(const f32x4*)(p.w2s + (size_t)e * p.H + row);
    sq = *(const f32x4*)(p.w2s + (size_t)e * p.H + row + 8);
  }
  f32x4 accp = {}, accq = {};
  cold_kloop<FP8, U>(ap, aq, bp, ok, (int)rowb, accp, accq, cold_rot(r));
  f32x4 vp = diag_sum(accp), vq = diag_sum(accq);
  if (holder && ok) {
    if (FP8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vp[i] *= sp[i] * hs;
        vq[i] *= sq[i] * hs;
      }
    }
    store_y<WT>(p, slot, row, vp);
    store_y<WT>(p, slot, row + 8, vq);
  }
}

// Hot FC2 tiles r0 .. r0+NT-1 (NT per wave): tile r is output rows
// [16r, 16r+16).
template <bool FP8, int MT, int NT>
__device__ __forceinline__ void fc2_hot_pass(const Fc2Args& p, int e, int r0, int b, int M,
                                             int m, int t0, uint8_t* lds) {
  const int lane = threadIdx.x & 63, g = lane >> 4, rho = lane & 15;
  const size_t rowb = (size_t)p.I * (FP8 ? 1 : 2);
  const uint8_t* a[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n)
    a[n] = (const uint8_t*)p.w2 + ((size_t)e * p.H + (r0 + n) * 16 + rho) * rowb + 16 * g;
  Stage st;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ti = t0 + (threadIdx.x >> 4) + 16 * i;
    const int slot = ti < m ? p.sorted_ids[(size_t)b * M + ti] : p.S;
    st.src[i] = slot < p.S ? (const uint8_t*)p.h + (size_t)slot * rowb : nullptr;
  }
  f32x4 acc[NT][4] = {};
  hot_kloop<FP8, MT, NT>(a, st, (int)rowb, lds, acc);
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int row = (r0 + n) * 16 + 4 * g;
    f32x4 sc = {1.f, 1.f, 1.f, 1.f};
    if (FP8) sc = *(const f32x4*)(p.w2s + (size_t)e * p.H + row);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int ti = t0 + 16 * t + rho;
      const int slot = ti < m ? p.sorted_ids[(size_t)b * M + ti] : p.S;
      if (slot < p.S) {
        f32x4 v = acc[n][t];
        if (FP8) {
          const float hs = p.hs[slot];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] *= sc[i] * hs;
        }
        store_y(p, slot, row, v);
      }
    }
  }
}

template <bool FP8>
struct Fc2Hot {
  static constexpr bool kOcts = !FP8;
  static constexpr bool kOctsIfFull = false;
  static constexpr bool kOctsOneRound = true;
  static constexpr bool kResetQueue = true;  // see finish_queue
  template <int MT, int NT>
  static __device__ __forceinline__ void pass(const Fc2Args& p, int e, int r0, int b, int M,
                                              int m, int t0, uint8_t* lds) {
    fc2_hot_pass<FP8, MT, NT>(p, e, r0, b, M, m, t0, lds);
  }
};

// ----------------------------------------- W8A16: e4m3 weights, bf16 x ---
// Weight-only FP8 ("vLLM SM architecture adaptation", sections 4.2 and 5.2:
// FP8 weights dequantised on the fly for 16-bit matrix cores). A tile's
// codes stream as in the cold path (half-split rows, whole 128-byte lines,
// non-temporal): a lane's 16 codes of one line are converted to two bf16x8
// MFMA fragments by v_cvt_pk_f32_fp8 (exact: every e4m3 value is a bf16
// value) and paired with the 16 bf16 activations of the same k. The
// per-output-channel scale multiplies the fp32 sum once.

// 16 e4m3 codes (byte order = k order) -> two bf16x8 fragments.
__device__ __forceinline__ void e4m3x16_to_bf16(const u32x4& q, bf16x8& f0, bf16x8& f1) {
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[i], false);  // codes 4i, 4i+1
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[i], true);   // codes 4i+2, 4i+3
    // exact values: the bf16 pattern is the float's upper half
    w[2 * i] = (__float_as_uint(lo[0]) >> 16) | (__float_as_uint(lo[1]) & 0xffff0000u);
    w[2 * i + 1] = (__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xffff0000u);
  }
  f0 = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
  f1 = __builtin_bit_cast(bf16x8, u32x4{w[4], w[5], w[6], w[7]});
}

template <int U>
struct W8Group {
  u32x4 p[U], q[U];     // 16 codes of tiles P and Q per chunk
  u32x4 b0[U], b1[U];   // the 16 matching bf16 activations
  __device__ __forceinline__ void issue(const uint8_t* __restrict__ ap,
                                        const uint8_t* __restrict__ aq,
                                        const uint8_t* __restrict__ bp, bool ok, int c) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      p[u] = __builtin_nontemporal_load((const u32x4*)(ap + (size_t)(c + u) * 128));
      q[u] = __builtin_nontemporal_load((const u32x4*)(aq + (size_t)(c + u) * 128));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      b0[u] = b1[u] = u32x4{0, 0, 0, 0};
      if (ok) {
        b0[u] = *(const u32x4*)(bp + (size_t)(c + u) * 256);
        b1[u] = *(const u32x4*)(bp + (size_t)(c + u) * 256 + 16);
      }
    }
  }
  __device__ __forceinline__ void compute(f32x4& accp, f32x4& accq) const {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bf16x8 x0 = __builtin_bit_cast(bf16x8, b0[u]), x1 = __builtin_bit_cast(bf16x8, b1[u]);
      bf16x8 f0, f1;
      e4m3x16_to_bf16(p[u], f0, f1);
      accp = mfma_bf16(f0, x0, accp);
      accp = mfma_bf16(f1, x1, accp);
      e4m3x16_to_bf16(q[u], f0, f1);
      accq = mfma_bf16(f0, x0, accq);
      accq = mfma_bf16(f1, x1, accq);
    }
  }
};

// accp/accq += codes of tiles P/Q (ap, aq: this lane's 16-byte piece of each
// 128-byte line) . bf16 token tile (bp: the matching 32 bytes of each
// 256-byte activation chunk) over kbytes = K bytes of codes per row, the groups
// in the rotated order of cold_kloop (16-token decode: FC1 135.5 -> 134.1 us,
// FC2 72.3 -> 70.6 us).
template <int U>
__device__ __forceinline__ void w8_kloop(const uint8_t* __restrict__ ap,
                                         const uint8_t* __restrict__ aq,
                                         const uint8_t* __restrict__ bp, bool ok, int kbytes,
                                         f32x4& accp, f32x4& accq, int rot) {
  const int nch = kbytes / 128;
  const int ngrp = nch / U;
  const int s0 = ngrp > 0 ? rot % ngrp : 0;  // rotated group order, as cold_kloop
  W8Group<U> g0, g1;
  if (ngrp > 0) g0.issue(ap, aq, bp, ok, rot_chunk<U>(0, s0, ngrp));
  int g = 0;
  for (; g + 1 < ngrp; g += 2) {
    g1.issue(ap, aq, bp, ok, rot_chunk<U>(g + 1, s0, ngrp));
    g0.compute(accp, accq);
    if (g + 2 < ngrp) g0.issue(ap, aq, bp, ok, rot_chunk<U>(g + 2, s0, ngrp));
    g1.compute(accp, accq);
  }
  if (g < ngrp) g0.compute(accp, accq);
  for (int c = ngrp * U; c < nch; ++c) {
    W8Group<1> one;
    one.issue(ap + (size_t)c * 128, aq + (size_t)c * 128, bp + (size_t)c * 256, ok, 0);
    one.compute(accp, accq);
  }
}

// Byte offsets of this lane's piece in the half-split layout: codes at
// half*64 + kgroup*16 of each 128-byte line, activations at twice that.
__device__ __forceinline__ int w8_code_off() { return half_split_off(); }
__device__ __forceinline__ int w8_act_off() { return 2 * half_split_off(); }

constexpr int kW8U = 2;  // code chunks per pipeline group (FC1; FC2's shorter rows take 1)

// Cold FC1 tile r of the W8A16 path (layout as fc1_cold).
__device__ __forceinline__ void fc1_cold_w8(const Fc1Args& p, int e, int r, int slot) {
  const int lane = threadIdx.x & 63;
  const size_t rowq = (size_t)p.H;      // code bytes per weight row
  const size_t rowx = (size_t)p.H * 2;  // bytes per activation row
  const uint8_t* w = (const uint8_t*)p.w1 + (size_t)e * 2 * p.I * rowq;
  const uint8_t* ap = w + (size_t)(r * 8 + (lane & 7)) * rowq + w8_code_off();
  const uint8_t* aq = w + (size_t)(p.I + r * 8 + (lane & 7)) * rowq + w8_code_off();
  const bool ok = slot < p.S;
  const uint8_t* bp = (const uint8_t*)p.x + (size_t)(ok ? slot / p.k : 0) * rowx + w8_act_off();
  const bool holder = (lane & 8) == 0 && lane < 32;
  const int col = r * 8 + 4 * (lane >> 4);
  f32x4 sg = {1.f, 1.f, 1.f, 1.f}, su = sg;
  if (holder) {
    sg = *(const f32x4*)(p.w1s + (size_t)e * 2 * p.I + col);
    su = *(const f32x4*)(p.w1s + (size_t)e * 2 * p.I + p.I + col);
  }
  f32x4 accp = {}, accq = {};
  w8_kloop<kW8U>(ap, aq, bp, ok, (int)rowq, accp, accq, cold_rot(r));
  f32x4 g = diag_sum(accp), u = diag_sum(accq);
  if (holder && ok) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      g[i] *= sg[i];
      u[i] *= su[i];
    }
    store_h<false>(p, slot, col, g, u);
  }
}

// Cold FC1 tile r of the W8A16 path computed by all 4 waves of the workgroup,
// one K quarter each (as fc1_cold_sliced).
__device__ __forceinline__ void fc1_cold_w8_sliced(const Fc1Args& p, int e, int r, int slot,
                                                   f32x4* __restrict__ red, int j) {
  const int lane = threadIdx.x & 63, w8 = threadIdx.x >> 6;
  const size_t rowq = (size_t)p.H;      // code bytes per weight row
  const size_t rowx = (size_t)p.H * 2;  // bytes per activation row
  const int nch = (int)(rowq / 128);
  const int c0 = kslice(nch, w8), c1 = kslice(nch, w8 + 1);
  const uint8_t* w = (const uint8_t*)p.w1 + (size_t)e * 2 * p.I * rowq;
  const uint8_t* ap = w + (size_t)(r * 8 + (lane & 7)) * rowq + w8_code_off() + (size_t)c0 * 128;
  const uint8_t* aq =
      w + (size_t)(p.I + r * 8 + (lane & 7)) * rowq + w8_code_off() + (size_t)c0 * 128;
  const bool ok = slot < p.S;
  const uint8_t* bp = (const uint8_t*)p.x + (size_t)(ok ? slot / p.k : 0) * rowx + w8_act_off() +
                      (size_t)c0 * 256;
  const bool fin = w8 == (j & 3);
  const bool holder = (lane & 8) == 0 && lane < 32;
  const int col = r * 8 + 4 * (lane >> 4);
  f32x4 sg = {1.f, 1.f, 1.f, 1.f}, su = sg;
  if (fin && holder) {
    sg = *(const f32x4*)(p.w1s + (size_t)e * 2 * p.I + col);
    su = *(const f32x4*)(p.w1s + (size_t)e * 2 * p.I + p.I + col);
  }
  f32x4 accp = {}, accq = {};
  w8_kloop<kW8U>(ap, aq, bp, ok, (c1 - c0) * 128, accp, accq, cold_rot(r));
  if (!sliced_reduce(red, j, accp, accq)) return;
  f32x4 g = diag_sum(accp), u = diag_sum(accq);
  if (holder && ok) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      g[i] *= sg[i];
      u[i] *= su[i];
    }
    store_h<false>(p, slot, col, g, u);
  }
}

// Cold FC2 tile r of the W8A16 path (layout as fc2_cold).
__device__ __forceinline__ void fc2_cold_w8(const Fc2Args& p, int e, int r, int slot) {
  const int lane = threadIdx.x & 63;
  const size_t rowq = (size_t)p.I;
  const size_t rowh = (size_t)p.I * 2;
  const uint8_t* w = (const uint8_t*)p.w2 + (size_t)e * p.H * rowq;
  const uint8_t* ap = w + (size_t)(r * 16 + (lane & 7)) * rowq + w8_code_off();
  const uint8_t* aq = w + (size_t)(r * 16 + 8 + (lane & 7)) * rowq + w8_code_off();
  const bool ok = slot < p.S;
  const uint8_t* bp = (const uint8_t*)p.h + (size_t)(ok ? slot : 0) * rowh + w8_act_off();
  const bool holder = (lane & 8) == 0 && lane < 32;
  const int row = r * 16 + 4 * (lane >> 4);
  f32x4 sp = {1.f, 1.f, 1.f, 1.f}, sq = sp;
  if (holder) {
    sp = *(const f32x4*)(p.w2s + (size_t)e * p.H + row);
    sq = *(const f32x4*)(p.w2s + (size_t)e * p.H + row + 8);
  }
  f32x4 accp = {}, accq = {};
  w8_kloop<1>(ap, aq, bp, ok, (int)rowq, accp, accq, cold_rot(r));  // short rows: occupancy over depth
  f32x4 vp = diag_sum(accp), vq = diag_sum(accq);
  if (holder && ok) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      vp[i] *= sp[i];
      vq[i] *= sq[i];
    }
    store_y(p, slot, row, vp);
    store_y(p, slot, row + 8, vq);
  }
}

// ------------------------------- block-scaled FP8: 128x128 weight blocks ---
// Block-wise FP8 ("vLLM SM architecture adaptation": section 4.1's block FP8
// MoE backends, section 4.2's block-wise DeepGEMM MoE, section 9's figure:
// dequantisation inside the GEMM loop). Weights carry one fp32 scale per
// 128 x 128 block, activations one per 128 consecutive elements of a row
// (x per token, h per slot), so every 128-byte line of a weight row and of
// an activation row is exactly one K-block. A line's partial dot product is
// formed apart from the others and scaled by (weight block scale) x
// (activation group scale) into the fp32 sum. The half-split tiles of the
// cold path carry both halves of the SAME line in D's two diagonal blocks,
// so the 16x16x32 fp8 MFMA (8 codes per lane) keeps each MFMA inside one
// line: a lane's 16 codes of a line are two MFMAs into a fresh partial,
// which is scaled per lane (its column is its token) and added.

template <int U>
struct BlkGroup {
  u32x4 p[U], q[U], b[U];  // 16 codes of tiles P, Q and of the token per line
  float sa[U];             // activation group scale of this lane's token per line
  float sp[U], sq[U];      // weight block scales of tiles P and Q per line
  // Every lane loads its token's codes and scales, also a lane without a
  // token: its callers point it at row 0, which exists, and its products stay
  // in its own output column, which is never stored (a load under a condition
  // costs register copies that wait for the load).
  __device__ __forceinline__ void issue(const uint8_t* __restrict__ ap,
                                        const uint8_t* __restrict__ aq,
                                        const uint8_t* __restrict__ bp,
                                        const float* __restrict__ as,
                                        const float* __restrict__ wsp,
                                        const float* __restrict__ wsq, int c) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      p[u] = __builtin_nontemporal_load((const u32x4*)(ap + (size_t)(c + u) * 128));
      q[u] = __builtin_nontemporal_load((const u32x4*)(aq + (size_t)(c + u) * 128));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      b[u] = *(const u32x4*)(bp + (size_t)(c + u) * 128);
      sa[u] = as[c + u];
      sp[u] = wsp[c + u];
      sq[u] = wsq[c + u];
    }
  }
  __device__ __forceinline__ void compute(f32x4& accp, f32x4& accq) const {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const u32x2 b0{b[u].x, b[u].y}, b1{b[u].z, b[u].w};
      f32x4 tp = mfma_fp8_k32(u32x2{p[u].x, p[u].y}, b0, f32x4{0.f, 0.f, 0.f, 0.f});
      tp = mfma_fp8_k32(u32x2{p[u].z, p[u].w}, b1, tp);
      f32x4 tq = mfma_fp8_k32(u32x2{q[u].x, q[u].y}, b0, f32x4{0.f, 0.f, 0.f, 0.f});
      tq = mfma_fp8_k32(u32x2{q[u].z, q[u].w}, b1, tq);
      const float fp = sp[u] * sa[u], fq = sq[u] * sa[u];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        accp[i] = fmaf(tp[i], fp, accp[i]);
        accq[i] = fmaf(tq[i], fq, accq[i]);
      }
    }
  }
};

// accp/accq = sum over the kbytes/128 lines of a row of the scaled line
// partials of tiles P and Q. as: the lane's token's group scales; wsp/wsq:
// the block-scale rows of P's and Q's row block. rot: group order as in
// cold_kloop; FC2 rotates (16-token decode: 70.8 -> 69.0 us), FC1 does not
// (133.5 -> 139.5 us rotated, in this loop's in-place form).
template <int U>
__device__ __forceinline__ void blk_kloop(const uint8_t* __restrict__ ap,
                                          const uint8_t* __restrict__ aq,
                                          const uint8_t* __restrict__ bp,
                                          const float* __restrict__ as,
                                          const float* __restrict__ wsp,
                                          const float* __restrict__ wsq, int kbytes,
                                          f32x4& accp, f32x4& accq, int rot) {
  const int nch = kbytes / 128;
  const int ngrp = nch / U;
  const int s0 = ngrp > 0 ? rot % ngrp : 0;  // rotated group order, as cold_kloop
  BlkGroup<U> g0, g1;
  if (ngrp > 0) g0.issue(ap, aq, bp, as, wsp, wsq, rot_chunk<U>(0, s0, ngrp));
  int g = 0;
  // no condition in the steady-state loop and each set refilled in place
  // after its MFMAs (the barriers keep the refill behind them), so one group
  // stays in flight while the other is consumed. Measured on the 16-token
  // decode shapes: FC1 137.4 -> 132.2 us; the same form in cold_kloop and
  // w8_kloop measured 2-5 % slower than their looser schedule and is not used
  // there.
  for (; g + 2 < ngrp; g += 2) {
    g1.issue(ap, aq, bp, as, wsp, wsq, rot_chunk<U>(g + 1, s0, ngrp));
    g0.compute(accp, accq);
    __builtin_amdgcn_sched_barrier(0);
    g0.issue(ap, aq, bp, as, wsp, wsq, rot_chunk<U>(g + 2, s0, ngrp));
    g1.compute(accp, accq);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (g + 1 < ngrp) {
    g1.issue(ap, aq, bp, as, wsp, wsq, rot_chunk<U>(g + 1, s0, ngrp));
    g0.compute(accp, accq);
    g1.compute(accp, accq);
  } else if (g < ngrp) {
    g0.compute(accp, accq);
  }
  for (int c = ngrp * U; c < nch; ++c) {
    BlkGroup<1> one;
    one.issue(ap, aq, bp, as, wsp, wsq, c);
    one.compute(accp, accq);
  }
}

constexpr int kBlk = 128;   // block edge (weights) and group length (activations)
constexpr int kBlkU = 2;    // lines per pipeline group (FC1; FC2's shorter rows take 1)

// Cold FC1 tile r of the block-scaled path (layout as fc1_cold). x: codes
// [T, H]; xs: group scales [T, H/128]; w1s: block scales [E, 2I/128, H/128].
__device__ __forceinline__ void fc1_cold_blk(const Fc1Args& p, int e, int r, int slot) {
  const int lane = threadIdx.x & 63;
  const int kb = p.H / kBlk, nb = 2 * p.I / kBlk;
  const int off = half_split_off();
  const uint8_t* w = (const uint8_t*)p.w1 + (size_t)e * 2 * p.I * p.H;
  const uint8_t* ap = w + (size_t)(r * 8 + (lane & 7)) * p.H + off;
  const uint8_t* aq = w + (size_t)(p.I + r * 8 + (lane & 7)) * p.H + off;
  const bool ok = slot < p.S;
  const int t = ok ? slot / p.k : 0;
  const uint8_t* bp = (const uint8_t*)p.x + (size_t)t * p.H + off;
  const float* as = p.xs + (size_t)t * kb;
  const float* wsp = p.w1s + ((size_t)e * nb + (r * 8) / kBlk) * kb;
  const float* wsq = p.w1s + ((size_t)e * nb + (p.I + r * 8) / kBlk) * kb;
  f32x4 accp = {}, accq = {};
  blk_kloop<kBlkU>(ap, aq, bp, as, wsp, wsq, p.H, accp, accq, 0);  // unrotated: see blk_kloop
  const f32x4 g = diag_sum(accp), u = diag_sum(accq);
  if ((lane & 8) == 0 && lane < 32 && ok) store_h<true>(p, slot, r * 8 + 4 * (lane >> 4), g, u);
}

// Cold FC1 tile r of the block-scaled path computed by all 4 waves of the
// workgroup, one K quarter (a run of whole 128-column blocks) each.
__device__ __forceinline__ void fc1_cold_blk_sliced(const Fc1Args& p, int e, int r, int slot,
                                                    f32x4* __restrict__ red, int j) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int kb = p.H / kBlk, nb = 2 * p.I / kBlk;
  const int c0 = kslice(kb, w), c1 = kslice(kb, w + 1);
  const int off = half_split_off() + c0 * 128;
  const uint8_t* wt = (const uint8_t*)p.w1 + (size_t)e * 2 * p.I * p.H;
  const uint8_t* ap = wt + (size_t)(r * 8 + (lane & 7)) * p.H + off;
  const uint8_t* aq = wt + (size_t)(p.I + r * 8 + (lane & 7)) * p.H + off;
  const bool ok = slot < p.S;
  const int t = ok ? slot / p.k : 0;
  const uint8_t* bp = (const uint8_t*)p.x + (size_t)t * p.H + off;
  const float* as = p.xs + (size_t)t * kb + c0;
  const float* wsp = p.w1s + ((size_t)e * nb + (r * 8) / kBlk) * kb + c0;
  const float* wsq = p.w1s + ((size_t)e * nb + (p.I + r * 8) / kBlk) * kb + c0;
  f32x4 accp = {}, accq = {};
  blk_kloop<kBlkU>(ap, aq, bp, as, wsp, wsq, (c1 - c0) * 128, accp, accq, 0);
  if (!sliced_reduce(red, j, accp, accq)) return;
  const f32x4 g = diag_sum(accp), u = diag_sum(accq);
  if ((lane & 8) == 0 && lane < 32 && ok) store_h<true>(p, slot, r * 8 + 4 * (lane >> 4), g, u);
}

// Cold FC2 tile r of the block-scaled path (layout as fc2_cold). h: codes
// [S, I]; hs: group scales [S, I/128]; w2s: block scales [E, H/128, I/128].
// Both 8-row halves of the tile lie in one 128-row block.
__device__ __forceinline__ void fc2_cold_blk(const Fc2Args& p, int e, int r, int slot) {
  const int lane = threadIdx.x & 63;
  const int kb = p.I / kBlk, nb = p.H / kBlk;
  const int off = half_split_off();
  const uint8_t* w = (const uint8_t*)p.w2 + (size_t)e * p.H * p.I;
  const uint8_t* ap = w + (size_t)(r * 16 + (lane & 7)) * p.I + off;
  const uint8_t* aq = w + (size_t)(r * 16 + 8 + (lane & 7)) * p.I + off;
  const bool ok = slot < p.S;
  const int s = ok ? slot : 0;
  const uint8_t* bp = (const uint8_t*)p.h + (size_t)s * p.I + off;
  const float* as = p.hs + (size_t)s * kb;
  const float* ws = p.w2s + ((size_t)e * nb + (r * 16) / kBlk) * kb;
  f32x4 accp = {}, accq = {};
  blk_kloop<1>(ap, aq, bp, as, ws, ws, p.I, accp, accq, cold_rot(r));  // short rows: occupancy over depth
  const f32x4 vp = diag_sum(accp), vq = diag_sum(accq);
  if ((lane & 8) == 0 && lane < 32 && ok) {
    const int row = r * 16 + 4 * (lane >> 4);
    store_y(p, slot, row, vp);
    store_y(p, slot, row + 8, vq);
  }
}

// ------------------------------------------------- persistent kernels ---

// Work list: (block, quad of 4 consecutive tiles), one quad per workgroup
// step, wave w taking tile 4q + w. With HOT, a block of up to 8 tokens runs
// one cold pass and a bigger block the LDS-staged passes. Without HOT every
// block runs cold passes of 8 tokens: the host picks that launch when blocks
// of more than 8 tokens are unlikely (T <= 16 tokens), where it needs far
// fewer registers, so more waves stream weights at once; it stays correct for
// any block, reading the weights once per 8 tokens.
template <bool FP8, bool HOT, typename Args, void (*Cold_)(const Args&, int, int, int),
          typename HotOps>
struct QuadRunner {
  const Args& p;
  int M, w, ti;
  int cur_b = -1, e = 0, m = 0;
  int cslot = 0;  // this lane's slot in the block's first cold pass (S: none)
  uint8_t* lds;
  __device__ QuadRunner(const Args& a, uint8_t* l)
      : p(a), M(1 << a.log2m), w(threadIdx.x >> 6), ti(threadIdx.x & 7), lds(l) {}
  // NT = 1: quad q of block b, wave w taking tile 4q + w; NT = 2: oct q,
  // wave w taking tiles 8q + 2w and 8q + 2w + 1 (a hot block's token rows are
  // then staged once for twice the weight rows)
  __device__ __forceinline__ void enter(int b) {
    if (b != cur_b) {
      cur_b = b;
      e = p.block_expert[b];
      m = (unsigned)e < (unsigned)p.E ? block_valid(p.sorted_ids, b, M, p.S) : 0;
      cslot = ti < m ? p.sorted_ids[(size_t)b * M + ti] : p.S;
    }
  }
  // Tile r of a cold block (at most kColdMax tokens) as one unit of the whole
  // workgroup, K-sliced over its 4 waves by Sliced_; j counts the
  // workgroup's sliced tiles.
  template <void (*Sliced_)(const Args&, int, int, int, f32x4*, int)>
  __device__ __forceinline__ void run_sliced(int b, int r, f32x4* __restrict__ red, int& j) {
    enter(b);
    if (m > 0) Sliced_(p, e, r, cslot, red, j++);
  }
  template <int NT>
  __device__ __forceinline__ void run(int b, int q) {
    const int r = NT == 1 ? q * 4 + w : q * 8 + 2 * w;
    enter(b);
    if (HOT && m > kColdMax) {
      for (int t0 = 0; t0 < m; t0 += kHotTok) {
        const int mt = min(4, (m - t0 + 15) >> 4);
        if (mt == 1) HotOps::template pass<1, NT>(p, e, r, b, M, m, t0, lds);
        else if (mt == 2) HotOps::template pass<2, NT>(p, e, r, b, M, m, t0, lds);
        else if (mt == 3) HotOps::template pass<3, NT>(p, e, r, b, M, m, t0, lds);
        else HotOps::template pass<4, NT>(p, e, r, b, M, m, t0, lds);
      }
    } else {
#pragma unroll
      for (int n = 0; n < NT; ++n)
        for (int t0 = 0; t0 < m; t0 += kColdMax) {
          const int slot =
              t0 == 0 ? cslot : (t0 + ti < m ? p.sorted_ids[(size_t)b * M + t0 + ti] : p.S);
          Cold_(p, e, r + n, slot);
        }
    }
  }
};

// Work list: (block, quad of 4 consecutive tiles), wave w of a workgroup
// taking tile 4q + w. With HOT, a block of up to 8 tokens runs one cold pass
// and a bigger block the LDS-staged passes. Without HOT every block runs cold
// passes of 8 tokens: the host picks that launch when blocks of more than 8
// tokens are unlikely (T <= 16 tokens), where it needs far fewer registers,
// so more waves stream weights at once; it stays correct for any block,
// reading the weights once per 8 tokens. With DYN, units are handed out by a
// QuadQueue over the hot-first block order (hot_first_order): the octs of the
// hot blocks, then the quads of the others (or, given Sliced_, their single
// tiles, each K-sliced over the workgroup's 4 waves: a quarter of a quad's
// cost, so the units that fill the tail behind the long hot ones are fine
// grained); else each workgroup takes one contiguous equal share of the quad
// list.
template <bool FP8, bool HOT, bool DYN, typename Args, void (*Cold_)(const Args&, int, int, int),
          typename HotOps, void (*Sliced_)(const Args&, int, int, int, f32x4*, int) = nullptr>
__device__ __forceinline__ void run_quads(const Args& p, int n_rt, uint8_t* lds) {
  const int M = 1 << p.log2m;
  const int nb = num_blocks(p.num_padded, p.S, p.E, p.log2m);
  const int qpb = n_rt >> 2;  // quads per block (n_rt is a multiple of 4)
  QuadRunner<FP8, HOT, Args, Cold_, HotOps> qr(p, lds);
  if constexpr (!DYN) {
    const Share sh = wg_share((long)nb * qpb, p.remap);
    for (long qd = sh.q0; qd < sh.q1; ++qd) qr.template run<1>((int)(qd / qpb), (int)(qd % qpb));
  } else {
    auto* slots = (volatile __attribute__((address_space(3))) int*)(lds + 2 * kHotTok * kLdsRow);
    int* ord = (int*)(lds + kHotLds);
    // (the staging buffers, not in use yet, serve as its scratch)
    const int nh = hot_first_order(p.sorted_ids, p.block_expert, nb, M, p.S, p.E, ord,
                                   ord + kOrdMax, (int*)lds);
    // hot blocks as octs (two tiles per wave) where the policy takes them
    bool octs = HotOps::kOcts && nh >= 0 && (n_rt & 7) == 0;
    if (HotOps::kOctsIfFull && octs) octs = 2L * nh * (n_rt >> 3) >= (long)gridDim.x;
    const int hnt = octs ? 2 : 1;
    const bool order = nh >= 0 && (n_rt & (4 * hnt - 1)) == 0;
    const int hpb = n_rt / (4 * hnt);           // units per hot block
    const int hot_units = order ? nh * hpb : 0;  // they come first
    // kOctsOneRound: hot octs beyond one per workgroup run as two quads each
    // (the end of the hot list: the least hot blocks), so the hot work that
    // starts in a second round is half as coarse
    int oct_units = hot_units, hq_units = 0;
    if constexpr (HotOps::kOctsOneRound) {
      if (octs && order && hot_units > (int)gridDim.x) {
        oct_units = gridDim.x;
        hq_units = 2 * (hot_units - oct_units);
      }
    }
    const int hot_all = oct_units + hq_units;
    // cold units per block: single sliced tiles where the order proves the
    // blocks cold, else quads (run<1> then also serves hot blocks)
    const bool sliced = Sliced_ != nullptr && order;
    const int cpb = sliced ? n_rt : qpb;
    // the staging buffers of the hot passes double as the sliced tiles'
    // partial sums: units are separated by the barrier in next()
    f32x4* red = (f32x4*)lds;
    static_assert(2 * kRedF4 * 16 <= 2 * kHotTok * kLdsRow, "sliced partials fit the staging");
    int j = 0;
    QuadQueue qq(p.queue, hot_all + (nb - (order ? nh : 0)) * cpb, p.remap);
    for (int u = qq.first(p.remap); u >= 0; u = qq.next(slots)) {
      const bool hot = u < hot_all;
      if (hot && u >= oct_units) {  // a hot quad: quad qi of the hot list
        const int qi = 2 * oct_units + (u - oct_units);
        qr.template run<1>(ord[qi / (2 * hpb)], qi % (2 * hpb));
        continue;
      }
      const int v = hot ? u : u - hot_all, per = hot ? hpb : cpb;
      const int b = order ? ord[(hot ? 0 : nh) + v / per] : v / per;
      if (order && !hot) qq.early();  // a cold unit: short
      if constexpr (HotOps::kOcts) {
        if (octs && hot) {
          qr.template run<2>(b, v % per);
          continue;
        }
      }
      if constexpr (Sliced_ != nullptr) {
        if (sliced && !hot) qr.template run_sliced<Sliced_>(b, v % per, red, j);
        else qr.template run<1>(b, v % per);
      } else {
        qr.template run<1>(b, v % per);
      }
    }
    if constexpr (HotOps::kResetQueue) finish_queue(p.queue, 1);
  }
}

template <bool FP8, bool HOT>
__global__ __launch_bounds__(256) void fc1_kernel(Fc1Args p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[HOT ? kHotLdsTotal : 16];
  run_quads<FP8, HOT, HOT, Fc1Args, fc1_cold<FP8, cold_u<FP8, HOT>()>, Fc1Hot<FP8>,
            fc1_cold_sliced<FP8, cold_u<FP8, false>()>>(p, p.I >> 3, lds);
}

// Whether an FC1 launch of T tokens (at most 16: the cold-only launches) runs
// K-sliced tiles rather than one tile per wave.
__host__ __device__ constexpr bool sliced_fc1(bool bf16, int T) {
  return bf16 || T <= kColdMax;
}

// The (block, tile) work list of a K-sliced FC1 launch: a workgroup takes a
// contiguous share and its 4 waves compute each tile together; blocks of more
// than 8 tokens run one such tile per 8 tokens.
template <void (*Tile)(const Fc1Args&, int, int, int, f32x4*, int)>
__device__ __forceinline__ void run_sliced_fc1(const Fc1Args& p, f32x4* __restrict__ red) {
  const int M = 1 << p.log2m, nb = num_blocks(p.num_padded, p.S, p.E, p.log2m), tpb = p.I >> 3;
  const int ti = threadIdx.x & 7;
  const Share sh = wg_share((long)nb * tpb, p.remap);
  int j = 0, cur_b = -1, e = 0, m = 0;
  for (long u = sh.q0; u < sh.q1; ++u) {
    const int b = (int)(u / tpb), r = (int)(u % tpb);
    if (b != cur_b) {
      cur_b = b;
      e = p.block_expert[b];
      m = (unsigned)e < (unsigned)p.E ? block_valid(p.sorted_ids, b, M, p.S) : 0;
    }
    for (int t0 = 0; t0 < m; t0 += kColdMax, ++j) {
      const int slot = t0 + ti < m ? p.sorted_ids[(size_t)b * M + t0 + ti] : p.S;
      Tile(p, e, r, slot, red, j);
    }
  }
}

// Cold-only FC1 launch with K-sliced tiles: the work list is (block, tile) and
// the 4 waves of a workgroup compute each tile together, one K quarter each,
// so four times as many waves stream weights as with one tile per wave, each
// along a dependent load chain a quarter as long. Blocks of more than 8 tokens
// run one such tile per 8 tokens. Taken for bf16 up to 16 tokens and for the
// other formats up to 8 (sliced_fc1()): measured with kernel traces at E = 64,
// H = 4096, I = 1536, k = 8 against one tile per wave, bf16 FC1 111.8 -> 91.3 us
// at 4 tokens, 243.1 -> 237.1 us at 16; fp8 58.1 -> 49.0 us at 4 tokens but
// 125.0 -> 126.8 us at 16; W8A16 and block FP8 5-8 % slower at 16 tokens.
template <bool FP8>
__global__ __launch_bounds__(256) void fc1_sliced_kernel(Fc1Args p) {
  __shared__ f32x4 red[2 * kRedF4];
  run_sliced_fc1<fc1_cold_sliced<FP8, cold_u<FP8, false>()>>(p, red);
}

template <bool FP8, bool HOT>
__global__ __launch_bounds__(256) void fc2_kernel(Fc2Args p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[HOT ? kHotLdsTotal : 16];
  // (no K-sliced cold tiles here: FC2's rows are short, and measured at 64
  // tokens, top-8 of 128 experts, 123.7 -> 162 us in bf16, 77.8 -> 99.7 in fp8)
  run_quads<FP8, HOT, HOT, Fc2Args, fc2_cold<FP8, cold_u<FP8, HOT>()>, Fc2Hot<FP8>>(p, p.H >> 4,
                                                                                   lds);
}

// W8A16 runs every block by cold passes of 8 tokens (the weights stream once
// per 8 tokens of a block): a decode path.
__global__ __launch_bounds__(256) void fc1_w8a16_kernel(Fc1Args p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[16];
  run_quads<false, false, false, Fc1Args, fc1_cold_w8, Fc1Hot<false>>(p, p.I >> 3,
                                                                                     lds);
}

// W8A16 FC1 with K-sliced tiles, for at most 8 tokens (see fc1_sliced_kernel).
__global__ __launch_bounds__(256) void fc1_w8a16_sliced_kernel(Fc1Args p) {
  __shared__ f32x4 red[2 * kRedF4];
  run_sliced_fc1<fc1_cold_w8_sliced>(p, red);
}

__global__ __launch_bounds__(256) void fc2_w8a16_kernel(Fc2Args p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[16];
  run_quads<false, false, false, Fc2Args, fc2_cold_w8, Fc2Hot<false>>(p, p.H >> 4,
                                                                                     lds);
}

// Block-scaled FP8 runs every block by cold passes of 8 tokens, like W8A16.
__global__ __launch_bounds__(256) void fc1_blk_kernel(Fc1Args p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[16];
  run_quads<true, false, false, Fc1Args, fc1_cold_blk, Fc1Hot<true>>(p, p.I >> 3,
                                                                                  lds);
}

// Block-scaled FC1 with K-sliced tiles, for at most 8 tokens.
__global__ __launch_bounds__(256, 3) void fc1_blk_sliced_kernel(Fc1Args p) {
  __shared__ f32x4 red[2 * kRedF4];
  run_sliced_fc1<fc1_cold_blk_sliced>(p, red);
}

__global__ __launch_bounds__(256) void fc2_blk_kernel(Fc2Args p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[16];
  run_quads<true, false, false, Fc2Args, fc2_cold_blk, Fc2Hot<true>>(p, p.H >> 4,
                                                                                  lds);
}

// ------------------------------------------- dense tiles (big blocks) ---
// For blocks of up to 256 tokens (prefill) the projection is a real grouped
// GEMM: a 512-thread workgroup multiplies a 256-row weight tile by the block's
// 256-token tile, both staged through LDS 64 k-elements (128 bytes) at a time.
// Weight tiles stream from HBM and get three LDS stages (two chunks in
// flight while one is multiplied); token tiles come from the caches and get
// two; together 160 KB, one workgroup per CU. Its 8 waves each own 64 rows
// x 128 tokens (4 x 8 MFMA 16x16x32 tiles, 128 accumulators), so each staged
// byte feeds 64..128 MFMAs per k-step. Units (block, 256-row tile) are ordered
// expert by expert, row tile by row tile with the expert's blocks innermost,
// and dealt round-robin to a virtual workgroup index laid out XCD by XCD, so
// blocks of one expert that share a weight tile run together on one XCD and
// the tile crosses HBM once.

constexpr int kDRows = 256;   // weight rows per unit
constexpr int kDTok = 256;    // tokens per unit
constexpr int kDThreads = 512;
constexpr int kDChunk = 128;  // bytes of K per stage (64 bf16, two MFMA k-steps) = one LDS row
constexpr int kDTile = kDRows * kDChunk;  // bytes of one staged operand tile (32 KB)
constexpr int kDAStages = 3;              // weight-tile ring
constexpr int kDBStages = 2;              // token-tile ring
constexpr int kDLds = (kDAStages + kDBStages) * kDTile;
constexpr int kDALoads = 4;  // direct-to-LDS loads per wave for one weight tile
// A block whose expert's tokens spill a little past one block (a "tail" of
// at most kDTail tokens in the expert's next and last block) takes those
// tokens into its own unit, so the weight tile streams once for both: the
// tail rows sit past the 256 token rows of the token stage, in two more
// 16-token groups. To fit, the merging ring keeps two weight stages instead
// of three (two 32 KB weight stages and two 36 KB token stages, 136 KB).
constexpr int kDTail = 32;
template <bool MG>
struct DRing {
  static constexpr int kAStages = MG ? 2 : kDAStages;
  static constexpr int kBTile = (kDTok + (MG ? kDTail : 0)) * kDChunk;
  static constexpr int kLds = kAStages * kDTile + kDBStages * kBTile;
};
static_assert(DRing<false>::kLds == kDLds && DRing<true>::kLds <= 160 * 1024, "LDS ring");
// LDS rows are 128 bytes (8 columns of 16 bytes) with no padding; column c of
// row r sits at column c ^ (r & 7), conflict-free for the MFMA fragment
// reads (16 consecutive rows, one column) on gfx950.

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Staging by direct-to-LDS loads: one load instruction of a wave writes 1 KB
// of LDS in lane order (lane l -> bytes 16 l..16 l+15), i.e. 8 whole LDS rows,
// and reads 8 whole 128-byte lines. Wave w stages rows [32 w, 32 w + 32) of
// each operand with 4 instructions; lane l fills physical column l & 7 of row
// l >> 3 of its 8-row group, so it loads the logical column (l & 7) ^ (l >> 3).
// Token groups lying wholly past the block's tokens are not loaded (their
// MFMA columns are never stored).
struct DenseStage {
  const uint8_t* arow[4];  // this lane's source weight rows (+ logical column)
  const uint8_t* brow[4];  // this lane's source token rows (+ logical column)
  int bgroups;             // this wave's token groups holding real tokens (0..4)
  // merged tail (waves 0..3 stage its 8-row groups, to token rows 256 + 8 w)
  const uint8_t* trow;
  bool tload;              // this wave's tail group holds tokens
  __device__ __forceinline__ void issue_a(uint8_t* __restrict__ tile, int c) const {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < kDALoads; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(arow[i] + (size_t)c * kDChunk),
                                       (lds_ptr_t)(tile + (32 * w + 8 * i) * kDChunk), 16, 0, 0);
  }
  template <bool MG = false>
  __device__ __forceinline__ void issue_b(uint8_t* __restrict__ tile, int c) const {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < bgroups)
        __builtin_amdgcn_global_load_lds((const void*)(brow[i] + (size_t)c * kDChunk),
                                         (lds_ptr_t)(tile + (32 * w + 8 * i) * kDChunk), 16, 0, 0);
    if (MG && tload)
      __builtin_amdgcn_global_load_lds((const void*)(trow + (size_t)c * kDChunk),
                                       (lds_ptr_t)(tile + (kDTok + 8 * w) * kDChunk), 16, 0, 0);
  }
};

// Row of this lane in staging instruction i, and its logical 16-byte column.
__device__ __forceinline__ int dstage_row(int i) {
  return 32 * (threadIdx.x >> 6) + 8 * i + ((threadIdx.x & 63) >> 3);
}
__device__ __forceinline__ int dstage_col() {
  const int l = threadIdx.x & 63;
  return ((l & 7) ^ (l >> 3)) * 16;
}
// Number of 8-row token groups of wave w holding at least one of the m tokens.
__device__ __forceinline__ int dstage_bgroups(int m) {
  const int first = 32 * (threadIdx.x >> 6);
  return max(0, min(4, (m - first + 7) >> 3));
}

// acc[i][j] += A rows (64*wr + 16i ..) . B tokens (128*wc + 16j ..), j < NJ,
// over one chunk. bf16: two MFMA k-steps; per k-step the fragments are read,
// then the MFMAs run on them. fp8 (e4m3 codes, 128 per chunk row): one
// 16x16x128 MFMA per tile pair; a lane's 32 bytes are the 16-byte columns
// (lane >> 4) and 4 + (lane >> 4) of its row (the two the bf16 path reads for
// its two k-steps), the same in A and B, so every product pairs equal k.
// Waves whose tokens end early use NJ < 8.
// TAIL (bf16): the wave also multiplies its 16-token group of a merged tail
// (token rows 256 + 16 wc ..) into acct.
template <int NJ, bool FP8, bool TAIL = false>
__device__ __forceinline__ void dense_compute(const uint8_t* __restrict__ ta,
                                              const uint8_t* __restrict__ tb, int wr, int wc,
                                              f32x4 (&acc)[4][8], f32x4 (&acct)[4]) {
  const int lane = threadIdx.x & 63;
  // fragment rows are 16-aligned bases + (lane & 15), so row & 7 == lane & 7
  const uint8_t* pa = ta + (64 * wr + (lane & 15)) * kDChunk;
  const uint8_t* pb = tb + (128 * wc + (lane & 15)) * kDChunk;
  if constexpr (FP8) {
    const int c0 = ((lane >> 4) ^ (lane & 7)) << 4, c1 = ((4 + (lane >> 4)) ^ (lane & 7)) << 4;
    Frag<true> fa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i].lds(pa + i * 16 * kDChunk + c0, c1 - c0);
    // B fragments one token group ahead (all twelve at once would not fit
    // beside the accumulators at two waves per SIMD)
    Frag<true> fb[2];
    fb[0].lds(pb + c0, c1 - c0);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (j + 1 < NJ) fb[(j + 1) & 1].lds(pb + (j + 1) * 16 * kDChunk + c0, c1 - c0);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][j] = mfma_fp8(fa[i].v, fb[j & 1].v, acc[i][j]);
    }
    return;
  }
  const uint8_t* pt = tb + (kDTok + 16 * wc + (lane & 15)) * kDChunk;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int cs = (((s << 2) + (lane >> 4)) ^ (lane & 7)) << 4;
    bf16x8 fa[4], fb[NJ > 0 ? NJ : 1], ft;
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = *(const bf16x8*)(pa + i * 16 * kDChunk + cs);
#pragma unroll
    for (int j = 0; j < NJ; ++j) fb[j] = *(const bf16x8*)(pb + j * 16 * kDChunk + cs);
    if constexpr (TAIL) ft = *(const bf16x8*)(pt + cs);
    // all reads of the k-step are issued before its first MFMA, so their
    // latencies overlap instead of one read per 4 MFMAs
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][j] = mfma_bf16(fa[i], fb[j], acc[i][j]);
    if constexpr (TAIL) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acct[i] = mfma_bf16(fa[i], ft, acct[i]);
    }
  }
}

// Wait until at most N vector-memory loads of this wave are outstanding
// (s_waitcnt with expcnt and lgkmcnt left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0xF70 | N);
}

// Workgroup barrier for the staging ring: waits for this wave's LDS reads
// (lgkmcnt 0), so the stage it read may be refilled, then meets the other
// waves, each of which has already waited for its own loads of the next
// stage. __syncthreads would also drain the loads still in flight for later
// stages (its fences wait for vmcnt 0, which tracks direct-to-LDS loads);
// compiler-only fences keep LDS accesses from being moved across instead.
__device__ __forceinline__ void ring_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt: no wait
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// The whole K loop of one unit; all 512 threads take part. While chunk c is
// multiplied, the token tile of chunk c+1 and the weight tiles of chunks c+1
// and c+2 are in flight (MG, the merging ring: chunk c+1 of both). Loads
// retire in issue order, so waiting for all but the newest weight tile's
// loads leaves chunk c+1 complete. tj: this wave multiplies a merged tail's
// token group as well (MG). nj = 16-token
// groups of this wave holding tokens (0 = idle wave, which only stages).
// The chunks are walked from chunk rot mod nch on, wrapping around. FC2
// passes cold_rot(row tile): the blocks sharing a weight tile stay in step (it
// is read once from HBM and served to the partner from L2) while the units of
// other row tiles start elsewhere in K. FC1 passes cold_rot(block): the row
// tiles sharing a block's 2 MB token tile stay in step instead, which measured
// better there. Prefill workload, kernel traces (one box each): against the
// same loop with rot = 0, e4m3 FC1 784 -> 627 us, bf16 FC2 587 -> 579 us, bf16
// FC1 unchanged (1104 us); FC1 keyed by block instead of row tile, bf16
// 1086 -> 1065 us, e4m3 623 -> 619 us (FC2 keyed by block: 571 -> 580 us, so
// FC2 keeps the row tile). The change also left bf16 FC1 without the 36 bytes
// of scratch per lane it had spilled (the compiler places the per-unit values
// differently).
template <bool FP8, bool MG = false>
__device__ __forceinline__ void dense_kloop(const DenseStage& st, int kbytes, int nj, bool tj,
                                            int wr, int wc, uint8_t* __restrict__ lds,
                                            f32x4 (&acc)[4][8], f32x4 (&acct)[4], int rot) {
  using R = DRing<MG>;
  const int nch = kbytes / kDChunk;  // at least 2 (K >= 128)
  // chunks in rotated order (as the cold tiles): the c-th chunk walked
  const int s0 = rot % nch;
  auto kc = [&](int c) {
    const int x = c + s0;
    return x >= nch ? x - nch : x;
  };
  // tile addresses are computed from the LDS base so they stay in the LDS
  // address space
  uint8_t* const ra = lds;
  uint8_t* const rb = lds + R::kAStages * kDTile;
  auto compute = [&](const uint8_t* ta, const uint8_t* tb) {
    if (MG && tj) {  // a merged tail rides on a full block: nj is 8, or 0 past a 128-block
      if (nj > 0)
        dense_compute<8, FP8, MG>(ta, tb, wr, wc, acc, acct);
      else
        dense_compute<0, FP8, MG>(ta, tb, wr, wc, acc, acct);
    } else if (nj > 4)
      dense_compute<8, FP8>(ta, tb, wr, wc, acc, acct);
    else if (nj > 2)
      dense_compute<4, FP8>(ta, tb, wr, wc, acc, acct);
    else if (nj > 0)
      dense_compute<2, FP8>(ta, tb, wr, wc, acc, acct);
  };
  if constexpr (MG) {
    // two stages of each operand: chunk c+1 is in flight while c is multiplied
    st.issue_a(ra, kc(0));
    st.issue_b<MG>(rb, kc(0));
    wait_vm<0>();
    ring_barrier();
    for (int c = 0; c < nch; ++c) {
      if (c + 1 < nch) {
        st.issue_b<MG>(rb + ((c + 1) & 1) * R::kBTile, kc(c + 1));
        st.issue_a(ra + ((c + 1) & 1) * kDTile, kc(c + 1));
      }
      compute(ra + (c & 1) * kDTile, rb + (c & 1) * R::kBTile);
      wait_vm<0>();
      ring_barrier();
    }
    return;
  }
  st.issue_a(ra, kc(0));
  st.issue_b(rb, kc(0));
  st.issue_a(ra + kDTile, kc(1));
  wait_vm<kDALoads>();
  ring_barrier();
  int ia = 0;  // weight stage of chunk c
  for (int c = 0; c < nch; ++c) {
    const int ia2 = ia == 0 ? 2 : ia - 1;  // weight stage of chunk c+2
    if (c + 1 < nch) st.issue_b(rb + ((c + 1) & 1) * kDTile, kc(c + 1));
    if (c + 2 < nch) st.issue_a(ra + ia2 * kDTile, kc(c + 2));
    compute(ra + ia * kDTile, rb + (c & 1) * kDTile);
    if (c + 2 < nch)
      wait_vm<kDALoads>();
    else
      wait_vm<0>();
    ring_barrier();
    ia = ia == 2 ? 0 : ia + 1;
  }
}

// Unit scheduler of the dense kernels. The unit list is cut into 8 contiguous
// shares, one per XCD; a workgroup takes the next unit of its own XCD's share
// from an atomic counter and, when that share is drained, helps with the
// others. Taking units in list order keeps the blocks that share a weight
// tile running side by side on one XCD, so the tile is fetched from HBM once
// and served to the partner from L2. Which workgroup computes a unit never
// changes the result. With remap off, units are dealt round-robin instead.

__device__ __forceinline__ int hw_xcc_id() {
  int v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & (kQueues - 1);
}

struct DenseSched {
  int* cnt;  // kQueues counters, zero at launch
  int units, per, q0, qi, next_static;
  bool dyn;
  __device__ DenseSched(int* c, int n, int remap)
      : cnt(c), units(n), per((n + kQueues - 1) / kQueues), q0(hw_xcc_id()), qi(0),
        next_static(blockIdx.x), dyn(remap != 0) {}
  // Next unit of this workgroup, or -1. Uses the first 4 bytes of the (idle)
  // staging LDS to broadcast the pick.
  __device__ __forceinline__ int next(uint8_t* __restrict__ lds) {
    if (!dyn) {
      const int u = next_static;
      next_static += gridDim.x;
      return u < units ? u : -1;
    }
    if (threadIdx.x == 0) {
      int u = -1;
      for (; qi < kQueues; ++qi) {
        const int q = (q0 + qi) & (kQueues - 1);
        const int lo = q * per, n = min(units, lo + per) - lo;
        if (n <= 0) continue;
        const int t = atomicAdd(cnt + q, 1);
        if (t < n) {
          u = lo + t;
          break;
        }
      }
      *(volatile __attribute__((address_space(3))) int*)lds = u;
    }
    __syncthreads();
    const int u = *(volatile __attribute__((address_space(3))) int*)lds;
    __syncthreads();
    return u;
  }
};

__global__ void zero_counters_kernel(int* __restrict__ c, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) c[i] = 0;
}

// First block and length of the run of blocks with expert e containing bn
// (block_expert is non-decreasing). Wave-wide probes of 64 blocks.
__device__ __forceinline__ void find_run(const int32_t* __restrict__ block_expert, int nb, int bn,
                                         int e, int& fb, int& q) {
  const int lane = threadIdx.x & 63;
  int lo = bn;
  for (;;) {
    const int i = lo - 64 + lane;
    const uint64_t m = __ballot(i >= 0 && block_expert[i] == e);
    if (m == ~0ull) {
      lo -= 64;
      continue;
    }
    lo = lo - 64 + (63 - __clzll(~m)) + 1;
    break;
  }
  int hi = bn + 1;
  for (;;) {
    const int i = hi + lane;
    const uint64_t m = __ballot(i < nb && block_expert[i] == e);
    if (m == ~0ull) {
      hi += 64;
      continue;
    }
    hi += __ffsll((long long)~m) - 1;
    break;
  }
  fb = lo;
  q = hi - lo;
}

// Map unit u of the (expert, row tile, block) order to (row tile r, block b).
// With MG, a run (the blocks of one expert) of two or more blocks whose last
// block holds at most kDTail tokens has that block merged into the one
// before it: merge is set, and tail_m is the last block's token count.
struct UnitMap {
  int nb, n_rt;
  int run_b0 = 0, run_q = 0, e = 0;
  long run_u0 = 0, run_u1 = 0;
  int tail_m = 0;
  bool merge = false;
  template <bool MG = false>
  __device__ __forceinline__ void locate(const int32_t* __restrict__ block_expert, int u, int& r,
                                         int& b, const int32_t* __restrict__ sorted_ids = nullptr,
                                         int M = 0, int S = 0) {
    if (u >= run_u1 || u < run_u0) {
      const int bn = (int)(u / n_rt);
      e = block_expert[bn];
      find_run(block_expert, nb, bn, e, run_b0, run_q);
      run_u0 = (long)run_b0 * n_rt;
      run_u1 = run_u0 + (long)run_q * n_rt;
      if (MG) {
        tail_m = run_q >= 2 ? block_valid(sorted_ids, run_b0 + run_q - 1, M, S) : kDTail + 1;
        merge = tail_m <= kDTail;
      }
    }
    const long loc = u - run_u0;
    r = (int)(loc / run_q);
    b = run_b0 + (int)(loc % run_q);
  }
};

// FC1 of prefill-sized blocks; FP8: e4m3 x codes and weights, scaled per
// weight row and per token in the epilogue; h is written in bf16 either way.
// bf16 merges tails (UnitMap); the fp8 tiles keep three weight stages.
template <bool FP8>
__global__ __launch_bounds__(kDThreads) void dense_fc1_kernel(Fc1Args p) {
  constexpr bool MG = !FP8;
  __shared__ __attribute__((aligned(16))) uint8_t lds[DRing<MG>::kLds];
  const int M = 1 << p.log2m;
  const int nb = num_blocks(p.num_padded, p.S, p.E, p.log2m);
  const int n_rt = (2 * p.I) / kDRows;  // 128 gate + 128 up rows per unit
  const int units = nb * n_rt;
  const int w = threadIdx.x >> 6, wr = w & 3, wc = w >> 2, lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const size_t rowb = (size_t)p.H * (FP8 ? 1 : 2);
  UnitMap um{nb, n_rt};
  DenseSched sched(p.queue, units, p.remap);
  for (int u; (u = sched.next(lds)) >= 0;) {
    int r, b;
    um.locate<MG>(p.block_expert, u, r, b, p.sorted_ids, M, p.S);
    const int e = um.e;
    int mb = (unsigned)e < (unsigned)p.E ? block_valid(p.sorted_ids, b, M, p.S) : 0;
    int tm = 0;  // tokens of a tail merged into this unit (block b + 1)
    if (MG && um.merge) {
      const int last = um.run_b0 + um.run_q - 1;
      if (b == last)
        mb = 0;  // computed with block b - 1
      else if (b == last - 1)
        tm = um.tail_m;
    }
    for (int t0 = 0; t0 < mb; t0 += kDTok) {  // one pass: M <= kDTok
      const int m = mb - t0;
      DenseStage st;
      const int col = dstage_col();
      const int slot0 = p.sorted_ids[(size_t)b * M + t0];  // a valid row for idle columns
      st.bgroups = dstage_bgroups(m);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // unit rows: 16-row MFMA tiles of 8 gate rows + the matching 8 up rows
        const int rho = dstage_row(i), tt = rho >> 4, wi = rho & 15;
        const int wrow = wi < 8 ? (r * 128 + tt * 8 + wi) : (p.I + r * 128 + tt * 8 + wi - 8);
        st.arow[i] = (const uint8_t*)p.w1 + ((size_t)e * 2 * p.I + wrow) * rowb + col;
        const int slot = rho < m ? p.sorted_ids[(size_t)b * M + t0 + rho] : slot0;
        st.brow[i] = (const uint8_t*)p.x + (size_t)(slot / p.k) * rowb + col;
      }
      if constexpr (MG) {
        const int tr = 8 * w + (lane >> 3);  // waves 0..3: tail rows 8 w ..
        st.tload = w < 4 && 8 * w < tm;
        const int ts = w < 4 && tr < tm ? p.sorted_ids[(size_t)(b + 1) * M + tr] : slot0;
        st.trow = (const uint8_t*)p.x + (size_t)(ts / p.k) * rowb + col;
      }
      f32x4 acc[4][8] = {}, acct[4] = {};
      const int nj = min(8, max(0, (m - 128 * wc + 15) >> 4));
      const bool tj = tm > 16 * wc;
      dense_kloop<FP8, MG>(st, (int)rowb, nj, tj, wr, wc, lds, acc, acct, cold_rot(b));
      if constexpr (MG) {
        if (tj) {
          const int ti = 16 * wc + (lane & 15);
          const int slot = ti < tm ? p.sorted_ids[(size_t)(b + 1) * M + ti] : p.S;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = __shfl_xor(acct[i][q], 32);
            if (lane < 32 && slot < p.S)
              store_h<false>(p, slot, r * 128 + (4 * wr + i) * 8 + 4 * g, acct[i], o);
          }
        }
      }
      if (nj == 0) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int ti = 128 * wc + 16 * j + (lane & 15);
        const int slot = ti < m ? p.sorted_ids[(size_t)b * M + t0 + ti] : p.S;
        if constexpr (FP8) {
          // lanes 0..31 hold gate rows, 32..63 the matching up rows
          const float xs = slot < p.S ? p.xs[slot / p.k] : 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tt = 4 * wr + i;
            const int srow =
                g < 2 ? (r * 128 + tt * 8 + 4 * g) : (p.I + r * 128 + tt * 8 + 4 * (g - 2));
            const f32x4 sc = *(const f32x4*)(p.w1s + (size_t)e * 2 * p.I + srow);
            f32x4 v, o;
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = acc[i][j][q] * (sc[q] * xs);
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = __shfl_xor(v[q], 32);
            // h in bf16 (the per-slot quantiser reads it next)
            if (lane < 32 && slot < p.S) store_h<false>(p, slot, r * 128 + tt * 8 + 4 * g, v, o);
          }
          continue;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = __shfl_xor(acc[i][j][q], 32);
          if (lane < 32 && slot < p.S) {
            const int colh = r * 128 + (4 * wr + i) * 8 + 4 * g;
            uint32_t hb[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) hb[q] = f32_to_bf16_rne(silu_mul(acc[i][j][q], o[q]));
            *(u32x2*)((uint16_t*)p.h + (size_t)slot * p.I + colh) =
                u32x2{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
          }
        }
      }
    }
  }
}

// FC2 of prefill-sized blocks; FP8: e4m3 h codes and weights, scaled per
// weight row and per slot in the epilogue. Tails are not merged here: on the
// prefill workload FC2 ran 567 us unmerged on three weight stages, 589 us on
// two, 571 us merged on two (one box, kernel traces), so FC2 keeps three.
template <bool FP8>
__global__ __launch_bounds__(kDThreads) void dense_fc2_kernel(Fc2Args p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kDLds];
  const int M = 1 << p.log2m;
  const int nb = num_blocks(p.num_padded, p.S, p.E, p.log2m);
  const int n_rt = (p.H + kDRows - 1) / kDRows;  // the last row tile may be partial
  const int units = nb * n_rt;
  const int w = threadIdx.x >> 6, wr = w & 3, wc = w >> 2, lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const size_t rowb = (size_t)p.I * (FP8 ? 1 : 2);
  UnitMap um{nb, n_rt};
  DenseSched sched(p.queue, units, p.remap);
  for (int u; (u = sched.next(lds)) >= 0;) {
    int r, b;
    um.locate(p.block_expert, u, r, b);
    const int e = um.e;
    const int mb = (unsigned)e < (unsigned)p.E ? block_valid(p.sorted_ids, b, M, p.S) : 0;
    for (int t0 = 0; t0 < mb; t0 += kDTok) {
      const int m = mb - t0;
      DenseStage st;
      const int col = dstage_col();
      const int slot0 = p.sorted_ids[(size_t)b * M + t0];  // a valid row for idle columns
      st.bgroups = dstage_bgroups(m);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rho = dstage_row(i);
        const int wrow = min(r * kDRows + rho, p.H - 1);  // rows past H: loaded, never stored
        st.arow[i] = (const uint8_t*)p.w2 + ((size_t)e * p.H + wrow) * rowb + col;
        const int slot = rho < m ? p.sorted_ids[(size_t)b * M + t0 + rho] : slot0;
        st.brow[i] = (const uint8_t*)p.h + (size_t)slot * rowb + col;
      }
      f32x4 acc[4][8] = {}, acct[4];
      const int nj = min(8, max(0, (m - 128 * wc + 15) >> 4));
      dense_kloop<FP8>(st, (int)rowb, nj, false, wr, wc, lds, acc, acct, cold_rot(r));
      if (nj == 0) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int ti = 128 * wc + 16 * j + (lane & 15);
        const int slot = ti < m ? p.sorted_ids[(size_t)b * M + t0 + ti] : p.S;
        if (slot < p.S) {
          const float hs = FP8 ? p.hs[slot] : 1.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = r * kDRows + 64 * wr + 16 * i + 4 * g;
            if (row < p.H) {
              f32x4 v = acc[i][j];
              if constexpr (FP8) {
                const f32x4 sc = *(const f32x4*)(p.w2s + (size_t)e * p.H + row);
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] *= sc[q] * hs;
              }
              store_y(p, slot, row, v);
            }
          }
        }
      }
    }
  }
  finish_queue(p.queue, kQueues);
}

// ----------------------------------------------- per-row FP8 quantiser ---
// One wave per row: absmax, scale = absmax/448 (1 for a zero row), then
// code = e4m3fn(v / scale); both divisions are correctly rounded fp32.
__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const u32x4 q = *(const u32x4*)p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_bits_to_f32(q[i] & 0xffffu);
    v[2 * i + 1] = bf16_bits_to_f32(q[i] >> 16);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}

// Encode 8 values of a row at column c with the row's scale (WT as store_h).
template <bool WT>
__device__ __forceinline__ void quant_store8(const float (&v)[8], float scale,
                                             uint8_t* __restrict__ codes, int c) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= f32_to_e4m3fn(v[i] / scale) << (8 * i);
    hi |= f32_to_e4m3fn(v[4 + i] / scale) << (8 * i);
  }
  if (WT) {
    st_dev((uint32_t*)(codes + c), lo);
    st_dev((uint32_t*)(codes + c) + 1, hi);
  } else {
    *(u32x2*)(codes + c) = u32x2{lo, hi};
  }
}

// One row of C elements by the calling wave: codes and its scale (WT as
// store_h). A lane takes 8 consecutive elements at each of the columns
// lane*8 + 512*b; up to kQB such vectors per lane are loaded together (all
// in flight at once) and, for rows of at most 512*kQB elements, kept in
// registers between the absmax and the encoding.
constexpr int kQB = 8;
template <typename InT, bool WT = false>
__device__ __forceinline__ void quant_row(const InT* __restrict__ row, int C,
                                          uint8_t* __restrict__ codes, float* __restrict__ scale_out) {
  const int lane = threadIdx.x & 63;
  constexpr int step = kWave * 8;
  float amax = 0.f;
  if (C <= step * kQB) {
    float v[kQB][8];
#pragma unroll
    for (int b = 0; b < kQB; ++b) {
      const int c = lane * 8 + b * step;
      if (c < C) {
        load8(row + c, v[b]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[b][i] = 0.f;
      }
    }
#pragma unroll
    for (int b = 0; b < kQB; ++b)
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[b][i]));
    amax = wave_max(amax);
    const float scale = amax == 0.f ? 1.0f : amax / 448.0f;
#pragma unroll
    for (int b = 0; b < kQB; ++b) {
      const int c = lane * 8 + b * step;
      if (c < C) quant_store8<WT>(v[b], scale, codes, c);
    }
    if (lane == 0) {
      if (WT) st_dev(scale_out, scale);
      else *scale_out = scale;
    }
    return;
  }
  for (int c0 = lane * 8; c0 < C; c0 += step * kQB) {
    float v[kQB][8];
#pragma unroll
    for (int b = 0; b < kQB; ++b) {
      const int c = c0 + b * step;
      if (c < C) {
        load8(row + c, v[b]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[b][i] = 0.f;
      }
    }
#pragma unroll
    for (int b = 0; b < kQB; ++b)
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[b][i]));
  }
  amax = wave_max(amax);
  const float scale = amax == 0.f ? 1.0f : amax / 448.0f;
  for (int c0 = lane * 8; c0 < C; c0 += step * kQB) {
    float v[kQB][8];
#pragma unroll
    for (int b = 0; b < kQB; ++b) {
      const int c = c0 + b * step;
      if (c < C) load8(row + c, v[b]);
    }
#pragma unroll
    for (int b = 0; b < kQB; ++b) {
      const int c = c0 + b * step;
      if (c < C) quant_store8<WT>(v[b], scale, codes, c);
    }
  }
  if (lane == 0) {
    if (WT) st_dev(scale_out, scale);
    else *scale_out = scale;
  }
}

template <typename InT>
__global__ __launch_bounds__(256) void quant_rows_kernel(const InT* __restrict__ in, int R, int C,
                                                         uint8_t* __restrict__ codes,
                                                         float* __restrict__ scales) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  quant_row<InT>(in + (size_t)r * C, C, codes + (size_t)r * C, scales + r);
}

// One row per 256-thread workgroup: the same codes and scale as quant_row
// (the absmax is exact in any order), with the per-element division and
// encoding spread over 4 times as many lanes. Rows of at most 2048*kQB
// elements (every row of this library's shapes).
template <typename InT>
__global__ __launch_bounds__(256) void quant_rows_wg_kernel(const InT* __restrict__ in, int C,
                                                            uint8_t* __restrict__ codes,
                                                            float* __restrict__ scales) {
  __shared__ float wmax[4];
  const int r = blockIdx.x, t = threadIdx.x;
  const InT* row = in + (size_t)r * C;
  uint8_t* crow = codes + (size_t)r * C;
  constexpr int step = 256 * 8;
  float v[kQB][8];
#pragma unroll
  for (int b = 0; b < kQB; ++b) {
    const int c = t * 8 + b * step;
    if (c < C) {
      load8(row + c, v[b]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[b][i] = 0.f;
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int b = 0; b < kQB; ++b)
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[b][i]));
  amax = wave_max(amax);
  if ((t & 63) == 0) wmax[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float scale = amax == 0.f ? 1.0f : amax / 448.0f;
#pragma unroll
  for (int b = 0; b < kQB; ++b) {
    const int c = t * 8 + b * step;
    if (c < C) quant_store8<false>(v[b], scale, crow, c);
  }
  if (t == 0) scales[r] = scale;
}

// Row quantiser launch: a workgroup per row while the rows are few (fewer than
// one wave per SIMD of the chip), else a wave per row.
template <typename InT>
static void launch_quant_rows(const InT* in, int R, int C, uint8_t* codes, float* scales,
                              hipStream_t stream) {
  if (R <= 1024 && C <= 256 * 8 * kQB)
    quant_rows_wg_kernel<InT><<<R, 256, 0, stream>>>(in, C, codes, scales);
  else
    quant_rows_kernel<InT><<<(R + 3) / 4, 256, 0, stream>>>(in, R, C, codes, scales);
}

// Per-group FP8 quantiser: groups of 128 consecutive elements of a row, 16
// lanes per group (8 elements each), four groups per wave; the decisions of
// quant_rows_kernel within each group. scales: [R, C/128].
template <typename InT>
__global__ __launch_bounds__(256) void quant_groups_kernel(const InT* __restrict__ in, int R,
                                                           int C, uint8_t* __restrict__ codes,
                                                           float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int G = C / kBlk;
  const long n = (long)R * G;
  const long gi = ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  const bool live = gi < n;  // a 16-lane row is live or not as a whole
  const size_t at = live ? (size_t)(gi / G) * C + (size_t)(gi % G) * kBlk + (lane & 15) * 8 : 0;
  float v[8] = {};
  if (live) load8(in + at, v);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  // max over the 16 lanes of the group (DPP inside one row)
  amax = fmaxf(amax, wave_partner<0>(amax));
  amax = fmaxf(amax, wave_partner<1>(amax));
  amax = fmaxf(amax, wave_partner<2>(amax));
  amax = fmaxf(amax, wave_partner<3>(amax));
  const float scale = amax == 0.f ? 1.0f : amax / 448.0f;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= f32_to_e4m3fn(v[i] / scale) << (8 * i);
    hi |= f32_to_e4m3fn(v[4 + i] / scale) << (8 * i);
  }
  if (live) {
    *(u32x2*)(codes + at) = u32x2{lo, hi};
    if ((lane & 15) == 0) scales[gi] = scale;
  }
}

// ----------------------------------------------------------- combine ---
// out[t, n] = sum_j w[t, j] * y[t*k + j, n], fp32 in j order, one rounding.
__device__ __forceinline__ void load8y(const float* p, float (&v)[8]) { load8(p, v); }
__device__ __forceinline__ void load8y(const uint16_t* p, float (&v)[8]) { load8(p, v); }

// Slots whose expert id lies outside [0, E) belong to another shard: their y
// rows were never written and they add nothing.
// Outputs [8i, 8i+8) of the flattened [T, H] result (H a multiple of 8).
template <typename YT, typename OutT>
__device__ __forceinline__ void combine8(const YT* __restrict__ y, const float* __restrict__ w,
                                         const int32_t* __restrict__ ids, int E, int H, int k,
                                         OutT* __restrict__ out, long i) {
  const int per_row = H >> 3;
  const int t = (int)(i / per_row), n = (int)(i % per_row) * 8;
  float acc[8] = {};
  // up to 8 slots at a time: all their loads are issued before the sum, which
  // then runs in j order and leaves out the slots of other shards (their y rows
  // are read, in bounds, but never added)
  for (int j0 = 0; j0 < k; j0 += 8) {
    const int jn = min(8, k - j0);
    float v[8][8], wj[8];
    bool mine[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      mine[u] = false;
      wj[u] = 0.f;
      if (u < jn) {
        const size_t s = (size_t)t * k + j0 + u;
        mine[u] = (unsigned)ids[s] < (unsigned)E;
        wj[u] = w[s];
        load8y(y + s * H + n, v[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (mine[u]) {
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += wj[u] * v[u][q];
      }
    }
  }
  if constexpr (sizeof(OutT) == 2) {
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = f32_to_bf16_rne(acc[2 * q]) | (f32_to_bf16_rne(acc[2 * q + 1]) << 16);
    *(u32x4*)(out + (size_t)t * H + n) = o;
  } else {
    *(f32x4*)(out + (size_t)t * H + n) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *(f32x4*)(out + (size_t)t * H + n + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
}

template <typename YT, typename OutT>
__global__ __launch_bounds__(256) void combine_kernel(const YT* __restrict__ y,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ ids, int E,
                                                      int T, int H, int k,
                                                      OutT* __restrict__ out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)T * (H >> 3)) return;
  combine8<YT, OutT>(y, w, ids, E, H, k, out, i);
}

// A combine for H not a multiple of 8 (fp32 path): one thread per element.
__global__ __launch_bounds__(256) void combine_f32_scalar_kernel(const float* __restrict__ y,
                                                                 const float* __restrict__ w,
                                                                 const int32_t* __restrict__ ids,
                                                                 int E, int T, int H, int k,
                                                                 float* __restrict__ out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)T * H) return;
  const int t = (int)(i / H), n = (int)(i % H);
  float acc = 0.f;
  for (int j = 0; j < k; ++j)
    if ((unsigned)ids[(size_t)t * k + j] < (unsigned)E)
      acc += w[(size_t)t * k + j] * y[((size_t)t * k + j) * H + n];
  out[i] = acc;
}

// ------------------------------------------------------------- fp32 ---
// Plain path for small problems: one wave per (sorted position, output
// column), lanes split K, wave-sum reduction.
__global__ __launch_bounds__(256) void fc1_f32_kernel(const float* __restrict__ x,
                                                      const float* __restrict__ w1,
                                                      const int32_t* __restrict__ sorted_ids,
                                                      const int32_t* __restrict__ block_expert,
                                                      const int32_t* __restrict__ num_padded,
                                                      int E, int H, int I, int k, int S,
                                                      int log2m, float* __restrict__ h) {
  const int lane = threadIdx.x & 63;
  const long W = (long)gridDim.x * 4;
  const long total = ((long)num_blocks(num_padded, S, E, log2m) << log2m) * I;
  for (long u = (long)blockIdx.x * 4 + (threadIdx.x >> 6); u < total; u += W) {
    const int pos = (int)(u / I), n = (int)(u % I);
    const int slot = sorted_ids[pos];
    if (slot >= S) continue;
    const int e = block_expert[pos >> log2m];
    if ((unsigned)e >= (unsigned)E) continue;
    const float* xr = x + (size_t)(slot / k) * H;
    const float* gr = w1 + ((size_t)e * 2 * I + n) * H;
    const float* ur = gr + (size_t)I * H;
    float gs = 0.f, us = 0.f;
    for (int c = lane * 4; c < H; c += kWave * 4) {
      const f32x4 xv = *(const f32x4*)(xr + c), gv = *(const f32x4*)(gr + c),
                  uv = *(const f32x4*)(ur + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        gs += gv[q] * xv[q];
        us += uv[q] * xv[q];
      }
    }
    gs = wave_sum(gs);
    us = wave_sum(us);
    if (lane == 0) h[(size_t)slot * I + n] = silu_mul(gs, us);
  }
}

__global__ __launch_bounds__(256) void fc2_f32_kernel(const float* __restrict__ h,
                                                      const float* __restrict__ w2,
                                                      const int32_t* __restrict__ sorted_ids,
                                                      const int32_t* __restrict__ block_expert,
                                                      const int32_t* __restrict__ num_padded,
                                                      int E, int H, int I, int S, int log2m,
                                                      float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const long W = (long)gridDim.x * 4;
  const long total = ((long)num_blocks(num_padded, S, E, log2m) << log2m) * H;
  for (long u = (long)blockIdx.x * 4 + (threadIdx.x >> 6); u < total; u += W) {
    const int pos = (int)(u / H), n = (int)(u % H);
    const int slot = sorted_ids[pos];
    if (slot >= S) continue;
    const int e = block_expert[pos >> log2m];
    if ((unsigned)e >= (unsigned)E) continue;
    const float* hr = h + (size_t)slot * I;
    const float* wr = w2 + ((size_t)e * H + n) * I;
    float s = 0.f;
    for (int c = lane * 4; c < I; c += kWave * 4) {
      const f32x4 hv = *(const f32x4*)(hr + c), wv = *(const f32x4*)(wr + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) s += wv[q] * hv[q];
    }
    s = wave_sum(s);
    if (lane == 0) y[(size_t)slot * H + n] = s;
  }
}

// ------------------------------------ bf16 / fp8, any multiple of 8 ---
// Shapes whose H or I is not a multiple of 128 (every kernel above stages
// whole 128-byte lines of a row): one wave per (aligned position, output
// column), lanes split K in vectors of 8 elements, as the fp32 path. The
// weights are read once per slot instead of once per block: a fallback for
// such shapes, not a performance path. FP8: e4m3 codes decoded exactly to
// fp32 (v_cvt_pk_f32_fp8), the per-row weight scale and the per-token /
// per-slot activation scale applied to the fp32 sum.

__device__ __forceinline__ void load8e(const uint16_t* p, float (&v)[8]) { load8(p, v); }
__device__ __forceinline__ void load8e(const uint8_t* p, float (&v)[8]) {
  const u32x2 q = *(const u32x2*)p;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[i], false);  // codes 4i, 4i+1
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[i], true);   // codes 4i+2, 4i+3
    v[4 * i] = lo[0];
    v[4 * i + 1] = lo[1];
    v[4 * i + 2] = hi[0];
    v[4 * i + 3] = hi[1];
  }
}

// FC1: h[s, n] = SiLU(g) * u; bf16 h in bf16, FP8 h in fp32 (quantised next).
template <bool FP8>
__global__ __launch_bounds__(256) void gen_fc1_kernel(Fc1Args p) {
  using ET = typename std::conditional<FP8, uint8_t, uint16_t>::type;
  const int lane = threadIdx.x & 63;
  const long W = (long)gridDim.x * 4;
  const long total = ((long)num_blocks(p.num_padded, p.S, p.E, p.log2m) << p.log2m) * p.I;
  for (long u = (long)blockIdx.x * 4 + (threadIdx.x >> 6); u < total; u += W) {
    const int pos = (int)(u / p.I), n = (int)(u % p.I);
    const int slot = p.sorted_ids[pos];
    if (slot >= p.S) continue;
    const int e = p.block_expert[pos >> p.log2m];
    if ((unsigned)e >= (unsigned)p.E) continue;
    const int t = slot / p.k;
    const ET* xr = (const ET*)p.x + (size_t)t * p.H;
    const ET* gr = (const ET*)p.w1 + ((size_t)e * 2 * p.I + n) * p.H;
    const ET* ur = gr + (size_t)p.I * p.H;
    float gs = 0.f, us = 0.f;
    for (int c = lane * 8; c < p.H; c += kWave * 8) {
      float xv[8], gv[8], uv[8];
      load8e(xr + c, xv);
      load8e(gr + c, gv);
      load8e(ur + c, uv);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        gs += gv[q] * xv[q];
        us += uv[q] * xv[q];
      }
    }
    gs = wave_sum(gs);
    us = wave_sum(us);
    if (lane == 0) {
      if constexpr (FP8) {
        const float xs = p.xs[t];
        gs *= p.w1s[(size_t)e * 2 * p.I + n] * xs;
        us *= p.w1s[(size_t)e * 2 * p.I + p.I + n] * xs;
        ((float*)p.h)[(size_t)slot * p.I + n] = silu_mul(gs, us);
      } else {
        ((uint16_t*)p.h)[(size_t)slot * p.I + n] = (uint16_t)f32_to_bf16_rne(silu_mul(gs, us));
      }
    }
  }
}

// FC2: y[s, n] = W2[e, n, :] . h[s, :]; bf16 y in bf16, FP8 y in fp32.
template <bool FP8>
__global__ __launch_bounds__(256) void gen_fc2_kernel(Fc2Args p) {
  using ET = typename std::conditional<FP8, uint8_t, uint16_t>::type;
  const int lane = threadIdx.x & 63;
  const long W = (long)gridDim.x * 4;
  const long total = ((long)num_blocks(p.num_padded, p.S, p.E, p.log2m) << p.log2m) * p.H;
  for (long u = (long)blockIdx.x * 4 + (threadIdx.x >> 6); u < total; u += W) {
    const int pos = (int)(u / p.H), n = (int)(u % p.H);
    const int slot = p.sorted_ids[pos];
    if (slot >= p.S) continue;
    const int e = p.block_expert[pos >> p.log2m];
    if ((unsigned)e >= (unsigned)p.E) continue;
    const ET* hr = (const ET*)p.h + (size_t)slot * p.I;
    const ET* wr = (const ET*)p.w2 + ((size_t)e * p.H + n) * p.I;
    float s = 0.f;
    for (int c = lane * 8; c < p.I; c += kWave * 8) {
      float hv[8], wv[8];
      load8e(hr + c, hv);
      load8e(wr + c, wv);
#pragma unroll
      for (int q = 0; q < 8; ++q) s += wv[q] * hv[q];
    }
    s = wave_sum(s);
    if (lane == 0) {
      if constexpr (FP8)
        ((float*)p.y)[(size_t)slot * p.H + n] = s * (p.w2s[(size_t)e * p.H + n] * p.hs[slot]);
      else
        ((uint16_t*)p.y)[(size_t)slot * p.H + n] = (uint16_t)f32_to_bf16_rne(s);
    }
  }
}

// --------------------------------------------- single-launch small path ---
// For batches of at most kSmallMaxT tokens the whole layer runs as one
// cooperative persistent kernel ("vLLM SM architecture adaptation", section
// 4.3: for a batch of at most 8 tokens the grouped-GEMM path's launch
// overhead is what a single-kernel path avoids). Phases, separated by grid
// barriers: routing (one wave per token; FP8: other waves quantise x rows) |
// alignment, rebuilt by every workgroup in LDS from the routed ids, then FC1 |
// (FP8: quantise h rows) | FC2 | combine. Every block of such a batch is cold,
// so FC1 and FC2 are exactly the cold passes of the separate launches, over
// units of (expert, up to 8 of its slots) instead of aligned blocks; results
// equal theirs bit for bit.

constexpr int kSmallMaxT = 16;
constexpr int kSmallMaxS = 256;     // slots (one per thread of a workgroup)
constexpr int kSmallMaxE = 1024;
constexpr int kBarInts = 512;       // barrier words, zero at launch
constexpr int kBarTop = 256, kBarGen = 288, kBarErr = 511;

struct SmallArgs {
  const float* logits;
  const uint16_t* x;
  const void* w1;
  const float* w1s;
  const void* w2;
  const float* w2s;
  int T, E, H, I, k, renorm, remap;
  int32_t* ids;
  float* wts;
  uint8_t* xq;     // FP8: codes and scales of x
  float* xs;
  void* h;         // bf16 [S, I] or f32 [S, I] (FP8)
  uint8_t* hq;     // FP8: codes and scales of h
  float* hs;
  void* y;         // bf16 [S, H] or f32 [S, H] (FP8)
  uint16_t* out;
  int* bar;        // kBarInts words: group counters at 32*g (g < 8), top, gen, error
};

// Grid barrier over all workgroups of a cooperative launch (all resident).
// Two levels: workgroup g arrives on the counter of group g & 7, the last of
// a group on the top counter, the last group raises the generation word the
// others poll. Counters only grow within a launch, so barrier j waits for
// the generation to reach j. Everything a phase hands to the next one is
// written with device-scope stores (through to where every XCD reads; the
// L2s of the XCDs are not coherent with each other), so a release needs
// only those stores to have completed, not a write-back of the whole L2
// (one per workgroup and barrier cost ~0.1 ms in all on MI355X); one
// acquire per workgroup then drops stale cached lines before the next
// phase reads. A wait gives up after 2^18 polls (each a
// device-scope load and a short sleep: well under a second) and raises the
// error word, so the kernel always ends.
struct GridSync {
  int* bar;
  int j = 0;
  __device__ __forceinline__ void sync() {
    ++j;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's device-scope stores are done
    __syncthreads();
    if (threadIdx.x == 0) {
      const int per_group = (int)gridDim.x >> 3;
      if (atomicAdd(bar + 32 * (blockIdx.x & 7), 1) == j * per_group - 1 &&
          atomicAdd(bar + kBarTop, 1) == j * 8 - 1)
        atomicMax(bar + kBarGen, j);
      int spins = 0;
      while (__hip_atomic_load(bar + kBarGen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < j) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins > (1 << 18)) {
          atomicMax(bar + kBarErr, j);
          break;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // drop stale cached lines
    }
    __syncthreads();
  }
};

// The work units of a batch: (expert, up to 8 of its slots), experts
// ascending, slots ascending within an expert; built from the routed ids by
// every workgroup (S <= 256: one slot per thread).
struct SmallPlan {
  int ids[kSmallMaxS];
  int rank[kSmallMaxS];    // position of the slot among its expert's slots
  int sorted[kSmallMaxS];  // slots by (expert, slot)
  int ue[kSmallMaxS];      // unit -> expert
  int upos[kSmallMaxS];    // unit -> its first position in sorted
  int ulen[kSmallMaxS];    // unit -> slots (1..8)
  int nunits;
};

__device__ __forceinline__ void small_plan(const int32_t* __restrict__ ids, int S, int E,
                                           SmallPlan& P) {
  const int s = threadIdx.x;
  const int e = s < S ? ids[s] : -1;
  if (s < S) P.ids[s] = e;
  __syncthreads();
  const bool valid = s < S && (unsigned)e < (unsigned)E;
  int rank = 0, below = 0, cnt = 0;
  if (valid) {
    for (int q = 0; q < S; ++q) {
      const int f = P.ids[q];
      rank += (f == e) & (q < s);
      cnt += f == e;
      below += (unsigned)f < (unsigned)e;  // slots of lower experts (never an invalid id)
    }
  }
  P.rank[s] = valid ? rank : -1;
  __syncthreads();
  const bool starts = valid && (rank & 7) == 0;
  if (valid) {
    int ubase = 0;  // units of lower experts
    for (int q = 0; q < S; ++q) {
      const int f = P.ids[q];
      ubase += ((unsigned)f < (unsigned)e) & ((P.rank[q] & 7) == 0);
    }
    const int pos = below + rank;
    P.sorted[pos] = s;
    if (starts) {
      const int u = ubase + (rank >> 3);
      P.ue[u] = e;
      P.upos[u] = pos;
      P.ulen[u] = min(8, cnt - rank);
    }
  }
  const int n = __syncthreads_count(starts);
  if (s == 0) P.nunits = n;
  __syncthreads();
}

// FC1 over (unit, tile) shares, each tile of 8 h columns K-sliced over the 4
// waves, or over (unit, quad) shares with one tile per wave, by the rule of
// the cold-only FC1 launches (so the results are the same bits).
// WT: device-scope stores (the reader is in the same kernel on another XCD).
template <bool FP8, bool WT>
__device__ __forceinline__ void small_fc1(const SmallArgs& a, const SmallPlan& P,
                                          f32x4* __restrict__ red) {
  const int ti = threadIdx.x & 7;
  const int S = a.T * a.k;
  const Fc1Args f{FP8 ? (const void*)a.xq : (const void*)a.x, a.xs, a.w1, a.w1s, nullptr,
                  nullptr, nullptr, a.H, a.I, a.k, S, 0, a.remap, a.h, nullptr, a.E};
  if (!sliced_fc1(!FP8, a.T)) {
    const int w = threadIdx.x >> 6, qpu = a.I >> 5;
    const Share sh = wg_share((long)P.nunits * qpu, a.remap);
    for (long qd = sh.q0; qd < sh.q1; ++qd) {
      const int u = (int)(qd / qpu), r = (int)(qd % qpu) * 4 + w;
      const int slot = ti < P.ulen[u] ? P.sorted[P.upos[u] + ti] : S;
      fc1_cold<FP8, cold_u<FP8, false>(), WT>(f, P.ue[u], r, slot);
    }
    return;
  }
  const int tpu = a.I >> 3;
  const Share sh = wg_share((long)P.nunits * tpu, a.remap);
  int j = 0;
  for (long t = sh.q0; t < sh.q1; ++t, ++j) {
    const int u = (int)(t / tpu), r = (int)(t % tpu);
    const int slot = ti < P.ulen[u] ? P.sorted[P.upos[u] + ti] : S;
    fc1_cold_sliced<FP8, cold_u<FP8, false>(), WT>(f, P.ue[u], r, slot, red, j);
  }
}

// FC2 over (unit, quad) shares: a quad is 4 tiles of 16 output rows.
template <bool FP8, bool WT>
__device__ __forceinline__ void small_fc2(const SmallArgs& a, const SmallPlan& P) {
  const int w = threadIdx.x >> 6, ti = threadIdx.x & 7;
  const int S = a.T * a.k;
  const Fc2Args f{FP8 ? (const void*)a.hq : (const void*)a.h, a.hs, a.w2, a.w2s, nullptr,
                  nullptr, nullptr, a.H, a.I, S, 0, a.remap, a.y, FP8 ? 0 : 1, nullptr, a.E};
  const int qpu = a.H >> 6;
  const Share sh = wg_share((long)P.nunits * qpu, a.remap);
  for (long qd = sh.q0; qd < sh.q1; ++qd) {
    const int u = (int)(qd / qpu), r = (int)(qd % qpu) * 4 + w;
    const int slot = ti < P.ulen[u] ? P.sorted[P.upos[u] + ti] : S;
    fc2_cold<FP8, cold_u<FP8, false>(), WT>(f, P.ue[u], r, slot);
  }
}

// The split form of the small path: FC1 and FC2 as launches of their own that
// each rebuild the plan from the routed ids (one launch per step and no
// alignment kernel: the routed ids are all they need).
template <bool FP8>
__global__ __launch_bounds__(256) void small_fc1_kernel(SmallArgs a) {
  __shared__ SmallPlan P;
  __shared__ f32x4 red[2 * kRedF4];
  small_plan(a.ids, a.T * a.k, a.E, P);
  small_fc1<FP8, false>(a, P, red);
}
template <bool FP8>
__global__ __launch_bounds__(256) void small_fc2_kernel(SmallArgs a) {
  __shared__ SmallPlan P;
  small_plan(a.ids, a.T * a.k, a.E, P);
  small_fc2<FP8, false>(a, P);
}

template <bool FP8, int VPL>
__global__ __launch_bounds__(256) void small_forward_kernel(SmallArgs a) {
  __shared__ SmallPlan P;
  __shared__ f32x4 red[2 * kRedF4];
  GridSync gs{a.bar};
  const int w = threadIdx.x >> 6;
  const int gw = blockIdx.x * 4 + w;  // global wave
  const int nw = gridDim.x * 4;
  const int S = a.T * a.k;
  // routing, and the x quantiser of the FP8 path
  if (gw < a.T) {
    float v[VPL];
    load_logits<VPL>(a.logits, gw, a.E, v);
    route_token<VPL, true>(v, gw, a.E, a.k, a.renorm, a.ids, a.wts, nullptr);
  } else if (FP8 && gw < 2 * a.T) {
    const int t = gw - a.T;
    quant_row<uint16_t, true>(a.x + (size_t)t * a.H, a.H, a.xq + (size_t)t * a.H, a.xs + t);
  }
  gs.sync();
  small_plan(a.ids, S, a.E, P);
  small_fc1<FP8, true>(a, P, red);
  gs.sync();
  if constexpr (FP8) {
    for (int r = gw; r < S; r += nw)
      quant_row<float, true>((const float*)a.h + (size_t)r * a.I, a.I, a.hq + (size_t)r * a.I,
                             a.hs + r);
    gs.sync();
  }
  small_fc2<FP8, true>(a, P);
  gs.sync();
  const long n8 = (long)a.T * (a.H >> 3);
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long)gridDim.x * 256) {
    if (FP8)
      combine8<float, uint16_t>((const float*)a.y, a.wts, a.ids, a.E, a.H, a.k, a.out, i);
    else
      combine8<uint16_t, uint16_t>((const uint16_t*)a.y, a.wts, a.ids, a.E, a.H, a.k, a.out, i);
  }
}

// -------------------------------------------------------- host side ---

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

FfnWorkspace ffn_workspace_layout(int T, int E, int H, int I, int k, int dtype) {
  FfnWorkspace L{};
  const size_t S = (size_t)T * k;
  size_t o = 0;
  auto put = [&](size_t& off, size_t& bytes, size_t n) {
    off = o;
    bytes = n;
    o = align_up(o + n, 256);
  };
  const size_t hbytes = dtype == MOE_DTYPE_BF16 ? 2 : 4;
  put(L.h_off, L.h_bytes, S * I * hbytes);
  if (dtype == MOE_DTYPE_FP8 || dtype == MOE_DTYPE_FP8_BLOCK) {
    // one scale per row (FP8) or per 128-element group of a row (block FP8)
    const size_t hg = dtype == MOE_DTYPE_FP8 ? 1 : (size_t)I / kBlk;
    const size_t xg = dtype == MOE_DTYPE_FP8 ? 1 : (size_t)H / kBlk;
    put(L.hq_off, L.hq_bytes, S * I);
    put(L.hs_off, L.hs_bytes, S * hg * 4);
    put(L.xq_off, L.xq_bytes, (size_t)T * H);
    put(L.xs_off, L.xs_bytes, (size_t)T * xg * 4);
  }
  put(L.y_off, L.y_bytes, S * H * (dtype == MOE_DTYPE_BF16 ? 2 : 4));
  put(L.q_off, L.q_bytes, S ? kQueueInts * sizeof(int) : 0);
  put(L.plan_off, L.plan_bytes, S && E > 0 ? gemm_plan_ints((int)S, E) * sizeof(int) : 0);
  L.total = o;
  return L;
}

// Resident-capacity grid of a persistent kernel on the current device,
// rounded down to a multiple of 8 (one share per XCD). Cached per device and
// kernel.
template <typename K>
static int persistent_grid(K kernel, int threads = 256) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  int& c = cache[{dev, (const void*)kernel}];
  if (c == 0) {
    int cus = 0, occ = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, 0) != hipSuccess ||
        occ < 1)
      occ = 1;
    c = cus * occ;
    c = c >= 8 ? (c / 8) * 8 : 8;
  }
  return c;
}

static int ilog2(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

// The stages a call runs: those named (all when none is), PREP with FC1
// unless the caller has run it already (MOE_FFN_PREPARED).
static unsigned stages(unsigned flags) {
  constexpr unsigned kAll =
      MOE_FFN_STAGE_PREP | MOE_FFN_STAGE_FC1 | MOE_FFN_STAGE_FC2 | MOE_FFN_STAGE_COMBINE;
  unsigned s = flags & kAll;
  if (!s) s = kAll;
  if ((s & MOE_FFN_STAGE_FC1) && !(flags & MOE_FFN_PREPARED)) s |= MOE_FFN_STAGE_PREP;
  return s;
}

static hipError_t launch_combine(const FfnProblem& p, const FfnWorkspace& L, int dtype,
                                 hipStream_t stream) {
  const void* y = (const char*)p.workspace + L.y_off;
  if (p.H % 8 == 0) {
    const long n = (long)p.T * (p.H / 8);
    const dim3 grid((unsigned)((n + 255) / 256));
    if (dtype == MOE_DTYPE_BF16)
      combine_kernel<uint16_t, uint16_t><<<grid, 256, 0, stream>>>(
          (const uint16_t*)y, p.topk_weights, p.topk_ids, p.E, p.T, p.H, p.k, (uint16_t*)p.out);
    else if (dtype == MOE_DTYPE_FP8)
      combine_kernel<float, uint16_t><<<grid, 256, 0, stream>>>(
          (const float*)y, p.topk_weights, p.topk_ids, p.E, p.T, p.H, p.k, (uint16_t*)p.out);
    else
      combine_kernel<float, float><<<grid, 256, 0, stream>>>(
          (const float*)y, p.topk_weights, p.topk_ids, p.E, p.T, p.H, p.k, (float*)p.out);
  } else {
    const long n = (long)p.T * p.H;
    combine_f32_scalar_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(
        (const float*)y, p.topk_weights, p.topk_ids, p.E, p.T, p.H, p.k, (float*)p.out);
  }
  return hipGetLastError();
}

// bf16 / fp8 FFN for H or I not a multiple of 128 (gen_fc1_kernel,
// gen_fc2_kernel), with the stages, workspace and combine of the paths below.
template <bool FP8>
static hipError_t launch_ffn_gen(const FfnProblem& p, hipStream_t stream) {
  const int dtype = FP8 ? MOE_DTYPE_FP8 : MOE_DTYPE_BF16;
  const FfnWorkspace L = ffn_workspace_layout(p.T, p.E, p.H, p.I, p.k, dtype);
  const unsigned st = stages(p.flags);
  const int S = p.T * p.k, log2m = ilog2(p.block_m);
  char* ws = (char*)p.workspace;
  void* h = ws + L.h_off;
  void* y = ws + L.y_off;
  uint8_t* hq = FP8 ? (uint8_t*)(ws + L.hq_off) : nullptr;
  float* hs = FP8 ? (float*)(ws + L.hs_off) : nullptr;
  uint8_t* xq = FP8 ? (uint8_t*)(ws + L.xq_off) : nullptr;
  float* xs = FP8 ? (float*)(ws + L.xs_off) : nullptr;
  constexpr int grid = 1024;
  hipError_t err;
  if (FP8 && (st & MOE_FFN_STAGE_PREP)) {
    launch_quant_rows<uint16_t>((const uint16_t*)p.x, p.T, p.H, xq, xs, stream);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_FC1) {
    Fc1Args a{FP8 ? (const void*)xq : p.x, xs, p.w1, p.w1_scale, p.sorted_ids, p.block_expert,
              p.num_padded, p.H, p.I, p.k, S, log2m, 0, h, nullptr, p.E};
    gen_fc1_kernel<FP8><<<grid, 256, 0, stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_FC2) {
    if (FP8) {
      launch_quant_rows<float>((const float*)h, S, p.I, hq, hs, stream);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    Fc2Args a{FP8 ? (const void*)hq : h, hs, p.w2, p.w2_scale, p.sorted_ids, p.block_expert,
              p.num_padded, p.H, p.I, S, log2m, 0, y, FP8 ? 0 : 1, nullptr, p.E};
    gen_fc2_kernel<FP8><<<grid, 256, 0, stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_COMBINE) return launch_combine(p, L, dtype, stream);
  return hipSuccess;
}

hipError_t launch_ffn_bf16(const FfnProblem& p, hipStream_t stream) {
  if (p.H % 128 != 0 || p.I % 128 != 0) return launch_ffn_gen<false>(p, stream);
  const FfnWorkspace L = ffn_workspace_layout(p.T, p.E, p.H, p.I, p.k, MOE_DTYPE_BF16);
  const unsigned st = stages(p.flags);
  const int remap = (p.flags & MOE_FFN_NO_XCD_REMAP) ? 0 : 1;
  const int S = p.T * p.k, log2m = ilog2(p.block_m);
  void* h = (char*)p.workspace + L.h_off;
  float* y = (float*)((char*)p.workspace + L.y_off);
  int* queue = (int*)((char*)p.workspace + L.q_off);  // FC1: [0, 8), FC2: [8, 16)
  int* plan = (int*)((char*)p.workspace + L.plan_off);
  hipError_t err;
  // prefill-sized blocks, on request: 256 x 256 tiles over token ranges
  if ((p.flags & MOE_FFN_RANGE_GEMM) && p.block_m >= 128 && gemm_supported(p.T, p.k, p.H, p.I)) {
    if (st & (MOE_FFN_STAGE_FC1 | MOE_FFN_STAGE_FC2)) {
      err = launch_gemm_plan(p.sorted_ids, p.block_expert, p.num_padded, S, p.E, log2m, plan,
                             queue, stream);
      if (err != hipSuccess) return err;
    }
    if (st & MOE_FFN_STAGE_FC1) {
      err = launch_gemm_fc1(p.x, p.w1, p.sorted_ids, plan, queue, p.H, p.I, p.k, S, remap, h,
                            stream);
      if (err != hipSuccess) return err;
    }
    if (st & MOE_FFN_STAGE_FC2) {
      err = launch_gemm_fc2(h, p.w2, p.sorted_ids, plan, queue + kQueues, p.H, p.I, S, remap, y,
                            stream);
      if (err != hipSuccess) return err;
    }
    if (st & MOE_FFN_STAGE_COMBINE) return launch_combine(p, L, MOE_DTYPE_BF16, stream);
    return hipSuccess;
  }
  const bool dense = p.block_m >= 128;  // prefill-sized blocks: grouped GEMM tiles
  const bool hot = p.T > 2 * kColdMax;  // see run_quads
  if ((dense || hot) && (st & MOE_FFN_STAGE_PREP)) {  // (FC2 without PREP: finish_queue)
    zero_counters_kernel<<<1, 64, 0, stream>>>(queue, kQueueInts);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_FC1) {
    Fc1Args a{p.x, nullptr, p.w1, nullptr, p.sorted_ids, p.block_expert, p.num_padded,
              p.H, p.I, p.k, S, log2m, remap, h, queue, p.E};
    if (dense)
      dense_fc1_kernel<false><<<persistent_grid(dense_fc1_kernel<false>, kDThreads), kDThreads, 0,
                                stream>>>(a);
    else if (hot)
      fc1_kernel<false, true><<<persistent_grid(fc1_kernel<false, true>), 256, 0, stream>>>(a);
    else
      fc1_sliced_kernel<false><<<persistent_grid(fc1_sliced_kernel<false>), 256, 0, stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_FC2) {
    Fc2Args a{h, nullptr, p.w2, nullptr, p.sorted_ids, p.block_expert, p.num_padded,
              p.H, p.I, S, log2m, remap, y, 1, queue + kQueues, p.E};
    if (dense)
      dense_fc2_kernel<false><<<persistent_grid(dense_fc2_kernel<false>, kDThreads), kDThreads, 0,
                                stream>>>(a);
    else if (hot)
      fc2_kernel<false, true><<<persistent_grid(fc2_kernel<false, true>), 256, 0, stream>>>(a);
    else
      fc2_kernel<false, false><<<persistent_grid(fc2_kernel<false, false>), 256, 0, stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_COMBINE) return launch_combine(p, L, MOE_DTYPE_BF16, stream);
  return hipSuccess;
}

hipError_t launch_ffn_fp8(const FfnProblem& p, hipStream_t stream) {
  if (p.H % 128 != 0 || p.I % 128 != 0) return launch_ffn_gen<true>(p, stream);
  const FfnWorkspace L = ffn_workspace_layout(p.T, p.E, p.H, p.I, p.k, MOE_DTYPE_FP8);
  const unsigned st = stages(p.flags);
  const int remap = (p.flags & MOE_FFN_NO_XCD_REMAP) ? 0 : 1;
  const int S = p.T * p.k, log2m = ilog2(p.block_m);
  char* ws = (char*)p.workspace;
  float* h = (float*)(ws + L.h_off);
  uint8_t* hq = (uint8_t*)(ws + L.hq_off);
  float* hs = (float*)(ws + L.hs_off);
  uint8_t* xq = (uint8_t*)(ws + L.xq_off);
  float* xs = (float*)(ws + L.xs_off);
  float* y = (float*)(ws + L.y_off);
  int* queue = (int*)(ws + L.q_off);    // FC1: [0, 8), FC2: [8, 16)
  const bool hot = p.T > 2 * kColdMax;  // see run_quads
  // prefill-sized blocks: the grouped-GEMM tiles on fp8 MFMA (two 128-code
  // chunks of K at least)
  const bool dense = p.block_m >= 128 && p.H >= 256 && p.I >= 256;
  hipError_t err;
  if ((dense || hot) && (st & MOE_FFN_STAGE_PREP)) {  // (FC2 without PREP: finish_queue)
    zero_counters_kernel<<<1, 64, 0, stream>>>(queue, kQueueInts);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_PREP) {
    launch_quant_rows<uint16_t>((const uint16_t*)p.x, p.T, p.H, xq, xs, stream);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_FC1) {
    Fc1Args a{xq, xs, p.w1, p.w1_scale, p.sorted_ids, p.block_expert, p.num_padded,
              p.H, p.I, p.k, S, log2m, remap, h, queue, p.E};
    if (dense)
      dense_fc1_kernel<true><<<persistent_grid(dense_fc1_kernel<true>, kDThreads), kDThreads, 0,
                               stream>>>(a);
    else if (hot)
      fc1_kernel<true, true><<<persistent_grid(fc1_kernel<true, true>), 256, 0, stream>>>(a);
    else if (sliced_fc1(false, p.T))
      fc1_sliced_kernel<true><<<persistent_grid(fc1_sliced_kernel<true>), 256, 0, stream>>>(a);
    else
      fc1_kernel<true, false><<<persistent_grid(fc1_kernel<true, false>), 256, 0, stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_FC2) {
    if (dense)  // the grouped-GEMM tiles leave h in bf16
      launch_quant_rows<uint16_t>((const uint16_t*)h, S, p.I, hq, hs, stream);
    else
      launch_quant_rows<float>(h, S, p.I, hq, hs, stream);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    // the grouped-GEMM tiles write y in bf16 (as the bf16 path does: at
    // prefill sizes y is the largest intermediate), the streaming kernels in f32
    Fc2Args a{hq, hs, p.w2, p.w2_scale, p.sorted_ids, p.block_expert, p.num_padded,
              p.H, p.I, S, log2m, remap, y, dense ? 1 : 0, queue + kQueues, p.E};
    if (dense)
      dense_fc2_kernel<true><<<persistent_grid(dense_fc2_kernel<true>, kDThreads), kDThreads, 0,
                               stream>>>(a);
    else if (hot)
      fc2_kernel<true, true><<<persistent_grid(fc2_kernel<true, true>), 256, 0, stream>>>(a);
    else
      fc2_kernel<true, false><<<persistent_grid(fc2_kernel<true, false>), 256, 0, stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_COMBINE)
    return launch_combine(p, L, dense ? MOE_DTYPE_BF16 : MOE_DTYPE_FP8, stream);
  return hipSuccess;
}

hipError_t launch_ffn_w8a16(const FfnProblem& p, hipStream_t stream) {
  const FfnWorkspace L = ffn_workspace_layout(p.T, p.E, p.H, p.I, p.k, MOE_DTYPE_BF16);
  const unsigned st = stages(p.flags);
  const int remap = (p.flags & MOE_FFN_NO_XCD_REMAP) ? 0 : 1;
  const int S = p.T * p.k, log2m = ilog2(p.block_m);
  void* h = (char*)p.workspace + L.h_off;
  void* y = (char*)p.workspace + L.y_off;
  hipError_t err;
  if (st & MOE_FFN_STAGE_FC1) {
    Fc1Args a{p.x, nullptr, p.w1, p.w1_scale, p.sorted_ids, p.block_expert, p.num_padded,
              p.H, p.I, p.k, S, log2m, remap, h, nullptr, p.E};
    if (sliced_fc1(false, p.T))
      fc1_w8a16_sliced_kernel<<<persistent_grid(fc1_w8a16_sliced_kernel), 256, 0, stream>>>(a);
    else
      fc1_w8a16_kernel<<<persistent_grid(fc1_w8a16_kernel), 256, 0, stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_FC2) {
    Fc2Args a{h, nullptr, p.w2, p.w2_scale, p.sorted_ids, p.block_expert, p.num_padded,
              p.H, p.I, S, log2m, remap, y, 1, nullptr, p.E};
    fc2_w8a16_kernel<<<persistent_grid(fc2_w8a16_kernel), 256, 0, stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_COMBINE) return launch_combine(p, L, MOE_DTYPE_BF16, stream);
  return hipSuccess;
}

hipError_t launch_ffn_fp8_block(const FfnProblem& p, hipStream_t stream) {
  const FfnWorkspace L = ffn_workspace_layout(p.T, p.E, p.H, p.I, p.k, MOE_DTYPE_FP8_BLOCK);
  const unsigned st = stages(p.flags);
  const int remap = (p.flags & MOE_FFN_NO_XCD_REMAP) ? 0 : 1;
  const int S = p.T * p.k, log2m = ilog2(p.block_m);
  char* ws = (char*)p.workspace;
  float* h = (float*)(ws + L.h_off);
  uint8_t* hq = (uint8_t*)(ws + L.hq_off);
  float* hs = (float*)(ws + L.hs_off);
  uint8_t* xq = (uint8_t*)(ws + L.xq_off);
  float* xs = (float*)(ws + L.xs_off);
  float* y = (float*)(ws + L.y_off);
  hipError_t err;
  if (st & MOE_FFN_STAGE_PREP) {
    const long ng = (long)p.T * (p.H / kBlk);
    quant_groups_kernel<uint16_t><<<(unsigned)((ng + 15) / 16), 256, 0, stream>>>(
        (const uint16_t*)p.x, p.T, p.H, xq, xs);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_FC1) {
    Fc1Args a{xq, xs, p.w1, p.w1_scale, p.sorted_ids, p.block_expert, p.num_padded,
              p.H, p.I, p.k, S, log2m, remap, h, nullptr, p.E};
    if (sliced_fc1(false, p.T))
      fc1_blk_sliced_kernel<<<persistent_grid(fc1_blk_sliced_kernel), 256, 0, stream>>>(a);
    else
      fc1_blk_kernel<<<persistent_grid(fc1_blk_kernel), 256, 0, stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_FC2) {
    const long ng = (long)S * (p.I / kBlk);
    quant_groups_kernel<float><<<(unsigned)((ng + 15) / 16), 256, 0, stream>>>(h, S, p.I, hq, hs);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    Fc2Args a{hq, hs, p.w2, p.w2_scale, p.sorted_ids, p.block_expert, p.num_padded,
              p.H, p.I, S, log2m, remap, y, 0, nullptr, p.E};
    fc2_blk_kernel<<<persistent_grid(fc2_blk_kernel), 256, 0, stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_COMBINE) return launch_combine(p, L, MOE_DTYPE_FP8, stream);
  return hipSuccess;
}

static_assert(kSmallKernelTokens == kSmallMaxT && kSmallExperts == kSmallMaxE &&
              kSmallKernelSlots == kSmallMaxS, "small-path limits");

// Carve-up of the small-batch forward's workspace beyond the small kernels:
// the alignment outputs, then the FFN workspace.
struct SmallAligned {
  int block_m;
  size_t cap, be_off, np_off, ffn_off, total;
};
static SmallAligned small_aligned_layout(int T, int E, int H, int I, int k, int dtype) {
  SmallAligned L;
  L.block_m = default_block_m(T, E, k);
  L.cap = align_capacity((long)T * k, E, L.block_m);
  L.be_off = align_up(L.cap * sizeof(int32_t), 256);
  L.np_off = L.be_off + align_up(L.cap / L.block_m * sizeof(int32_t), 256);
  L.ffn_off = L.np_off + 256;
  L.total = L.ffn_off + ffn_workspace_layout(T, E, H, I, k, dtype).total;
  return L;
}

size_t small_workspace_bytes(int T, int E, int H, int I, int k, int dtype) {
  if (!small_kernels(T, k)) return small_aligned_layout(T, E, H, I, k, dtype).total;
  return align_up(ffn_workspace_layout(T, 0, H, I, k, dtype).total, 256) + kBarInts * sizeof(int);
}

template <bool FP8>
static hipError_t launch_small(const SmallProblem& p, const SmallArgs& a, hipStream_t stream) {
  void* args[] = {(void*)&a};
  auto go = [&](auto kernel) {
    const int grid = persistent_grid(kernel);
    return hipLaunchCooperativeKernel(kernel, dim3(grid), dim3(256), args, 0, stream);
  };
  if (p.E <= 64) return go(small_forward_kernel<FP8, 1>);
  if (p.E <= 256) return go(small_forward_kernel<FP8, 4>);
  return go(small_forward_kernel<FP8, 16>);
}

// The split small path: route, (fp8: quantise x), FC1, (fp8: quantise h), FC2,
// combine, each its own launch; FC1 and FC2 plan from the routed ids.
template <bool FP8>
static hipError_t launch_small_split(const SmallProblem& p, const SmallArgs& a,
                                     hipStream_t stream) {
  hipError_t err;
  if ((err = launch_route_topk(p.logits, p.T, p.E, p.k, p.renorm, p.ids, p.wts, stream)) !=
      hipSuccess)
    return err;
  const int S = p.T * p.k;
  if (FP8) {
    launch_quant_rows<uint16_t>(a.x, p.T, p.H, a.xq, a.xs, stream);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  small_fc1_kernel<FP8><<<persistent_grid(small_fc1_kernel<FP8>), 256, 0, stream>>>(a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (FP8) {
    launch_quant_rows<float>((const float*)a.h, S, p.I, a.hq, a.hs, stream);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  small_fc2_kernel<FP8><<<persistent_grid(small_fc2_kernel<FP8>), 256, 0, stream>>>(a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const long n8 = (long)p.T * (p.H / 8);
  const dim3 grid((unsigned)((n8 + 255) / 256));
  if (FP8)
    combine_kernel<float, uint16_t><<<grid, 256, 0, stream>>>(
        (const float*)a.y, p.wts, p.ids, p.E, p.T, p.H, p.k, (uint16_t*)p.out);
  else
    combine_kernel<uint16_t, uint16_t><<<grid, 256, 0, stream>>>(
        (const uint16_t*)a.y, p.wts, p.ids, p.E, p.T, p.H, p.k, (uint16_t*)p.out);
  return hipGetLastError();
}

// Batches beyond the small kernels: routing, alignment at the default block
// size and the FFN launchers, in the forward's own workspace (the same kernels
// and results as the separate calls).
static hipError_t launch_small_aligned(const SmallProblem& p, hipStream_t stream) {
  const SmallAligned L = small_aligned_layout(p.T, p.E, p.H, p.I, p.k, p.dtype);
  char* ws = (char*)p.workspace;
  int32_t* sorted_ids = (int32_t*)ws;
  int32_t* block_expert = (int32_t*)(ws + L.be_off);
  int32_t* num_padded = (int32_t*)(ws + L.np_off);
  const int S = p.T * p.k;
  hipError_t err;
  if ((err = launch_route_topk(p.logits, p.T, p.E, p.k, p.renorm, p.ids, p.wts, stream)) !=
      hipSuccess)
    return err;
  if ((err = launch_align(p.ids, S, p.E, L.block_m, (int)L.cap, sorted_ids, block_expert,
                          num_padded, stream)) != hipSuccess)
    return err;
  const bool fp8 = p.dtype == MOE_DTYPE_FP8;
  const FfnProblem f{p.x, p.w1, fp8 ? p.w1_scale : nullptr, p.w2, fp8 ? p.w2_scale : nullptr,
                     p.ids, p.wts, sorted_ids, block_expert, num_padded,
                     p.T, p.E, p.H, p.I, p.k, L.block_m, p.flags & MOE_FFN_NO_XCD_REMAP,
                     ws + L.ffn_off, p.out};
  return fp8 ? launch_ffn_fp8(f, stream) : launch_ffn_bf16(f, stream);
}

hipError_t launch_forward_small(const SmallProblem& p, hipStream_t stream) {
  if (!small_kernels(p.T, p.k)) return launch_small_aligned(p, stream);
  const bool fp8 = p.dtype == MOE_DTYPE_FP8;
  const FfnWorkspace L = ffn_workspace_layout(p.T, 0, p.H, p.I, p.k, p.dtype);
  char* ws = (char*)p.workspace;
  int* bar = (int*)(ws + align_up(L.total, 256));
  SmallArgs a{p.logits, (const uint16_t*)p.x, p.w1, p.w1_scale, p.w2, p.w2_scale,
              p.T, p.E, p.H, p.I, p.k, p.renorm, (p.flags & MOE_FFN_NO_XCD_REMAP) ? 0 : 1,
              p.ids, p.wts,
              fp8 ? (uint8_t*)(ws + L.xq_off) : nullptr, fp8 ? (float*)(ws + L.xs_off) : nullptr,
              ws + L.h_off,
              fp8 ? (uint8_t*)(ws + L.hq_off) : nullptr, fp8 ? (float*)(ws + L.hs_off) : nullptr,
              ws + L.y_off, (uint16_t*)p.out, bar};
  if (!(p.flags & MOE_FORWARD_ONE_KERNEL))
    return fp8 ? launch_small_split<true>(p, a, stream) : launch_small_split<false>(p, a, stream);
  zero_counters_kernel<<<1, 256, 0, stream>>>(bar, kBarInts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return fp8 ? launch_small<true>(p, a, stream) : launch_small<false>(p, a, stream);
}

// Scratch of the allocation-free small-batch forward: one copy of this array
// per GPU, zero at load, held until the process ends. In host code its name
// is only a stand-in: kernels get the device address hipGetSymbolAddress
// returns for the current device, fetched once per device and kept. Every
// call on a GPU reuses the same bytes; whatever must start at zero (the
// one-kernel mode's barrier words) is cleared by a kernel in each call.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* a = nullptr;
    err = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (a == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_ffn_f32(const FfnProblem& p, hipStream_t stream) {
  const FfnWorkspace L = ffn_workspace_layout(p.T, p.E, p.H, p.I, p.k, MOE_DTYPE_F32);
  const unsigned st = stages(p.flags);
  const int S = p.T * p.k, log2m = ilog2(p.block_m);
  float* h = (float*)((char*)p.workspace + L.h_off);
  float* y = (float*)((char*)p.workspace + L.y_off);
  hipError_t err;
  const int grid = 1024;
  if (st & MOE_FFN_STAGE_FC1) {
    fc1_f32_kernel<<<grid, 256, 0, stream>>>((const float*)p.x, (const float*)p.w1,
                                             p.sorted_ids, p.block_expert, p.num_padded, p.E,
                                             p.H, p.I, p.k, S, log2m, h);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_FC2) {
    fc2_f32_kernel<<<grid, 256, 0, stream>>>(h, (const float*)p.w2, p.sorted_ids,
                                             p.block_expert, p.num_padded, p.E, p.H, p.I, S,
                                             log2m, y);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_COMBINE) return launch_combine(p, L, MOE_DTYPE_F32, stream);
  return hipSuccess;
}

}  // namespace moe
