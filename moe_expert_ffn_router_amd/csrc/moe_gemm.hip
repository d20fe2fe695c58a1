// Grouped GEMM of the expert FFN for prefill-sized batches: FC1 (gate|up) +
// SiLU-and-mul and FC2, bf16 operands, fp32 accumulation, on gfx950's matrix
// cores.
//
// Pages: "vLLM SM architecture adaptation", sections 4.3 and 9: one fused
// kernel runs the MoE layer over all experts as a grouped GEMM once tokens per
// expert make it a real contraction; "vLLM support for NVIDIA Vera Rubin
// NVL72", section "Locality domain": FC1 and FC2 are the expert projections;
// V100 fork article, "wall 2": silu_and_mul between FC1 and FC2.
//
// Design (MI355X, one workgroup per CU). A unit is (token range, 256-row
// weight tile): a token range is up to 256 consecutive tokens of one expert's
// run in the aligned list (an expert with m tokens is cut into ceil(m/256)
// ranges of equal size, so no unit is a sliver), and its 256 x 256 output tile
// is owned by one workgroup of 4 waves, one per SIMD. Wave (wr, wc) computes
// 128 weight rows x half of the range's 16-token groups (8 x 8 MFMA
// 16x16x32 tiles, 256 fp32 accumulators held in AGPRs), so every byte read
// from LDS feeds 8 MFMAs. Waves 0-1 stage the weight tile into a 5-deep LDS
// ring and waves 2-3 the token tile into a 4-deep ring, 32 k-elements (64
// bytes of every row) per stage, with raw buffer loads straight into LDS;
// each wave reads the next k-step's fragments while its MFMAs run on the
// current ones. Units come from 8 per-XCD queues over the list ordered
// (expert, row tile, range), so the ranges of one expert sharing a weight
// tile, and the row tiles sharing a token range, run side by side on one XCD
// and meet in its L2.
#include "moe_common.h"
#include "moe_launch.h"

#include <map>
#include <mutex>

namespace moe {
namespace gemm {

constexpr int kRows = 256;                    // weight rows per unit
constexpr int kTok = 256;                     // tokens per range (at most)
constexpr int kThreads = 256;                 // 4 waves, one per SIMD
constexpr int kChunk = 64;                    // bytes of K per stage = 32 bf16 = one MFMA k-step
constexpr int kAStages = 5;                   // weight ring: loads issued 4 k-steps ahead
constexpr int kBStages = 4;                   // token ring: 3 k-steps ahead
constexpr int kTile = kRows * kChunk;         // 16 KB: one operand, one stage
constexpr int kLdsB = kAStages * kTile;       // token ring after the weight ring
constexpr int kLdsMisc = kLdsB + kBStages * kTile;  // 144 KB: mailbox word
constexpr int kLdsTok = kLdsMisc + 64;        // token slots of the current and next range
constexpr int kLds = kLdsTok + 2 * kTok * 4;
constexpr int kQueues = 8;

typedef __attribute__((address_space(3))) void* lds_ptr_t;
// Word 3 of a raw buffer resource on gfx9-family chips: 32-bit data format,
// no swizzle, no stride.
constexpr int kRsrcWord3 = 0x00020000;
// A buffer offset past any buffer here (all are under 2 GiB): the load
// returns zeros and reads no memory.
constexpr uint32_t kOOB = 0xFFFFFFF0u;

// ------------------------------------------------------------ the plan ---
// Token ranges of the aligned list, written by plan_kernel into the
// workspace: word 0 = number of ranges R, then per range (expert, first
// position in sorted_ids, tokens, first range of the expert | ranges of the
// expert << 20). An expert's tokens are the valid prefix
// of its run of blocks; expert e with m tokens gets J = ceil(m/256) ranges,
// range j covering tokens [j*m/J, (j+1)*m/J).

__device__ __forceinline__ int num_blocks(const int32_t* __restrict__ num_padded, int S, int E,
                                          int log2m) {
  const long M = 1L << log2m;
  const long cap = (S + (long)min(E, S) * (M - 1) + M - 1) >> log2m;
  const long nb = (long)max(num_padded[0], 0) >> log2m;
  return (int)min(nb, cap);
}

// First block in [0, nb) whose expert is >= e (block_expert is non-decreasing).
__device__ __forceinline__ int lower_bound(const int32_t* __restrict__ be, int nb, int e) {
  int lo = 0, hi = nb;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (be[mid] < e) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ sorted_ids,
                                                    const int32_t* __restrict__ block_expert,
                                                    const int32_t* __restrict__ num_padded,
                                                    int S, int E, int log2m,
                                                    int* __restrict__ plan, int max_ranges,
                                                    int* __restrict__ queues) {
  __shared__ int scan[1024];
  const int t = threadIdx.x;
  if (t < 2 * kQueues) queues[t] = 0;
  const int nb = num_blocks(num_padded, S, E, log2m);
  const int M = 1 << log2m;
  int total = 0;
  for (int e0 = 0; e0 < E; e0 += 1024) {  // E <= 1024: one pass
    const int e = e0 + t;
    int pos = 0, m = 0, J = 0;
    if (e < E) {
      const int lo = lower_bound(block_expert, nb, e);
      const int hi = lower_bound(block_expert, nb, e + 1);
      if (hi > lo) {
        // tokens of the last block: its valid entries form a prefix
        const int32_t* last = sorted_ids + (size_t)(hi - 1) * M;
        int a = 0, b = M;
        while (a < b) {
          const int mid = (a + b) >> 1;
          if ((unsigned)last[mid] < (unsigned)S) a = mid + 1;
          else b = mid;
        }
        pos = lo * M;
        m = (hi - 1 - lo) * M + a;
        J = (m + kTok - 1) / kTok;
      }
    }
    // exclusive scan of J over the workgroup (Hillis-Steele in LDS)
    scan[t] = J;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      const int v = t >= d ? scan[t - d] : 0;
      __syncthreads();
      scan[t] += v;
      __syncthreads();
    }
    const int base = total + scan[t] - J;
    // (the region holds every range of a consistent alignment; the clamp only
    // keeps a corrupt one inside it)
    for (int j = 0; j < J && base + j < max_ranges; ++j) {
      const int a = (int)((long)j * m / J), b = (int)((long)(j + 1) * m / J);
      int4* r = (int4*)(plan + 4) + base + j;
      *r = int4{e, pos + a, b - a, base | (J << 20)};
    }
    total += scan[1023];
    __syncthreads();
  }
  if (t == 0) plan[0] = min(total, max_ranges);
}

// ------------------------------------------------------------- staging ---
// LDS rows are 64 bytes (4 columns of 16 bytes); column c of row r is stored
// at column c ^ ((r >> 2) & 3), so the fragment reads (16 consecutive rows,
// one column) and their 8- or 16-lane phases hit distinct banks. One
// direct-to-LDS load of a wave writes 1 KB in lane order: lane l fills
// physical column l & 3 of row l >> 2 of a 16-row group, so it loads logical
// column (l & 3) ^ (l >> 4) of its row.

__device__ __forceinline__ int stage_col() {
  const int l = threadIdx.x & 63;
  return ((l & 3) ^ (l >> 4)) * 16;
}
// LDS byte offset of this lane's fragment in a 16-row tile: row l & 15,
// logical column l >> 4.
__device__ __forceinline__ int frag_off() {
  const int l = threadIdx.x & 63;
  return (l & 15) * kChunk + (((l >> 4) ^ ((l >> 2) & 3)) << 4);
}

// A value the compiler may not see is the same in every lane of the wave.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// s_waitcnt vmcnt(VM) lgkmcnt(LGKM) (expcnt never waited); 15 = no LDS wait.
template <int VM, int LGKM>
__device__ __forceinline__ void wait_cnt() {
  static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "waitcnt");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (0x7 << 4) | (LGKM << 8));
}

// Workgroup barrier of the staging ring: only a compiler fence around
// s_barrier (no wait for loads still in flight for later stages); the waits
// that make the barrier meaningful are explicit before it.
__device__ __forceinline__ void ring_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

struct GemmArgs {
  const uint8_t* a;     // weights: FC1 w1 [E, 2I, H], FC2 w2 [E, H, I] (bf16)
  const uint8_t* b;     // activations: FC1 x [T, H], FC2 h [S, I] (bf16)
  const int32_t* sorted_ids;
  const int* plan;      // written by plan_kernel
  int* queue;           // kQueues counters, zero at launch
  uint16_t* out;        // FC1: h [S, I] bf16; FC2: y [S, H] bf16
  int K;                // reduction length: H (FC1) or I (FC2)
  int rows;             // weight rows per expert: 2I (FC1) or H (FC2)
  int n_rt;             // 256-row tiles per expert
  int I, H, k, S;
  int remap;
};

// Staging roles: waves 0 and 1 stage the weight tile (128 rows each), waves 2
// and 3 the token tile (128 rows each), 8 loads of 1 KB per wave and k-step
// (rows past the range's tokens stage zeros).
// A wave's vmcnt then counts only its own operand's loads, so the deeper
// weight ring is never held up by the token ring's waits.
constexpr int kLoads = 8;

// Token slots of a range live in LDS (one of two tables, by unit parity):
// entry t is the slot of the range's token t (0 for t >= m, an entry never
// used). load_tok copies them from sorted_ids straight into LDS, one
// direct-to-LDS load per wave (64 entries), so no register waits for them;
// the load counts in the wave's vmcnt like a staging load.
__device__ __forceinline__ void load_tok(const GemmArgs& p, const int4& rg, uint8_t* lds,
                                         int buf) {
  const int w = uni(threadIdx.x >> 6), t = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.sorted_ids, (short)0, 0x7FFFFFF0, kRsrcWord3);
  const uint32_t off = t < rg.z ? (uint32_t)(rg.y + t) * 4u : kOOB;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rs, (lds_ptr_t)(lds + kLdsTok + (buf * kTok + 64 * w) * 4), 4, (int)off, 0, 0, 0);
}
__device__ __forceinline__ int tok(const uint8_t* lds, int buf, int t) {
  return ((const int*)(lds + kLdsTok))[buf * kTok + t];
}

// One unit as this lane needs it: the 8 rows it stages, as 32-bit byte
// offsets (already including its column) into a wave-uniform buffer (the
// expert's weight matrix or the activations, `bytes` long), and the
// wave-uniform shape of the range. Staging goes through buffer loads, whose
// range check returns zeros for an offset past the buffer without touching
// memory: rows that are staged but never used (tokens past the range's,
// weight rows past H) get the offset kOOB and cost no HBM traffic.
struct Unit {
  const uint8_t* base;
  uint32_t bytes;
  uint32_t off[8];
  int pos, m, r, j0, nj;
  int nk;  // k-steps of the unit
};

__device__ __forceinline__ const uint8_t* uni_ptr(const uint8_t* v) {
  const uint64_t a = (uint64_t)v;
  return (const uint8_t*)(((uint64_t)(uint32_t)uni((int)(a >> 32)) << 32) |
                          (uint32_t)uni((int)(uint32_t)a));
}

// Unit u of the list ordered (expert, 256-row tile, range): its range entry
// and row tile. Two dependent reads of the plan.
__device__ __forceinline__ int first_range_unit(const GemmArgs& p, int u) {
  return u / p.n_rt;  // some range of the unit's expert
}
__device__ __forceinline__ int unit_range(const GemmArgs& p, int u, const int4& some, int& r) {
  const int R0 = some.w & 0xFFFFF, J = max(some.w >> 20, 1);
  const int v = u - R0 * p.n_rt;
  r = v / J;
  return R0 + v % J;
}
// The plan is read through the constant address space (it is not written
// while the kernel runs), so its wave-uniform reads are scalar loads.
typedef const __attribute__((address_space(4))) int plan_int;
__device__ __forceinline__ int4 plan_entry(const GemmArgs& p, int rho) {
  plan_int* q = (plan_int*)(p.plan + 4 + 4 * (size_t)rho);
  return int4{q[0], q[1], q[2], q[3]};
}

template <bool FC1>
__device__ __forceinline__ void make_unit(const GemmArgs& p, const int4& rg, int r,
                                          const uint8_t* lds, int buf, Unit& U) {
  U.pos = uni(rg.y);
  U.m = uni(rg.z);
  U.r = uni(r);
  U.nk = uni(p.K / 32);
  const int e = uni(rg.x);
  const int w = uni(threadIdx.x >> 6), l = threadIdx.x & 63;
  const int col = stage_col();
  const uint32_t rowb = (uint32_t)p.K * 2;
  if (w < 2) {
    U.base = uni_ptr(p.a + (size_t)e * p.rows * rowb);
    U.bytes = uni((int)((uint32_t)p.rows * rowb));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rho = 128 * w + 16 * i + (l >> 2);  // unit row 0..255
      int wrow;
      if (FC1) {  // 16-row MFMA tiles of 8 gate rows + the matching 8 up rows
        const int tau = rho >> 4, wi = rho & 15;
        wrow = wi < 8 ? r * 128 + tau * 8 + wi : p.I + r * 128 + tau * 8 + wi - 8;
      } else {
        wrow = r * kRows + rho;  // rows past H: zeros, never stored
      }
      U.off[i] = wrow < p.rows ? (uint32_t)wrow * rowb + col : kOOB;
    }
  } else {
    U.base = uni_ptr(p.b);
    U.bytes = uni((int)((uint32_t)(FC1 ? p.S / p.k : p.S) * rowb));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = 128 * (w - 2) + 16 * i + (l >> 2);
      const int s = tok(lds, buf, t);
      const uint32_t row = FC1 ? (uint32_t)(s / p.k) : (uint32_t)s;
      // tokens past the range's (and a slot past S, which only a corrupt
      // alignment holds) stage zeros
      U.off[i] = t < U.m && (unsigned)s < (unsigned)p.S ? row * rowb + col : kOOB;
    }
  }
  const int G = (U.m + 15) >> 4;  // 16-token groups holding tokens
  const int G0 = (G + 1) >> 1;
  const int wc = w >> 1;
  U.j0 = uni(wc ? G0 : 0);
  U.nj = uni(wc ? G - G0 : G0);
}

// This wave's 8 staging loads of k-step c into ring slot q of its operand.
// The buffer starts at k-step c's column, so the range check covers every
// byte a load reads. A k-step past the unit's last is issued against an
// empty buffer: it loads zeros and reads no memory, which keeps the count of
// loads in flight the same at every k-step (so are the waits).
__device__ __forceinline__ void issue(const Unit& U, uint8_t* lds, int q, int c) {
  const int w = uni(threadIdx.x >> 6);
  const int nrec = c < U.nk ? (int)(U.bytes - (uint32_t)c * kChunk) : 0;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(U.base + (size_t)c * kChunk), (short)0, nrec, kRsrcWord3);
  uint8_t* t = lds + (w < 2 ? q * kTile + (128 * w) * kChunk
                            : kLdsB + q * kTile + (128 * (w - 2)) * kChunk);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(t + 16 * i * kChunk), 16,
                                             (int)U.off[i], 0, 0, 0);
}

// Fragments of one k-step: this wave's 8 weight tiles and 8 token groups.
struct Frags {
  bf16x8 a[8], b[8];
};

__device__ __forceinline__ void read_frags(Frags& f, const uint8_t* lds, int qa, int qb, int wr,
                                           int j0) {
  const uint8_t* pa = lds + qa * kTile + (128 * wr) * kChunk + frag_off();
  const uint8_t* pb = lds + kLdsB + qb * kTile + (16 * j0) * kChunk + frag_off();
#pragma unroll
  for (int i = 0; i < 8; ++i) f.a[i] = *(const bf16x8*)(pa + 16 * i * kChunk);
#pragma unroll
  for (int j = 0; j < 8; ++j) f.b[j] = *(const bf16x8*)(pb + 16 * j * kChunk);
}

// The MFMAs of one k-step on fragments `f`; with READ, the next k-step's
// fragments (ring slot QN) are read into `g` meanwhile, one LDS read every
// few MFMAs, all in the first half of the step so that they have landed by
// its end.
template <int NJ, bool READ>
__device__ __forceinline__ void mma(f32x4 (&acc)[8][8], const Frags& f, Frags& g,
                                    const uint8_t* lds, int qa, int qb, int wr, int j0) {
  if constexpr (READ) read_frags(g, lds, qa, qb, wr, j0);
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i][j] = mfma_bf16(f.a[i], f.b[j], acc[i][j]);
  if constexpr (READ && NJ > 0) {
    constexpr int kN = 8 * NJ;                       // MFMAs of the step
    constexpr int kM = kN / 32 > 0 ? kN / 32 : 1;    // MFMAs per group
    constexpr int kG = kN / kM < 16 ? kN / kM : 16;  // groups (at most one per read)
    constexpr int kR = (16 + kG - 1) / kG;           // LDS reads per group
#pragma unroll
    for (int s = 0; s < kG; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x100, kR, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, kM, 0);  // MFMA
    }
  }
}

// ----------------------------------------------------------- scheduler ---
// Units are cut into kQueues contiguous shares, one per XCD; a workgroup
// takes the next unit of its own XCD's share and, once that is drained, helps
// the others. Which workgroup computes a unit never changes the result.
__device__ __forceinline__ int hw_xcc_id() {
  int v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & (kQueues - 1);
}

struct Sched {
  int* cnt;
  int units, per, q0, qi, t;
  __device__ Sched(int* c, int n, int remap)
      : cnt(c), units(n), per((n + kQueues - 1) / kQueues), q0(remap ? hw_xcc_id() : 0), qi(0),
        t(0) {}
  __device__ int lo(int i) const { return ((q0 + i) & (kQueues - 1)) * per; }
  __device__ int size(int i) const { return min(units, lo(i) + per) - lo(i); }
  // Thread 0 only. request() takes a ticket from the current queue without
  // looking at it (the atomic's latency can hide under other work);
  // resolve() turns it into a unit, moving on to the next queue (and waiting
  // for its ticket) when the current one is drained; -1 once all are.
  __device__ void request() {
    while (qi < kQueues && size(qi) <= 0) ++qi;
    if (qi < kQueues)
      t = __hip_atomic_fetch_add(
          (__attribute__((address_space(1))) int*)(cnt + ((q0 + qi) & (kQueues - 1))), 1,
          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ int resolve() {
    while (qi < kQueues) {
      if (t < size(qi)) return lo(qi) + t;
      ++qi;
      request();
    }
    return -1;
  }
};

// Scheduling state carried through a unit's K loop: the next unit is picked
// by thread 0 before the loop (an atomic whose latency the loop hides),
// published through LDS at k-step kPub and read by every wave after the next
// barrier; its range entry and token slots, and this unit's output slots,
// are fetched a few k-steps later, so none of them waits at the unit's end.
struct Lookahead {
  int nxt;  // every thread, from k-step kPub + 1 on: the next unit (or -1)
  int4 nrg; // its range entry
  int nr;   // its row tile
};
constexpr int kPub = 3;               // used when a unit has at least kHookSteps k-steps
constexpr int kHookSteps = kPub + 10;  // the hooks (up to k-step kPub + 5) and the
                                       // waits covering their loads

template <bool FC1>
__device__ __forceinline__ void lookahead(const GemmArgs& p, Lookahead& L, Sched& sched,
                                          uint8_t* lds, int* mail, int nbuf, int s) {
  if (s == kPub) {
    if (threadIdx.x == 0) mail[0] = sched.resolve();
  } else if (s == kPub + 1) {
    L.nxt = uni(mail[0]);
    if (L.nxt >= 0) L.nrg = plan_entry(p, first_range_unit(p, L.nxt));
  } else if (s == kPub + 3) {
    if (L.nxt >= 0) L.nrg = plan_entry(p, unit_range(p, L.nxt, L.nrg, L.nr));
  } else if (s == kPub + 5) {
    // lands within 4 k-steps: the waits of k-step kPub + 9 cover it
    if (L.nxt >= 0) load_tok(p, L.nrg, lds, nbuf);
  }
}

// k-step s of a unit (weight slot qa = s mod 5, token slot qb = s mod 4):
// wait until this wave's fragments of k-step s have arrived and its loads of
// k-step s + 1 have landed (the loads of the 3 weight / 2 token k-steps
// after it may stay in flight), meet the other waves (then slots qa, qb have
// been read by all and k-step s + 1 is complete everywhere), refill slot qa
// with k-step s + 5 and slot qb with k-step s + 4, then multiply while
// reading k-step s + 1's fragments (at the last k-step these are zeros or
// stale, read and never used).
constexpr int kWaitA = kLoads * (kAStages - 2);
constexpr int kWaitB = kLoads * (kBStages - 2);

template <int NJ, bool FC1>
__device__ __forceinline__ void kstep(const GemmArgs& p, f32x4 (&acc)[8][8], const Frags& f,
                                      Frags& g, const Unit& U, Lookahead& L, Sched& sched,
                                      uint8_t* lds, int* mail, int nbuf, int s, int& qa,
                                      int& qb, int wa, int wr, bool hooks) {
  // (the LDS wait is unconditional so the compiler's own wait insertion sees it
  // on every path into the MFMAs)
  wait_cnt<63, 0>();
  if (wa)
    wait_cnt<kWaitA, 15>();
  else
    wait_cnt<kWaitB, 15>();
  ring_barrier();
  if (hooks && s <= kPub + 9) lookahead<FC1>(p, L, sched, lds, mail, nbuf, s);
  if (wa)
    issue(U, lds, qa, s + kAStages);
  else
    issue(U, lds, qb, s + kBStages);
  qa = qa == kAStages - 1 ? 0 : qa + 1;
  qb = qb == kBStages - 1 ? 0 : qb + 1;
  mma<NJ, true>(acc, f, g, lds, qa, qb, wr, U.j0);
}

// All k-steps of unit U (nk even): weight slots 0..4 hold (or are loading)
// k-steps 0..4, token slots 0..3 k-steps 0..3, and k-step 0 has landed
// everywhere. Leaves the loads of the 4 weight / 3 token k-steps past the
// last in flight (zeros, into slots no wave reads before they land).
template <int NJ, bool FC1>
__device__ __forceinline__ void kloop(const GemmArgs& p, f32x4 (&acc)[8][8], Frags& f0,
                                      Frags& f1, const Unit& U, Lookahead& L, Sched& sched,
                                      uint8_t* lds, int* mail, int nbuf, int nk, int wr) {
  const bool hooks = nk >= kHookSteps;
  const int wa = uni(threadIdx.x >> 7 == 0);  // weight-staging wave
  int qa = 0, qb = 0;
  read_frags(f0, lds, 0, 0, wr, U.j0);
  for (int s = 0; s < nk; s += 2) {
    kstep<NJ, FC1>(p, acc, f0, f1, U, L, sched, lds, mail, nbuf, s, qa, qb, wa, wr, hooks);
    kstep<NJ, FC1>(p, acc, f1, f0, U, L, sched, lds, mail, nbuf, s + 1, qa, qb, wa, wr, hooks);
  }
}

// ----------------------------------------------------------- epilogues ---

// SiLU(g) * u = g u / (1 + 2^(-g log2 e)), with the hardware exp2 and
// reciprocal (about 1 ulp each; the result is rounded to bf16).
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// FC1: D rows 0..7 of tile i (lanes 0..31) are 8 gate rows and rows 8..15
// (lanes 32..63) the matching up rows of 16-row tile tau = 8 wr + i, 4 rows
// per lane (q = 0..3). One v_permlane32_swap pairs gate and up of q = 0 in
// the low lanes and of q = 2 in the high lanes, another those of q = 1 and 3,
// so every lane forms two h values: columns 4 g + 2 hi + {0, 1} of the tile,
// hi = lane / 32, g = (lane / 16) % 2.
template <int NJ>
__device__ __forceinline__ void store_fc1(const GemmArgs& p, const Unit& U, int wr,
                                          const f32x4 (&acc)[8][8], const uint8_t* lds,
                                          int buf) {
  const int l = threadIdx.x & 63, hi = l >> 5, g = (l >> 4) & 1;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int t = 16 * (U.j0 + j) + (l & 15);
    const int slot = t < U.m ? tok(lds, buf, t) : p.S;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[i][j][0]),
                                                        __float_as_uint(acc[i][j][2]), false, false);
      const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[i][j][1]),
                                                        __float_as_uint(acc[i][j][3]), false, false);
      // low lanes: (gate, up) = (s[0], s[1]) of q = 0 / 1; high lanes: (s[0], s[1]) of q = 2 / 3
      const float h0 = silu_mul(__uint_as_float(s02[0]), __uint_as_float(s02[1]));
      const float h1 = silu_mul(__uint_as_float(s13[0]), __uint_as_float(s13[1]));
      if ((unsigned)slot < (unsigned)p.S) {
        const int col = U.r * 128 + (8 * wr + i) * 8 + 4 * g + 2 * hi;
        *(uint32_t*)(p.out + (size_t)slot * p.I + col) = pack_bf16(h0, h1);
      }
    }
  }
}

// FC2: D rows 4 g .. 4 g + 3 of tile i are 4 consecutive output rows of the
// lane's token: one 8-byte store of y (bf16).
template <int NJ>
__device__ __forceinline__ void store_fc2(const GemmArgs& p, const Unit& U, int wr,
                                          const f32x4 (&acc)[8][8], const uint8_t* lds,
                                          int buf) {
  const int l = threadIdx.x & 63, g = l >> 4;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int t = 16 * (U.j0 + j) + (l & 15);
    const int slot = t < U.m ? tok(lds, buf, t) : p.S;
    if ((unsigned)slot >= (unsigned)p.S) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = U.r * kRows + 128 * wr + 16 * i + 4 * g;
      if (row < p.H)
        *(u32x2*)(p.out + (size_t)slot * p.H + row) =
            u32x2{pack_bf16(acc[i][j][0], acc[i][j][1]), pack_bf16(acc[i][j][2], acc[i][j][3])};
    }
  }
}

// ------------------------------------------------------------- kernels ---

// The first k-steps of a unit: 5 into the weight ring, 4 into the token ring.
__device__ __forceinline__ void issue_prologue(const Unit& U, uint8_t* lds) {
  const int n = (threadIdx.x >> 7) == 0 ? kAStages : kBStages;
  for (int c = 0; c < n; ++c) issue(U, lds, c, c);
}

// One unit whose wave has NJ token groups (the accumulators live only here,
// so each variant keeps them in place): its K loop, the next unit picked and
// its first k-steps staged, then this unit's results written. Returns whether
// there is a next unit (then U is it).
template <int NJ, bool FC1>
__device__ __forceinline__ bool run_unit(const GemmArgs& p, Unit& U, Sched& sched, uint8_t* lds,
                                         int* mail, int buf, int nk, int wr) {
  Lookahead L;
  if (threadIdx.x == 0) sched.request();
  L.nxt = -1;
  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // k-step 0 has landed (the later ring slots may still be loading; loads in
  // flight before the prologue, zeros of the last unit, land first)
  if ((threadIdx.x >> 7) == 0)
    wait_cnt<(kAStages - 1) * kLoads, 15>();
  else
    wait_cnt<(kBStages - 1) * kLoads, 15>();
  ring_barrier();
  Frags f0, f1;
  kloop<NJ, FC1>(p, acc, f0, f1, U, L, sched, lds, mail, buf ^ 1, nk, wr);
  if (nk < kHookSteps) {  // short units: the lookahead steps, done here
    if (threadIdx.x == 0) mail[0] = sched.resolve();
    __syncthreads();
    L.nxt = uni(mail[0]);
    if (L.nxt >= 0) {
      L.nrg = plan_entry(p, unit_range(p, L.nxt, plan_entry(p, first_range_unit(p, L.nxt)), L.nr));
      load_tok(p, L.nrg, lds, buf ^ 1);
      wait_cnt<0, 15>();
    }
    __syncthreads();
  }
  // every wave has read the unit's last k-step (what it may still read or
  // have landing is zeros past it): stage the next unit's first k-steps
  // while this unit's results are written
  Unit N = U;
  if (L.nxt >= 0) {
    make_unit<FC1>(p, L.nrg, L.nr, lds, buf ^ 1, N);
    issue_prologue(N, lds);
  }
  if (FC1)
    store_fc1<NJ>(p, U, wr, acc, lds, buf);
  else
    store_fc2<NJ>(p, U, wr, acc, lds, buf);
  U = N;
  return L.nxt >= 0;
}

template <bool FC1>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
  int* mail = (int*)(lds + kLdsMisc);
  const int units = ((plan_int*)p.plan)[0] * p.n_rt;
  const int nk = p.K / 32;  // k-steps, a multiple of 4
  const int wr = uni((threadIdx.x >> 6) & 1);  // weight half of the tile
  Sched sched(p.queue, units, p.remap);
  if (threadIdx.x == 0) {
    sched.request();
    mail[0] = sched.resolve();
  }
  __syncthreads();
  int u = uni(mail[0]);
  __syncthreads();
  if (u < 0) return;
  int buf = 0;  // token table of the current unit
  Unit U;
  {
    int r;
    const int4 rg = plan_entry(p, unit_range(p, u, plan_entry(p, first_range_unit(p, u)), r));
    load_tok(p, rg, lds, 0);
    wait_cnt<0, 15>();
    __syncthreads();
    make_unit<FC1>(p, rg, r, lds, 0, U);
  }
  issue_prologue(U, lds);
  for (;;) {
    bool more;
    switch (U.nj) {
      case 8: more = run_unit<8, FC1>(p, U, sched, lds, mail, buf, nk, wr); break;
      case 7: more = run_unit<7, FC1>(p, U, sched, lds, mail, buf, nk, wr); break;
      case 6: more = run_unit<6, FC1>(p, U, sched, lds, mail, buf, nk, wr); break;
      case 5: more = run_unit<5, FC1>(p, U, sched, lds, mail, buf, nk, wr); break;
      case 4: more = run_unit<4, FC1>(p, U, sched, lds, mail, buf, nk, wr); break;
      case 3: more = run_unit<3, FC1>(p, U, sched, lds, mail, buf, nk, wr); break;
      case 2: more = run_unit<2, FC1>(p, U, sched, lds, mail, buf, nk, wr); break;
      case 1: more = run_unit<1, FC1>(p, U, sched, lds, mail, buf, nk, wr); break;
      default: more = run_unit<0, FC1>(p, U, sched, lds, mail, buf, nk, wr); break;
    }
    if (!more) {
      wait_cnt<0, 0>();  // no load may still write this workgroup's LDS at exit
      break;
    }
    buf ^= 1;
  }
}

}  // namespace gemm

// ---------------------------------------------------------------- host ---

static long plan_ranges(int S, int E) {
  return ((long)S + gemm::kTok - 1) / gemm::kTok + (E < S ? E : S);
}

size_t gemm_plan_ints(int S, int E) { return 4 + 4 * (size_t)plan_ranges(S, E); }

bool gemm_supported(int T, int k, int H, int I) {
  // k-steps of both projections (K / 32) a multiple of 4 and at least 8; every
  // staged buffer (x [T, H], h [T k, I], one expert's w1 [2I, H]) under 2 GiB,
  // so its rows are 32-bit offsets and kOOB lies past it
  const double lim = 2147483648.0;
  return H % 128 == 0 && I % 128 == 0 && H >= 256 && I >= 256 && T >= 0 && k >= 1 &&
         2.0 * T * H < lim && 2.0 * T * k * I < lim && 4.0 * I * H < lim;
}

static int gemm_grid(const void* kernel) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  int& c = cache[{dev, kernel}];
  if (c == 0) {
    int cus = 0, occ = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void*)kernel, gemm::kThreads,
                                                     0) != hipSuccess ||
        occ < 1)
      occ = 1;
    c = cus * occ;
  }
  return c;
}

hipError_t launch_gemm_plan(const int32_t* sorted_ids, const int32_t* block_expert,
                            const int32_t* num_padded, int S, int E, int log2m, int* plan,
                            int* queues, hipStream_t stream) {
  gemm::plan_kernel<<<1, 1024, 0, stream>>>(sorted_ids, block_expert, num_padded, S, E, log2m,
                                            plan, (int)plan_ranges(S, E), queues);
  return hipGetLastError();
}

hipError_t launch_gemm_fc1(const void* x, const void* w1, const int32_t* sorted_ids,
                           const int* plan, int* queue, int H, int I, int k, int S, int remap,
                           void* h, hipStream_t stream) {
  gemm::GemmArgs a{(const uint8_t*)w1, (const uint8_t*)x, sorted_ids, plan, queue,
                   (uint16_t*)h, H, 2 * I, I / 128, I, H, k, S, remap};
  auto kern = gemm::gemm_kernel<true>;
  kern<<<gemm_grid((const void*)kern), gemm::kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_fc2(const void* h, const void* w2, const int32_t* sorted_ids,
                           const int* plan, int* queue, int H, int I, int S, int remap, void* y,
                           hipStream_t stream) {
  gemm::GemmArgs a{(const uint8_t*)w2, (const uint8_t*)h, sorted_ids, plan, queue,
                   (uint16_t*)y, I, H, (H + gemm::kRows - 1) / gemm::kRows, I, H, 1, S, remap};
  auto kern = gemm::gemm_kernel<false>;
  kern<<<gemm_grid((const void*)kern), gemm::kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace moe
