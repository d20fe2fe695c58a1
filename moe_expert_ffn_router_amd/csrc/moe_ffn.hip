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
// Design (MI355X): FC1 and FC2 are weight streams. The work of a projection
// is a list of units (aligned block b, 16-row weight tile r); the list length
// comes from num_padded on the device, so the host never synchronises. A
// persistent grid sized to the resident capacity gives every wave one
// contiguous, equal share of the list; with the XCD remap on, the waves of one
// XCD (workgroup id mod 8) own one contiguous share, so each XCD's L2 serves a
// contiguous slice of (expert, rows). Per unit a wave streams its 16 weight
// rows straight from HBM into MFMA A-fragments (64 contiguous bytes per row per
// load instruction), gathers the block's token rows into B-fragments (L2
// resident) and accumulates 16x16 tiles with v_mfma; no LDS, no barriers.
// FC1 interleaves 8 gate rows and the matching 8 up rows in one tile, so
// SiLU(gate)*up is formed in registers after one lane swap.
#include "moe_common.h"
#include "moe_launch.h"

#include <mutex>

#include "../../include/moe.h"

namespace moe {

// ------------------------------------------------- work partitioning ---

struct WaveRange {
  long u0, u1;
};

__device__ __forceinline__ WaveRange wave_range(long total, int remap) {
  int wg = blockIdx.x;
  const int G = gridDim.x;
  if (remap && (G & 7) == 0) wg = (wg & 7) * (G >> 3) + (wg >> 3);
  const long wave = (long)wg * 4 + (threadIdx.x >> 6);
  const long W = (long)G * 4;
  return {total * wave / W, total * (wave + 1) / W};
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

// Slot of column (lane & 15) of token tile t of the group starting at t0.
__device__ __forceinline__ void group_slots(const int32_t* __restrict__ sorted_ids, int b, int M,
                                            int S, int m_valid, int t0, int (&slot)[4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int i = t0 + t * 16 + (lane & 15);
    slot[t] = i < m_valid ? sorted_ids[(size_t)b * M + i] : S;
  }
}

// ------------------------------------------------------- bf16 K loop ---
// acc[t] += A(16 rows, this lane: a_ptr) . B_t(16 tokens, this lane: b_ptr[t])
// over K elements; one k-step is 32 elements (64 bytes per row).
template <int MT, int U>
__device__ __forceinline__ void kloop_bf16(const uint16_t* __restrict__ a_ptr,
                                           const uint16_t* const (&b_ptr)[4], const bool (&ok)[4],
                                           int K, f32x4 (&acc)[4]) {
  const int nks = K >> 5;
  int ks = 0;
  for (; ks + U <= nks; ks += U) {
    bf16x8 a[U], b[MT][U];
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = *(const bf16x8*)(a_ptr + (size_t)(ks + u) * 32);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        b[t][u] = bf16x8{};
        if (ok[t]) b[t][u] = *(const bf16x8*)(b_ptr[t] + (size_t)(ks + u) * 32);
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = mfma_bf16(a[u], b[t][u], acc[t]);
  }
  for (; ks < nks; ++ks) {
    const bf16x8 a = *(const bf16x8*)(a_ptr + (size_t)ks * 32);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      bf16x8 b{};
      if (ok[t]) b = *(const bf16x8*)(b_ptr[t] + (size_t)ks * 32);
      acc[t] = mfma_bf16(a, b, acc[t]);
    }
  }
}

// -------------------------------------------------------- fp8 K loop ---
// One k-step is 128 e4m3 bytes per row. A lane's 32 operand bytes are the
// 16 bytes at 16*g and the 16 bytes at 64 + 16*g of the step (g = lane >> 4),
// so each load instruction reads 64 contiguous bytes per row; B uses the same
// placement, which keeps every product paired with its own k.
__device__ __forceinline__ i32x8 load_fp8_frag(const uint8_t* __restrict__ p) {
  const u32x4 lo = *(const u32x4*)p;
  const u32x4 hi = *(const u32x4*)(p + 64);
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
               (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int MT, int U>
__device__ __forceinline__ void kloop_fp8(const uint8_t* __restrict__ a_ptr,
                                          const uint8_t* const (&b_ptr)[4], const bool (&ok)[4],
                                          int K, f32x4 (&acc)[4]) {
  const int nks = K >> 7;
  int ks = 0;
  for (; ks + U <= nks; ks += U) {
    i32x8 a[U], b[MT][U];
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = load_fp8_frag(a_ptr + (size_t)(ks + u) * 128);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        b[t][u] = i32x8{};
        if (ok[t]) b[t][u] = load_fp8_frag(b_ptr[t] + (size_t)(ks + u) * 128);
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = mfma_fp8(a[u], b[t][u], acc[t]);
  }
  for (; ks < nks; ++ks) {
    const i32x8 a = load_fp8_frag(a_ptr + (size_t)ks * 128);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      i32x8 b{};
      if (ok[t]) b = load_fp8_frag(b_ptr[t] + (size_t)ks * 128);
      acc[t] = mfma_fp8(a, b, acc[t]);
    }
  }
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// ---------------------------------------------------------- FC1 bf16 ---

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
};

template <int MT>
__device__ __forceinline__ void fc1_bf16_group(const Fc1Args& p, int e, int r, const int (&slot)[4]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, rho = lane & 15;
  const int row = rho < 8 ? (r * 8 + rho) : (p.I + r * 8 + rho - 8);
  const uint16_t* a_ptr =
      (const uint16_t*)p.w1 + ((size_t)e * 2 * p.I + row) * p.H + 8 * g;
  const uint16_t* b_ptr[4];
  bool ok[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    ok[t] = t < MT && slot[t] < p.S;
    b_ptr[t] = (const uint16_t*)p.x + (size_t)(ok[t] ? slot[t] / p.k : 0) * p.H + 8 * g;
  }
  f32x4 acc[4] = {};
  kloop_bf16<MT, 8 / MT>(a_ptr, b_ptr, ok, p.H, acc);
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    f32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __shfl_xor(acc[t][i], 32);
    if (lane < 32 && ok[t]) {
      uint32_t hb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) hb[i] = f32_to_bf16_rne(silu_mul(acc[t][i], o[i]));
      *(u32x2*)((uint16_t*)p.h + (size_t)slot[t] * p.I + r * 8 + 4 * g) =
          u32x2{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
    }
  }
}

template <int MT>
__device__ __forceinline__ void fc1_fp8_group(const Fc1Args& p, int e, int r, const int (&slot)[4]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, rho = lane & 15;
  const int row = rho < 8 ? (r * 8 + rho) : (p.I + r * 8 + rho - 8);
  const uint8_t* a_ptr = (const uint8_t*)p.w1 + ((size_t)e * 2 * p.I + row) * p.H + 16 * g;
  const uint8_t* b_ptr[4];
  bool ok[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    ok[t] = t < MT && slot[t] < p.S;
    b_ptr[t] = (const uint8_t*)p.x + (size_t)(ok[t] ? slot[t] / p.k : 0) * p.H + 16 * g;
  }
  f32x4 acc[4] = {};
  kloop_fp8<MT, (MT == 1 ? 4 : (MT == 2 ? 2 : 1))>(a_ptr, b_ptr, ok, p.H, acc);
  // this lane's D rows: 4*g + i; gate rows for g < 2, up rows for g >= 2
  const int nrow0 = (g < 2) ? (r * 8 + 4 * g) : (p.I + r * 8 + 4 * (g - 2));
  const f32x4 ws = *(const f32x4*)(p.w1s + (size_t)e * 2 * p.I + nrow0);
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const float xs = ok[t] ? p.xs[slot[t] / p.k] : 0.f;
    f32x4 v, o;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = acc[t][i] * ws[i] * xs;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __shfl_xor(v[i], 32);
    if (lane < 32 && ok[t]) {
      f32x4 hv;
#pragma unroll
      for (int i = 0; i < 4; ++i) hv[i] = silu_mul(v[i], o[i]);
      *(f32x4*)((float*)p.h + (size_t)slot[t] * p.I + r * 8 + 4 * g) = hv;
    }
  }
}

template <bool FP8>
__global__ __launch_bounds__(256) void fc1_kernel(Fc1Args p) {
  const int M = 1 << p.log2m;
  const int nb = p.num_padded[0] >> p.log2m;
  const int n_rt = p.I >> 3;
  const WaveRange wr = wave_range((long)nb * n_rt, p.remap);
  int cur_b = -1, e = 0, m_valid = 0;
  for (long u = wr.u0; u < wr.u1; ++u) {
    const int b = (int)(u / n_rt), r = (int)(u % n_rt);
    if (b != cur_b) {
      cur_b = b;
      e = p.block_expert[b];
      m_valid = block_valid(p.sorted_ids, b, M, p.S);
    }
    for (int t0 = 0; t0 < m_valid; t0 += 64) {
      int slot[4];
      group_slots(p.sorted_ids, b, M, p.S, m_valid, t0, slot);
      const int mt = min(4, (m_valid - t0 + 15) >> 4);
      if (FP8) {
        if (mt == 1) fc1_fp8_group<1>(p, e, r, slot);
        else if (mt == 2) fc1_fp8_group<2>(p, e, r, slot);
        else if (mt == 3) fc1_fp8_group<3>(p, e, r, slot);
        else fc1_fp8_group<4>(p, e, r, slot);
      } else {
        if (mt == 1) fc1_bf16_group<1>(p, e, r, slot);
        else if (mt == 2) fc1_bf16_group<2>(p, e, r, slot);
        else if (mt == 3) fc1_bf16_group<3>(p, e, r, slot);
        else fc1_bf16_group<4>(p, e, r, slot);
      }
    }
  }
}

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
  float* y;            // f32 [S, H]
};

template <int MT, bool FP8>
__device__ __forceinline__ void fc2_group(const Fc2Args& p, int e, int r, const int (&slot)[4]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, rho = lane & 15;
  const size_t arow = (size_t)e * p.H + r * 16 + rho;
  bool ok[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) ok[t] = t < MT && slot[t] < p.S;
  f32x4 acc[4] = {};
  if (FP8) {
    const uint8_t* a_ptr = (const uint8_t*)p.w2 + arow * p.I + 16 * g;
    const uint8_t* b_ptr[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      b_ptr[t] = (const uint8_t*)p.h + (size_t)(ok[t] ? slot[t] : 0) * p.I + 16 * g;
    kloop_fp8<MT, (MT == 1 ? 4 : (MT == 2 ? 2 : 1))>(a_ptr, b_ptr, ok, p.I, acc);
  } else {
    const uint16_t* a_ptr = (const uint16_t*)p.w2 + arow * p.I + 8 * g;
    const uint16_t* b_ptr[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      b_ptr[t] = (const uint16_t*)p.h + (size_t)(ok[t] ? slot[t] : 0) * p.I + 8 * g;
    kloop_bf16<MT, 8 / MT>(a_ptr, b_ptr, ok, p.I, acc);
  }
  f32x4 ws = {1.f, 1.f, 1.f, 1.f};
  if (FP8) ws = *(const f32x4*)(p.w2s + (size_t)e * p.H + r * 16 + 4 * g);
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    if (!ok[t]) continue;
    f32x4 v = acc[t];
    if (FP8) {
      const float hs = p.hs[slot[t]];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = v[i] * ws[i] * hs;
    }
    *(f32x4*)(p.y + (size_t)slot[t] * p.H + r * 16 + 4 * g) = v;
  }
}

template <bool FP8>
__global__ __launch_bounds__(256) void fc2_kernel(Fc2Args p) {
  const int M = 1 << p.log2m;
  const int nb = p.num_padded[0] >> p.log2m;
  const int n_rt = p.H >> 4;
  const WaveRange wr = wave_range((long)nb * n_rt, p.remap);
  int cur_b = -1, e = 0, m_valid = 0;
  for (long u = wr.u0; u < wr.u1; ++u) {
    const int b = (int)(u / n_rt), r = (int)(u % n_rt);
    if (b != cur_b) {
      cur_b = b;
      e = p.block_expert[b];
      m_valid = block_valid(p.sorted_ids, b, M, p.S);
    }
    for (int t0 = 0; t0 < m_valid; t0 += 64) {
      int slot[4];
      group_slots(p.sorted_ids, b, M, p.S, m_valid, t0, slot);
      const int mt = min(4, (m_valid - t0 + 15) >> 4);
      if (mt == 1) fc2_group<1, FP8>(p, e, r, slot);
      else if (mt == 2) fc2_group<2, FP8>(p, e, r, slot);
      else if (mt == 3) fc2_group<3, FP8>(p, e, r, slot);
      else fc2_group<4, FP8>(p, e, r, slot);
    }
  }
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

template <typename InT>
__global__ __launch_bounds__(256) void quant_rows_kernel(const InT* __restrict__ in, int R, int C,
                                                         uint8_t* __restrict__ codes,
                                                         float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const InT* row = in + (size_t)r * C;
  float amax = 0.f;
  for (int c = lane * 8; c < C; c += kWave * 8) {
    float v[8];
    load8(row + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = wave_max(amax);
  const float scale = amax == 0.f ? 1.0f : amax / 448.0f;
  for (int c = lane * 8; c < C; c += kWave * 8) {
    float v[8];
    load8(row + c, v);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= f32_to_e4m3fn(v[i] / scale) << (8 * i);
      hi |= f32_to_e4m3fn(v[4 + i] / scale) << (8 * i);
    }
    *(u32x2*)(codes + (size_t)r * C + c) = u32x2{lo, hi};
  }
  if (lane == 0) scales[r] = scale;
}

// ----------------------------------------------------------- combine ---
// out[t, n] = sum_j w[t, j] * y[t*k + j, n], fp32 in j order, one rounding.
template <typename OutT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const float* __restrict__ w, int T, int H,
                                                      int k, OutT* __restrict__ out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const int per_row = H >> 3;
  if (i >= (long)T * per_row) return;
  const int t = (int)(i / per_row), n = (int)(i % per_row) * 8;
  float acc[8] = {};
  for (int j = 0; j < k; ++j) {
    const float wj = w[(size_t)t * k + j];
    const float* yr = y + ((size_t)t * k + j) * H + n;
    const f32x4 a = *(const f32x4*)yr, b = *(const f32x4*)(yr + 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[q] += wj * a[q];
      acc[4 + q] += wj * b[q];
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

// A combine for H not a multiple of 8 (fp32 path): one thread per element.
__global__ __launch_bounds__(256) void combine_f32_scalar_kernel(const float* __restrict__ y,
                                                                 const float* __restrict__ w,
                                                                 int T, int H, int k,
                                                                 float* __restrict__ out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)T * H) return;
  const int t = (int)(i / H), n = (int)(i % H);
  float acc = 0.f;
  for (int j = 0; j < k; ++j) acc += w[(size_t)t * k + j] * y[((size_t)t * k + j) * H + n];
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
                                                      int H, int I, int k, int S, int log2m,
                                                      float* __restrict__ h) {
  const int lane = threadIdx.x & 63;
  const long W = (long)gridDim.x * 4;
  const long total = (long)num_padded[0] * I;
  for (long u = (long)blockIdx.x * 4 + (threadIdx.x >> 6); u < total; u += W) {
    const int pos = (int)(u / I), n = (int)(u % I);
    const int slot = sorted_ids[pos];
    if (slot >= S) continue;
    const int e = block_expert[pos >> log2m];
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
                                                      int H, int I, int S, int log2m,
                                                      float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const long W = (long)gridDim.x * 4;
  const long total = (long)num_padded[0] * H;
  for (long u = (long)blockIdx.x * 4 + (threadIdx.x >> 6); u < total; u += W) {
    const int pos = (int)(u / H), n = (int)(u % H);
    const int slot = sorted_ids[pos];
    if (slot >= S) continue;
    const int e = block_expert[pos >> log2m];
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

// -------------------------------------------------------- host side ---

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

FfnWorkspace ffn_workspace_layout(int T, int H, int I, int k, int dtype) {
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
  if (dtype == MOE_DTYPE_FP8) {
    put(L.hq_off, L.hq_bytes, S * I);
    put(L.hs_off, L.hs_bytes, S * 4);
    put(L.xq_off, L.xq_bytes, (size_t)T * H);
    put(L.xs_off, L.xs_bytes, (size_t)T * 4);
  }
  put(L.y_off, L.y_bytes, S * H * 4);
  L.total = o;
  return L;
}

// Resident-capacity grid of a persistent kernel on the current device,
// rounded down to a multiple of 8 (one share per XCD). Cached per device.
template <typename K>
static int persistent_grid(K kernel, int slot) {
  static std::mutex mu;
  static int cache[64][8];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  int& c = cache[dev][slot];
  if (c == 0) {
    int cus = 0, occ = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, 256, 0) != hipSuccess ||
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

static unsigned stages(unsigned flags) {
  const unsigned s = flags & (MOE_FFN_STAGE_FC1 | MOE_FFN_STAGE_FC2 | MOE_FFN_STAGE_COMBINE);
  return s ? s : (MOE_FFN_STAGE_FC1 | MOE_FFN_STAGE_FC2 | MOE_FFN_STAGE_COMBINE);
}

static hipError_t launch_combine(const FfnProblem& p, const FfnWorkspace& L, bool bf16_out,
                                 hipStream_t stream) {
  const float* y = (const float*)((char*)p.workspace + L.y_off);
  if (p.H % 8 == 0) {
    const long n = (long)p.T * (p.H / 8);
    const dim3 grid((unsigned)((n + 255) / 256));
    if (bf16_out)
      combine_kernel<uint16_t><<<grid, 256, 0, stream>>>(y, p.topk_weights, p.T, p.H, p.k,
                                                         (uint16_t*)p.out);
    else
      combine_kernel<float><<<grid, 256, 0, stream>>>(y, p.topk_weights, p.T, p.H, p.k,
                                                      (float*)p.out);
  } else {
    const long n = (long)p.T * p.H;
    combine_f32_scalar_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(
        y, p.topk_weights, p.T, p.H, p.k, (float*)p.out);
  }
  return hipGetLastError();
}

hipError_t launch_ffn_bf16(const FfnProblem& p, hipStream_t stream) {
  const FfnWorkspace L = ffn_workspace_layout(p.T, p.H, p.I, p.k, MOE_DTYPE_BF16);
  const unsigned st = stages(p.flags);
  const int remap = (p.flags & MOE_FFN_NO_XCD_REMAP) ? 0 : 1;
  const int S = p.T * p.k, log2m = ilog2(p.block_m);
  void* h = (char*)p.workspace + L.h_off;
  float* y = (float*)((char*)p.workspace + L.y_off);
  hipError_t err;
  if (st & MOE_FFN_STAGE_FC1) {
    Fc1Args a{p.x, nullptr, p.w1, nullptr, p.sorted_ids, p.block_expert, p.num_padded,
              p.H, p.I, p.k, S, log2m, remap, h};
    fc1_kernel<false><<<persistent_grid(fc1_kernel<false>, 0), 256, 0, stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_FC2) {
    Fc2Args a{h, nullptr, p.w2, nullptr, p.sorted_ids, p.block_expert, p.num_padded,
              p.H, p.I, S, log2m, remap, y};
    fc2_kernel<false><<<persistent_grid(fc2_kernel<false>, 1), 256, 0, stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_COMBINE) return launch_combine(p, L, true, stream);
  return hipSuccess;
}

hipError_t launch_ffn_fp8(const FfnProblem& p, hipStream_t stream) {
  const FfnWorkspace L = ffn_workspace_layout(p.T, p.H, p.I, p.k, MOE_DTYPE_FP8);
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
  if (st & MOE_FFN_STAGE_FC1) {
    quant_rows_kernel<uint16_t><<<(p.T + 3) / 4, 256, 0, stream>>>((const uint16_t*)p.x, p.T,
                                                                   p.H, xq, xs);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    Fc1Args a{xq, xs, p.w1, p.w1_scale, p.sorted_ids, p.block_expert, p.num_padded,
              p.H, p.I, p.k, S, log2m, remap, h};
    fc1_kernel<true><<<persistent_grid(fc1_kernel<true>, 2), 256, 0, stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_FC2) {
    quant_rows_kernel<float><<<(S + 3) / 4, 256, 0, stream>>>(h, S, p.I, hq, hs);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    Fc2Args a{hq, hs, p.w2, p.w2_scale, p.sorted_ids, p.block_expert, p.num_padded,
              p.H, p.I, S, log2m, remap, y};
    fc2_kernel<true><<<persistent_grid(fc2_kernel<true>, 3), 256, 0, stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_COMBINE) return launch_combine(p, L, true, stream);
  return hipSuccess;
}

hipError_t launch_ffn_f32(const FfnProblem& p, hipStream_t stream) {
  const FfnWorkspace L = ffn_workspace_layout(p.T, p.H, p.I, p.k, MOE_DTYPE_F32);
  const unsigned st = stages(p.flags);
  const int S = p.T * p.k, log2m = ilog2(p.block_m);
  float* h = (float*)((char*)p.workspace + L.h_off);
  float* y = (float*)((char*)p.workspace + L.y_off);
  hipError_t err;
  const int grid = 1024;
  if (st & MOE_FFN_STAGE_FC1) {
    fc1_f32_kernel<<<grid, 256, 0, stream>>>((const float*)p.x, (const float*)p.w1,
                                             p.sorted_ids, p.block_expert, p.num_padded, p.H,
                                             p.I, p.k, S, log2m, h);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_FC2) {
    fc2_f32_kernel<<<grid, 256, 0, stream>>>(h, (const float*)p.w2, p.sorted_ids,
                                             p.block_expert, p.num_padded, p.H, p.I, S, log2m,
                                             y);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (st & MOE_FFN_STAGE_COMBINE) return launch_combine(p, L, false, stream);
  return hipSuccess;
}

}  // namespace moe
