// Device helpers shared by the MoE kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ------------------------------------------------------------ formats ---

// bfloat16 bits -> float (exact).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bfloat16 bits, round to nearest even: add just under half an ulp of
// the 16-bit result, plus one when the kept LSB is odd, then truncate. A NaN
// stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// float -> OCP e4m3fn code (1 sign, 4 exponent bits with bias 7, 3 mantissa
// bits, no infinities, max 448), round to nearest even, magnitudes above 448
// saturate to 448. The sign is kept, so a negative value that rounds to zero
// gives 0x80. NaN input is outside the contract.
__device__ __forceinline__ uint32_t f32_to_e4m3fn(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.0f);
  const uint32_t au = __float_as_uint(a);
  if (au < 0x3c800000u) {                 // a < 2^-6: subnormal grid, step 2^-9
    const float q = rintf(a * 512.0f);     // exact scaling, then ties-to-even
    return sign | (uint32_t)q;             // q == 8 is the smallest normal (code 0x08)
  }
  // normal: keep 3 mantissa bits with round-to-nearest-even; a carry out of
  // the mantissa bumps the exponent, which is what RNE requires
  const uint32_t r = au + 0x7ffffu + ((au >> 20) & 1u);
  const uint32_t ex = (r >> 23) - 127u + 7u;
  return sign | (ex << 3) | ((r >> 20) & 7u);
}

// ----------------------------------------------------- wave reductions ---
// Partner exchange of step s of a wave64 reduction. Steps 0..3 are DPP moves
// inside rows of 16 lanes (quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror), each pairing the two halves of a group of 2,
// 4, 8, 16 lanes; steps 4 and 5 pair lane l with l ^ 16 and l ^ 32 through
// gfx950's v_permlane16_swap / v_permlane32_swap (swapping a register with a
// copy of itself leaves, in lanes of even rows / the low half, the partner's
// value in the second result and elsewhere in the first). Combining a value
// with its partner's at every step leaves the same combination over all 64
// lanes in every lane (bit-identical when the combination is commutative),
// with no LDS traffic.
template <int STEP>
__device__ __forceinline__ int wave_partner(int v) {
  if constexpr (STEP == 0) {
    return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  } else if constexpr (STEP == 1) {
    return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  } else if constexpr (STEP == 2) {
    return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
  } else if constexpr (STEP == 3) {
    return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
  } else if constexpr (STEP == 4) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return ((threadIdx.x >> 4) & 1) == 0 ? (int)r[1] : (int)r[0];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (threadIdx.x & 32) == 0 ? (int)r[1] : (int)r[0];
  }
}
template <int STEP>
__device__ __forceinline__ float wave_partner(float v) {
  return __int_as_float(wave_partner<STEP>(__float_as_int(v)));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, wave_partner<0>(v));
  v = fmaxf(v, wave_partner<1>(v));
  v = fmaxf(v, wave_partner<2>(v));
  v = fmaxf(v, wave_partner<3>(v));
  v = fmaxf(v, wave_partner<4>(v));
  return fmaxf(v, wave_partner<5>(v));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += wave_partner<0>(v);
  v += wave_partner<1>(v);
  v += wave_partner<2>(v);
  v += wave_partner<3>(v);
  v += wave_partner<4>(v);
  return v + wave_partner<5>(v);
}

// ------------------------------------------------------------- MFMA ---
// Fragment conventions of the 16x16 MFMAs on gfx950 (lane l of a wave64):
//   A (16 x K): lane l holds row (l & 15), k-group (l >> 4)
//   B (K x 16): lane l holds column (l & 15), k-group (l >> 4)
//   D (16x16) : lane l holds rows 4*(l >> 4) + i, i = 0..3, column (l & 15)
// A dot product is invariant under any permutation of K applied to A and B
// alike, so the kernels place bytes in each k-group in the order that makes
// their global loads contiguous; A and B always use the same placement.

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x16x128 with both operands OCP fp8 e4m3 (format code 0) and unit block
// scales (E8M0 exponent 127 = 2^0).
__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& a, const i32x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// A device-scope store: written through to the point where every XCD sees
// it (the L2 of one XCD is not coherent with the others' within a kernel).
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float* p, float v) {
  st_dev((uint32_t*)p, __float_as_uint(v));
}
__device__ __forceinline__ void st_dev(int32_t* p, int32_t v) { st_dev((uint32_t*)p, (uint32_t)v); }

// 16x16x32 with both operands OCP fp8 e4m3: 8 codes per lane (one k-group).
__device__ __forceinline__ f32x4 mfma_fp8_k32(const u32x2& a, const u32x2& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(long, a),
                                                    __builtin_bit_cast(long, b), c, 0, 0, 0);
}

}  // namespace moe
