// nsnq_device.hpp -- device-side building blocks shared by the libnsnq kernels
// (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nsnq {

constexpr int kDim = 128;        // head dimension d
constexpr int kCodewords = 256;  // codebook size (uint8 codes)
constexpr int kWave = 64;

typedef _Float16 half_t;
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t uint4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float h2f(uint16_t bits) { return (float)__builtin_bit_cast(half_t, bits); }
__device__ __forceinline__ uint16_t f2h(float x) { return __builtin_bit_cast(uint16_t, (half_t)x); }

// Value held by lane (lane ^ M).  DPP for M = 1, 2, 8 (quad permutes and the
// row rotation by 8 are exactly these XORs within a 16-lane row), the LDS
// swizzle unit for 4 and 16, v_permlane32_swap for 32.
template <int M>
__device__ __forceinline__ float xlane(float v) {
  const int iv = __builtin_bit_cast(int, v);
  if constexpr (M == 1) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, true));
  else if constexpr (M == 2) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, true));
  else if constexpr (M == 4) return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(iv, 0x101F));
  else if constexpr (M == 8) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(iv, 0x128, 0xF, 0xF, true));
  else if constexpr (M == 16) return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(iv, 0x401F));
  else {
    static_assert(M == 32, "lane xor");
    const auto r = __builtin_amdgcn_permlane32_swap((unsigned)iv, (unsigned)iv, false, false);
    const unsigned lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    return __builtin_bit_cast(float, lane < 32 ? r[1] : r[0]);
  }
}

// Runtime-mask butterfly partner (any lane xor), through the LDS crossbar.
__device__ __forceinline__ float xshfl(float v, int mask) { return __shfl_xor(v, mask, kWave); }

// All-reduce over the WIDTH lanes that share lane / WIDTH (WIDTH a power of
// two).  Within a row of 16 lanes: the two quad exchanges, then the half-row
// and row mirrors (lane 7 - i and 15 - i, which pair each reduced quad /
// half-row with the other one), all by DPP folded into the operation.  Across
// rows: the LDS-crossbar swizzle for the odd/even row pair (one VALU op fewer
// than the row swap, which needs two copies of its operand and a select) and
// the half-wave swap of xlane<32>.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int WIDTH, typename Op>
__device__ __forceinline__ float group_reduce(float v, Op op) {
  if constexpr (WIDTH >= 2) v = op(v, dpp_f<0xB1>(v));   // quad_perm 1,0,3,2
  if constexpr (WIDTH >= 4) v = op(v, dpp_f<0x4E>(v));   // quad_perm 2,3,0,1
  if constexpr (WIDTH >= 8) v = op(v, dpp_f<0x141>(v));  // row_half_mirror
  if constexpr (WIDTH >= 16) v = op(v, dpp_f<0x140>(v)); // row_mirror
  if constexpr (WIDTH >= 32) v = op(v, xlane<16>(v));
  if constexpr (WIDTH >= 64) v = op(v, xlane<32>(v));
  return v;
}
struct AddOp {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct MaxOp {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) { return group_reduce<WIDTH>(v, AddOp{}); }
template <int WIDTH>
__device__ __forceinline__ float group_max(float v) { return group_reduce<WIDTH>(v, MaxOp{}); }

// Unnormalised Sylvester-order Walsh-Hadamard transform of a 128-vector held
// E consecutive elements per lane, in 128/E consecutive lanes (element
// c = lane_in_group * E + e).  Result u_c = sum_j (-1)^popcount(c & j) x_j.
// Cross-lane stage with partner p: lower lane x + p, upper lane p - x.
template <int M, int E>
__device__ __forceinline__ void fwht_stage(float (&x)[E], int lane) {
  const float sgn = (lane & M) ? -1.f : 1.f;
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = fmaf(x[e], sgn, xlane<M>(x[e]));
}

template <int E>
__device__ __forceinline__ void fwht128(float (&x)[E], int lane) {
#pragma unroll
  for (int h = 1; h < E; h <<= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if ((e & h) == 0) {
        float a = x[e], b = x[e + h];
        x[e] = a + b;
        x[e + h] = a - b;
      }
    }
  }
  constexpr int LANES = kDim / E;
  if constexpr (LANES >= 2) fwht_stage<1>(x, lane);
  if constexpr (LANES >= 4) fwht_stage<2>(x, lane);
  if constexpr (LANES >= 8) fwht_stage<4>(x, lane);
  if constexpr (LANES >= 16) fwht_stage<8>(x, lane);
  if constexpr (LANES >= 32) fwht_stage<16>(x, lane);
  if constexpr (LANES >= 64) fwht_stage<32>(x, lane);
}

// Walsh-Hadamard transform in the encoder's lane layout: E consecutive
// channels per lane, 128 / E lanes per token (lane `l` of the token's group).
// The in-lane stages are the usual butterflies.  Every cross-lane stage is one
// DPP-fused multiply-add t <- t + c t', with t' the partner lane's value and
// c = -1 on the lane whose stage bit is set (that lane keeps the negated
// difference).  The first cross-lane stage pairs lanes l and l ^ 7 (the
// half-row mirror: DPP has no xor-4 exchange), then l ^ 1, l ^ 2, l ^ 8 and,
// for E = 4, l ^ 16 through the swizzle.  Composed over GF(2), the stages give
// the Sylvester transform with lane l holding the channels of slot hslot(l),
// in order, times hsign(l).
__device__ __forceinline__ int hslot(int l) { return l ^ ((((l >> 1) ^ l) & 1) << 2); }  // bit 2 ^= bit 0 ^ bit 1
__device__ __forceinline__ float hsign(int l) {
  return ((__builtin_popcount(l) + ((l >> 2) & ((l >> 1) ^ l))) & 1) ? -1.f : 1.f;
}
// One DPP stage over the lane's E values: x[e] += c * partner(x[e]) as
// v_fmac_f32_dpp (the compiler keeps a separate DPP move otherwise).  The
// leading s_nop covers the wait a DPP read needs after a VALU write of its
// register, which the compiler cannot see inside the block.
#define NSNQ_HSTAGE4(DPP)                                                                    \
  asm("s_nop 1\n\t"                                                                          \
      "v_fmac_f32_dpp %0, %0, %4 " DPP " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"        \
      "v_fmac_f32_dpp %1, %1, %4 " DPP " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"        \
      "v_fmac_f32_dpp %2, %2, %4 " DPP " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"        \
      "v_fmac_f32_dpp %3, %3, %4 " DPP " row_mask:0xf bank_mask:0xf bound_ctrl:1"              \
      : "+v"(x[e]), "+v"(x[e + 1]), "+v"(x[e + 2]), "+v"(x[e + 3])                            \
      : "v"(c))
template <int BIT, int E>
__device__ __forceinline__ void hstage(float (&x)[E], int l) {
  const float c = ((l >> BIT) & 1) ? -1.f : 1.f;
#pragma unroll
  for (int e = 0; e < E; e += 4) {
    if constexpr (BIT == 2) NSNQ_HSTAGE4("row_half_mirror");
    else if constexpr (BIT == 0) NSNQ_HSTAGE4("quad_perm:[1,0,3,2]");
    else if constexpr (BIT == 1) NSNQ_HSTAGE4("quad_perm:[2,3,0,1]");
    else NSNQ_HSTAGE4("row_ror:8");
  }
}
#undef NSNQ_HSTAGE4
template <int E>
__device__ __forceinline__ void fwht_lanes(float (&x)[E], int l) {
  static_assert(E == 4 || E == 8, "4 or 8 channels per lane");
#pragma unroll
  for (int h = 1; h < E; h <<= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if ((e & h) == 0) {
        const float a = x[e], b = x[e + h];
        x[e] = a + b;
        x[e + h] = a - b;
      }
    }
  }
  hstage<2>(x, l);  // row_half_mirror: l ^ 7
  hstage<0>(x, l);  // quad_perm 1,0,3,2: l ^ 1
  hstage<1>(x, l);  // quad_perm 2,3,0,1: l ^ 2
  hstage<3>(x, l);  // row_ror 8: l ^ 8
  if constexpr (E == 4) {
    const float c = ((l >> 4) & 1) ? -1.f : 1.f;
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = fmaf(xlane<16>(x[e]), c, x[e]);
  }
}

// 1/sqrt(128)
constexpr float kInvSqrtD = 0.088388347648318440550f;

// Power-of-two scaling of fp16 weights.  For the largest magnitude xmax of a
// set of non-negative weights, x * 2^f16_headroom_exp(xmax) < 2^15 for every
// member: the scaled set fits fp16 (max 65504) and its largest members keep
// full fp16 precision, whatever the magnitude of the unscaled weights.  The
// exponent is uniform over the wave (the reduction gives every lane the same
// maximum).
__device__ __forceinline__ int f16_headroom_exp(float xmax) {
  return __builtin_amdgcn_readfirstlane(15 - __builtin_amdgcn_frexp_expf(xmax));
}
__device__ __forceinline__ float pow2f(int e) { return __builtin_amdgcn_ldexpf(1.f, e); }

// Maximum over the 64 lanes of a wave of non-negative floats, through their
// bit patterns (which order like the values): integer maxima need none of the
// NaN canonicalisation that fmaxf carries.
__device__ __forceinline__ float wave_max_nonneg(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0xB1, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x4E, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x141, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x140, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_ds_swizzle((int)u, 0x401F));
  return fmaxf(__builtin_bit_cast(float, u), xlane<32>(__builtin_bit_cast(float, u)));
}

// Raw buffer resource over `bytes` bytes at `base` (gfx9 descriptor): loads
// at or past the end return zeros and touch no memory, so a prefetch past the
// last chunk needs no branch.
typedef __amdgpu_buffer_rsrc_t buf_rsrc_t;
__device__ __forceinline__ buf_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ uint4_t buf_load_b128(buf_rsrc_t r, int off) {
  return __builtin_bit_cast(uint4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load_b32(buf_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

}  // namespace nsnq
