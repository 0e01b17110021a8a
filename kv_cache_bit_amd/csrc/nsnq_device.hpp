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

// Butterfly partner exchange inside a wave.
__device__ __forceinline__ float xshfl(float v, int mask) { return __shfl_xor(v, mask, kWave); }

// Sum over the `width` lanes that share lane / width (width a power of two).
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = 1; m < WIDTH; m <<= 1) v += xshfl(v, m);
  return v;
}

template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = 1; m < WIDTH; m <<= 1) v = fmaxf(v, xshfl(v, m));
  return v;
}

// Unnormalised Sylvester-order Walsh-Hadamard transform of a 128-vector held
// E consecutive elements per lane, in 128/E consecutive lanes (element
// c = lane_in_group * E + e).  Result u_c = sum_j (-1)^popcount(c & j) x_j.
template <int E>
__device__ __forceinline__ void fwht128(float (&x)[E], int lane) {
  // in-lane stages: element bits
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
  // cross-lane stages: lane bits
  constexpr int LANES = kDim / E;
#pragma unroll
  for (int m = 1; m < LANES; m <<= 1) {
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float p = xshfl(x[e], m);
      x[e] = upper ? (p - x[e]) : (x[e] + p);
    }
  }
}

// 1/sqrt(128)
constexpr float kInvSqrtD = 0.088388347648318440550f;

}  // namespace nsnq
