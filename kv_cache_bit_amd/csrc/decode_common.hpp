// decode_common.hpp -- pieces shared by the two compressed-cache decode
// kernels (LUT scoring in decode.hip, matrix-core scoring in decode_mfma.hip).
#pragma once

#include <atomic>

#include "nsnq_device.hpp"
#include "nsnq_launch.hpp"

namespace nsnq {

// Blocks of R tokens one split may span.
constexpr int kMaxSplitBlocks = 16;

// Lets `kernel` use up to 160 KB of dynamic LDS, once per device of the
// process (the attribute is per device); `set` is the caller's per-kernel
// record of the devices done.  Threads making a first call on one device at
// the same time may both set the attribute: the call is idempotent, and the
// record is atomic.
inline hipError_t allow_lds(const void* kernel, std::atomic<bool> (&set)[kMaxDevices]) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (!set[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    set[dev].store(true, std::memory_order_release);
  }
  return hipSuccess;
}

// Block-wide reduction of GH values per thread (max or sum); red is 4*GH floats.
template <int GH, bool MAX>
__device__ __forceinline__ void block_reduce(float (&v)[GH], float* red, int lane, int wave) {
#pragma unroll
  for (int g = 0; g < GH; ++g) v[g] = MAX ? group_max<kWave>(v[g]) : group_sum<kWave>(v[g]);
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GH; ++g) red[wave * GH + g] = v[g];
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < GH; ++g) {
    float r0 = red[g], r1 = red[GH + g], r2 = red[2 * GH + g], r3 = red[3 * GH + g];
    v[g] = MAX ? fmaxf(fmaxf(r0, r1), fmaxf(r2, r3)) : (r0 + r1) + (r2 + r3);
  }
  __syncthreads();
}


// Residual split: fp16 keys and values, one query token per head.
template <int GH>
__device__ __forceinline__ void decode_residual(const DecodeArgs& a, int nt, float* qf, float* sc, float* ov,
                                                float* red, float* ws_base, int64_t ws_head, int64_t unit) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int TS = 128;
  const uint16_t* kr = a.kresid + unit * a.R * kDim;
  const uint16_t* vr = a.vresid + unit * a.R * kDim;
  __syncthreads();
  // scores: one thread per token, the whole key row in flight at once
  if (tid < nt) {
    const uint4* row = reinterpret_cast<const uint4*>(kr + (int64_t)tid * kDim);
    uint4 kv[16];
#pragma unroll
    for (int ch = 0; ch < 16; ++ch) kv[ch] = row[ch];
    float acc[GH];
#pragma unroll
    for (int g = 0; g < GH; ++g) acc[g] = 0.f;
    if (a.rope_cos) {
      // keys stored before RoPE: rotate the pairs (c, c + 64) by the token's
      // position (after the n_quant compressed tokens of the row)
      const int64_t pos = (int64_t)a.rope_pos0 + row_quant(a, (int)(unit / a.Hkv)) + tid;
      const float4* cs4 = reinterpret_cast<const float4*>(a.rope_cos + pos * (kDim / 2));
      const float4* sn4 = reinterpret_cast<const float4*>(a.rope_sin + pos * (kDim / 2));
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) {
        const uint32_t lo4[4] = {kv[ch].x, kv[ch].y, kv[ch].z, kv[ch].w};
        const uint32_t hi4[4] = {kv[ch + 8].x, kv[ch + 8].y, kv[ch + 8].z, kv[ch + 8].w};
        const float4 ca = cs4[2 * ch], cb = cs4[2 * ch + 1], sa = sn4[2 * ch], sb = sn4[2 * ch + 1];
        const float cv[8] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w};
        const float sv[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t wl = lo4[i >> 1], wh = hi4[i >> 1];
          const float k0 = h2f((i & 1) ? (wl >> 16) : (wl & 0xffff));
          const float k1 = h2f((i & 1) ? (wh >> 16) : (wh & 0xffff));
          const float r0 = fmaf(k0, cv[i], -k1 * sv[i]);
          const float r1 = fmaf(k1, cv[i], k0 * sv[i]);
          const int c = ch * 8 + i;
#pragma unroll
          for (int g = 0; g < GH; ++g)
            acc[g] = fmaf(qf[g * kDim + c], r0, fmaf(qf[g * kDim + c + 64], r1, acc[g]));
        }
      }
    } else {
#pragma unroll
      for (int ch = 0; ch < 16; ++ch) {
        const uint32_t w4[4] = {kv[ch].x, kv[ch].y, kv[ch].z, kv[ch].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float k0 = h2f(w4[i] & 0xffff), k1 = h2f(w4[i] >> 16);
          const int c = ch * 8 + 2 * i;
#pragma unroll
          for (int g = 0; g < GH; ++g) acc[g] = fmaf(qf[g * kDim + c], k0, fmaf(qf[g * kDim + c + 1], k1, acc[g]));
        }
      }
    }
#pragma unroll
    for (int g = 0; g < GH; ++g) sc[g * TS + tid] = acc[g] * a.scale_log2;
  }
  __syncthreads();
  float m[GH], l[GH];
#pragma unroll
  for (int g = 0; g < GH; ++g) m[g] = -INFINITY;
  for (int t = tid; t < nt; t += 256)
#pragma unroll
    for (int g = 0; g < GH; ++g) m[g] = fmaxf(m[g], sc[g * TS + t]);
  block_reduce<GH, true>(m, red, lane, wave);
#pragma unroll
  for (int g = 0; g < GH; ++g) l[g] = 0.f;
  for (int t = tid; t < nt; t += 256)
#pragma unroll
    for (int g = 0; g < GH; ++g) {
      const float pr = exp2f(sc[g * TS + t] - m[g]);
      sc[g * TS + t] = pr;
      l[g] += pr;
    }
  block_reduce<GH, false>(l, red, lane, wave);
  // values: wave per token row, lanes own channels (2 lane, 2 lane + 1)
  float o0[GH], o1[GH];
#pragma unroll
  for (int g = 0; g < GH; ++g) o0[g] = o1[g] = 0.f;
#pragma unroll 8
  for (int t = wave; t < nt; t += 4) {
    const uint32_t vv = *reinterpret_cast<const uint32_t*>(vr + (int64_t)t * kDim + 2 * lane);
    const float v0 = h2f(vv & 0xffff), v1 = h2f(vv >> 16);
#pragma unroll
    for (int g = 0; g < GH; ++g) {
      const float pr = sc[g * TS + t];
      o0[g] = fmaf(pr, v0, o0[g]);
      o1[g] = fmaf(pr, v1, o1[g]);
    }
  }
#pragma unroll
  for (int g = 0; g < GH; ++g) {
    ov[(wave * GH + g) * kDim + 2 * lane] = o0[g];
    ov[(wave * GH + g) * kDim + 2 * lane + 1] = o1[g];
  }
  __syncthreads();
  for (int o = tid; o < GH * kDim; o += 256) {
    const int g = o / kDim, c = o % kDim;
    const float sum = (ov[(0 * GH + g) * kDim + c] + ov[(1 * GH + g) * kDim + c]) +
                      (ov[(2 * GH + g) * kDim + c] + ov[(3 * GH + g) * kDim + c]);
    ws_base[g * ws_head + c] = sum;
    if (c == 0) {
      ws_base[g * ws_head + kDim] = m[g];
      ws_base[g * ws_head + kDim + 1] = l[g];
    }
  }
}

}  // namespace nsnq
