// aux.hip -- dequantisation and k-means codebook fitting (gfx950).

#include "nsnq_device.hpp"
#include "nsnq_launch.hpp"

namespace nsnq {

// ---------------------------------------------------------------------------
// Dequant: x_hat = N1 * (N2 * D H c_hat + MU_block), D = diag(signs).  Same lane layout as the
// encoder (one sub-vector per lane, S lanes per token); the Hadamard inverse is
// the forward transform (H symmetric, orthonormal).  64 tokens per group.
template <int SUB>
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
  constexpr int S = kDim / SUB;
  constexpr int TPR = kWave / S;
  constexpr int TPB = 64;                // tokens per work-group
  constexpr int ROWS = TPB / 4 / TPR;
  __shared__ float cbf[kCodewords * SUB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane % S, tir = lane / S;
  // lane `slot` takes the codeword of its slot; the transform (DPP stages,
  // as in the encoder) leaves it holding the channels of output slot
  // hslot(slot) times hsign(slot), which the scale undoes
  const int oslot = hslot(slot);
  const int unit = blockIdx.y;
  // per-lane bases, then 32-bit token offsets per row (R is 64 or 128: the
  // block of token t is t >> lgR)
  const int lgR = __builtin_ctz(a.R);
  const int i0 = blockIdx.x * TPB + wave * (TPB / 4) + tir;  // output token of row 0
  const int tlast = a.tok0 + a.ntok - 1;                      // loads of rows past the end re-read the last token
  const uint8_t* codes_u = a.codes + (int64_t)unit * a.cap * S + slot;
  const uint32_t* scales_u = reinterpret_cast<const uint32_t*>(a.scales) + (int64_t)unit * a.cap;
  const uint16_t* mu_u = a.mu + (int64_t)unit * (a.cap >> lgR) * kDim + oslot * SUB;
  // every row's codes, scales and block-mean channels are requested before
  // the codebook goes to LDS, so their latency overlaps the codebook's
  uint32_t code[ROWS], s2[ROWS], mw[ROWS][SUB / 2];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int t = min(a.tok0 + i0 + r * TPR, tlast);
    code[r] = codes_u[t * S];
    if (!a.dq) {
      s2[r] = scales_u[t];
      // the block mean's SUB channels of the output slot, one 8- or 16-byte load
      const uint16_t* mp = mu_u + (t >> lgR) * kDim;
      if constexpr (SUB == 4) {
        const uint2 m2 = *reinterpret_cast<const uint2*>(mp);
        mw[r][0] = m2.x;
        mw[r][1] = m2.y;
      } else {
        const uint4 m4 = *reinterpret_cast<const uint4*>(mp);
        mw[r][0] = m4.x;
        mw[r][1] = m4.y;
        mw[r][2] = m4.z;
        mw[r][3] = m4.w;
      }
    }
  }
  for (int i = threadIdx.x; i < kCodewords * SUB; i += 256) cbf[i] = h2f(a.codebook[i]);
  float sc[SUB];  // 1/sqrt(d), the lane's transform sign and the randomised-Hadamard sign of each output channel
#pragma unroll
  for (int e = 0; e < SUB; ++e)
    sc[e] = kInvSqrtD * hsign(slot) * (a.signs ? (float)a.signs[oslot * SUB + e] : 1.f);
  __syncthreads();
  const int64_t o_u = ((int64_t)unit * a.ntok + i0) * kDim + oslot * SUB;  // output element of row 0
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int i = i0 + r * TPR;  // output token
    const bool act = i < a.ntok;
    const bool live = !a.seq_quant || a.tok0 + i < a.seq_quant[unit / a.H];  // ragged: past the row's end -> 0
    const int t = min(a.tok0 + i, tlast);                                   // cache token
    const int64_t blk = (int64_t)unit * (a.cap >> lgR) + (t >> lgR);
    float n1, n2, mv[SUB];
    if (a.dq) {
      const uint8_t* rec = reinterpret_cast<const uint8_t*>(a.scales) + blk * dq_record_bytes(a.R);
      const uint32_t tq = dq_token(rec, a.R, t & (a.R - 1));
      n1 = dq_value(dq_s1_params(rec, a.R), tq >> 16);
      n2 = h2f(tq & 0xffff);
      const uint8_t* mrec = reinterpret_cast<const uint8_t*>(a.mu) + blk * kDqMuRecord;
#pragma unroll
      for (int e = 0; e < SUB; e += 2) dq_mu_pair(mrec, (oslot * SUB + e) / 2, mv[e], mv[e + 1]);
    } else {
      n1 = h2f(s2[r] & 0xffff);
      n2 = h2f(s2[r] >> 16);
#pragma unroll
      for (int e = 0; e < SUB; e += 2) {
        mv[e] = h2f(mw[r][e / 2] & 0xffff);
        mv[e + 1] = h2f(mw[r][e / 2] >> 16);
      }
    }
    float x[SUB];
#pragma unroll
    for (int e = 0; e < SUB; ++e) x[e] = cbf[code[r] * SUB + e];
    fwht_lanes<SUB>(x, slot);
#pragma unroll
    for (int e = 0; e < SUB; ++e) x[e] = live ? n1 * fmaf(n2, x[e] * sc[e], mv[e]) : 0.f;
    if (act) {
      // the output slot's SUB values in one store per lane; the lanes of a
      // token cover its 256 (fp16) or 512 (fp32) bytes
      const int64_t o = o_u + (int64_t)(r * TPR) * kDim;
      if (a.out_f16) {
        uint32_t w[SUB / 2];
#pragma unroll
        for (int e = 0; e < SUB; e += 2) w[e / 2] = (uint32_t)f2h(x[e]) | ((uint32_t)f2h(x[e + 1]) << 16);
        uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + o;
        if constexpr (SUB == 4) *reinterpret_cast<uint2*>(out) = uint2{w[0], w[1]};
        else *reinterpret_cast<uint4*>(out) = uint4{w[0], w[1], w[2], w[3]};
      } else {
        float4* out = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + o);
#pragma unroll
        for (int e = 0; e < SUB; e += 4) out[e / 4] = float4{x[e], x[e + 1], x[e + 2], x[e + 3]};
      }
    }
  }
}

hipError_t launch_dequant(const DequantArgs& a, int sub, int n_units, hipStream_t stream) {
  dim3 grid((a.ntok + 63) / 64, n_units), block(256);
  if (sub == 4) hipLaunchKernelGGL(dequant_kernel<4>, grid, block, 0, stream, a);
  else if (sub == 8) hipLaunchKernelGGL(dequant_kernel<8>, grid, block, 0, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// k-means (Lloyd).  Iteration = assign (nearest centroid, ties to the lowest
// index) with per-group LDS accumulation of member sums (fp64), counts and
// distortion, flushed to global fp64 accumulators; then a one-group update
// that moves non-empty centroids to their means and clears the accumulators
// for the next iteration.
//
// Assignment on the matrix cores, as the encoder's distance products:
// centroids are the rows and samples the columns of v_mfma_f32_32x32x16_f16
// tiles, and K carries
//   [x_hi, x_hi, x_lo] . [-2 c_hi, -2 c_lo, -2 c_hi] + [xx_hi, xx_lo, 1, 1] . [1, 1, cc_hi, cc_lo]
// with the fp32 sample x and centroid c split into fp16 halves (x = x_hi +
// x_lo), xx = |x|^2 and cc = |c|^2 + 2^-12 likewise, so a tile holds
// D = |x - c|^2 + 2^-12 up to the rounding of the fp32 sums and the dropped
// x_lo c_lo term (~1e-6 absolute for unit-scale data).  D's bits with the low
// byte replaced by the centroid index give packed keys whose unsigned minimum
// is the argmin (ties, and distances within 2^-15 relative, to the lowest
// index).  The winner's distortion is then recomputed in fp32 difference form.
// Samples with an element of magnitude >= 2^5 or |x|^2 >= 2^10, and every
// sample when a centroid is outside those bounds, take a per-lane fp32 loop
// over the centroids instead, where fp16 halves or the expanded form would
// lose accuracy.  At 1 bit (SUB = 8) the terms fill two K = 16 products.
constexpr float kKmMaxAbs = 32.f, kKmMaxSq = 1024.f;
constexpr float kKmEps = 0.000244140625f;  // 2^-12: keeps D > 0 through rounding

__device__ __forceinline__ uint32_t km_pack(half_t a, half_t b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}
__device__ __forceinline__ half8_t km_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(half8_t, uint4_t{a, b, c, d});
}
// (hi, lo) fp16 halves of v
__device__ __forceinline__ void km_split(float v, half_t& hi, half_t& lo) {
  hi = (half_t)v;
  lo = (half_t)(v - (float)hi);
}

template <int SUB>
__global__ __launch_bounds__(256) void kmeans_assign_kernel(KmeansArgs a) {
  constexpr int KS = SUB / 4;  // K = 16 products per 32-centroid tile
  __shared__ float cent[kCodewords * SUB];
  __shared__ double lsum[kCodewords * SUB];
  __shared__ double lcnt[kCodewords];
  __shared__ double ldist[4];
  __shared__ half8_t sA[8][KS][kWave];  // A operands, [tile][product][lane]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kCodewords * SUB; i += 256) {
    cent[i] = a.cent[i];
    lsum[i] = 0.0;
  }
  lcnt[tid] = 0.0;
  __syncthreads();
  // any centroid outside the products' range?  (one block-wide vote)
  bool cbad;
  {
    float cc = 0.f, mx = 0.f;
#pragma unroll
    for (int e = 0; e < SUB; ++e) {
      const float v = cent[tid * SUB + e];
      cc = fmaf(v, v, cc);
      mx = fmaxf(mx, fabsf(v));
    }
    cbad = __syncthreads_or(!(mx < kKmMaxAbs && cc < kKmMaxSq));
  }
  // A operands: tile t, lane (row i = lane % 32, K half kb = lane / 32),
  // centroid 32 t + i; wave w builds tiles 2 w, 2 w + 1
  const int ri = lane & 31, kb = lane >> 5;
#pragma unroll
  for (int t = 2 * wave; t < 2 * wave + 2; ++t) {
    const float* c = cent + (32 * t + ri) * SUB;
    half_t h[SUB], l[SUB];
    float cc = 0.f;
#pragma unroll
    for (int e = 0; e < SUB; ++e) {
      km_split(c[e], h[e], l[e]);
      cc = fmaf(c[e], c[e], cc);
    }
    half_t cch, ccl;
    km_split(cc + kKmEps, cch, ccl);
    const half_t one = (half_t)1.f, zero = (half_t)0.f;
    if constexpr (SUB == 4) {
      // kb 0: [-2 c_hi, -2 c_lo]; kb 1: [-2 c_hi, 1, 1, cc_hi, cc_lo]
      const uint32_t w0 = km_pack(-2 * h[0], -2 * h[1]), w1 = km_pack(-2 * h[2], -2 * h[3]);
      sA[t][0][lane] = kb == 0 ? km_half8(w0, w1, km_pack(-2 * l[0], -2 * l[1]), km_pack(-2 * l[2], -2 * l[3]))
                               : km_half8(w0, w1, km_pack(one, one), km_pack(cch, ccl));
    } else {
      // product 0: kb 0 [-2 c_hi], kb 1 [-2 c_lo]; product 1: kb 0 [-2 c_hi], kb 1 [1, 1, cc_hi, cc_lo, 0 ..]
      const half8_t hh = km_half8(km_pack(-2 * h[0], -2 * h[1]), km_pack(-2 * h[2], -2 * h[3]),
                                  km_pack(-2 * h[4], -2 * h[5]), km_pack(-2 * h[6], -2 * h[7]));
      const half8_t ll = km_half8(km_pack(-2 * l[0], -2 * l[1]), km_pack(-2 * l[2], -2 * l[3]),
                                  km_pack(-2 * l[4], -2 * l[5]), km_pack(-2 * l[6], -2 * l[7]));
      sA[t][0][lane] = kb == 0 ? hh : ll;
      sA[t][KS - 1][lane] = kb == 0 ? hh : km_half8(km_pack(one, one), km_pack(cch, ccl), km_pack(zero, zero), 0u);
    }
  }
  __syncthreads();
  const float16_t zacc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  double dl = 0.0;
  // each wave takes 64 samples per step, one per lane
  for (int64_t p0 = ((int64_t)blockIdx.x * 4 + wave) * 64; p0 < a.n; p0 += (int64_t)gridDim.x * 256) {
    const int64_t p = p0 + lane;
    const bool valid = p < a.n;
    float x[SUB];
    float xx = 0.f, mx = 0.f;
#pragma unroll
    for (int e = 0; e < SUB; ++e) {
      x[e] = valid ? a.samples[p * SUB + e] : 0.f;
      xx = fmaf(x[e], x[e], xx);
      mx = fmaxf(mx, fabsf(x[e]));
    }
    const bool fast = !cbad && mx < kKmMaxAbs && xx < kKmMaxSq;
    // this lane's K halves: P (K 0-7), Q (K 8-15) of each product
    uint32_t P[KS][4], Q[KS][4];
    {
      half_t h[SUB], l[SUB], xh, xl;
#pragma unroll
      for (int e = 0; e < SUB; ++e) km_split(fast ? x[e] : 0.f, h[e], l[e]);
      km_split(fast ? xx : 0.f, xh, xl);
      const half_t one = (half_t)1.f, zero = (half_t)0.f;
      if constexpr (SUB == 4) {
        P[0][0] = km_pack(h[0], h[1]);
        P[0][1] = km_pack(h[2], h[3]);
        P[0][2] = P[0][0];
        P[0][3] = P[0][1];
        Q[0][0] = km_pack(l[0], l[1]);
        Q[0][1] = km_pack(l[2], l[3]);
        Q[0][2] = km_pack(xh, xl);
        Q[0][3] = km_pack(one, one);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          P[0][i] = Q[0][i] = km_pack(h[2 * i], h[2 * i + 1]);
          P[KS - 1][i] = km_pack(l[2 * i], l[2 * i + 1]);
        }
        Q[KS - 1][0] = km_pack(xh, xl);
        Q[KS - 1][1] = km_pack(one, one);
        Q[KS - 1][2] = Q[KS - 1][3] = km_pack(zero, zero);
      }
    }
    // B operands: columns = the samples of lanes 0-31 (B0) and 32-63 (B1);
    // lane (n, kb) holds K 8 kb .. 8 kb + 7 of column n
    half8_t B0[KS], B1[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      uint32_t b0[4], b1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const auto r = __builtin_amdgcn_permlane32_swap(P[k][i], Q[k][i], false, false);
        b0[i] = r[0];
        b1[i] = r[1];
      }
      B0[k] = km_half8(b0[0], b0[1], b0[2], b0[3]);
      B1[k] = km_half8(b1[0], b1[1], b1[2], b1[3]);
    }
    // keys carry the index within the lane's rows (a constant per
    // accumulator); the lane's row offset 4 kb is added before the two
    // halves meet.  The mask sits in a VGPR so each key is one v_and_or_b32
    // with the index as its scalar operand.
    uint32_t vmask;
    asm("v_mov_b32 %0, %1" : "=v"(vmask) : "s"(0xffffff00u));
    uint32_t best0 = 0xffffffffu, best1 = 0xffffffffu;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      float16_t d0 = zacc, d1 = zacc;
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const half8_t A = sA[t][k][lane];
        d0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, B0[k], d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, B1[k], d1, 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        // accumulator q holds centroid 32 t + 8 (q / 4) + 4 kb + q % 4
        const uint32_t k = 32u * t + 8u * (q >> 2) + (q & 3);
        best0 = min(best0, (__float_as_uint(d0[q]) & vmask) | k);
        best1 = min(best1, (__float_as_uint(d1[q]) & vmask) | k);
      }
      __builtin_amdgcn_sched_barrier(0);  // one tile's accumulators live at a time
    }
    // lane l: the two half-lists of sample p0 + l
    uint32_t key;
    {
      const auto r = __builtin_amdgcn_permlane32_swap(best0 + 4u * kb, best1 + 4u * kb, false, false);
      key = min(r[0], r[1]);
    }
    int best = (int)(key & 0xffu);
    if (!fast && valid) {
      float bd = INFINITY;
      best = 0;
      for (int k = 0; k < kCodewords; ++k) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < SUB; ++e) {
          const float df = x[e] - cent[k * SUB + e];
          d = fmaf(df, df, d);
        }
        if (d < bd) {
          bd = d;
          best = k;
        }
      }
    }
    if (valid) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < SUB; ++e) {
        const float df = x[e] - cent[best * SUB + e];
        d = fmaf(df, df, d);
      }
#pragma unroll
      for (int e = 0; e < SUB; ++e) atomicAdd(&lsum[best * SUB + e], (double)x[e]);
      atomicAdd(&lcnt[best], 1.0);
      dl += (double)d;
    }
  }
  // wave sum of the distortion
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) dl += __shfl_xor(dl, m, kWave);
  if (lane == 0) ldist[wave] = dl;
  __syncthreads();
  for (int i = tid; i < kCodewords * SUB; i += 256)
    if (lsum[i] != 0.0) atomicAdd(&a.sums[i], lsum[i]);
  if (lcnt[tid] != 0.0) atomicAdd(&a.counts[tid], lcnt[tid]);
  if (tid == 0) atomicAdd(a.dsum, (ldist[0] + ldist[1]) + (ldist[2] + ldist[3]));
}

template <int SUB>
__global__ __launch_bounds__(256) void kmeans_update_kernel(KmeansArgs a) {
  const int k = threadIdx.x;
  const double cnt = a.counts[k];
  if (cnt > 0.0) {
#pragma unroll
    for (int e = 0; e < SUB; ++e) a.cent[k * SUB + e] = (float)(a.sums[k * SUB + e] / cnt);
  }
#pragma unroll
  for (int e = 0; e < SUB; ++e) a.sums[k * SUB + e] = 0.0;
  a.counts[k] = 0.0;
  __syncthreads();
  if (k == 0) {
    if (a.distortion) a.distortion[a.it] = (float)(*a.dsum / ((double)a.n * SUB));
    *a.dsum = 0.0;
  }
}

__global__ void kmeans_clear_kernel(double* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0.0;
}

__global__ void kmeans_finish_kernel(KmeansArgs a, int total) {
  for (int i = threadIdx.x; i < total; i += blockDim.x) a.codebook[i] = f2h(a.cent[i]);
}

hipError_t launch_kmeans_iter(const KmeansArgs& a, int sub, hipStream_t stream) {
  // two groups per CU: each group flushes 256 (SUB + 1) fp64 sums with global
  // atomics, which at 2048 groups cost more than the assignment itself
  const int64_t want = (a.n + 255) / 256;
  const int grid = (int)(want < 512 ? want : 512);
  if (sub == 4) {
    hipLaunchKernelGGL(kmeans_assign_kernel<4>, dim3(grid), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(kmeans_update_kernel<4>, dim3(1), dim3(256), 0, stream, a);
  } else if (sub == 8) {
    hipLaunchKernelGGL(kmeans_assign_kernel<8>, dim3(grid), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(kmeans_update_kernel<8>, dim3(1), dim3(256), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Cosine refinement of the codebook: full-batch gradient descent on the mean
// of 1 - cos(x, x_hat) over head vectors x [n][128], x_hat the concatenation of
// the nearest codewords of x's sub-vectors.  One group of S lanes per vector,
// one sub-vector per lane; the gradient d(1 - cos)/d x_hat of each sub-vector
// goes to its codeword through fp64 LDS sums, flushed to the global sums.

template <int SUB>
__global__ __launch_bounds__(256) void finetune_grad_kernel(KmeansArgs a) {
  constexpr int S = kDim / SUB;
  constexpr int VPW = kWave / S;  // vectors per wave
  __shared__ float cent[kCodewords * SUB];
  __shared__ double lsum[kCodewords * SUB];
  __shared__ double ldist[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = lane % S;
  for (int i = tid; i < kCodewords * SUB; i += 256) {
    cent[i] = a.cent[i];
    lsum[i] = 0.0;
  }
  __syncthreads();
  double dl = 0.0;
  const int64_t nvec = a.n;  // head vectors
  const int64_t stride = (int64_t)gridDim.x * 4 * VPW;
  for (int64_t v0 = ((int64_t)blockIdx.x * 4 + wave) * VPW; v0 < nvec; v0 += stride) {
    const int64_t v = v0 + lane / S;
    const bool act = v < nvec;
    float x[SUB];
#pragma unroll
    for (int e = 0; e < SUB; ++e) x[e] = act ? a.samples[v * kDim + slot * SUB + e] : 0.f;
    float bd = INFINITY;
    int best = 0;
    for (int k = 0; k < kCodewords; ++k) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < SUB; ++e) {
        const float df = x[e] - cent[k * SUB + e];
        d = fmaf(df, df, d);
      }
      if (d < bd) {
        bd = d;
        best = k;
      }
    }
    float xh[SUB], ax = 0.f, xx = 0.f, hh = 0.f;
#pragma unroll
    for (int e = 0; e < SUB; ++e) {
      xh[e] = cent[best * SUB + e];
      ax = fmaf(x[e], xh[e], ax);
      xx = fmaf(x[e], x[e], xx);
      hh = fmaf(xh[e], xh[e], hh);
    }
    ax = group_sum<S>(ax);
    xx = group_sum<S>(xx);
    hh = group_sum<S>(hh);
    if (act) {
      if (xx > 0.f && hh > 0.f) {
        const float nx = sqrtf(xx), nh = sqrtf(hh);
        const float cosv = ax / (nx * nh);
        const float gx = 1.f / (nx * nh), gh = cosv / hh;
#pragma unroll
        for (int e = 0; e < SUB; ++e) atomicAdd(&lsum[best * SUB + e], (double)(gh * xh[e] - gx * x[e]));
        if (slot == 0) dl += 1.0 - (double)cosv;
      } else if (slot == 0) {
        dl += 1.0;
      }
    }
  }
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) dl += __shfl_xor(dl, m, kWave);
  if (lane == 0) ldist[wave] = dl;
  __syncthreads();
  for (int i = tid; i < kCodewords * SUB; i += 256)
    if (lsum[i] != 0.0) atomicAdd(&a.sums[i], lsum[i]);
  if (tid == 0) atomicAdd(a.dsum, (ldist[0] + ldist[1]) + (ldist[2] + ldist[3]));
}

template <int SUB>
__global__ __launch_bounds__(256) void finetune_update_kernel(KmeansArgs a) {
  const int k = threadIdx.x;
#pragma unroll
  for (int e = 0; e < SUB; ++e) {
    a.cent[k * SUB + e] = (float)((double)a.cent[k * SUB + e] - a.lr * (a.sums[k * SUB + e] / (double)a.n));
    a.sums[k * SUB + e] = 0.0;
  }
  __syncthreads();
  if (k == 0) {
    if (a.distortion) a.distortion[a.it] = (float)(*a.dsum / (double)a.n);
    *a.dsum = 0.0;
  }
}

hipError_t launch_finetune_iter(const KmeansArgs& a, int sub, hipStream_t stream) {
  const int vpb = 4 * (kWave / (kDim / sub));
  const int64_t want = (a.n + vpb - 1) / vpb;
  const int grid = (int)(want < 2048 ? want : 2048);
  if (sub == 4) {
    hipLaunchKernelGGL(finetune_grad_kernel<4>, dim3(grid), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(finetune_update_kernel<4>, dim3(1), dim3(256), 0, stream, a);
  } else if (sub == 8) {
    hipLaunchKernelGGL(finetune_grad_kernel<8>, dim3(grid), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(finetune_update_kernel<8>, dim3(1), dim3(256), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_kmeans_init(const float* src, float* cent, int sub, hipStream_t stream) {
  hipError_t e = hipMemcpyAsync(cent, src, sizeof(float) * kCodewords * sub, hipMemcpyDeviceToDevice, stream);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t launch_kmeans_clear(double* acc, int n, hipStream_t stream) {
  hipLaunchKernelGGL(kmeans_clear_kernel, dim3(1), dim3(256), 0, stream, acc, n);
  return hipGetLastError();
}

hipError_t launch_kmeans_finish(const KmeansArgs& a, int sub, hipStream_t stream) {
  hipLaunchKernelGGL(kmeans_finish_kernel, dim3(1), dim3(256), 0, stream, a, kCodewords * sub);
  return hipGetLastError();
}

}  // namespace nsnq
