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
  const int unit = blockIdx.y;
  for (int i = threadIdx.x; i < kCodewords * SUB; i += 256) cbf[i] = h2f(a.codebook[i]);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int i = blockIdx.x * TPB + wave * (TPB / 4) + r * TPR + tir;  // output token
    const bool act = i < a.ntok;
    const bool live = !a.seq_quant || a.tok0 + i < a.seq_quant[unit / a.H];  // ragged: past the row's end -> 0
    const int t = a.tok0 + (act ? i : 0);                               // cache token
    const int64_t ct = (int64_t)unit * a.cap + t;
    const int64_t blk = (int64_t)unit * (a.cap / a.R) + t / a.R;
    const uint32_t code = a.codes[ct * S + slot];
    float n1, n2, mv[SUB];
    if (a.dq) {
      const uint8_t* rec = reinterpret_cast<const uint8_t*>(a.scales) + blk * dq_record_bytes(a.R);
      const uint32_t tq = dq_token(rec, a.R, t % a.R);
      n1 = dq_value(dq_s1_params(rec, a.R), tq >> 16);
      n2 = h2f(tq & 0xffff);
      const uint8_t* mrec = reinterpret_cast<const uint8_t*>(a.mu) + blk * kDqMuRecord;
#pragma unroll
      for (int e = 0; e < SUB; e += 2) dq_mu_pair(mrec, (slot * SUB + e) / 2, mv[e], mv[e + 1]);
    } else {
      const uint32_t sc = reinterpret_cast<const uint32_t*>(a.scales)[ct];
      n1 = h2f(sc & 0xffff);
      n2 = h2f(sc >> 16);
      const uint16_t* mp = a.mu + blk * kDim + slot * SUB;
#pragma unroll
      for (int e = 0; e < SUB; ++e) mv[e] = h2f(mp[e]);
    }
    float x[SUB];
#pragma unroll
    for (int e = 0; e < SUB; ++e) x[e] = cbf[code * SUB + e];
    fwht128<SUB>(x, lane);
#pragma unroll
    for (int e = 0; e < SUB; ++e) {
      const float sg = a.signs ? (float)a.signs[slot * SUB + e] : 1.f;
      x[e] = live ? n1 * fmaf(n2, x[e] * (kInvSqrtD * sg), mv[e]) : 0.f;
    }
    if (act) {
      const int64_t o = ((int64_t)unit * a.ntok + i) * kDim + slot * SUB;
      if (a.out_f16) {
        uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + o;
#pragma unroll
        for (int e = 0; e < SUB; ++e) out[e] = f2h(x[e]);
      } else {
        float* out = reinterpret_cast<float*>(a.out) + o;
#pragma unroll
        for (int e = 0; e < SUB; ++e) out[e] = x[e];
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
// k-means (Lloyd).  Iteration = assign (fp32 squared distances in difference
// form, ties to the lowest index) with per-group LDS accumulation of member
// sums (fp64), counts and distortion, flushed to global fp64 accumulators;
// then a one-group update that moves non-empty centroids to their means and
// clears the accumulators for the next iteration.

template <int SUB>
__global__ __launch_bounds__(256) void kmeans_assign_kernel(KmeansArgs a) {
  __shared__ float cent[kCodewords * SUB];
  __shared__ double lsum[kCodewords * SUB];
  __shared__ double lcnt[kCodewords];
  __shared__ double ldist[4];
  const int tid = threadIdx.x;
  for (int i = tid; i < kCodewords * SUB; i += 256) {
    cent[i] = a.cent[i];
    lsum[i] = 0.0;
  }
  lcnt[tid] = 0.0;
  __syncthreads();
  double dl = 0.0;
  for (int64_t p = (int64_t)blockIdx.x * 256 + tid; p < a.n; p += (int64_t)gridDim.x * 256) {
    float x[SUB];
#pragma unroll
    for (int e = 0; e < SUB; ++e) x[e] = a.samples[p * SUB + e];
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
#pragma unroll
    for (int e = 0; e < SUB; ++e) atomicAdd(&lsum[best * SUB + e], (double)x[e]);
    atomicAdd(&lcnt[best], 1.0);
    dl += (double)bd;
  }
  // wave sum of the distortion
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) dl += __shfl_xor(dl, m, kWave);
  if ((tid & 63) == 0) ldist[tid >> 6] = dl;
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
  const int64_t want = (a.n + 255) / 256;
  const int grid = (int)(want < 2048 ? want : 2048);
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
