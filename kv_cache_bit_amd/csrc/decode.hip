// decode.hip -- split-K decode attention over the NSNQuant-compressed cache,
// the LSE combine, and an fp16-cache comparator (gfx950).
//
// For a key stored as codes c_t, scales (N1, N2) and block mean MU_b,
//   q . k_hat_t = N1 (N2 (Hq) . c_hat_t + q . MU_b),
// and (Hq) . c_hat_t = sum_j LUT_j[c_tj] with LUT_j[c] = (Hq)_j . C[c] (the j-th
// s-element slice).  For the values,
//   sum_t p_t v_hat_t = H^T( sum_j sum_c Hist_j[c] C[c] ) + sum_b beta_b MU_b,
//   Hist_j[c] = sum_{t: c_tj = c} p_t N1_t N2_t,   beta_b = sum_{t in b} p_t N1_t.
// So a work-group streams only codes and fp16 scalars from HBM: pass 1 gathers
// LUT entries (LDS) into scores; pass 2 forms sum_t w_t c_hat_t in the Hadamard
// domain by gathering codewords from LDS (each lane owns 16 channels and a
// strided subset of tokens).  That is the codeword histogram Hist_j[c] applied
// to the codebook without materialising it: LDS float atomics serialise on
// gfx950.  The inverse Hadamard runs once per split.  Residual fp16 tokens get
// a split of their own.

#include "nsnq_device.hpp"
#include "nsnq_launch.hpp"

namespace nsnq {


constexpr int kLutStride = 257;  // odd row stride: finish-step reads hit distinct banks

struct DecodeSmem {
  // offsets in floats
  int qf, qr, cbf, lut, sc, qmu, beta, om, red, vred, total;
};

// Blocks of R tokens one split may span (mean-term registers per wave: 4).
constexpr int kMaxSplitBlocks = 16;

__host__ __device__ inline DecodeSmem decode_smem(int sub, int gh, int split_tokens, int R) {
  const int S = kDim / sub;
  const int nb = split_tokens / R;
  DecodeSmem s;
  int o = 0;
  s.qf = o; o += gh * kDim;
  s.qr = o; o += gh * kDim;
  s.cbf = o; o += kCodewords * sub;
  s.lut = o; o += gh * S * kLutStride;
  s.sc = o; o += gh * split_tokens;
  s.qmu = o; o += gh * nb;
  s.beta = o; o += gh * nb;
  s.om = o; o += gh * kDim;
  s.red = o; o += 2 * 4 * gh;
  s.vred = o; o += 4 * gh * kDim;
  s.total = o;
  return s;
}

size_t decode_lds_bytes(int sub, int gh, int split_tokens, int R) {
  return (size_t)decode_smem(sub, gh, split_tokens, R).total * sizeof(float);
}

int decode_max_split_tokens(int sub, int gh, int R) {
  const size_t cap = 160 * 1024;
  int best = 0;
  for (int ts = R; ts <= kMaxSplitBlocks * R; ts += R)
    if (decode_lds_bytes(sub, gh, ts, R) <= cap) best = ts;
  return best;
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

template <int S>
__device__ __forceinline__ void load_codes(const uint8_t* p, uint32_t (&cw)[S / 4]) {
#pragma unroll
  for (int i = 0; i < S / 16; ++i) {
    const uint4 v4 = *reinterpret_cast<const uint4*>(p + 16 * i);
    cw[4 * i] = v4.x; cw[4 * i + 1] = v4.y; cw[4 * i + 2] = v4.z; cw[4 * i + 3] = v4.w;
  }
}

// Residual split: fp16 keys and values, one query token per head.
template <int GH>
__device__ __forceinline__ void decode_residual(const DecodeArgs& a, float* qf, float* sc, float* ov, float* red,
                                                float* ws_base, int64_t ws_head, int64_t unit, int TS) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nt = a.n_resid;
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

template <int SUB, int GH>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr int S = kDim / SUB;
  constexpr int CW = S / 4;  // 32-bit words of codes per token
  extern __shared__ float smem[];
  const int TS = a.split_tokens;
  const DecodeSmem L = decode_smem(SUB, GH, TS, a.R);
  float* qf = smem + L.qf;
  float* qr = smem + L.qr;
  float* cbf = smem + L.cbf;
  float* lut = smem + L.lut;
  float* sc = smem + L.sc;
  float* qmu = smem + L.qmu;
  float* beta = smem + L.beta;
  float* om = smem + L.om;
  float* red = smem + L.red;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x;
  const int groups = a.G / GH;
  const int hg = blockIdx.y % groups;
  const int bk = blockIdx.y / groups;
  const int b = bk / a.Hkv, hk = bk % a.Hkv;
  const int h0 = hk * a.G + hg * GH;
  const int64_t unit = (int64_t)b * a.Hkv + hk;
  const int nbmu = a.cap / a.R;
  float* ws_base = a.ws + ((int64_t)b * a.Hq + h0) * a.nsplit * (kDim + 2) + (int64_t)split * (kDim + 2);
  const int64_t ws_head = (int64_t)a.nsplit * (kDim + 2);

  for (int i = tid; i < GH * kDim; i += 256) {
    const int g = i / kDim, c = i % kDim;
    qf[i] = h2f(a.q[((int64_t)b * a.Hq + h0 + g) * kDim + c]);
  }

  if (split >= a.nsplit_q) {
    decode_residual<GH>(a, qf, sc, lut, red, ws_base, ws_head, unit, TS);
    return;
  }

  // ---------------- compressed tokens ----------------
  const int t0 = split * TS;
  const int ntok = min(TS, a.n_quant - t0);
  const int nb = ntok / a.R;
  const uint8_t* kc = a.kcodes + (unit * a.cap + t0) * S;
  const uint32_t* ks = reinterpret_cast<const uint32_t*>(a.kscales) + unit * a.cap + t0;
  const uint8_t* vc = a.vcodes + (unit * a.cap + t0) * S;
  const uint32_t* vs = reinterpret_cast<const uint32_t*>(a.vscales) + unit * a.cap + t0;
  const int iters = (ntok + 255) / 256;

  // issue the first token loads and the block means before the LUT work
  uint32_t kcw[CW], ksc = 0, vsc = 0;
  if (tid < ntok) {
    load_codes<S>(kc + (int64_t)tid * S, kcw);
    ksc = ks[tid];
    vsc = vs[tid];
  }
  uint32_t kmu_r[kMaxSplitBlocks / 4], vmu_r[kMaxSplitBlocks / 4];
#pragma unroll
  for (int i = 0; i < kMaxSplitBlocks / 4; ++i) {
    const int bl = wave + 4 * i;
    kmu_r[i] = vmu_r[i] = 0;
    if (bl < nb) {
      const int64_t row = (unit * nbmu + t0 / a.R + bl) * kDim + 2 * lane;
      kmu_r[i] = *reinterpret_cast<const uint32_t*>(a.kmu + row);
      vmu_r[i] = *reinterpret_cast<const uint32_t*>(a.vmu + row);
    }
  }
  for (int i = tid; i < kCodewords * SUB; i += 256) cbf[i] = h2f(a.codebook[i]);
  for (int i = tid; i < GH * kDim; i += 256) om[i] = 0.f;
  __syncthreads();

  // rotate the queries (one wave per head); q . MU_b per block
  if (wave < GH) {
    float x[2] = {qf[wave * kDim + 2 * lane], qf[wave * kDim + 2 * lane + 1]};
    fwht128<2>(x, lane);
    qr[wave * kDim + 2 * lane] = x[0] * kInvSqrtD;
    qr[wave * kDim + 2 * lane + 1] = x[1] * kInvSqrtD;
  }
#pragma unroll
  for (int i = 0; i < kMaxSplitBlocks / 4; ++i) {
    const int bl = wave + 4 * i;
    if (bl < nb) {
      const float m0 = h2f(kmu_r[i] & 0xffff), m1 = h2f(kmu_r[i] >> 16);
#pragma unroll
      for (int g = 0; g < GH; ++g) {
        float d = fmaf(qf[g * kDim + 2 * lane], m0, qf[g * kDim + 2 * lane + 1] * m1);
        d = group_sum<kWave>(d);
        if (lane == 0) qmu[g * nb + bl] = d;
      }
    }
  }
  __syncthreads();

  // LUT_j[c] = (Hq)_j . C[c]; thread = codeword
  {
    const int c = tid;
    float cv[SUB];
#pragma unroll
    for (int e = 0; e < SUB; ++e) cv[e] = cbf[c * SUB + e];
#pragma unroll
    for (int g = 0; g < GH; ++g) {
#pragma unroll 8
      for (int j = 0; j < S; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < SUB; ++e) acc = fmaf(qr[g * kDim + j * SUB + e], cv[e], acc);
        lut[(g * S + j) * kLutStride + c] = acc;
      }
    }
  }
  __syncthreads();

  // pass 1: scores from K codes
  float m[GH];
#pragma unroll
  for (int g = 0; g < GH; ++g) m[g] = -INFINITY;
  for (int it = 0; it < iters; ++it) {
    const int t = it * 256 + tid;
    if (t < ntok) {
      if (it > 0) {
        load_codes<S>(kc + (int64_t)t * S, kcw);
        ksc = ks[t];
      }
      const float n1 = h2f(ksc & 0xffff), n2 = h2f(ksc >> 16);
      const int bl = t / a.R;
#pragma unroll
      for (int g = 0; g < GH; ++g) {
        const float* lg = lut + g * S * kLutStride;
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int j = 0; j < S; j += 2) {
          acc0 += lg[j * kLutStride + ((kcw[j >> 2] >> (8 * (j & 3))) & 0xffu)];
          acc1 += lg[(j + 1) * kLutStride + ((kcw[(j + 1) >> 2] >> (8 * ((j + 1) & 3))) & 0xffu)];
        }
        const float sv = a.scale_log2 * n1 * fmaf(n2, acc0 + acc1, qmu[g * nb + bl]);
        sc[g * TS + t] = sv;
        m[g] = fmaxf(m[g], sv);
      }
    }
  }
  block_reduce<GH, true>(m, red, lane, wave);

  // softmax weights times the V scales: w_t = p_t N1_t N2_t, beta_b += p_t N1_t
  for (int i = tid; i < GH * nb; i += 256) beta[i] = 0.f;
  float l[GH];
#pragma unroll
  for (int g = 0; g < GH; ++g) l[g] = 0.f;
  __syncthreads();
  for (int it = 0; it < iters; ++it) {
    const int t = it * 256 + tid;
    float pn1[GH];
#pragma unroll
    for (int g = 0; g < GH; ++g) pn1[g] = 0.f;
    if (t < ntok) {
      if (it > 0) vsc = vs[t];
      const float n1 = h2f(vsc & 0xffff), n2 = h2f(vsc >> 16);
#pragma unroll
      for (int g = 0; g < GH; ++g) {
        const float pr = exp2f(sc[g * TS + t] - m[g]);
        l[g] += pr;
        pn1[g] = pr * n1;
        sc[g * TS + t] = pr * n1 * n2;
      }
    }
    // a wave's 64 tokens lie in one mean block (64 divides R, splits are R-aligned)
    const int bl = (it * 256 + wave * 64) / a.R;
#pragma unroll
    for (int g = 0; g < GH; ++g) {
      const float sum = group_sum<kWave>(pn1[g]);
      if (lane == 0 && bl < nb) atomicAdd(beta + g * nb + bl, sum);
    }
  }
  block_reduce<GH, false>(l, red, lane, wave);  // also publishes w_t in sc

  // pass 2: o_hat = sum_t w_t c_hat_t.  Lane (sq, tg) owns 16 channels (4 slots
  // at 2 bits, 2 at 1 bit) and tokens tg, tg + 32, ...
  constexpr int SPT = 16 / SUB;  // slots per thread
  const int sq = tid & 7, tg = tid >> 3;
  float acc[GH][16];
#pragma unroll
  for (int g = 0; g < GH; ++g)
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[g][c] = 0.f;
  const uint8_t* vrow = vc + sq * SPT;
  for (int t = tg; t < ntok; t += 32) {
    uint32_t cw;
    if constexpr (SPT == 4) cw = *reinterpret_cast<const uint32_t*>(vrow + (int64_t)t * S);
    else cw = *reinterpret_cast<const uint16_t*>(vrow + (int64_t)t * S);
    float wg[GH];
#pragma unroll
    for (int g = 0; g < GH; ++g) wg[g] = sc[g * TS + t];
#pragma unroll
    for (int si = 0; si < SPT; ++si) {
      const uint32_t code = (cw >> (8 * si)) & 0xffu;
      const float4* cp = reinterpret_cast<const float4*>(cbf + code * SUB);
#pragma unroll
      for (int hh = 0; hh < SUB / 4; ++hh) {
        const float4 c4 = cp[hh];
#pragma unroll
        for (int g = 0; g < GH; ++g) {
          float* ag = &acc[g][si * SUB + 4 * hh];
          ag[0] = fmaf(wg[g], c4.x, ag[0]);
          ag[1] = fmaf(wg[g], c4.y, ag[1]);
          ag[2] = fmaf(wg[g], c4.z, ag[2]);
          ag[3] = fmaf(wg[g], c4.w, ag[3]);
        }
      }
    }
  }
  // reduce over the 8 token groups of the wave (lane bits 3..5), then the waves
#pragma unroll
  for (int g = 0; g < GH; ++g)
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      float v = acc[g][c];
      v += xshfl(v, 8);
      v += xshfl(v, 16);
      v += xshfl(v, 32);
      acc[g][c] = v;
    }
  float* vred = smem + L.vred;
  if (lane < 8) {
#pragma unroll
    for (int g = 0; g < GH; ++g)
#pragma unroll
      for (int c = 0; c < 16; ++c) vred[(wave * GH + g) * kDim + sq * 16 + c] = acc[g][c];
  }
  __syncthreads();
  for (int o = tid; o < GH * kDim; o += 256) {
    const int g = o / kDim, c = o % kDim;
    qr[o] = (vred[(0 * GH + g) * kDim + c] + vred[(1 * GH + g) * kDim + c]) +
            (vred[(2 * GH + g) * kDim + c] + vred[(3 * GH + g) * kDim + c]);
  }
  // mean terms: sum_b beta_b MU_b, from the V means this wave prefetched
#pragma unroll
  for (int i = 0; i < kMaxSplitBlocks / 4; ++i) {
    const int bl = wave + 4 * i;
    if (bl < nb) {
      const float m0 = h2f(vmu_r[i] & 0xffff), m1 = h2f(vmu_r[i] >> 16);
#pragma unroll
      for (int g = 0; g < GH; ++g) {
        const float be = beta[g * nb + bl];
        atomicAdd(om + g * kDim + 2 * lane, be * m0);
        atomicAdd(om + g * kDim + 2 * lane + 1, be * m1);
      }
    }
  }
  __syncthreads();
  // inverse Hadamard of o_hat (one wave per head) plus the mean terms
  if (wave < GH) {
    const int g = wave;
    float x[2] = {qr[g * kDim + 2 * lane], qr[g * kDim + 2 * lane + 1]};
    fwht128<2>(x, lane);
    float* wo = ws_base + g * ws_head;
    wo[2 * lane] = fmaf(x[0], kInvSqrtD, om[g * kDim + 2 * lane]);
    wo[2 * lane + 1] = fmaf(x[1], kInvSqrtD, om[g * kDim + 2 * lane + 1]);
    if (lane == 0) {
      wo[kDim] = m[g];
      wo[kDim + 1] = l[g];
    }
  }
}

// out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i.  The (m_i, l_i) pairs
// go through LDS so every load is issued before any is consumed.

__global__ __launch_bounds__(128) void combine_kernel(CombineArgs a) {
  __shared__ float ml[2 * kMaxSplits];
  __shared__ float red[2];
  const int bh = blockIdx.x;
  const int c = threadIdx.x;
  const float* w = a.ws + (int64_t)bh * a.nsplit * (kDim + 2);
  float M = -INFINITY;
  for (int i = c; i < a.nsplit; i += 128) {
    const float mi = w[i * (kDim + 2) + kDim];
    ml[2 * i] = mi;
    ml[2 * i + 1] = w[i * (kDim + 2) + kDim + 1];
    M = fmaxf(M, mi);
  }
  M = group_max<kWave>(M);
  if ((c & 63) == 0) red[c >> 6] = M;
  __syncthreads();
  M = fmaxf(red[0], red[1]);
  float num = 0.f, den = 0.f;
  int i = 0;
  for (; i + 8 <= a.nsplit; i += 8) {
    float o[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) o[u] = w[(i + u) * (kDim + 2) + c];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float f = exp2f(ml[2 * (i + u)] - M);
      num = fmaf(f, o[u], num);
      den = fmaf(f, ml[2 * (i + u) + 1], den);
    }
  }
  for (; i < a.nsplit; ++i) {
    const float f = exp2f(ml[2 * i] - M);
    num = fmaf(f, w[i * (kDim + 2) + c], num);
    den = fmaf(f, ml[2 * i + 1], den);
  }
  a.out[(int64_t)bh * kDim + c] = f2h(num / den);
}

template <int SUB, int GH>
static hipError_t launch_decode_t(const DecodeArgs& a, int B, size_t lds, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_split_kernel<SUB, GH>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid(a.nsplit, B * a.Hkv * (a.G / GH)), block(256);
  hipLaunchKernelGGL((decode_split_kernel<SUB, GH>), grid, block, lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int sub, int gh, int B, size_t lds, hipStream_t stream) {
  if (sub == 4) {
    if (gh == 1) return launch_decode_t<4, 1>(a, B, lds, stream);
    if (gh == 2) return launch_decode_t<4, 2>(a, B, lds, stream);
    if (gh == 4) return launch_decode_t<4, 4>(a, B, lds, stream);
  } else if (sub == 8) {
    if (gh == 1) return launch_decode_t<8, 1>(a, B, lds, stream);
    if (gh == 2) return launch_decode_t<8, 2>(a, B, lds, stream);
    if (gh == 4) return launch_decode_t<8, 4>(a, B, lds, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_combine(const CombineArgs& a, int B, hipStream_t stream) {
  hipLaunchKernelGGL(combine_kernel, dim3(B * a.Hq), dim3(128), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp16 comparator: one work-group per (batch row, KV head, split); the G query
// heads of the KV head share every K/V read.  Scores: each lane owns one token
// of the wave's 64 and forms its G dot products from the token row (read as
// 16-byte chunks) against the queries in LDS.  Values: one wave per token row,
// lanes own 2 channels.
template <int G>
__global__ __launch_bounds__(256) void fp16_decode_kernel(Fp16DecodeArgs a) {
  extern __shared__ float smem[];
  const int TS = a.split_tokens;
  float* qf = smem;                 // [G][128]
  float* sc = qf + G * kDim;        // [G][TS]
  float* ov = sc + G * TS;          // [4][G][128]
  float* red = ov + 4 * G * kDim;   // [4][G]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x;
  const int bk = blockIdx.y;
  const int b = bk / a.Hkv, hk = bk % a.Hkv;
  const int h0 = hk * G;
  const int t0 = split * TS;
  const int nt = min(TS, a.T - t0);
  const uint16_t* K = a.k + ((int64_t)bk * a.T + t0) * kDim;
  const uint16_t* V = a.v + ((int64_t)bk * a.T + t0) * kDim;
  for (int i = tid; i < G * kDim; i += 256) qf[i] = h2f(a.q[((int64_t)b * a.Hq + h0) * kDim + i]);
  __syncthreads();
  for (int t = tid; t < nt; t += 256) {
    float acc[G];
    _Pragma("unroll") for (int g = 0; g < G; ++g) acc[g] = 0.f;
    const uint4* row = reinterpret_cast<const uint4*>(K + (int64_t)t * kDim);
#pragma unroll 4
    for (int ch = 0; ch < 16; ++ch) {
      const uint4 v4 = row[ch];
      const uint32_t w[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float k0 = h2f(w[i] & 0xffff), k1 = h2f(w[i] >> 16);
        const int c = ch * 8 + 2 * i;
        _Pragma("unroll") for (int g = 0; g < G; ++g) acc[g] = fmaf(qf[g * kDim + c], k0, fmaf(qf[g * kDim + c + 1], k1, acc[g]));
      }
    }
    _Pragma("unroll") for (int g = 0; g < G; ++g) sc[g * TS + t] = acc[g] * a.scale_log2;
  }
  __syncthreads();
  // max and sum per head (G <= 8)
  float m[G], l[G];
  _Pragma("unroll") for (int g = 0; g < G; ++g) {
    float v = -INFINITY;
    for (int t = tid; t < nt; t += 256) v = fmaxf(v, sc[g * TS + t]);
    m[g] = group_max<kWave>(v);
  }
  if (lane == 0)
    _Pragma("unroll") for (int g = 0; g < G; ++g) red[wave * G + g] = m[g];
  __syncthreads();
  _Pragma("unroll") for (int g = 0; g < G; ++g)
    m[g] = fmaxf(fmaxf(red[g], red[G + g]), fmaxf(red[2 * G + g], red[3 * G + g]));
  __syncthreads();
  _Pragma("unroll") for (int g = 0; g < G; ++g) {
    float v = 0.f;
    for (int t = tid; t < nt; t += 256) {
      const float p = exp2f(sc[g * TS + t] - m[g]);
      sc[g * TS + t] = p;
      v += p;
    }
    l[g] = group_sum<kWave>(v);
  }
  if (lane == 0)
    _Pragma("unroll") for (int g = 0; g < G; ++g) red[wave * G + g] = l[g];
  __syncthreads();
  _Pragma("unroll") for (int g = 0; g < G; ++g) l[g] = (red[g] + red[G + g]) + (red[2 * G + g] + red[3 * G + g]);
  // values
  float o0[G], o1[G];
  _Pragma("unroll") for (int g = 0; g < G; ++g) o0[g] = o1[g] = 0.f;
  for (int t = wave; t < nt; t += 4) {
    const uint32_t vv = *reinterpret_cast<const uint32_t*>(V + (int64_t)t * kDim + 2 * lane);
    const float v0 = h2f(vv & 0xffff), v1 = h2f(vv >> 16);
    _Pragma("unroll") for (int g = 0; g < G; ++g) {
      const float p = sc[g * TS + t];
      o0[g] = fmaf(p, v0, o0[g]);
      o1[g] = fmaf(p, v1, o1[g]);
    }
  }
  _Pragma("unroll") for (int g = 0; g < G; ++g) {
    ov[(wave * G + g) * kDim + 2 * lane] = o0[g];
    ov[(wave * G + g) * kDim + 2 * lane + 1] = o1[g];
  }
  __syncthreads();
  for (int o = tid; o < G * kDim; o += 256) {
    const int g = o / kDim, c = o % kDim;
    const float s = (ov[(0 * G + g) * kDim + c] + ov[(1 * G + g) * kDim + c]) +
                    (ov[(2 * G + g) * kDim + c] + ov[(3 * G + g) * kDim + c]);
    float* wo = a.ws + (((int64_t)b * a.Hq + h0 + g) * a.nsplit + split) * (kDim + 2);
    wo[c] = s;
    if (c == 0) {
      wo[kDim] = m[g];
      wo[kDim + 1] = l[g];
    }
  }
}

template <int G>
static hipError_t launch_fp16_t(const Fp16DecodeArgs& a, int B, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fp16_decode_kernel<G>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const size_t lds = fp16_decode_lds_bytes(G, a.split_tokens);
  hipLaunchKernelGGL((fp16_decode_kernel<G>), dim3(a.nsplit, B * a.Hkv), dim3(256), lds, stream, a);
  return hipGetLastError();
}

size_t fp16_decode_lds_bytes(int G, int split_tokens) {
  return sizeof(float) * ((size_t)G * kDim + (size_t)G * split_tokens + 4 * (size_t)G * kDim + 4 * G);
}

hipError_t launch_fp16_decode(const Fp16DecodeArgs& a, int B, hipStream_t stream) {
  switch (a.G) {
    case 1: return launch_fp16_t<1>(a, B, stream);
    case 2: return launch_fp16_t<2>(a, B, stream);
    case 4: return launch_fp16_t<4>(a, B, stream);
    case 8: return launch_fp16_t<8>(a, B, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nsnq
