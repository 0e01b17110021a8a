// fp16_decode.hip -- decode attention over an uncompressed fp16 K/V cache,
// the comparator the compressed cache is measured against (gfx950).
//
// One work-group of 4 waves per (batch row, KV head, split); the G query heads
// of a KV head share every K/V read.  Each wave streams steps of 32 tokens
// (16 KB), the next step's loads in flight while the current one is used:
//   scores  on the matrix cores: v_mfma_f32_16x16x32_f16 with the K rows as
//           the A operand (lane (m16, kb) loads 8 channels of token m16, the
//           16 bytes the operand needs, straight from memory) and the queries
//           as B (fp16 inputs, so the products are exact in the fp32 sums);
//   softmax online per head, with a lazily moved reference as in the
//           compressed-cache kernels;
//   values  lane (c8, tr) loads 8 channels of tokens 4 j + tr and accumulates
//           p v with mixed-precision fmas; the step's p go through LDS.
// Every load is a 16-byte buffer load bounded by the split, so a step past
// the end reads zeros without touching memory and needs no branch.

#include "nsnq_device.hpp"
#include "nsnq_launch.hpp"
#include "decode_common.hpp"

namespace nsnq {

namespace {
constexpr int kStep = 32;       // tokens per wave step
constexpr float kLazy16 = 3.f;  // log2 headroom of the running reference
}  // namespace

template <int G>
__global__ __launch_bounds__(256) void fp16_decode_kernel(Fp16DecodeArgs a) {
  __shared__ float pbuf[4][2][G][4][8];      // per wave and step parity: p as [head][tr][j], token 4 j + tr
  __shared__ float mrg[4][G][kDim + 2];      // per wave: m, l, o
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m16 = lane & 15, kb = lane >> 4;  // score layout: token row m16, channel block kb
  const int c8 = lane & 15, tr = lane >> 4;   // value layout: channels 8 c8 .., tokens 4 j + tr
  const int split = blockIdx.x, bk = blockIdx.y;
  const int b = bk / a.Hkv, hk = bk % a.Hkv;
  const int h0 = hk * G;
  const int t0 = split * a.split_tokens;
  const int nt = max(0, min(a.split_tokens, a.T - t0));
  const int nsteps = (nt + kStep - 1) / kStep;
  const uint16_t* K = a.k + ((int64_t)bk * a.T + t0) * kDim;
  const uint16_t* V = a.v + ((int64_t)bk * a.T + t0) * kDim;
  const buf_rsrc_t rk = make_rsrc(K, nt * kDim * 2), rv = make_rsrc(V, nt * kDim * 2);

  // B operands: q[head m16][32 i + 8 kb .. + 7] (zeros for columns >= G)
  half8_t qb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4_t w = {0u, 0u, 0u, 0u};
    if (m16 < G) w = *reinterpret_cast<const uint4_t*>(a.q + ((int64_t)b * a.Hq + h0 + m16) * kDim + 32 * i + 8 * kb);
    qb[i] = __builtin_bit_cast(half8_t, w);
  }

  struct StepLd {
    uint4_t k[2][4];  // [tile][k-step]: token 16 tile + m16, channels 32 ks + 8 kb
    uint4_t v[8];     // token 4 j + tr, channels 8 c8
  };
  auto load = [&](int st, StepLd& r) {
    const int tb = st * kStep;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int i = 0; i < 4; ++i) r.k[tau][i] = buf_load_b128(rk, ((tb + 16 * tau + m16) * kDim + 32 * i + 8 * kb) * 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) r.v[j] = buf_load_b128(rv, ((tb + 4 * j + tr) * kDim + 8 * c8) * 2);
  };

  float m = -INFINITY, l = 0.f;  // head m16's reference and this lane's share of its sum
  float acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;

  auto step = [&](int st, const StepLd& r, int par) {
    // scores of tokens 16 tau + 4 kb + e for head m16
    float s[8];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      float4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, r.k[tau][i]), qb[i], c, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = st * kStep + 16 * tau + 4 * kb + e;
        s[4 * tau + e] = t < nt ? c[e] * a.scale_log2 : -INFINITY;
      }
    }
    float cm = s[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cm = fmaxf(cm, s[e]);
    if (__builtin_amdgcn_ballot_w64(cm > m + kLazy16)) {
      // move every head's reference to its exact maximum so far
      cm = fmaxf(cm, xlane<16>(cm));
      cm = fmaxf(cm, xlane<32>(cm));
      const float mn = fmaxf(m, cm);
      const float al = mn == -INFINITY ? 1.f : exp2f(m - mn);
      m = mn;
      l *= al;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float ag = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, al), g));
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] *= ag;
      }
    }
    float* pb = &pbuf[wave][par][0][0][0];
    if (m16 < G) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // token 16 tau + 4 kb + e = 4 j + tr with tr = e, j = 4 tau + kb
          const float p = exp2f(s[4 * tau + e] - m);
          l += p;
          pb[(m16 * 4 + e) * 8 + 4 * tau + kb] = p;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float4* pr = reinterpret_cast<const float4*>(pb + (g * 4 + tr) * 8);
      const float4 p0 = pr[0], p1 = pr[1];
      const float pj[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t w4[4] = {r.v[j][0], r.v[j][1], r.v[j][2], r.v[j][3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[g][2 * e] = fmaf(pj[j], h2f(w4[e] & 0xffff), acc[g][2 * e]);
          acc[g][2 * e + 1] = fmaf(pj[j], h2f(w4[e] >> 16), acc[g][2 * e + 1]);
        }
      }
    }
  };

  // steps wave, wave + 4, ... with two buffers in turn: the next step's loads
  // are in flight while the current one is used
  int st = wave;
  if (st < nsteps) {
    StepLd x0, x1;
    load(st, x0);
    for (;;) {
      load(st + 4, x1);
      step(st, x0, 0);
      st += 4;
      if (st >= nsteps) break;
      load(st + 4, x0);
      step(st, x1, 1);
      st += 4;
      if (st >= nsteps) break;
    }
  }

  // reduce within the wave: l over the lanes of each head, acc over tr
  l += xlane<16>(l);
  l += xlane<32>(l);
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[g][e];
      v += xlane<16>(v);
      v += xlane<32>(v);
      acc[g][e] = v;
    }
  if (lane < G) {
    mrg[wave][lane][0] = m;
    mrg[wave][lane][1] = l;
  }
  if (tr == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) mrg[wave][g][2 + 8 * c8 + e] = acc[g][e];
  }
  __syncthreads();
  for (int o = tid; o < G * kDim; o += 256) {
    const int g = o / kDim, c = o % kDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mrg[w][g][0]);
    float sum = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = mrg[w][g][0] == -INFINITY ? 0.f : exp2f(mrg[w][g][0] - M);
      sum = fmaf(f, mrg[w][g][2 + c], sum);
      lsum = fmaf(f, mrg[w][g][1], lsum);
    }
    float* wo = a.ws + (((int64_t)b * a.Hq + h0 + g) * a.nsplit + split) * (kDim + 2);
    wo[c] = sum;
    if (c == 0) {
      wo[kDim] = M;
      wo[kDim + 1] = lsum;
    }
  }
}

size_t fp16_decode_lds_bytes(int G, int split_tokens) {
  (void)split_tokens;
  return sizeof(float) * (size_t)(4 * 2 * G * 32 + 4 * G * (kDim + 2));
}

template <int G>
static hipError_t launch_fp16_t(const Fp16DecodeArgs& a, int B, hipStream_t stream) {
  hipLaunchKernelGGL((fp16_decode_kernel<G>), dim3(a.nsplit, B * a.Hkv), dim3(256), 0, stream, a);
  return hipGetLastError();
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
