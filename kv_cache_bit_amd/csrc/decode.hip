// decode.hip -- split-K decode attention over the NSNQuant-compressed cache,
// the LSE combine, and an fp16-cache comparator (gfx950).
//
// For a key stored as codes c_t, scales (N1, N2) and block mean MU_b,
//   q . k_hat_t = N1 (N2 (Hq) . c_hat_t + q . MU_b),
// and (Hq) . c_hat_t = sum_j LUT_j[c_tj] with LUT_j[c] = (Hq)_j . C[c] (the j-th
// s-element slice).  For the values,
//   sum_t p_t v_hat_t = H^T( sum_j sum_c Hist_j[c] C[c] ) + sum_b beta_b MU_b,
//   Hist_j[c] = sum_{t: c_tj = c} p_t N1_t N2_t,   beta_b = sum_{t in b} p_t N1_t.
// A split streams only packed codes and fp16 scalars from HBM; the codebook
// product and the inverse Hadamard run once per split.  Residual fp16 tokens
// get a split of their own.

#include "nsnq_device.hpp"
#include "nsnq_launch.hpp"
#include "decode_common.hpp"

namespace nsnq {


constexpr int kLutStride = 257;  // odd row stride: finish-step reads hit distinct banks

// ---------------------------------------------------------------------------
// Compressed-token split: single streaming pass with online softmax.
//
// The work-group builds the query LUTs once; then each wave streams its own
// 64-token chunks (chunks w, w + 4, ... of the split) with the next chunk's
// codes and scalars already in flight:
//   scores  lane = token: s_t = N1 (N2 sum_j LUT_j[c_tj] + q . MU_b)
//   softmax running max / sum per head; the value accumulators are rescaled
//           when the max moves
//   values  lane (sq, tg) owns 16 Hadamard-domain channels (slots 4 sq..4 sq+3
//           at 2 bits, 2 sq, 2 sq + 1 at 1 bit) and tokens 8 tg .. 8 tg + 7 of
//           the chunk: acc += w_t C[c_tj] with w_t = p_t N1_t N2_t, codewords
//           gathered from the fp16 codebook in LDS;
//   means   the block-mean term sum_t p_t N1_t MU_b is accumulated per chunk
//           (2 channels per lane).
// At the end the waves merge through LDS, the Hadamard-domain sum goes through
// one inverse transform, and the split's (m, l, o) partial is written.

constexpr int kChunk = 64;
constexpr float kLazyMax = 3.f;  // log2 headroom of the running softmax reference

struct DecodeSmem {
  // offsets in floats
  int qf, qr, cbh, lut, wbuf, qmu, vst, total;
};

__host__ __device__ constexpr DecodeSmem decode_smem(int sub, int gh, int split_tokens, int R) {
  (void)split_tokens;
  (void)R;
  const int S = kDim / sub;
  DecodeSmem s{};
  int o = 0;
  s.qf = o; o += gh * kDim;
  s.qr = o; o += gh * kDim;
  s.cbh = o; o += kCodewords * sub / 2;      // fp16 codebook
  s.lut = o; o += gh * S * kLutStride;       // LUTs; reused for the wave merge
  s.wbuf = o; o += 4 * gh * kChunk;          // per-wave chunk weights
  s.qmu = o; o += kMaxSplitBlocks * gh;      // q . KMU_b of the split's blocks
  s.vst = o; o += (sub == 8 && gh == 1) ? 4 * kChunk * 16 / 4 : 0;  // per-wave V codes [64][16] (matrix-core values)
  s.total = o;
  return s;
}

size_t decode_lds_bytes(int sub, int gh, int split_tokens, int R) {
  return (size_t)decode_smem(sub, gh, split_tokens, R).total * sizeof(float);
}

int decode_max_split_tokens(int sub, int gh, int R) {
  (void)sub;
  (void)gh;
  return kMaxSplitBlocks * R;
}

// LDS loads at absolute byte addresses.  The split kernel has no static LDS,
// so its dynamic segment (smem) starts at address 0: an address is the
// shifted code byte (one SDWA shift) plus a constant folded into the
// instruction's offset field.
__device__ __forceinline__ float lds_f32(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) float*>(static_cast<size_t>(addr));
}
__device__ __forceinline__ uint4_t lds_u32x4(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) uint4_t*>(static_cast<size_t>(addr));
}
typedef uint32_t lds_u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 lds_u32x2(uint32_t addr) {
  const lds_u32x2_t v = *reinterpret_cast<const __attribute__((address_space(3))) lds_u32x2_t*>(static_cast<size_t>(addr));
  return make_uint2(v.x, v.y);
}

template <int S>
__device__ __forceinline__ void load_codes(const uint8_t* p, uint32_t (&cw)[S / 4]) {
#pragma unroll
  for (int i = 0; i < S / 16; ++i) {
    const uint4 v4 = *reinterpret_cast<const uint4*>(p + 16 * i);
    cw[4 * i] = v4.x; cw[4 * i + 1] = v4.y; cw[4 * i + 2] = v4.z; cw[4 * i + 3] = v4.w;
  }
}

// One query head per group (no RoPE): registers capped for 4 waves per SIMD
// at 2 bits (two chunk buffers in turn) and 5 at 1 bit (one buffer, copied),
// without spilling; the wider variants keep the compiler's choice.
template <int SUB, int GH, bool DQ, bool ROPE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(GH == 1 && !ROPE ? 4 : 1))) void decode_split_kernel(DecodeArgs a) {
  constexpr bool kPingPong = SUB == 4;
  // one head at 1 bit: the value sum on the matrix cores (see the values below)
  constexpr bool kMV = SUB == 8 && GH == 1 && !ROPE;
  constexpr int S = kDim / SUB;
  constexpr int CW = S / 4;      // 32-bit words of codes per token
  constexpr int SPT = 16 / SUB;  // value slots per lane
  extern __shared__ float smem[];
  const DecodeSmem L = decode_smem(SUB, GH, a.split_tokens, a.R);
  constexpr DecodeSmem kL = decode_smem(SUB, GH, 0, 0);  // the same offsets, as constants
  float* qf = smem + L.qf;
  float* qr = smem + L.qr;
  uint16_t* cbh = reinterpret_cast<uint16_t*>(smem + L.cbh);
  float* lut = smem + L.lut;
  float* qmus = smem + L.qmu;

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
    float* red = lut + 4 * GH * kDim;
    decode_residual<GH>(a, row_resid(a, b), qf, lut + 4 * GH * kDim + 8 * GH, lut, red, ws_base, ws_head, unit);
    return;
  }

  const int t0 = split * a.split_tokens;
  const int ntok = max(0, min(a.split_tokens, row_quant(a, b) - t0));  // 0: empty partial
  const int nchunk = ntok / kChunk;
  const uint8_t* kc = a.kcodes + (unit * a.cap + t0) * S;
  const uint32_t* ks = reinterpret_cast<const uint32_t*>(a.kscales) + unit * a.cap + t0;
  const uint8_t* vc = a.vcodes + (unit * a.cap + t0) * S;
  const uint32_t* vs = reinterpret_cast<const uint32_t*>(a.vscales) + unit * a.cap + t0;
  const uint16_t* kmu = a.kmu + (unit * nbmu + t0 / a.R) * kDim;
  const uint16_t* vmu = a.vmu + (unit * nbmu + t0 / a.R) * kDim;
  const int64_t blk0 = unit * nbmu + t0 / a.R;  // first block of the split (record index)

  const int sq = lane & 7, tg = lane >> 3;
  // one chunk's loads for this lane
  struct ChunkRegs {
    uint32_t kcw[CW];
    uint32_t ksc, vsc;    // (n1, n2) fp16 pairs, or (q1 << 16 | n2) double-quantised
    uint32_t kpar, vpar;  // double-quantised: the block's (S1, Z1)
    // V block mean of channels 2 lane, 2 lane + 1: an fp16 pair, or two fp32
    // read-back values when double-quantised
    uint32_t vm[DQ ? 2 : 1];
    uint32_t vcw[8];
  };
  auto load_chunk = [&](int ch, ChunkRegs& r) {
    const int tl = ch * kChunk + lane;  // this lane's token for scores
    load_codes<S>(kc + (int64_t)tl * S, r.kcw);
    const int bl = (ch * kChunk) / a.R;
    if constexpr (DQ) {
      const int SRB = dq_record_bytes(a.R), tb = tl % a.R;
      const uint8_t* kr = reinterpret_cast<const uint8_t*>(a.kscales) + (blk0 + bl) * SRB;
      const uint8_t* vr = reinterpret_cast<const uint8_t*>(a.vscales) + (blk0 + bl) * SRB;
      r.ksc = dq_token(kr, a.R, tb);
      r.vsc = dq_token(vr, a.R, tb);
      r.kpar = dq_s1_params(kr, a.R);
      r.vpar = dq_s1_params(vr, a.R);
      float m0, m1;
      dq_mu_pair(reinterpret_cast<const uint8_t*>(a.vmu) + (blk0 + bl) * kDqMuRecord, lane, m0, m1);
      r.vm[0] = __float_as_uint(m0);
      r.vm[DQ ? 1 : 0] = __float_as_uint(m1);
    } else {
      r.ksc = ks[tl];
      r.vsc = vs[tl];
      r.vm[0] = *reinterpret_cast<const uint32_t*>(vmu + (int64_t)bl * kDim + 2 * lane);
    }
    if constexpr (kMV) {
      // the V code row of token `lane` (16 bytes), staged in LDS per chunk
      const uint4 v4 = *reinterpret_cast<const uint4*>(vc + (int64_t)tl * S);
      r.vcw[0] = v4.x; r.vcw[1] = v4.y; r.vcw[2] = v4.z; r.vcw[3] = v4.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint8_t* p = vc + (int64_t)(ch * kChunk + 8 * tg + i) * S + sq * SPT;
        if constexpr (SPT == 4) r.vcw[i] = *reinterpret_cast<const uint32_t*>(p);
        else r.vcw[i] = *reinterpret_cast<const uint16_t*>(p);
      }
    }
  };
  ChunkRegs cur;
  int ch = wave;
  if (ch < nchunk) load_chunk(ch, cur);

  for (int i = tid; i < kCodewords * SUB; i += 256) cbh[i] = a.codebook[i];
  __syncthreads();
  // rotate the queries (one wave per head): q' = H D q
  const float sg0 = a.signs ? (float)a.signs[2 * lane] : 1.f;
  const float sg1 = a.signs ? (float)a.signs[2 * lane + 1] : 1.f;
  if (wave < GH) {
    float x[2] = {qf[wave * kDim + 2 * lane] * sg0, qf[wave * kDim + 2 * lane + 1] * sg1};
    fwht128<2>(x, lane);
    qr[wave * kDim + 2 * lane] = x[0] * kInvSqrtD;
    qr[wave * kDim + 2 * lane + 1] = x[1] * kInvSqrtD;
  }
  __syncthreads();
  // LUT_j[c] = (Hq)_j . C[c]; thread = codeword (keys stored before RoPE
  // need no table: their dot products are formed from dequantised keys)
  if constexpr (!ROPE) {
    const int c = tid;
    float cv[SUB];
#pragma unroll
    for (int e = 0; e < SUB; ++e) cv[e] = h2f(cbh[c * SUB + e]);
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
    // q . KMU_b: the 16 lanes of a row share block b = tid / 16, each lane
    // takes 8 channels of every head and the row sums them
    if ((tid >> 4) < ntok / a.R) {
      const int bl = tid >> 4, c8 = tid & 15;
      float mk[8];
      if constexpr (DQ) {
        const uint8_t* mr = reinterpret_cast<const uint8_t*>(a.kmu) + (blk0 + bl) * kDqMuRecord;
#pragma unroll
        for (int e = 0; e < 8; e += 2) dq_mu_pair(mr, 4 * c8 + e / 2, mk[e], mk[e + 1]);
      } else {
        const uint4 m8 = *reinterpret_cast<const uint4*>(kmu + (int64_t)bl * kDim + 8 * c8);
        const uint32_t mw[4] = {m8.x, m8.y, m8.z, m8.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) mk[e] = h2f((e & 1) ? (mw[e >> 1] >> 16) : (mw[e >> 1] & 0xffff));
      }
#pragma unroll
      for (int g = 0; g < GH; ++g) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(qf[g * kDim + 8 * c8 + e], mk[e], d);
        d = group_sum<16>(d);
        if (c8 == 0) qmus[bl * GH + g] = d;
      }
    }
  }
  __syncthreads();

  float m[GH], l[GH], acc[GH][16], om0[GH], om1[GH];
#pragma unroll
  for (int g = 0; g < GH; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
    om0[g] = om1[g] = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[g][c] = 0.f;
  }
  float* wb = smem + L.wbuf + wave * GH * kChunk;
  // matrix-core values: tile e, row = slot, column 0 = sum_t (p N1 N2 / 8)_t
  // c_hat_t[8 slot + e] over the split's tokens (the other columns repeat it)
  float4_t vacc[kMV ? 8 : 1];
#pragma unroll
  for (int t = 0; t < (kMV ? 8 : 1); ++t) vacc[t] = float4_t{0.f, 0.f, 0.f, 0.f};
  uint8_t* const vstw = reinterpret_cast<uint8_t*>(smem + L.vst) + wave * kChunk * 16;
  const uint32_t vst_lds = (uint32_t)(reinterpret_cast<uintptr_t>(vstw) - reinterpret_cast<uintptr_t>(smem));
  const uint32_t wb_lds = (uint32_t)(reinterpret_cast<uintptr_t>(wb) - reinterpret_cast<uintptr_t>(smem));
  const int m16 = lane & 15, kb = lane >> 4;
  // keys stored before RoPE: lane (token group tt, j) dequantises channels
  // 8 j .. 8 j + 7 of token 4 pass + tt, rotates them and dots them with the
  // queries; the per-token dot products go through LDS (the LUT space)
  const int rj = lane & 15, rtt = lane >> 4;
  float* rsc = lut + wave * GH * kChunk;
  float rq[ROPE ? GH : 1][8], rsg[8];
  if constexpr (ROPE) {
#pragma unroll
    for (int g = 0; g < GH; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) rq[g][e] = qf[g * kDim + 8 * rj + e];
#pragma unroll
    for (int e = 0; e < 8; ++e) rsg[e] = (a.signs ? (float)a.signs[8 * rj + e] : 1.f) * kInvSqrtD;
  }

  // one chunk of this wave with its loads in `cur` (the next chunk's loads
  // are already in flight into the other buffer)
  auto chunk_step = [&](int ch, const ChunkRegs& cur) {
    if constexpr (kMV)
      *reinterpret_cast<uint4_t*>(vstw + lane * 16) = uint4_t{cur.vcw[0], cur.vcw[1], cur.vcw[2], cur.vcw[3]};
    float kn1, kn2, vn1, vn2, vm0, vm1;
    if constexpr (DQ) {
      kn1 = dq_value(cur.kpar, cur.ksc >> 16);
      kn2 = h2f(cur.ksc & 0xffff);
      vn1 = dq_value(cur.vpar, cur.vsc >> 16);
      vn2 = h2f(cur.vsc & 0xffff);
      vm0 = __uint_as_float(cur.vm[0]);
      vm1 = __uint_as_float(cur.vm[DQ ? 1 : 0]);
    } else {
      kn1 = h2f(cur.ksc & 0xffff);
      kn2 = h2f(cur.ksc >> 16);
      vn1 = h2f(cur.vsc & 0xffff);
      vn2 = h2f(cur.vsc >> 16);
      vm0 = h2f(cur.vm[0] & 0xffff);
      vm1 = h2f(cur.vm[0] >> 16);
    }
    if constexpr (ROPE) {
      // the chunk's block mean for channels 8 rj .. 8 rj + 7
      const int bl = (ch * kChunk) / a.R;
      float mk[8];
      if constexpr (DQ) {
        const uint8_t* mr = reinterpret_cast<const uint8_t*>(a.kmu) + (blk0 + bl) * kDqMuRecord;
#pragma unroll
        for (int e = 0; e < 8; e += 2) dq_mu_pair(mr, 4 * rj + e / 2, mk[e], mk[e + 1]);
      } else {
        const uint4 m8 = *reinterpret_cast<const uint4*>(kmu + (int64_t)bl * kDim + 8 * rj);
        const uint32_t mw[4] = {m8.x, m8.y, m8.z, m8.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) mk[e] = h2f((e & 1) ? (mw[e >> 1] >> 16) : (mw[e >> 1] & 0xffff));
      }
#pragma unroll 2
      for (int pass = 0; pass < kChunk / 4; ++pass) {
        const int tok = 4 * pass + rtt;
        const int64_t tc = (int64_t)ch * kChunk + tok;  // token in the split
        float x[8];
        if constexpr (SUB == 4) {
          const uint32_t c2 = *reinterpret_cast<const uint16_t*>(kc + tc * S + 2 * rj);
          const uint2 w0 = *reinterpret_cast<const uint2*>(cbh + (c2 & 0xffu) * 4);
          const uint2 w1 = *reinterpret_cast<const uint2*>(cbh + (c2 >> 8) * 4);
          const uint32_t w[4] = {w0.x, w0.y, w1.x, w1.y};
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = h2f((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffff));
        } else {
          const uint32_t c1 = kc[tc * S + rj];
          const uint4 w4 = *reinterpret_cast<const uint4*>(cbh + c1 * 8);
          const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = h2f((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffff));
        }
        fwht128<8>(x, lane);
        float tn1, tn2;
        if constexpr (DQ) {
          const uint8_t* kr = reinterpret_cast<const uint8_t*>(a.kscales) + (blk0 + bl) * dq_record_bytes(a.R);
          const uint32_t tq = dq_token(kr, a.R, (int)(tc % a.R));
          tn1 = dq_value(dq_s1_params(kr, a.R), tq >> 16);
          tn2 = h2f(tq & 0xffff);
        } else {
          const uint32_t sc = ks[tc];
          tn1 = h2f(sc & 0xffff);
          tn2 = h2f(sc >> 16);
        }
        const int64_t pos = (int64_t)a.rope_pos0 + t0 + tc;
        const float4* cs4 = reinterpret_cast<const float4*>(a.rope_cos + pos * (kDim / 2) + 8 * (rj & 7));
        const float4* sn4 = reinterpret_cast<const float4*>(a.rope_sin + pos * (kDim / 2) + 8 * (rj & 7));
        const float4 ca = cs4[0], cb = cs4[1], sa = sn4[0], sb = sn4[1];
        const float cv[8] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w};
        const float sv8[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
        // rotate-half pairs (c, c + 64): lanes rj < 8 hold c < 64, the partner is rj ^ 8
        const float ssg = rj < 8 ? -1.f : 1.f;
        float r[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float kk = tn1 * fmaf(tn2, x[e] * rsg[e], mk[e]);
          const float pk = xlane<8>(kk);
          r[e] = fmaf(kk, cv[e], ssg * pk * sv8[e]);
        }
#pragma unroll
        for (int g = 0; g < GH; ++g) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) d = fmaf(r[e], rq[g][e], d);
          d = group_sum<16>(d);
          if (rj == 0) rsc[g * kChunk + tok] = d;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
#pragma unroll
    for (int g = 0; g < GH; ++g) {
      float sv;
      if constexpr (ROPE) {
        sv = a.scale_log2 * rsc[g * kChunk + lane];
      } else {
        // score of this lane's token
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int j = 0; j < S; j += 2) {
          constexpr uint32_t base = 4u * kL.lut;
          const uint32_t o0 = base + 4u * (uint32_t)((g * S + j) * kLutStride);
          const uint32_t o1 = o0 + 4u * kLutStride;
          s0 += lds_f32(o0 + (((cur.kcw[j >> 2] >> (8 * (j & 3))) & 0xffu) << 2));
          s1 += lds_f32(o1 + (((cur.kcw[(j + 1) >> 2] >> (8 * ((j + 1) & 3))) & 0xffu) << 2));
        }
        const float qmu = qmus[((ch * kChunk) / a.R) * GH + g];
        sv = a.scale_log2 * kn1 * fmaf(kn2, s0 + s1, qmu);
      }
      // online softmax over the chunk.  The reference m moves only when a
      // score exceeds it by more than 2^3 (then to the exact maximum), so the
      // cross-lane maximum and the rescale are rare; l is a per-lane partial.
      float dl = sv - m[g];
      if (__builtin_amdgcn_ballot_w64(dl > kLazyMax)) {
        const float mn = fmaxf(m[g], group_max<kWave>(sv));
        const float alpha = exp2f(m[g] - mn);
        m[g] = mn;
        l[g] *= alpha;
        om0[g] *= alpha;
        om1[g] *= alpha;
        if constexpr (kMV) {
#pragma unroll
          for (int t = 0; t < 8; ++t) vacc[t] *= alpha;
        } else {
#pragma unroll
          for (int c = 0; c < 16; ++c) acc[g][c] *= alpha;
        }
        dl = sv - mn;
      }
      const float pr = exp2f(dl);
      l[g] += pr;
      const float pn1 = group_sum<kWave>(pr * vn1);
      om0[g] = fmaf(pn1, vm0, om0[g]);
      om1[g] = fmaf(pn1, vm1, om1[g]);
      if constexpr (kMV) {
        // fp16 p N1 N2 / 8: p <= 8 keeps the range of the p <= 1 weights
        reinterpret_cast<uint16_t*>(wb)[lane] = f2h(pr * vn1 * vn2 * 0.125f);
      } else {
        wb[g * kChunk + lane] = pr * vn1 * vn2;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if constexpr (kMV) {
      // values on the matrix cores, 32-token step c: lane (slot m16, kb)
      // supplies tokens 32 c + 8 kb + e; its 8 codewords, transposed with
      // v_perm_b32, give the A operand of each channel e of the slot
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const half8_t bw = __builtin_bit_cast(half8_t, lds_u32x4(wb_lds + 2 * (32 * c + 8 * kb)));
        const uint8_t* vrow = vstw + (32 * c + 8 * kb) * 16 + m16;
        uint32_t code[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) code[e] = vrow[e * 16];
        __builtin_amdgcn_sched_barrier(0);
        uint4_t cw[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) cw[e] = lds_u32x4((code[e] << 4) + 4u * kL.cbh);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ep = 0; ep < 8; ++ep) {
          const uint32_t sel = (ep & 1) ? 0x07060302u : 0x05040100u;
          uint32_t d[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) d[jj] = __builtin_amdgcn_perm(cw[2 * jj + 1][ep >> 1], cw[2 * jj][ep >> 1], sel);
          const half8_t A = __builtin_bit_cast(half8_t, uint4_t{d[0], d[1], d[2], d[3]});
          vacc[ep] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bw, vacc[ep], 0, 0, 0);
        }
      }
    } else {
    // values: tokens 8 tg .. 8 tg + 7 of the chunk, this lane's 16 channels
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float wg[GH];
#pragma unroll
      for (int g = 0; g < GH; ++g) wg[g] = wb[g * kChunk + 8 * tg + i];
#pragma unroll
      for (int si = 0; si < SPT; ++si) {
        const uint32_t caddr = ((cur.vcw[i] >> (8 * si)) & 0xffu) * (2u * SUB) + 4u * kL.cbh;
#pragma unroll
        for (int hh = 0; hh < SUB / 4; ++hh) {
          const uint2 c4 = lds_u32x2(caddr + 8u * hh);
          const float c0 = h2f(c4.x & 0xffff), c1 = h2f(c4.x >> 16);
          const float c2 = h2f(c4.y & 0xffff), c3 = h2f(c4.y >> 16);
#pragma unroll
          for (int g = 0; g < GH; ++g) {
            float* ag = &acc[g][si * SUB + 4 * hh];
            ag[0] = fmaf(wg[g], c0, ag[0]);
            ag[1] = fmaf(wg[g], c1, ag[1]);
            ag[2] = fmaf(wg[g], c2, ag[2]);
            ag[3] = fmaf(wg[g], c3, ag[3]);
          }
        }
      }
    }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  if constexpr (kPingPong) {
    // two buffers in turn, so no register copies between chunks
    ChunkRegs alt;
    for (; ch < nchunk; ch += 8) {
      if (ch + 4 < nchunk) load_chunk(ch + 4, alt);
      chunk_step(ch, cur);
      if (ch + 4 >= nchunk) break;
      if (ch + 8 < nchunk) load_chunk(ch + 8, cur);
      chunk_step(ch + 4, alt);
    }
  } else {
    for (; ch < nchunk; ch += 4) {
      ChunkRegs nxt;
      if (ch + 4 < nchunk) load_chunk(ch + 4, nxt);
      chunk_step(ch, cur);
      cur = nxt;
    }
  }

  // the per-lane sums of p
#pragma unroll
  for (int g = 0; g < GH; ++g) l[g] = group_sum<kWave>(l[g]);
  // token-group reduction inside the wave (lane bits 3..5)
#pragma unroll
  for (int g = 0; g < (kMV ? 0 : GH); ++g)
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      float v = acc[g][c];
      v += xlane<8>(v);
      v += xlane<16>(v);
      v += xlane<32>(v);
      acc[g][c] = v;
    }
  // merge the 4 waves through LDS (the LUT space is free now)
  __syncthreads();
  float* mrg = lut;  // [4 waves][GH][2 + 128 + 128]: m, l, acc, mean term
  constexpr int MS = 2 + 2 * kDim;
#pragma unroll
  for (int g = 0; g < GH; ++g) {
    float* r = mrg + (wave * GH + g) * MS;
    if (lane == 0) {
      r[0] = m[g];
      r[1] = l[g];
    }
    if constexpr (kMV) {
      // column 0: lane (0, kb) holds slots 4 kb .. 4 kb + 3 of every tile
      if (m16 == 0) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) r[2 + 8 * (4 * kb + rr) + t] = 8.f * vacc[t][rr];
      }
    } else if (lane < 8) {
#pragma unroll
      for (int c = 0; c < 16; ++c) r[2 + sq * 16 + c] = acc[g][c];
    }
    r[2 + kDim + 2 * lane] = om0[g];
    r[2 + kDim + 2 * lane + 1] = om1[g];
  }
  __syncthreads();
  if (wave < GH) {
    const int g = wave;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mrg[(w * GH + g) * MS]);
    float lsum = 0.f, x[2] = {0.f, 0.f}, om[2] = {0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float* r = mrg + (w * GH + g) * MS;
      const float f = r[0] == -INFINITY ? 0.f : exp2f(r[0] - M);
      lsum = fmaf(f, r[1], lsum);
      x[0] = fmaf(f, r[2 + 2 * lane], x[0]);
      x[1] = fmaf(f, r[2 + 2 * lane + 1], x[1]);
      om[0] = fmaf(f, r[2 + kDim + 2 * lane], om[0]);
      om[1] = fmaf(f, r[2 + kDim + 2 * lane + 1], om[1]);
    }
    fwht128<2>(x, lane);
    float* wo = ws_base + g * ws_head;
    wo[2 * lane] = fmaf(x[0], kInvSqrtD * sg0, om[0]);
    wo[2 * lane + 1] = fmaf(x[1], kInvSqrtD * sg1, om[1]);
    if (lane == 0) {
      wo[kDim] = M;
      wo[kDim + 1] = lsum;
    }
  }
}

// out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i, one group of 128
// lanes (channels) per (batch row, query head).  Every lane reads the splits'
// (m_i, l_i) itself (the same addresses for the whole group) and its channel
// of o_i, 32 splits at a time with all loads of a batch in flight together;
// the running maximum rescales the sums between batches.
__global__ __launch_bounds__(128) void combine_kernel(CombineArgs a) {
  constexpr int kBatch = 32;
  const int bh = blockIdx.x;
  const int c = threadIdx.x;
  const float* w = a.ws + (int64_t)bh * a.nsplit * (kDim + 2);
  float M = -INFINITY, num = 0.f, den = 0.f;
  for (int i0 = 0; i0 < a.nsplit; i0 += kBatch) {
    const int n = min(kBatch, a.nsplit - i0);
    float mi[kBatch], li[kBatch], oi[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float* r = w + (int64_t)(i0 + u) * (kDim + 2);
      mi[u] = u < n ? r[kDim] : -INFINITY;
      li[u] = u < n ? r[kDim + 1] : 0.f;
      oi[u] = u < n ? r[c] : 0.f;
    }
    float Mb = M;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) Mb = fmaxf(Mb, mi[u]);
    if (Mb == -INFINITY) continue;  // no tokens so far
    const float sc = exp2f(M - Mb);  // 0 while M is -inf
    num *= sc;
    den *= sc;
    M = Mb;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float f = exp2f(mi[u] - M);
      num = fmaf(f, oi[u], num);
      den = fmaf(f, li[u], den);
    }
  }
  // a row without tokens (ragged cache): zero output
  a.out[(int64_t)bh * kDim + c] = M == -INFINITY ? (uint16_t)0 : f2h(num / den);
}

template <int SUB, int GH, bool DQ, bool ROPE>
static hipError_t launch_decode_dq(const DecodeArgs& a, int B, size_t lds, hipStream_t stream) {
  static bool lds_set[kMaxDevices] = {};
  const hipError_t e = allow_lds(reinterpret_cast<const void*>(&decode_split_kernel<SUB, GH, DQ, ROPE>), lds_set);
  if (e != hipSuccess) return e;
  dim3 grid(a.nsplit, B * a.Hkv * (a.G / GH)), block(256);
  hipLaunchKernelGGL((decode_split_kernel<SUB, GH, DQ, ROPE>), grid, block, lds, stream, a);
  return hipGetLastError();
}

template <int SUB, int GH>
static hipError_t launch_decode_t(const DecodeArgs& a, int B, size_t lds, hipStream_t stream) {
  if (a.rope_cos)
    return a.dq ? launch_decode_dq<SUB, GH, true, true>(a, B, lds, stream)
                : launch_decode_dq<SUB, GH, false, true>(a, B, lds, stream);
  return a.dq ? launch_decode_dq<SUB, GH, true, false>(a, B, lds, stream)
              : launch_decode_dq<SUB, GH, false, false>(a, B, lds, stream);
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
  static bool lds_set[kMaxDevices] = {};
  const hipError_t e = allow_lds(reinterpret_cast<const void*>(&fp16_decode_kernel<G>), lds_set);
  if (e != hipSuccess) return e;
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
