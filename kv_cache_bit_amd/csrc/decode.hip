// decode.hip -- split-K decode attention over the NSNQuant-compressed cache
// with per-query lookup tables, and the LSE combine of the split partials
// (gfx950).
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
// Staged V code rows of the matrix-core value sum (1 bit, one head): token
// t's 16-byte row sits at 16 t + 16 (t / 8): the value step's lane groups
// read rows 8 apart, which without the padding share banks.
constexpr int kVstWave = kChunk * 16 + kChunk / 8 * 16;  // bytes per wave
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
  s.vst = o; o += (sub == 8 && gh == 1) ? 4 * kVstWave / 4 : 0;  // per-wave V codes [64][16] (matrix-core values)
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
  const int split = a.split_slow ? blockIdx.y : blockIdx.x;
  const int ux = a.split_slow ? blockIdx.x : blockIdx.y;
  const int groups = a.G / GH;
  const int hg = ux % groups;
  const int bk = ux / groups;
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

  const int sb0 = split_block(a, split), sb1 = split_block(a, split + 1);
  const int t0 = sb0 << a.lgR;
  const int ntok = max(0, min((sb1 - sb0) << a.lgR, row_quant(a, b) - t0));  // 0: empty partial
  const int nchunk = ntok / kChunk;
  const uint8_t* kc = a.kcodes + (unit * a.cap + t0) * S;
  const uint32_t* ks = reinterpret_cast<const uint32_t*>(a.kscales) + unit * a.cap + t0;
  const uint8_t* vc = a.vcodes + (unit * a.cap + t0) * S;
  const uint32_t* vs = reinterpret_cast<const uint32_t*>(a.vscales) + unit * a.cap + t0;
  const uint16_t* kmu = a.kmu + (unit * nbmu + (t0 >> a.lgR)) * kDim;
  const uint16_t* vmu = a.vmu + (unit * nbmu + (t0 >> a.lgR)) * kDim;
  const int64_t blk0 = unit * nbmu + (t0 >> a.lgR);  // first block of the split (record index)

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
  // Without double quantisation the chunk loads go through buffer resources
  // bounded by the split: a prefetch past the last chunk returns zeros without
  // touching memory, so prefetches are unconditional and the wait before a
  // chunk's use counts only the loads issued before it.
  constexpr bool kBuf = !DQ;
  const int nblk_split = (ntok + a.R - 1) >> a.lgR;
  const buf_rsrc_t rkc = make_rsrc(kc, ntok * S), rvc = make_rsrc(vc, ntok * S);
  const buf_rsrc_t rks = make_rsrc(ks, ntok * 4), rvs = make_rsrc(vs, ntok * 4);
  const buf_rsrc_t rvm = make_rsrc(vmu, nblk_split * kDim * 2);
  auto load_chunk = [&](int ch, ChunkRegs& r) {
    const int tl = ch * kChunk + lane;  // this lane's token for scores
    if constexpr (kBuf) {
#pragma unroll
      for (int i = 0; i < S / 16; ++i) {
        const uint4_t v4 = buf_load_b128(rkc, tl * S + 16 * i);
        r.kcw[4 * i] = v4[0]; r.kcw[4 * i + 1] = v4[1]; r.kcw[4 * i + 2] = v4[2]; r.kcw[4 * i + 3] = v4[3];
      }
      const int bl = (ch * kChunk) >> a.lgR;
      r.ksc = buf_load_b32(rks, tl * 4);
      r.vsc = buf_load_b32(rvs, tl * 4);
      r.vm[0] = buf_load_b32(rvm, (bl * kDim + 2 * lane) * 2);
      if constexpr (kMV) {
        const uint4_t v4 = buf_load_b128(rvc, tl * S);
        r.vcw[0] = v4[0]; r.vcw[1] = v4[1]; r.vcw[2] = v4[2]; r.vcw[3] = v4[3];
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int off = (ch * kChunk + 8 * tg + i) * S + sq * SPT;
          if constexpr (SPT == 4) r.vcw[i] = buf_load_b32(rvc, off);
          else r.vcw[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rvc, off, 0, 0);
        }
      }
      return;
    }
    load_codes<S>(kc + (int64_t)tl * S, r.kcw);
    const int bl = (ch * kChunk) >> a.lgR;
    if constexpr (DQ) {
      const int SRB = dq_record_bytes(a.R), tb = tl & (a.R - 1);
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
  if (kBuf || ch < nchunk) load_chunk(ch, cur);

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
    if ((tid >> 4) < (ntok >> a.lgR)) {
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
  // matrix-core values: the fp16 weights carry 2^(ev - 3), ev the smallest
  // headroom exponent of the wave's chunks so far (vacc is rescaled exactly
  // when it drops), so no N1 N2 overflows fp16 and no small one underflows;
  // 64 is above any chunk's exponent
  int ev = 64;
  uint8_t* const vstw = reinterpret_cast<uint8_t*>(smem + L.vst) + wave * kVstWave;
  const uint32_t wb_lds = (uint32_t)(reinterpret_cast<uintptr_t>(wb) - reinterpret_cast<uintptr_t>(smem));
  const int m16 = lane & 15, kb = lane >> 4;
  // Keys stored before RoPE are rebuilt 16 tokens at a time on the matrix
  // cores: H c_hat = (H_4 (x) H_32) c_hat, the 32-point factor as
  // v_mfma_f32_16x16x32_f16 products of the gathered codewords (A: token rows)
  // with +-1 operands, the 4-point factor over the four 32-channel blocks in
  // registers.  Lane (rj, rtt) then holds channels 32 ch + 2 rj + j (value
  // 2 ch + j, ch = 0..3, j = 0, 1) of tokens 4 rtt .. 4 rtt + 3 of the tile:
  // the RoPE pairs (c, c + 64) and their tables' columns (2 rj, 2 rj + 1 and
  // 32 + 2 rj, 33 + 2 rj) stay in the lane.  It scales, adds the block mean,
  // rotates and dots the pairs with the queries; a 16-lane sum gives each
  // token's score, which goes through LDS (the LUT space) to the softmax.
  const int rj = lane & 15, rtt = lane >> 4;
  float* rsc = lut + wave * GH * kChunk;
  float rq[ROPE ? GH : 1][8], rsg[8];
  half8_t hb[ROPE ? 2 : 1];  // B operands: H_32[8 rtt + e][2 rj + j]
  auto rch = [&](int v) { return 32 * (v >> 1) + 2 * rj + (v & 1); };  // channel of value v
  if constexpr (ROPE) {
#pragma unroll
    for (int g = 0; g < GH; ++g)
#pragma unroll
      for (int v = 0; v < 8; ++v) rq[g][v] = qf[g * kDim + rch(v)];
#pragma unroll
    for (int v = 0; v < 8; ++v) rsg[v] = (a.signs ? (float)a.signs[rch(v)] : 1.f) * kInvSqrtD;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        hb[j][e] = (__builtin_popcount((8 * rtt + e) & (2 * rj + j)) & 1) ? (half_t)-1.f : (half_t)1.f;
  }
  // One head: the scale, the sign and the two 4-point outputs of each RoPE
  // pair fold into the query.  For pair p = (c, j) (values 2 c + j and
  // 2 c + 4 + j, the blocks' transform outputs e0 + e1 and e0 - e1 with
  // (e0, e1) = (a0, a2) or (a1, a3)), q . rot(k) / N1 =
  //   cos (N2 A_W + A_M) + sin (N2 B_W + B_M),
  //   A_W = qa[p][0] e0 + qa[p][1] e1,  B_W = qa[p][2] e0 + qa[p][3] e1,
  // with A_M, B_M the block mean's share (per chunk).
  float qa[ROPE && GH == 1 ? 4 : 1][4];
  if constexpr (ROPE && GH == 1) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int vl = 2 * (p >> 1) + (p & 1), vh = vl + 4;
      const float Ql = rq[0][vl] * rsg[vl], Qh = rq[0][vh] * rsg[vh];
      const float Xl = rq[0][vh] * rsg[vl], Xh = -rq[0][vl] * rsg[vh];
      qa[p][0] = Ql + Qh;
      qa[p][1] = Ql - Qh;
      qa[p][2] = Xl + Xh;
      qa[p][3] = Xl - Xh;
    }
  }

  // one chunk of this wave with its loads in `cur` (the next chunk's loads
  // are already in flight into the other buffer)
  auto chunk_step = [&](int ch, const ChunkRegs& cur) {
    if constexpr (kMV)
      *reinterpret_cast<uint4_t*>(vstw + lane * 16 + (lane >> 3) * 16) = uint4_t{cur.vcw[0], cur.vcw[1], cur.vcw[2], cur.vcw[3]};
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
    if constexpr (kMV) {
      const int ec = f16_headroom_exp(wave_max_nonneg(fabsf(vn1 * vn2)));
      if (ec < ev) {
        const float f = pow2f(ec - ev);
#pragma unroll
        for (int t = 0; t < 8; ++t) vacc[t] *= f;
        ev = ec;
      }
    }
    if constexpr (ROPE) {
      // the chunk's block mean for this lane's channels (pairs 32 ch + 2 rj, + 1)
      const int bl = (ch * kChunk) >> a.lgR;
      float mk[8];
      if constexpr (DQ) {
        const uint8_t* mr = reinterpret_cast<const uint8_t*>(a.kmu) + (blk0 + bl) * kDqMuRecord;
#pragma unroll
        for (int c = 0; c < 4; ++c) dq_mu_pair(mr, 16 * c + rj, mk[2 * c], mk[2 * c + 1]);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t m2 = *reinterpret_cast<const uint32_t*>(kmu + (int64_t)bl * kDim + 32 * c + 2 * rj);
          mk[2 * c] = h2f(m2 & 0xffff);
          mk[2 * c + 1] = h2f(m2 >> 16);
        }
      }
      // one head: the block mean's share per RoPE pair (see qa)
      float mam[GH == 1 ? 4 : 1][2];
      if constexpr (GH == 1) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int vl = 2 * (p >> 1) + (p & 1), vh = vl + 4;
          mam[p][0] = fmaf(rq[0][vl], mk[vl], rq[0][vh] * mk[vh]);
          mam[p][1] = fmaf(rq[0][vh], mk[vl], -rq[0][vl] * mk[vh]);
        }
      }
      // the chunk's K code rows and (N1, N2) per token, staged in LDS (the
      // products read the codes of other lanes' tokens); the LUT space is
      // free here
      uint8_t* kst = reinterpret_cast<uint8_t*>(lut + 4 * GH * kChunk) + wave * (kChunk * (S + 8));
      float2* sst = reinterpret_cast<float2*>(kst + kChunk * S);
#pragma unroll
      for (int i = 0; i < S / 16; ++i)
        *reinterpret_cast<uint4_t*>(kst + lane * S + 16 * i) =
            uint4_t{cur.kcw[4 * i], cur.kcw[4 * i + 1], cur.kcw[4 * i + 2], cur.kcw[4 * i + 3]};
      sst[lane] = float2{kn1, kn2};
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const float4_t zacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
      for (int tt = 0; tt < kChunk / 16; ++tt) {
        // RoPE rows of this lane's four tokens, requested before the products
        float2 rc[4][2], rs[4][2];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t pos = (int64_t)a.rope_pos0 + t0 + (int64_t)ch * kChunk + 16 * tt + 4 * rtt + r;
          const float* cp = a.rope_cos + pos * (kDim / 2) + 2 * rj;
          const float* sp = a.rope_sin + pos * (kDim / 2) + 2 * rj;
          rc[r][0] = *reinterpret_cast<const float2*>(cp);
          rc[r][1] = *reinterpret_cast<const float2*>(cp + 32);
          rs[r][0] = *reinterpret_cast<const float2*>(sp);
          rs[r][1] = *reinterpret_cast<const float2*>(sp + 32);
        }
        // P[s][j]: token rows 16 tt + rj (A), 32-channel block s, columns 2 rj + j
        float4_t P[4][2];
        const int ta = 16 * tt + rj;
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
          half8_t A;
          if constexpr (SUB == 4) {
            const uint32_t c2 = *reinterpret_cast<const uint16_t*>(kst + ta * S + 8 * sb + 2 * rtt);
            const uint2 w0 = *reinterpret_cast<const uint2*>(cbh + (c2 & 0xffu) * 4);
            const uint2 w1 = *reinterpret_cast<const uint2*>(cbh + (c2 >> 8) * 4);
            A = __builtin_bit_cast(half8_t, uint4_t{w0.x, w0.y, w1.x, w1.y});
          } else {
            const uint32_t c1 = kst[ta * S + 4 * sb + rtt];
            A = __builtin_bit_cast(half8_t, *reinterpret_cast<const uint4_t*>(cbh + c1 * 8));
          }
          P[sb][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, hb[0], zacc, 0, 0, 0);
          P[sb][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, hb[1], zacc, 0, 0, 0);
        }
        if constexpr (GH == 1) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tok = 16 * tt + 4 * rtt + r;
            const float2 tsc = sst[tok];
            float aw = 0.f, am = 0.f;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const float a0 = P[0][j][r] + P[1][j][r], a1 = P[0][j][r] - P[1][j][r];
              const float a2 = P[2][j][r] + P[3][j][r], a3 = P[2][j][r] - P[3][j][r];
#pragma unroll
              for (int c = 0; c < 2; ++c) {
                const int p = 2 * c + j;
                const float e0 = c ? a1 : a0, e1 = c ? a3 : a2;
                const float AW = fmaf(qa[p][0], e0, qa[p][1] * e1);
                const float BW = fmaf(qa[p][2], e0, qa[p][3] * e1);
                const float cs = j ? rc[r][c].y : rc[r][c].x, sn = j ? rs[r][c].y : rs[r][c].x;
                aw = fmaf(cs, AW, aw);
                aw = fmaf(sn, BW, aw);
                am = fmaf(cs, mam[p][0], am);
                am = fmaf(sn, mam[p][1], am);
              }
            }
            const float d = group_sum<16>(fmaf(tsc.y, aw, am));
            if (rj == 0) rsc[tok] = tsc.x * d;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tok = 16 * tt + 4 * rtt + r;
            const float2 tsc = sst[tok];
            // 4-point transform over the blocks: value 2 ch + j
            float kk[8];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const float a0 = P[0][j][r] + P[1][j][r], a1 = P[0][j][r] - P[1][j][r];
              const float a2 = P[2][j][r] + P[3][j][r], a3 = P[2][j][r] - P[3][j][r];
              kk[j] = a0 + a2;
              kk[2 + j] = a1 + a3;
              kk[4 + j] = a0 - a2;
              kk[6 + j] = a1 - a3;
            }
            // k / N1 = N2 D H c_hat / sqrt(d) + mu, then the rotation of the pairs (ch, ch + 2)
#pragma unroll
            for (int v = 0; v < 8; ++v) kk[v] = fmaf(tsc.y * rsg[v], kk[v], mk[v]);
            float kr[8];
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
              for (int j = 0; j < 2; ++j) {
                const float lo = kk[2 * c + j], hi = kk[2 * c + 4 + j];
                const float cs = j ? rc[r][c].y : rc[r][c].x, sn = j ? rs[r][c].y : rs[r][c].x;
                kr[2 * c + j] = fmaf(lo, cs, -hi * sn);
                kr[2 * c + 4 + j] = fmaf(hi, cs, lo * sn);
              }
#pragma unroll
            for (int g = 0; g < GH; ++g) {
              float d = 0.f;
#pragma unroll
              for (int v = 0; v < 8; ++v) d = fmaf(kr[v], rq[g][v], d);
              d = group_sum<16>(d);
              if (rj == 0) rsc[g * kChunk + tok] = tsc.x * d;
            }
          }
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
        const float qmu = qmus[((ch * kChunk) >> a.lgR) * GH + g];
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
        // fp16 p N1 N2 2^(ev - 3) < 2^15 (p <= 8)
        reinterpret_cast<uint16_t*>(wb)[lane] = f2h(pr * (vn1 * vn2) * pow2f(ev - 3));
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
        const uint8_t* vrow = vstw + (32 * c + 8 * kb) * 16 + (4 * c + kb) * 16 + m16;
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
    // values: tokens 8 tg .. 8 tg + 7 of the chunk, this lane's 16 channels,
    // two tokens at a time: all eight codeword gathers are issued before the
    // first product (issued one by one next to their products, each gather's
    // bank-conflicted latency stalled the wave)
    constexpr int NG = SPT * (SUB / 4);  // 8-byte codeword pieces per token
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      float wg[2][GH];
      uint2 c4[2][NG];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int g = 0; g < GH; ++g) wg[t][g] = wb[g * kChunk + 8 * tg + i + t];
#pragma unroll
        for (int si = 0; si < SPT; ++si) {
          const uint32_t caddr = ((cur.vcw[i + t] >> (8 * si)) & 0xffu) * (2u * SUB) + 4u * kL.cbh;
#pragma unroll
          for (int hh = 0; hh < SUB / 4; ++hh) c4[t][si * (SUB / 4) + hh] = lds_u32x2(caddr + 8u * hh);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int n = 0; n < NG; ++n) {
          const float c0 = h2f(c4[t][n].x & 0xffff), c1 = h2f(c4[t][n].x >> 16);
          const float c2 = h2f(c4[t][n].y & 0xffff), c3 = h2f(c4[t][n].y >> 16);
#pragma unroll
          for (int g = 0; g < GH; ++g) {
            float* ag = &acc[g][4 * n];
            ag[0] = fmaf(wg[t][g], c0, ag[0]);
            ag[1] = fmaf(wg[t][g], c1, ag[1]);
            ag[2] = fmaf(wg[t][g], c2, ag[2]);
            ag[3] = fmaf(wg[t][g], c3, ag[3]);
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
      if (kBuf || ch + 4 < nchunk) load_chunk(ch + 4, alt);
      chunk_step(ch, cur);
      if (ch + 4 >= nchunk) break;
      if (kBuf || ch + 8 < nchunk) load_chunk(ch + 8, cur);
      chunk_step(ch + 4, alt);
    }
  } else {
    for (; ch < nchunk; ch += 4) {
      ChunkRegs nxt;
      if (kBuf || ch + 4 < nchunk) load_chunk(ch + 4, nxt);
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
          for (int rr = 0; rr < 4; ++rr) r[2 + 8 * (4 * kb + rr) + t] = pow2f(3 - ev) * vacc[t][rr];
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

// out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i for each (batch row,
// query head).  CPL channels per lane: one wave per head (CPL = 2) or two
// (CPL = 1, more waves for few heads).  The splits go in batches of NB
// (<= 64): lane u reads split u's (m_u, l_u) while the batch's o values of
// every lane are in flight (indexes past the batch re-read its last split, so
// no load sits behind a branch); one wave maximum and one exp2 per lane then
// give the split factors, which the channel sums read back with v_readlane
// (uniform split index; lanes past the batch hold factor 0).  A running
// maximum rescales the sums between batches.
template <int NB, int CPL>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  static_assert(NB <= kWave, "one split per lane");
  static_assert(CPL == 1 || CPL == 2, "one or two channels per lane");
  constexpr int WPH = 2 / CPL;  // waves per head
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bh = blockIdx.x * ((int)(blockDim.x >> 6) / WPH) + wave / WPH;
  if (bh >= a.nbh) return;  // the whole wave (and its partner)
  const int c0 = (wave % WPH) * kWave * CPL + CPL * lane;  // this lane's first channel
  constexpr int RS = kDim + 2;  // floats per partial
  const float* w = a.ws + (int64_t)bh * a.nsplit * RS;
  float M = -INFINITY, den = 0.f, n0 = 0.f, n1 = 0.f;
  for (int i0 = 0; i0 < a.nsplit; i0 += NB) {
    const int last = min(NB, a.nsplit - i0) - 1;
    const float* wb = w + (int64_t)i0 * RS;
    float mu = -INFINITY, lu = 0.f;
    if (lane <= last) {
      mu = wb[lane * RS + kDim];
      lu = wb[lane * RS + kDim + 1];
    }
    float2 o[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const float* r = wb + min(k, last) * RS + c0;
      if constexpr (CPL == 2) o[k] = *reinterpret_cast<const float2*>(r);
      else o[k] = float2{*r, 0.f};
    }
    const float Mb = fmaxf(M, group_max<kWave>(mu));
    if (Mb == -INFINITY) continue;  // no tokens so far
    const float sc = exp2f(M - Mb);  // 0 while M is -inf
    n0 *= sc;
    n1 *= sc;
    den *= sc;
    M = Mb;
    const float fu = exp2f(mu - M);  // 0 for lanes past the batch
    den += group_sum<kWave>(fu * lu);
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const float f = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fu), k));
      n0 = fmaf(f, o[k].x, n0);
      if constexpr (CPL == 2) n1 = fmaf(f, o[k].y, n1);
    }
  }
  // a row without tokens (ragged cache): zero output
  uint16_t* out = a.out + (int64_t)bh * kDim + c0;
  if constexpr (CPL == 2) {
    const uint32_t pair = M == -INFINITY ? 0u : ((uint32_t)f2h(n0 / den) | ((uint32_t)f2h(n1 / den) << 16));
    *reinterpret_cast<uint32_t*>(out) = pair;
  } else {
    *out = M == -INFINITY ? (uint16_t)0 : f2h(n0 / den);
  }
}

// Work-groups of a kernel variant the device holds at once (0 if unknown),
// cached per device in `cache` (0 = not asked yet, -1 = unknown).
static int resident_groups(const void* kernel, size_t lds, std::atomic<int> (&cache)[kMaxDevices]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 0;
  }
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, lds) != hipSuccess) per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
    (void)hipGetLastError();
    v = per_cu > 0 && cus > 0 ? per_cu * cus : -1;
    cache[dev].store(v, std::memory_order_relaxed);  // concurrent first queries store the same value
  }
  return v > 0 ? v : 0;
}

template <int SUB, int GH, bool DQ, bool ROPE>
static hipError_t launch_decode_dq(const DecodeArgs& a, int B, size_t lds, hipStream_t stream) {
  static std::atomic<bool> lds_set[kMaxDevices];
  static std::atomic<int> resident[kMaxDevices];
  const void* k = reinterpret_cast<const void*>(&decode_split_kernel<SUB, GH, DQ, ROPE>);
  const hipError_t e = allow_lds(k, lds_set);
  if (e != hipSuccess) return e;
  // When every compressed split fits the device at once, they go first and
  // the short residual groups fill in behind them; otherwise each row's
  // groups go together, so residual reads overlap the compressed splits.
  // Keys stored before RoPE: compressed splits first in every case (their
  // groups are long, so the residual groups are better left to the end).
  DecodeArgs c = a;
  const int units = B * a.Hkv * (a.G / GH);
  const int cap = resident_groups(k, lds, resident);
  c.split_slow = ROPE || (cap > 0 && (int64_t)a.nsplit_q * units <= cap) || units > 65535 ? 1 : 0;  // grid y <= 65535
  const dim3 grid = c.split_slow ? dim3(units, a.nsplit) : dim3(a.nsplit, units), block(256);
  hipLaunchKernelGGL((decode_split_kernel<SUB, GH, DQ, ROPE>), grid, block, lds, stream, c);
  return hipGetLastError();
}

template <int SUB, int GH>
static hipError_t launch_decode_t(const DecodeArgs& a, int B, size_t lds, hipStream_t stream) {
  if (a.rope_cos) {
    // keys stored before RoPE: groups of at most 2 heads (the planner's choice)
    if constexpr (GH > 2) return hipErrorInvalidValue;
    else
      return a.dq ? launch_decode_dq<SUB, GH, true, true>(a, B, lds, stream)
                  : launch_decode_dq<SUB, GH, false, true>(a, B, lds, stream);
  }
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

template <int CPL>
static void launch_combine_nb(const CombineArgs& c, dim3 grid, dim3 block, hipStream_t stream) {
  if (c.nsplit <= 4) hipLaunchKernelGGL((combine_kernel<4, CPL>), grid, block, 0, stream, c);
  else if (c.nsplit <= 8) hipLaunchKernelGGL((combine_kernel<8, CPL>), grid, block, 0, stream, c);
  else if (c.nsplit <= 16) hipLaunchKernelGGL((combine_kernel<16, CPL>), grid, block, 0, stream, c);
  else hipLaunchKernelGGL((combine_kernel<32, CPL>), grid, block, 0, stream, c);
}

hipError_t launch_combine(const CombineArgs& a, int B, hipStream_t stream) {
  CombineArgs c = a;
  c.nbh = B * a.Hq;
  // many heads: one wave per head, four heads per group; few heads: two
  // waves per head (one channel per lane), spread over more CUs
  if (c.nbh >= 4096) launch_combine_nb<2>(c, dim3((c.nbh + 3) / 4), dim3(256), stream);
  else launch_combine_nb<1>(c, dim3(c.nbh), dim3(128), stream);
  return hipGetLastError();
}

}  // namespace nsnq
