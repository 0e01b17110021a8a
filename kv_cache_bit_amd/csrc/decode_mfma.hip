// decode_mfma.hip -- decode attention over the compressed cache for grouped
// query heads, with the scoring and the value sum on the matrix cores (gfx950).
//
// The algebra is the one of decode.hip (technical summary sec. 4, Attention
// Computation): for a token stored as codes, (N1, N2) and block mean MU_b,
//   q . k_hat = N1 (N2 (H D q) . c_hat + q . MU_b),
//   sum_t p_t v_hat_t = D H^T sum_t (p_t N1_t N2_t) c_hat_t + sum_b (sum_{t in b} p_t N1_t) MU_b.
// Here the Hadamard-domain codewords c_hat_t are gathered once per token and
// shared by every query head of the KV head, instead of one table lookup per
// (token, slot, head):
//   scores  S[t][g] = sum_c c_hat_t[c] q'_g[c]: v_mfma_f32_16x16x32_f16 over
//           16-token x 16-head tiles; the A operand of a lane is the codeword
//           pair (2 bits) or the codeword (1 bit) of its token read straight
//           from the fp16 codebook in LDS; q' = H D q is split into fp16 high
//           and low parts (two products), so the scores keep fp32 accuracy;
//   values  O'[c][g] += sum_t c_hat_t[c] w_t[g] with w = p N1 N2 in fp16.  The
//           contraction runs over tokens, so a lane gathers the codewords of
//           its 8 tokens for one slot and transposes them in registers
//           (v_perm_b32) into one A operand per channel of the slot.  The
//           token order inside a 32-token step is the one the score tiles
//           leave in the lanes, so the B operand (the weights) needs no
//           exchange between lanes;
//   means   per 64-token chunk, beta = sum_t p_t N1_t and the running max are
//           kept in LDS and folded in once at the end of the split.
// Up to 16 query heads share a work-group, one MFMA column each.

#include "decode_common.hpp"

namespace nsnq {

namespace {

constexpr int kMChunk = 64;                                 // tokens per wave step
constexpr int kMaxChunks = kMaxSplitBlocks * 128 / kMChunk;  // per split (R <= 128)

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// (byte BYTE of w) << SH: the LDS byte offset of that code's codeword (8 bytes
// at 2 bits, SH = 3; 16 bytes at 1 bit, SH = 4), in one VALU op (SDWA byte
// select on the shifted operand).
#define NSNQ_CODE_SHL(SH, B) \
  asm("v_lshlrev_b32_sdwa %0, " #SH ", %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_" #B \
      : "=v"(r) : "v"(w))
template <int BYTE, int SH>
__device__ __forceinline__ uint32_t code_shl(uint32_t w) {
  static_assert(SH == 3 || SH == 4, "codeword size");
  uint32_t r;
  if constexpr (SH == 3) {
    if constexpr (BYTE == 0) NSNQ_CODE_SHL(3, 0);
    else if constexpr (BYTE == 1) NSNQ_CODE_SHL(3, 1);
    else if constexpr (BYTE == 2) NSNQ_CODE_SHL(3, 2);
    else NSNQ_CODE_SHL(3, 3);
  } else {
    if constexpr (BYTE == 0) NSNQ_CODE_SHL(4, 0);
    else if constexpr (BYTE == 1) NSNQ_CODE_SHL(4, 1);
    else if constexpr (BYTE == 2) NSNQ_CODE_SHL(4, 2);
    else NSNQ_CODE_SHL(4, 3);
  }
  return r;
}
#undef NSNQ_CODE_SHL

// LDS word at absolute byte address `addr`.  The kernel below declares no
// static LDS, so its dynamic LDS (and the codebook at offset 0) starts at
// address 0 and a code's byte offset is its LDS address.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2_t lds_b64(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x2_t*>(static_cast<size_t>(addr));
}
__device__ __forceinline__ uint4_t lds_b128(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) uint4_t*>(static_cast<size_t>(addr));
}

constexpr int cmax3(int a, int b, int c) { return a > b ? (a > c ? a : c) : (b > c ? b : c); }

// LDS layout in 4-byte words: a union of the main-loop, merge and residual
// views, then the per-chunk (beta, max) lists and the V block means, which
// live for the whole split.  The codebook sits at offset 0 so the gather
// addresses need no base.
template <int SUB, int GQ>
struct MfmaSmem {
  static constexpr int S = kDim / SUB;
  // main loop
  static constexpr int cbh = 0;                          // fp16 codebook [256][SUB]
  static constexpr int qf = cbh + kCodewords * SUB / 2;  // [GQ][128] queries
  static constexpr int qr = qf + GQ * kDim;              // [GQ][128] H D q / sqrt(d)
  static constexpr int qmu = qr + GQ * kDim;             // [kMaxSplitBlocks][GQ] q . KMU_b
  static constexpr int kmu = qmu + kMaxSplitBlocks * GQ;  // [kMaxSplitBlocks][128] fp32 K block means
  static constexpr int VSTW = kMChunk * S / 4 + 4 * kMChunk;  // per wave: V codes, 4 per-token factors
  static constexpr int vst = kmu + kMaxSplitBlocks * kDim;
  static constexpr int main_end = vst + 4 * VSTW;
  // merge of the four waves
  static constexpr int mrg = 0;  // [4][GQ][2 + 128]
  static constexpr int mrg_end = mrg + 4 * GQ * (kDim + 2);
  // residual split (decode_residual): qf as above, then scores, value partials, reductions
  static constexpr int rsc = qr;
  static constexpr int rov = rsc + GQ * 128;
  static constexpr int rred = rov + 4 * GQ * kDim;
  static constexpr int res_end = rred + 8 * GQ;
  // persistent
  static constexpr int bc = cmax3(main_end, mrg_end, res_end);  // [kMaxChunks][GQ] beta
  static constexpr int mc = bc + kMaxChunks * GQ;                // [kMaxChunks][GQ] max
  static constexpr int vmu = mc + kMaxChunks * GQ;               // [kMaxSplitBlocks][128] fp32 V block means
  static constexpr int total = vmu + kMaxSplitBlocks * kDim;
};

// Channel held by accumulator row `row` (0..15) of value tile `tile` (0..7).
template <int SUB>
__device__ __forceinline__ int value_channel(int tile, int row) {
  if constexpr (SUB == 4) return 4 * (16 * (tile >> 2) + row) + (tile & 3);
  else return 8 * row + tile;
}

}  // namespace

template <int SUB, int GQ, bool DQ>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a) {
  using L = MfmaSmem<SUB, GQ>;
  constexpr int S = kDim / SUB;
  extern __shared__ float smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m16 = lane & 15, kb = lane >> 4;
  const int split = blockIdx.x;
  const int groups = a.G / GQ;
  const int hg = blockIdx.y % groups;
  const int bk = blockIdx.y / groups;
  const int b = bk / a.Hkv, hk = bk % a.Hkv;
  const int h0 = hk * a.G + hg * GQ;
  const int64_t unit = (int64_t)b * a.Hkv + hk;
  const int nbmu = a.cap / a.R;
  float* ws_base = a.ws + ((int64_t)b * a.Hq + h0) * a.nsplit * (kDim + 2) + (int64_t)split * (kDim + 2);
  const int64_t ws_head = (int64_t)a.nsplit * (kDim + 2);

  float* qf = smem + L::qf;
  for (int i = tid; i < GQ * kDim; i += 256) qf[i] = h2f(a.q[((int64_t)b * a.Hq + h0) * kDim + i]);
  if (split >= a.nsplit_q) {
    decode_residual<GQ>(a, row_resid(a, b), qf, smem + L::rsc, smem + L::rov, smem + L::rred, ws_base, ws_head,
                        unit);
    return;
  }

  const int t0 = split * a.split_tokens;
  const int ntok = max(0, min(a.split_tokens, row_quant(a, b) - t0));  // 0: empty partial
  const int nchunk = ntok / kMChunk;
  const int nblk = ntok / a.R;
  const uint8_t* kc = a.kcodes + (unit * a.cap + t0) * S;
  const uint32_t* ks = reinterpret_cast<const uint32_t*>(a.kscales) + unit * a.cap + t0;
  const uint8_t* vc = a.vcodes + (unit * a.cap + t0) * S;
  const uint32_t* vs = reinterpret_cast<const uint32_t*>(a.vscales) + unit * a.cap + t0;
  const uint16_t* kmu = a.kmu + (unit * nbmu + t0 / a.R) * kDim;
  const uint16_t* vmu = a.vmu + (unit * nbmu + t0 / a.R) * kDim;
  const int64_t blk0 = unit * nbmu + t0 / a.R;  // first block of the split (record index)

  // One chunk's global loads for this lane: the K codes its score tiles need
  // (token 16 tau + m16, the 8 (2 bits) or 4 (1 bit) code bytes starting at
  // slot 8 kb / 4 kb), and token `lane`'s scales and V code row, which go
  // through LDS.
  constexpr int KCW = SUB == 4 ? 2 : 1;
  struct Ld {
    uint32_t kc[4][KCW];
    uint32_t ksc, vsc;    // (n1, n2) fp16 pairs, or (q1 << 16 | n2) double-quantised
    uint32_t kpar, vpar;  // double-quantised: the chunk's block (S1, Z1)
    uint4_t vcode[S / 16];
  };
  auto load = [&](int ch, Ld& r) {
    const int64_t base = (int64_t)ch * kMChunk;
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
      const uint8_t* p = kc + (base + 16 * tau + m16) * S + KCW * 4 * kb;
      if constexpr (SUB == 4) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        r.kc[tau][0] = v.x;
        r.kc[tau][1] = v.y;
      } else {
        r.kc[tau][0] = *reinterpret_cast<const uint32_t*>(p);
      }
    }
    if constexpr (DQ) {
      const int SRB = dq_record_bytes(a.R);
      const int64_t rb = blk0 + (int)(base / a.R);
      const int tb = (int)((base + lane) % a.R);
      const uint8_t* kr = reinterpret_cast<const uint8_t*>(a.kscales) + rb * SRB;
      const uint8_t* vr = reinterpret_cast<const uint8_t*>(a.vscales) + rb * SRB;
      r.ksc = dq_token(kr, a.R, tb);
      r.vsc = dq_token(vr, a.R, tb);
      r.kpar = dq_s1_params(kr, a.R);
      r.vpar = dq_s1_params(vr, a.R);
    } else {
      r.ksc = ks[base + lane];
      r.vsc = vs[base + lane];
    }
#pragma unroll
    for (int i = 0; i < S / 16; ++i) r.vcode[i] = *reinterpret_cast<const uint4_t*>(vc + (base + lane) * S + 16 * i);
  };
  Ld cur;
  int ch = wave;
  if (ch < nchunk) load(ch, cur);

  // ---- per-split set-up: codebook, rotated queries, q . KMU_b -------------
  uint32_t* cb32 = reinterpret_cast<uint32_t*>(smem + L::cbh);
  for (int i = tid; i < kCodewords * SUB / 2; i += 256) cb32[i] = reinterpret_cast<const uint32_t*>(a.codebook)[i];
  // the split's block means as fp32 (at most 16 blocks x 128 channels for K
  // and V), all loads in flight together
  {
    float2* kmul = reinterpret_cast<float2*>(smem + L::kmu);
    float2* vmul = reinterpret_cast<float2*>(smem + L::vmu);
    const int nw = nblk * kDim / 2;  // channel pairs
    float2 kt[4], vt[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + 256 * j;
      kt[j] = vt[j] = float2{0.f, 0.f};
      if (i < nw) {
        if constexpr (DQ) {
          const int bl = i / (kDim / 2), cp = i % (kDim / 2);
          dq_mu_pair(reinterpret_cast<const uint8_t*>(a.kmu) + (blk0 + bl) * kDqMuRecord, cp, kt[j].x, kt[j].y);
          dq_mu_pair(reinterpret_cast<const uint8_t*>(a.vmu) + (blk0 + bl) * kDqMuRecord, cp, vt[j].x, vt[j].y);
        } else {
          const uint32_t k2 = reinterpret_cast<const uint32_t*>(kmu)[i];
          const uint32_t v2 = reinterpret_cast<const uint32_t*>(vmu)[i];
          kt[j] = float2{h2f(k2 & 0xffff), h2f(k2 >> 16)};
          vt[j] = float2{h2f(v2 & 0xffff), h2f(v2 >> 16)};
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      kmul[tid + 256 * j] = kt[j];
      vmul[tid + 256 * j] = vt[j];
    }
  }
  __syncthreads();
  const float sg0 = a.signs ? (float)a.signs[2 * lane] : 1.f;
  const float sg1 = a.signs ? (float)a.signs[2 * lane + 1] : 1.f;
  float* qr = smem + L::qr;
  for (int g = wave; g < GQ; g += 4) {
    float x[2] = {qf[g * kDim + 2 * lane] * sg0, qf[g * kDim + 2 * lane + 1] * sg1};
    fwht128<2>(x, lane);
    qr[g * kDim + 2 * lane] = x[0] * kInvSqrtD;
    qr[g * kDim + 2 * lane + 1] = x[1] * kInvSqrtD;
  }
  float* qmu = smem + L::qmu;
  for (int i = tid; i < nblk * GQ; i += 256) {
    const int bl = i / GQ, g = i % GQ;
    const float4* mp = reinterpret_cast<const float4*>(smem + L::kmu) + bl * (kDim / 4);
    const float4* qg = reinterpret_cast<const float4*>(qf + g * kDim);
    float s0 = 0.f, s1 = 0.f;
#pragma unroll 8
    for (int c = 0; c < kDim / 4; ++c) {
      const float4 m4 = mp[c], q4 = qg[c];
      s0 = fmaf(q4.x, m4.x, s0);
      s1 = fmaf(q4.y, m4.y, s1);
      s0 = fmaf(q4.z, m4.z, s0);
      s1 = fmaf(q4.w, m4.w, s1);
    }
    qmu[i] = s0 + s1;
  }
  __syncthreads();
  // B operands of the score products: lane (head m16, k-block kb), MFMA i
  // holds channels 32 kb + 8 i .. + 7 of q', as fp16 high and low parts.
  half8_t bqh[4], bql[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = m16 < GQ ? qr[m16 * kDim + 32 * kb + 8 * i + e] : 0.f;
      const half_t hi = (half_t)v;
      bqh[i][e] = hi;
      bql[i][e] = (half_t)(v - (float)hi);
    }

  float* vst = smem + L::vst + wave * L::VSTW;
  uint8_t* vcl = reinterpret_cast<uint8_t*>(vst);  // [64][S] V codes
  // per-token factors: s = KA S + KB (q . KMU), w = p VC, beta += p VD
  float* fka = vst + kMChunk * S / 4;
  float* fkb = fka + kMChunk;
  float* fvc = fkb + kMChunk;
  float* fvd = fvc + kMChunk;
  float* bc = smem + L::bc;
  float* mc = smem + L::mc;

  float m = -INFINITY, l = 0.f;
  float4_t vacc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) vacc[t] = float4_t{0.f, 0.f, 0.f, 0.f};

  for (; ch < nchunk; ch += 4) {
    Ld nxt;
    if (ch + 4 < nchunk) load(ch + 4, nxt);
    // stage this chunk's V codes and token `lane`'s factors
#pragma unroll
    for (int i = 0; i < S / 16; ++i) *reinterpret_cast<uint4_t*>(vcl + lane * S + 16 * i) = cur.vcode[i];
    {
      float kn1, kn2, vn1, vn2;
      if constexpr (DQ) {
        kn1 = dq_value(cur.kpar, cur.ksc >> 16);
        kn2 = h2f(cur.ksc & 0xffff);
        vn1 = dq_value(cur.vpar, cur.vsc >> 16);
        vn2 = h2f(cur.vsc & 0xffff);
      } else {
        kn1 = h2f(cur.ksc & 0xffff);
        kn2 = h2f(cur.ksc >> 16);
        vn1 = h2f(cur.vsc & 0xffff);
        vn2 = h2f(cur.vsc >> 16);
      }
      const float kas = a.scale_log2 * kn1;
      fka[lane] = kas * kn2;
      fkb[lane] = kas;
      fvc[lane] = vn1 * vn2;
      fvd[lane] = vn1;
    }
    wave_sync();

    // scores: tile tau covers tokens 16 tau .. 16 tau + 15 (rows), heads (columns)
    float4_t sacc[4];
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
      half8_t A[4];
      if constexpr (SUB == 4) {
        uint32_t ad[8];
        const uint32_t w0 = cur.kc[tau][0], w1 = cur.kc[tau][1];
        ad[0] = code_shl<0, 3>(w0); ad[1] = code_shl<1, 3>(w0); ad[2] = code_shl<2, 3>(w0); ad[3] = code_shl<3, 3>(w0);
        ad[4] = code_shl<0, 3>(w1); ad[5] = code_shl<1, 3>(w1); ad[6] = code_shl<2, 3>(w1); ad[7] = code_shl<3, 3>(w1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x2_t c0 = lds_b64(ad[2 * i]);
          const u32x2_t c1 = lds_b64(ad[2 * i + 1]);
          A[i] = __builtin_bit_cast(half8_t, uint4_t{c0.x, c0.y, c1.x, c1.y});
        }
      } else {
        const uint32_t w0 = cur.kc[tau][0];
        uint32_t ad[4] = {code_shl<0, 4>(w0), code_shl<1, 4>(w0), code_shl<2, 4>(w0), code_shl<3, 4>(w0)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          A[i] = __builtin_bit_cast(half8_t, lds_b128(ad[i]));
        }
      }
      float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[i], bqh[i], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[i], bql[i], acc, 0, 0, 0);
      }
      sacc[tau] = acc;
    }
    // s = KA S + KB (q . KMU_b) for this lane's 16 tokens 16 tau + 4 kb + r
    const int bl = (ch * kMChunk) / a.R;
    const float qm = m16 < GQ ? qmu[bl * GQ + m16] : 0.f;
    float s[16];
    float cmax = -INFINITY;
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
      const float4 ka = *reinterpret_cast<const float4*>(fka + 16 * tau + 4 * kb);
      const float4 kbb = *reinterpret_cast<const float4*>(fkb + 16 * tau + 4 * kb);
      const float kav[4] = {ka.x, ka.y, ka.z, ka.w}, kbv[4] = {kbb.x, kbb.y, kbb.z, kbb.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = fmaf(kav[r], sacc[tau][r], kbv[r] * qm);
        s[4 * tau + r] = v;
        cmax = fmaxf(cmax, v);
      }
    }
    cmax = fmaxf(cmax, xlane<16>(cmax));
    cmax = fmaxf(cmax, xlane<32>(cmax));
    const float mn = fmaxf(m, cmax);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    float lsum = 0.f, beta = 0.f;
    half8_t bw[2];
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
      const float4 vc4 = *reinterpret_cast<const float4*>(fvc + 16 * tau + 4 * kb);
      const float4 vd4 = *reinterpret_cast<const float4*>(fvd + 16 * tau + 4 * kb);
      const float vcv[4] = {vc4.x, vc4.y, vc4.z, vc4.w}, vdv[4] = {vd4.x, vd4.y, vd4.z, vd4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[4 * tau + r] - mn);
        lsum += p;
        beta = fmaf(p, vdv[r], beta);
        bw[tau >> 1][4 * (tau & 1) + r] = (half_t)(p * vcv[r]);
      }
    }
    l = fmaf(l, alpha, lsum);
    beta += xlane<16>(beta);
    beta += xlane<32>(beta);
    if (kb == 0 && m16 < GQ) {
      bc[ch * GQ + m16] = beta;
      mc[ch * GQ + m16] = mn;
    }
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {  // the running max moved for some head
#pragma unroll
      for (int t = 0; t < 8; ++t) vacc[t] *= alpha;
    }

    // values: 32-token step c holds the rows of score tiles 2c and 2c + 1;
    // lane (m16, kb) supplies tokens 16 (2c + e/4) + 4 kb + e%4, e = 0..7
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      int toks[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) toks[e] = 16 * (2 * c + (e >> 2)) + 4 * kb + (e & 3);
      if constexpr (SUB == 4) {
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          u32x2_t cw[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) cw[e] = lds_b64((uint32_t)vcl[toks[e] * S + 16 * g2 + m16] << 3);
#pragma unroll
          for (int ep = 0; ep < 4; ++ep) {
            const uint32_t sel = (ep & 1) ? 0x07060302u : 0x05040100u;
            uint32_t d[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint32_t lo = (ep < 2) ? cw[2 * j].x : cw[2 * j].y;
              const uint32_t hi = (ep < 2) ? cw[2 * j + 1].x : cw[2 * j + 1].y;
              d[j] = __builtin_amdgcn_perm(hi, lo, sel);
            }
            const half8_t A = __builtin_bit_cast(half8_t, uint4_t{d[0], d[1], d[2], d[3]});
            vacc[4 * g2 + ep] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bw[c], vacc[4 * g2 + ep], 0, 0, 0);
          }
        }
      } else {
        uint4_t cw[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) cw[e] = lds_b128((uint32_t)vcl[toks[e] * S + m16] << 4);
#pragma unroll
        for (int ep = 0; ep < 8; ++ep) {
          const uint32_t sel = (ep & 1) ? 0x07060302u : 0x05040100u;
          uint32_t d[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            d[j] = __builtin_amdgcn_perm(cw[2 * j + 1][ep >> 1], cw[2 * j][ep >> 1], sel);
          }
          const half8_t A = __builtin_bit_cast(half8_t, uint4_t{d[0], d[1], d[2], d[3]});
          vacc[ep] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bw[c], vacc[ep], 0, 0, 0);
        }
      }
    }
    wave_sync();
    cur = nxt;
  }

  // ---- merge the four waves, inverse transform, mean term ------------------
  l += xlane<16>(l);
  l += xlane<32>(l);
  __syncthreads();  // the main-loop LDS views are dead from here on
  float* mrg = smem + L::mrg;
  constexpr int MS = kDim + 2;
  if (m16 < GQ) {
    float* r = mrg + (wave * GQ + m16) * MS;
    if (kb == 0) {
      r[0] = m;
      r[1] = l;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) r[2 + value_channel<SUB>(t, 4 * kb + rr)] = vacc[t][rr];
  }
  __syncthreads();
  for (int g = wave; g < GQ; g += 4) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mrg[(w * GQ + g) * MS]);
    float lsum = 0.f, x[2] = {0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float* r = mrg + (w * GQ + g) * MS;
      const float f = r[0] == -INFINITY ? 0.f : exp2f(r[0] - M);
      lsum = fmaf(f, r[1], lsum);
      x[0] = fmaf(f, r[2 + 2 * lane], x[0]);
      x[1] = fmaf(f, r[2 + 2 * lane + 1], x[1]);
    }
    fwht128<2>(x, lane);
    // sum over chunks of 2^(m_c - M) beta_c MU_b(c), channels 2 lane, 2 lane + 1
    const float2* vmul = reinterpret_cast<const float2*>(smem + L::vmu);
    float om0 = 0.f, om1 = 0.f;
    for (int ci = 0; ci < nchunk; ++ci) {
      const float f = exp2f(mc[ci * GQ + g] - M) * bc[ci * GQ + g];
      const float2 mu2 = vmul[((ci * kMChunk) / a.R) * (kDim / 2) + lane];
      om0 = fmaf(f, mu2.x, om0);
      om1 = fmaf(f, mu2.y, om1);
    }
    float* wo = ws_base + g * ws_head;
    wo[2 * lane] = fmaf(x[0], kInvSqrtD * sg0, om0);
    wo[2 * lane + 1] = fmaf(x[1], kInvSqrtD * sg1, om1);
    if (lane == 0) {
      wo[kDim] = M;
      wo[kDim + 1] = lsum;
    }
  }
}

size_t decode_mfma_lds_bytes(int sub, int gq) {
  int w = 0;
  if (sub == 4) {
    w = gq == 2 ? MfmaSmem<4, 2>::total : gq == 4 ? MfmaSmem<4, 4>::total
      : gq == 8 ? MfmaSmem<4, 8>::total : MfmaSmem<4, 16>::total;
  } else {
    w = gq == 2 ? MfmaSmem<8, 2>::total : gq == 4 ? MfmaSmem<8, 4>::total
      : gq == 8 ? MfmaSmem<8, 8>::total : MfmaSmem<8, 16>::total;
  }
  return (size_t)w * sizeof(float);
}

template <int SUB, int GQ, bool DQ>
static hipError_t launch_mfma_dq(const DecodeArgs& a, int B, hipStream_t stream) {
  const size_t lds = (size_t)MfmaSmem<SUB, GQ>::total * sizeof(float);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_mfma_kernel<SUB, GQ, DQ>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid(a.nsplit, B * a.Hkv * (a.G / GQ)), block(256);
  hipLaunchKernelGGL((decode_mfma_kernel<SUB, GQ, DQ>), grid, block, lds, stream, a);
  return hipGetLastError();
}

template <int SUB, int GQ>
static hipError_t launch_mfma_t(const DecodeArgs& a, int B, hipStream_t stream) {
  return a.dq ? launch_mfma_dq<SUB, GQ, true>(a, B, stream) : launch_mfma_dq<SUB, GQ, false>(a, B, stream);
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int sub, int gq, int B, hipStream_t stream) {
  if (sub == 4) {
    if (gq == 2) return launch_mfma_t<4, 2>(a, B, stream);
    if (gq == 4) return launch_mfma_t<4, 4>(a, B, stream);
    if (gq == 8) return launch_mfma_t<4, 8>(a, B, stream);
    if (gq == 16) return launch_mfma_t<4, 16>(a, B, stream);
  } else if (sub == 8) {
    if (gq == 2) return launch_mfma_t<8, 2>(a, B, stream);
    if (gq == 4) return launch_mfma_t<8, 4>(a, B, stream);
    if (gq == 8) return launch_mfma_t<8, 8>(a, B, stream);
    if (gq == 16) return launch_mfma_t<8, 16>(a, B, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace nsnq
