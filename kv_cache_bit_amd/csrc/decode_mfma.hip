// decode_mfma.hip -- decode attention over the compressed cache for grouped
// query heads, with the scoring and the value sum on the matrix cores (gfx950).
//
// The algebra is the one of decode.hip (technical summary sec. 4, Attention
// Computation): for a token stored as codes, (N1, N2) and block mean MU_b,
//   q . k_hat = N1 (N2 (H D q) . c_hat + q . MU_b),
//   sum_t p_t v_hat_t = D H^T sum_t (p_t N1_t N2_t) c_hat_t + sum_b (sum_{t in b} p_t N1_t) MU_b.
// Here the Hadamard-domain codewords c_hat_t are gathered once per token and
// shared by every query head of the KV head, instead of one table lookup per
// (token, slot, head).  The codewords are read straight from the fp16
// codebook in LDS; q' = H D q is split into fp16 high and low parts (two
// products), so the scores keep fp32 accuracy.
//   scores, up to 4 heads: one token per lane.  v_mfma_f32_4x4x4_16b_f16 with
//           the lane's codeword (4 channels) as the B operand and q' broadcast
//           from one of 16 A blocks (CBSZ / ABID), so every lane ends with its
//           token's score for each head;
//   scores, 8 or 16 heads: v_mfma_f32_16x16x32_f16 over 16-token x 16-head
//           tiles, the A operand of a lane being the codeword pair (2 bits) or
//           codeword (1 bit) of its token;
//   values  O'[c][g] += sum_t c_hat_t[c] w_t[g] with w = p N1 N2 in fp16,
//           v_mfma_f32_16x16x32_f16 contracting over tokens: a lane gathers
//           the codewords of its 8 tokens for one slot and transposes them in
//           registers (v_perm_b32) into one A operand per channel of the slot;
//   means   per 64-token chunk, beta = sum_t p_t N1_t and the softmax
//           reference are kept in LDS and folded in once at the end of the
//           split.
// Up to 16 query heads share a work-group.

#include <type_traits>
#include <utility>

#include "decode_common.hpp"

namespace nsnq {

namespace {

constexpr int kMChunk = 64;                                 // tokens per wave step
// Staged V code rows (up to 4 heads): token t's row sits at t S + 32 (t / 8)
// bytes, 32 bytes of padding after every 8 rows.  The value step's lane
// groups read rows 8 apart; without the padding those rows share banks.  At
// 2 bits a row holds its codes as pairs (slot j, slot j + 16), so one 16-bit
// read gives a lane both slots it gathers for.
constexpr int kVRowPad = 32;
__host__ __device__ constexpr int vcode_bytes(int S) { return kMChunk * S + kMChunk / 8 * kVRowPad; }
// Row stride (fp16 elements) of the staged value weights [8][kMChunk]: the
// value step reads rows m16 mod 8 at once, which with a 128-byte stride share
// banks.
constexpr int kPbStride = kMChunk + 8;
constexpr int kMaxChunks = kMaxSplitBlocks * 128 / kMChunk;  // per split (R <= 128)
static_assert(kMaxChunks <= 64, "the merge gives each chunk a lane");

// f(std::integral_constant<int, I>) for I = 0 .. N-1, unrolled at compile time
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

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
  // per wave: V codes and 4 per-token factors, or (up to 4 heads) two sets
  // of V codes and fp16 weights
  static constexpr int VSTW = GQ <= 4 ? 2 * (vcode_bytes(S) / 4 + 4 * kPbStride) : kMChunk * S / 4 + 4 * kMChunk;
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
  // up to 4 heads: one token per lane, scores from 4x4x4 blocks; more heads
  // fill the columns of 16x16x32 tiles instead
  constexpr bool T4 = GQ <= 4;
  extern __shared__ float smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m16 = lane & 15, kb = lane >> 4;
  const int split = a.split_slow ? blockIdx.y : blockIdx.x;
  const int ux = a.split_slow ? blockIdx.x : blockIdx.y;
  const int groups = a.G / GQ;
  const int hg = ux % groups;
  const int bk = ux / groups;
  const int b = bk / a.Hkv, hk = bk % a.Hkv;
  const int h0 = hk * a.G + hg * GQ;
  const int64_t unit = (int64_t)b * a.Hkv + hk;
  const int nbmu = a.cap / a.R;
  float* ws_base = a.ws + ((int64_t)b * a.Hq + h0) * a.nsplit * (kDim + 2) + (int64_t)split * (kDim + 2);
  const int64_t ws_head = (int64_t)a.nsplit * (kDim + 2);

  float* qf = smem + L::qf;
  // queries into registers first: every set-up load below is issued before
  // any of them is waited for
  constexpr int QPT = (GQ * kDim + 255) / 256;
  uint16_t qh[QPT];
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int i = tid + 256 * j;
    qh[j] = i < GQ * kDim ? a.q[((int64_t)b * a.Hq + h0) * kDim + i] : (uint16_t)0;
  }
  if (split >= a.nsplit_q) {
#pragma unroll
    for (int j = 0; j < QPT; ++j)
      if (tid + 256 * j < GQ * kDim) qf[tid + 256 * j] = h2f(qh[j]);
    decode_residual<GQ>(a, row_resid(a, b), qf, smem + L::rsc, smem + L::rov, smem + L::rred, ws_base, ws_head,
                        unit);
    return;
  }

  const int sb0 = split_block(a, split), sb1 = split_block(a, split + 1);
  const int t0 = sb0 << a.lgR;
  const int ntok = max(0, min((sb1 - sb0) << a.lgR, row_quant(a, b) - t0));  // 0: empty partial
  const int nchunk = ntok / kMChunk;
  const int nblk = (ntok >> a.lgR);
  const uint8_t* kc = a.kcodes + (unit * a.cap + t0) * S;
  const uint32_t* ks = reinterpret_cast<const uint32_t*>(a.kscales) + unit * a.cap + t0;
  const uint8_t* vc = a.vcodes + (unit * a.cap + t0) * S;
  const uint32_t* vs = reinterpret_cast<const uint32_t*>(a.vscales) + unit * a.cap + t0;
  const uint16_t* kmu = a.kmu + (unit * nbmu + (t0 >> a.lgR)) * kDim;
  const uint16_t* vmu = a.vmu + (unit * nbmu + (t0 >> a.lgR)) * kDim;
  const int64_t blk0 = unit * nbmu + (t0 >> a.lgR);  // first block of the split (record index)

  // One chunk's global loads for this lane: the K codes its score tiles need
  // (token 16 tau + m16, the 8 (2 bits) or 4 (1 bit) code bytes starting at
  // slot 8 kb / 4 kb), and token `lane`'s scales and V code row, which go
  // through LDS.
  constexpr int KCW = SUB == 4 ? 2 : 1;
  struct LdTile {
    uint32_t kc[4][KCW];  // K codes of token 16 tau + m16, slots KCW 4 kb ..
  };
  struct LdToken {
    uint4_t kc[S / 16];   // K code row of token `lane`
  };
  struct Ld : std::conditional_t<T4, LdToken, LdTile> {
    uint32_t ksc, vsc;    // (n1, n2) fp16 pairs, or (q1 << 16 | n2) double-quantised
    uint32_t kpar, vpar;  // double-quantised: the chunk's block (S1, Z1)
    uint4_t vcode[S / 16];
  };
  // Without double quantisation the chunk loads go through buffer resources
  // bounded by the split's tokens: a prefetch past the last chunk returns
  // zeros without touching memory, so every prefetch is issued unconditionally
  // and the wait before a chunk's use counts only the loads issued before it.
  constexpr bool kBuf = !DQ;
  const buf_rsrc_t rkc = make_rsrc(kc, ntok * S), rvc = make_rsrc(vc, ntok * S);
  const buf_rsrc_t rks = make_rsrc(ks, ntok * 4), rvs = make_rsrc(vs, ntok * 4);
  auto load = [&](int ch, Ld& r) {
    const int64_t base = (int64_t)ch * kMChunk;
    if constexpr (kBuf) {
      const int tb = ch * kMChunk;
      if constexpr (T4) {
#pragma unroll
        for (int i = 0; i < S / 16; ++i) r.kc[i] = buf_load_b128(rkc, (tb + lane) * S + 16 * i);
      } else {
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
          const int off = (tb + 16 * tau + m16) * S + KCW * 4 * kb;
          if constexpr (SUB == 4) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(rkc, off, 0, 0);
            r.kc[tau][0] = v[0];
            r.kc[tau][1] = v[1];
          } else {
            r.kc[tau][0] = buf_load_b32(rkc, off);
          }
        }
      }
      r.ksc = buf_load_b32(rks, (tb + lane) * 4);
      r.vsc = buf_load_b32(rvs, (tb + lane) * 4);
#pragma unroll
      for (int i = 0; i < S / 16; ++i) r.vcode[i] = buf_load_b128(rvc, (tb + lane) * S + 16 * i);
      return;
    }
    if constexpr (T4) {
#pragma unroll
      for (int i = 0; i < S / 16; ++i) r.kc[i] = *reinterpret_cast<const uint4_t*>(kc + (base + lane) * S + 16 * i);
    } else {
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
    }
    if constexpr (DQ) {
      const int SRB = dq_record_bytes(a.R);
      const int64_t rb = blk0 + (int)(base >> a.lgR);
      const int tb = (int)((base + lane) & (a.R - 1));
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
  // randomised-Hadamard signs of channels 2 lane, 2 lane + 1
  const float sg0 = a.signs ? (float)a.signs[2 * lane] : 1.f;
  const float sg1 = a.signs ? (float)a.signs[2 * lane + 1] : 1.f;

  // ---- per-split set-up: codebook, rotated queries, q . KMU_b -------------
  uint32_t* cb32 = reinterpret_cast<uint32_t*>(smem + L::cbh);
  constexpr int CPT = kCodewords * SUB / 2 / 256;  // codebook words per thread
  uint32_t cbw[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) cbw[j] = reinterpret_cast<const uint32_t*>(a.codebook)[tid + 256 * j];
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
    // the first chunk's loads queue behind the set-up loads, which are waited
    // for first
    if (kBuf || ch < nchunk) load(ch, cur);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      kmul[tid + 256 * j] = kt[j];
      vmul[tid + 256 * j] = vt[j];
    }
  }
#pragma unroll
  for (int j = 0; j < CPT; ++j) cb32[tid + 256 * j] = cbw[j];
#pragma unroll
  for (int j = 0; j < QPT; ++j)
    if (tid + 256 * j < GQ * kDim) qf[tid + 256 * j] = h2f(qh[j]);
  __syncthreads();
  float* qr = smem + L::qr;
  for (int g = wave; g < GQ; g += 4) {
    float x[2] = {qf[g * kDim + 2 * lane] * sg0, qf[g * kDim + 2 * lane + 1] * sg1};
    fwht128<2>(x, lane);
    qr[g * kDim + 2 * lane] = x[0] * kInvSqrtD;
    qr[g * kDim + 2 * lane + 1] = x[1] * kInvSqrtD;
  }
  // q . KMU_b: the 16 lanes of a row share block b = tid / 16, each lane
  // takes 8 channels of every head and the row sums them
  float* qmu = smem + L::qmu;
  if ((tid >> 4) < nblk) {
    const int bl = tid >> 4, c8 = tid & 15;
    const float4* mp = reinterpret_cast<const float4*>(smem + L::kmu) + bl * (kDim / 4) + 2 * c8;
    const float4 m0 = mp[0], m1 = mp[1];
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      const float4* qg = reinterpret_cast<const float4*>(qf + g * kDim) + 2 * c8;
      const float4 q0 = qg[0], q1 = qg[1];
      float d = q0.x * m0.x;
      d = fmaf(q0.y, m0.y, d);
      d = fmaf(q0.z, m0.z, d);
      d = fmaf(q0.w, m0.w, d);
      d = fmaf(q1.x, m1.x, d);
      d = fmaf(q1.y, m1.y, d);
      d = fmaf(q1.z, m1.z, d);
      d = fmaf(q1.w, m1.w, d);
      d = group_sum<16>(d);
      if (c8 == 0) qmu[bl * GQ + g] = d;
    }
  }
  __syncthreads();
  // the rotated queries q' as score-product operands, in fp16 high and low parts
  half8_t bqh[4], bql[4];
  half4_t qa[2][2];  // [fp16 high, low part][k-slice half]
  if constexpr (T4) {
    // A blocks of the score products: lane 4 j + i holds channels
    // 4 (16 h + j) .. + 3 of head i in qa[.][h]; a product broadcasts block
    // j of the slice it needs to all 16 blocks
    const int i = lane & 3, j = lane >> 2;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float4 v = *reinterpret_cast<const float4*>(qr + (i < GQ ? i : 0) * kDim + 4 * (16 * h + j));
      const float on = i < GQ ? 1.f : 0.f;
      const float x[4] = {v.x * on, v.y * on, v.z * on, v.w * on};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const half_t hi = (half_t)x[e];
        qa[0][h][e] = hi;
        qa[1][h][e] = (half_t)(x[e] - (float)hi);
      }
    }
  } else {
    // B operands: lane (head m16, k-block kb), product i holds channels
    // 32 kb + 8 i .. + 7 of q'
    const float4* qrow = reinterpret_cast<const float4*>(qr + (m16 < GQ ? m16 : 0) * kDim + 32 * kb);
    const float on = m16 < GQ ? 1.f : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v0 = qrow[2 * i], v1 = qrow[2 * i + 1];
      const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = v[e] * on;
        const half_t hi = (half_t)x;
        bqh[i][e] = hi;
        bql[i][e] = (half_t)(x - (float)hi);
      }
    }
  }

  // the wave's staging area; 8 or more heads: V codes [64][S], then the
  // per-token factors s = KA S + KB (q . KMU), w = p VC, beta += p VD
  float* vst = smem + L::vst + wave * L::VSTW;
  uint8_t* vcl = reinterpret_cast<uint8_t*>(vst);
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
  // The fp16 value weights of a chunk carry the factor 2^ev, ev the smallest
  // headroom exponent of the wave's chunks so far (it only decreases, and
  // vacc is rescaled exactly when it does), so that neither a large N1 N2
  // overflows fp16 nor a small one (short value vectors, a dominant token
  // elsewhere) underflows; vacc is scaled back at the end.  64 is above the
  // exponent of any chunk (the smallest fp16 product gives 62).
  int ev = 64;

  if constexpr (T4) {
    // ---- one token per lane ----------------------------------------------
    // Scores: row r, lane t of (sh + sl) is (H D q_r / sqrt d) . codewords
    // of token t, summed over 32 slices of 4 channels (two 8-channel
    // codewords' halves at 1 bit).  The running reference mr of each head
    // moves only when a score exceeds it by more than 2^3 (then to the exact
    // maximum), so the cross-lane maximum and the rescale are rare; p <= 8,
    // and p VC / 8 in fp16 keeps the range of p VC with p <= 1.
    // The loop is software-pipelined: a chunk is scored while the value
    // products of the chunk before it run, from a second set of buffers.
    constexpr float kLazy = 3.f;
    float mr[GQ], lp[GQ];
#pragma unroll
    for (int r = 0; r < GQ; ++r) {
      mr[r] = -INFINITY;
      lp[r] = 0.f;
    }
    // per-wave buffer pair: V codes [64][S] of a chunk (padded rows), then
    // p VC / 8 (columns 0..3) and p VD / 8 (columns 4..7) of its tokens, fp16
    // [8][kPbStride]
    constexpr int kBufB = vcode_bytes(S) + 8 * kPbStride * 2;
    uint8_t* const vbase = reinterpret_cast<uint8_t*>(vst);
    const uint32_t vbase_lds = (uint32_t)(reinterpret_cast<uintptr_t>(vst) - reinterpret_cast<uintptr_t>(smem));
    // A of the beta product: row 0 all ones
    half8_t aone;
#pragma unroll
    for (int e = 0; e < 8; ++e) aone[e] = (half_t)(m16 == 0 ? 1.f : 0.f);

    float4_t sh, sl;
    float kas, ka, wn12, wn1;  // N1 N2 and N1 of the lane's token (V)
    int eb0 = 0, eb1 = 0;   // beta weights' exponent of the chunk in buffer 0 / 1
    // stage chunk `c`'s V codes in buffer `bs`, score its tokens
    auto front = [&](const Ld& c, int bs) {
      uint8_t* vb = vbase + bs * kBufB;
      uint8_t* vrw = vb + lane * S + (lane >> 3) * kVRowPad;
      if constexpr (SUB == 4) {
        // bytes (2 j, 2 j + 1) = (code of slot j, code of slot j + 16)
        const uint32_t d[8] = {c.vcode[0][0], c.vcode[0][1], c.vcode[0][2], c.vcode[0][3],
                               c.vcode[1][0], c.vcode[1][1], c.vcode[1][2], c.vcode[1][3]};
        uint32_t pd[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) pd[k] = __builtin_amdgcn_perm(d[4 + k / 2], d[k / 2], (k & 1) ? 0x07030602u : 0x05010400u);
        *reinterpret_cast<uint4_t*>(vrw) = uint4_t{pd[0], pd[1], pd[2], pd[3]};
        *reinterpret_cast<uint4_t*>(vrw + 16) = uint4_t{pd[4], pd[5], pd[6], pd[7]};
      } else {
#pragma unroll
        for (int i = 0; i < S / 16; ++i) *reinterpret_cast<uint4_t*>(vrw + 16 * i) = c.vcode[i];
      }
      float kn1, kn2, vn1, vn2;
      if constexpr (DQ) {
        kn1 = dq_value(c.kpar, c.ksc >> 16);
        kn2 = h2f(c.ksc & 0xffff);
        vn1 = dq_value(c.vpar, c.vsc >> 16);
        vn2 = h2f(c.vsc & 0xffff);
      } else {
        kn1 = h2f(c.ksc & 0xffff);
        kn2 = h2f(c.ksc >> 16);
        vn1 = h2f(c.vsc & 0xffff);
        vn2 = h2f(c.vsc >> 16);
      }
      kas = a.scale_log2 * kn1;
      ka = kas * kn2;
      wn1 = vn1;
      wn12 = vn1 * vn2;
      sh = float4_t{0.f, 0.f, 0.f, 0.f};
      sl = float4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (SUB == 4) {
        // eight gathers in flight before their products (the scheduler would
        // otherwise wait for each gather next to its product)
        static_for<4>([&](auto bt_) {
          constexpr int bt = decltype(bt_)::value;
          u32x2_t cw[8];
          static_for<8>([&](auto i_) {
            constexpr int kk = 8 * bt + decltype(i_)::value;
            cw[decltype(i_)::value] = lds_b64(code_shl<kk & 3, 3>(c.kc[kk >> 4][(kk >> 2) & 3]));
          });
          __builtin_amdgcn_sched_barrier(0);
          static_for<8>([&](auto i_) {
            constexpr int kk = 8 * bt + decltype(i_)::value;
            const half4_t B = __builtin_bit_cast(half4_t, cw[decltype(i_)::value]);
            sh = __builtin_amdgcn_mfma_f32_4x4x4f16(qa[0][kk >> 4], B, sh, 4, kk & 15, 0);
            sl = __builtin_amdgcn_mfma_f32_4x4x4f16(qa[1][kk >> 4], B, sl, 4, kk & 15, 0);
          });
        });
      } else {
        static_for<16>([&](auto j_) {
          constexpr int j = decltype(j_)::value, kk = 2 * j;
          const uint4_t cw = lds_b128(code_shl<j & 3, 4>(c.kc[0][j >> 2]));
          const half4_t B0 = __builtin_bit_cast(half4_t, u32x2_t{cw.x, cw.y});
          const half4_t B1 = __builtin_bit_cast(half4_t, u32x2_t{cw.z, cw.w});
          sh = __builtin_amdgcn_mfma_f32_4x4x4f16(qa[0][kk >> 4], B0, sh, 4, kk & 15, 0);
          sl = __builtin_amdgcn_mfma_f32_4x4x4f16(qa[1][kk >> 4], B0, sl, 4, kk & 15, 0);
          sh = __builtin_amdgcn_mfma_f32_4x4x4f16(qa[0][kk >> 4], B1, sh, 4, (kk + 1) & 15, 0);
          sl = __builtin_amdgcn_mfma_f32_4x4x4f16(qa[1][kk >> 4], B1, sl, 4, (kk + 1) & 15, 0);
        });
      }
    };
    // softmax of the scored chunk `chk`, its weights into buffer `bs`
    auto weigh = [&](int chk, int bs) {
      // s = KA S + KB (q . KMU_b), in log2 units
      const int bl = (chk * kMChunk) >> a.lgR;
      float sc[GQ], dl[GQ];
      bool up = false;
#pragma unroll
      for (int r = 0; r < GQ; ++r) {
        sc[r] = fmaf(ka, sh[r] + sl[r], kas * qmu[bl * GQ + r]);
        dl[r] = sc[r] - mr[r];
        up = up || dl[r] > kLazy;
      }
      if (__builtin_amdgcn_ballot_w64(up)) {
        float as = 1.f;
#pragma unroll
        for (int r = 0; r < GQ; ++r) {
          const float mn = fmaxf(mr[r], group_max<64>(sc[r]));
          const float al = __builtin_amdgcn_exp2f(mr[r] - mn);
          mr[r] = mn;
          lp[r] *= al;
          dl[r] = sc[r] - mn;
          as = m16 == r ? al : as;
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) vacc[t] *= as;
      }
      // fp16 weights p N1 N2 2^(ev - 3) and p N1 2^(eb - 3): with p <= 8 they
      // stay below 2^15; beta's exponent is the chunk's own (each chunk's
      // beta is taken out separately)
      const int ec = f16_headroom_exp(wave_max_nonneg(fabsf(wn12)));
      const int eb = f16_headroom_exp(wave_max_nonneg(fabsf(wn1)));
      if (ec < ev) {
        const float f = pow2f(ec - ev);
#pragma unroll
        for (int t = 0; t < 8; ++t) vacc[t] *= f;
        ev = ec;
      }
      if (bs) eb1 = eb;
      else eb0 = eb;
      const float fw = wn12 * pow2f(ev - 3), fb = wn1 * pow2f(eb - 3);
      uint16_t* pb = reinterpret_cast<uint16_t*>(vbase + bs * kBufB + vcode_bytes(S));
#pragma unroll
      for (int r = 0; r < GQ; ++r) {
        const float pr = __builtin_amdgcn_exp2f(dl[r]);
        lp[r] += pr;
        pb[r * kPbStride + lane] = f2h(pr * fw);
        pb[(4 + r) * kPbStride + lane] = f2h(pr * fb);
      }
      if (lane == 0) {  // the references are uniform over the wave
#pragma unroll
        for (int r = 0; r < GQ; ++r) mc[chk * GQ + r] = mr[r];
      }
    };
    // value products of the weighed chunk `chk` in buffer `bs`; lane
    // (m16, kb) supplies tokens 32 c + 8 kb + e of step c
    auto back = [&](int chk, int bs) {
      const uint8_t* vb = vbase + bs * kBufB;
      const uint32_t pb_lds = vbase_lds + bs * kBufB + vcode_bytes(S);
      float4_t db = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const half8_t bw = __builtin_bit_cast(half8_t, lds_b128(pb_lds + 2 * ((m16 & 7) * kPbStride + 32 * c + 8 * kb)));
        const uint8_t* vrow = vb + (32 * c + 8 * kb) * S + (4 * c + kb) * kVRowPad + m16;
        if constexpr (SUB == 4) {
          // the code pairs (slot m16, slot m16 + 16) of the eight tokens
          const uint16_t* vrow16 = reinterpret_cast<const uint16_t*>(vrow - m16) + m16;
          uint32_t code2[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) code2[e] = vrow16[e * (S / 2)];
#pragma unroll
          for (int g2 = 0; g2 < 2; ++g2) {
            // all eight gathers, then the products
            __builtin_amdgcn_sched_barrier(0);
            u32x2_t cw[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) cw[e] = lds_b64(g2 ? code_shl<1, 3>(code2[e]) : code_shl<0, 3>(code2[e]));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ep = 0; ep < 4; ++ep) {
              const uint32_t sel = (ep & 1) ? 0x07060302u : 0x05040100u;
              uint32_t d[4];
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) {
                const uint32_t lo = (ep < 2) ? cw[2 * jj].x : cw[2 * jj].y;
                const uint32_t hi = (ep < 2) ? cw[2 * jj + 1].x : cw[2 * jj + 1].y;
                d[jj] = __builtin_amdgcn_perm(hi, lo, sel);
              }
              const half8_t A = __builtin_bit_cast(half8_t, uint4_t{d[0], d[1], d[2], d[3]});
              vacc[4 * g2 + ep] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bw, vacc[4 * g2 + ep], 0, 0, 0);
            }
          }
        } else {
          uint4_t cw[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) cw[e] = lds_b128((uint32_t)vrow[e * S] << 4);
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
        db = __builtin_amdgcn_mfma_f32_16x16x32_f16(aone, bw, db, 0, 0, 0);
      }
      // beta_r = sum p VD: row 0, column 4 + r of db (lanes 4 .. 4 + GQ - 1),
      // scaled back by the chunk's exponent
      if (m16 >= 4 && m16 < 4 + GQ && kb == 0) bc[chk * GQ + m16 - 4] = db[0] * pow2f(3 - (bs ? eb1 : eb0));
    };

    if (ch < nchunk) {
      {
        Ld nxt;
        if (kBuf || ch + 4 < nchunk) load(ch + 4, nxt);
        front(cur, 0);
        weigh(ch, 0);
        cur = nxt;
      }
      int chp = ch, bs = 1;
      for (ch += 4; ch < nchunk; ch += 4) {
        Ld nxt;
        if (kBuf || ch + 4 < nchunk) load(ch + 4, nxt);
        front(cur, bs);       // score this chunk ...
        back(chp, bs ^ 1);    // ... while the one before it meets its values
        weigh(ch, bs);
        chp = ch;
        bs ^= 1;
        cur = nxt;
      }
      back(chp, bs ^ 1);
    }
    // lane (m16 < GQ, kb): reference and sum of head m16; the value columns
    // hold p VC 2^(ev - 3)
    m = mr[0];
    l = 0.f;
#pragma unroll
    for (int r = 0; r < GQ; ++r) {
      const float lt = group_sum<64>(lp[r]);
      m = m16 == r ? mr[r] : m;
      l = m16 == r ? lt : l;
    }
    {
      const float f = pow2f(3 - ev);
#pragma unroll
      for (int t = 0; t < 8; ++t) vacc[t] *= f;
    }
  } else {
  for (; ch < nchunk; ch += 4) {
      Ld nxt;
      if (kBuf || ch + 4 < nchunk) load(ch + 4, nxt);
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
        // the chunk's value weights p N1 N2 (p <= 1) carry 2^ev in fp16
        const int ec = f16_headroom_exp(wave_max_nonneg(fabsf(vn1 * vn2)));
        if (ec < ev) {
          const float f = pow2f(ec - ev);
#pragma unroll
          for (int t = 0; t < 8; ++t) vacc[t] *= f;
          ev = ec;
        }
      }
      const float fwv = pow2f(ev);
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
      const int bl = (ch * kMChunk) >> a.lgR;
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
          bw[tau >> 1][4 * (tau & 1) + r] = (half_t)(p * vcv[r] * fwv);
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
  }

  // ---- merge the four waves, inverse transform, mean term ------------------
  if constexpr (!T4) {
    l += xlane<16>(l);
    l += xlane<32>(l);
    const float f = pow2f(-ev);
#pragma unroll
    for (int t = 0; t < 8; ++t) vacc[t] *= f;
  }
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
    // sum over chunks of 2^(m_c - M) beta_c MU_b(c), channels 2 lane, 2 lane + 1:
    // lane c weighs chunk c (a split has at most 32 chunks), then the weights
    // of each block's chunks meet its mean
    const float2* vmul = reinterpret_cast<const float2*>(smem + L::vmu);
    const float fch = lane < nchunk ? exp2f(mc[lane * GQ + g] - M) * bc[lane * GQ + g] : 0.f;
    const int cpb = a.R / kMChunk;
    float om0 = 0.f, om1 = 0.f;
    for (int bl = 0; bl < nblk; ++bl) {
      float f = 0.f;
      for (int j = 0; j < cpb; ++j)
        f += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fch), bl * cpb + j));
      const float2 mu2 = vmul[bl * (kDim / 2) + lane];
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
static int mfma_groups_per_cu() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(&decode_mfma_kernel<SUB, GQ, DQ>),
                                                   256, (size_t)MfmaSmem<SUB, GQ>::total * sizeof(float)) != hipSuccess)
    return 0;
  return n;
}

template <int SUB>
static int mfma_groups_per_cu_s(int gq, bool dq) {
  if (gq == 2) return dq ? mfma_groups_per_cu<SUB, 2, true>() : mfma_groups_per_cu<SUB, 2, false>();
  if (gq == 4) return dq ? mfma_groups_per_cu<SUB, 4, true>() : mfma_groups_per_cu<SUB, 4, false>();
  if (gq == 8) return dq ? mfma_groups_per_cu<SUB, 8, true>() : mfma_groups_per_cu<SUB, 8, false>();
  if (gq == 16) return dq ? mfma_groups_per_cu<SUB, 16, true>() : mfma_groups_per_cu<SUB, 16, false>();
  return 0;
}

int decode_mfma_resident_groups(int sub, int gq, bool dq) {
  // cached per device and kernel variant; 0 = unknown (no device, query
  // failed).  Concurrent first queries store the same value.
  static std::atomic<int> cache[kMaxDevices][2][5][2];  // [device][sub 4/8][log2 gq][dq], -1 = "unknown"
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 0;
  }
  const int si = sub == 8 ? 1 : 0;
  const int gi = gq == 2 ? 1 : gq == 4 ? 2 : gq == 8 ? 3 : gq == 16 ? 4 : 0;
  std::atomic<int>& slot = cache[dev][si][gi][dq ? 1 : 0];
  int v = slot.load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0;
    const int per_cu = sub == 4 ? mfma_groups_per_cu_s<4>(gq, dq) : mfma_groups_per_cu_s<8>(gq, dq);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
    (void)hipGetLastError();
    v = per_cu > 0 && cus > 0 ? per_cu * cus : -1;
    slot.store(v, std::memory_order_relaxed);
  }
  return v > 0 ? v : 0;
}

template <int SUB, int GQ, bool DQ>
static hipError_t launch_mfma_dq(const DecodeArgs& a, int B, hipStream_t stream) {
  const size_t lds = (size_t)MfmaSmem<SUB, GQ>::total * sizeof(float);
  static std::atomic<bool> lds_set[kMaxDevices];
  const hipError_t e = allow_lds(reinterpret_cast<const void*>(&decode_mfma_kernel<SUB, GQ, DQ>), lds_set);
  if (e != hipSuccess) return e;
  // compressed splits first when they all fit the device at once (see the
  // LUT kernel's launcher)
  DecodeArgs c = a;
  const int units = B * a.Hkv * (a.G / GQ);
  const int cap = decode_mfma_resident_groups(SUB, GQ, DQ);
  c.split_slow = (cap > 0 && (int64_t)a.nsplit_q * units <= cap) || units > 65535 ? 1 : 0;  // grid y <= 65535
  const dim3 grid = c.split_slow ? dim3(units, a.nsplit) : dim3(a.nsplit, units), block(256);
  hipLaunchKernelGGL((decode_mfma_kernel<SUB, GQ, DQ>), grid, block, lds, stream, c);
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
