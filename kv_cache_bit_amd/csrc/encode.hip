// encode.hip -- fused NSN + Hadamard + VQ encode of R-token blocks (gfx950).
//
// The unit of work is one block of R tokens of one (batch row, head) stream,
// K or V.  The exhaustive search runs one 8-wave work-group per block; the
// candidate-list search (2 bits) runs one persistent 16-wave group per CU and
// K/V half that loops over blocks.  Each lane holds one sub-vector (s = SUB
// elements) of one token, so a token occupies S = 128/SUB consecutive lanes
// and a wave "row" covers 64/S tokens.
//
//  1. token-wise normalisation to norm sqrt(d) (n1), kept in registers;
//  2. channel mean over the block (wave partial sums, LDS across waves);
//  3. second normalisation (n2), w = z / n2;
//  4. Walsh-Hadamard transform across the S lanes of a token, scaled by
//     1/sqrt(d) (its DPP stages leave each lane with a relabelled slot and a
//     sign: fwht_lanes in nsnq_device.hpp);
//  5. VQ: squared distances to all 256 codewords (or to the candidate list
//     of the sub-vector's orthant box) as an MFMA GEMM, then a per-lane
//     argmin on packed (distance | index) keys.
//
// Distance GEMM.  Codewords are the rows (M) and sub-vectors the columns (N)
// of v_mfma_f32_32x32x16_f16 tiles, so each lane receives 16 candidate
// codewords of ONE sub-vector per tile and the argmin runs in registers.  The
// K dimension carries, for each sub-vector u and codeword c,
//     [u_hi, u_lo] . [-2c, -2c]  +  [uu_hi, uu_lo, 1, 1] . [1, 1, b_hi, b_lo]
// with u = u_hi + u_lo split into two fp16 halves (22 significant bits),
// uu = ||u||^2 and b = ||c||^2 + eps likewise split, so the accumulator holds
// D = ||u - c||^2 + eps >= 0 to ~1e-6 absolute.  Positive floats order like
// their bit patterns; the low 8 mantissa bits are replaced by the codeword
// index and a v_min3_u32 chain yields the argmin (ties: lowest index).  The
// truncation costs at most 2^-15 relative, below the 1e-4 near-tie band.
// At 2 bits (SUB = 4) all terms fit one K = 16 instruction; at 1 bit
// (SUB = 8) the hi/lo products fill K = 16 and the bias terms go through a
// second 32x32x8 instruction.

#include <algorithm>
#include <type_traits>

#include "nsnq_device.hpp"
#include "nsnq_launch.hpp"

namespace nsnq {

// eps keeps the packed distance strictly positive despite rounding when a
// sub-vector sits on a codeword.
constexpr float kDistEps = 0.000244140625f;  // 2^-12
// n2 below this is rounding noise of the shift: treated as zero
constexpr float kN2Floor = 0.000244140625f;  // 2^-12

// Packed argmin key: the distance's bits with the low byte replaced by the
// codeword index.  With the mask in a VGPR and the index in an SGPR this is a
// single v_and_or_b32 (constant-bus limit: one scalar operand).
__device__ __forceinline__ uint32_t make_key(float dist, uint32_t vmask, uint32_t idx) {
  return (__float_as_uint(dist) & vmask) | idx;
}

// Packed fp16 pairs straight from fp32 products, each half written by one
// mixed-precision fma (v_fma_mixlo_f16 / v_fma_mixhi_f16; the compiler
// otherwise packs with a shift and an or per word):
//   mix_pair:     [f16(b s), f16(a s)]
//   mix_rem_pair: [f16(b s - h.hi), f16(a s - h.lo)], the fused remainders
//   mix_lo:       f16(a s) in the low half (the high half is left as it was)
//   mix_rem_lo:   [f16(a s - h.lo), h.lo]
__device__ __forceinline__ uint32_t mix_lo(float a, float s) {
  uint32_t w;
  asm("v_fma_mixlo_f16 %0, %1, %2, 0" : "=v"(w) : "v"(a), "v"(s));
  return w;
}
__device__ __forceinline__ uint32_t mix_pair(float a, float b, float s) {
  uint32_t w;
  asm("v_fma_mixlo_f16 %0, %1, %3, 0\n\tv_fma_mixhi_f16 %0, %2, %3, 0" : "=&v"(w) : "v"(a), "v"(b), "v"(s));
  return w;
}
__device__ __forceinline__ uint32_t mix_rem_pair(float a, float b, float s, uint32_t h) {
  uint32_t w;
  asm("v_fma_mixlo_f16 %0, %1, %3, -%4 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %0, %2, %3, -%4 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
      : "=&v"(w)
      : "v"(a), "v"(b), "v"(s), "v"(h));
  return w;
}
__device__ __forceinline__ uint32_t mix_rem_lo(float a, float s, uint32_t h) {
  uint32_t w = h;
  asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel_hi:[0,0,1]" : "+v"(w) : "v"(a), "v"(s), "v"(h));
  return w;
}

// words 2 and 3 of a token's 8-channel (1-bit) slice; a 4-channel slice has none
__device__ __forceinline__ uint32_t raw_hi(const uint2&, int) { return 0u; }
__device__ __forceinline__ uint32_t raw_hi(const uint4& r, int i) { return i ? r.w : r.z; }
__device__ __forceinline__ uint32_t pack_h2(half_t a, half_t b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ half8_t u32x4_to_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  uint4_t v = {a, b, c, d};
  return __builtin_bit_cast(half8_t, v);
}

__device__ __forceinline__ uint4_t half8_to_u32x4(half8_t h) { return __builtin_bit_cast(uint4_t, h); }

// Move lanes 0-31 / 32-63 between two registers (one v_permlane32_swap):
//   lo_out = [a(lanes 0-31), b(lanes 0-31) moved up]
//   hi_out = [a(lanes 32-63) moved down, b(lanes 32-63)]
__device__ __forceinline__ void half_swap(uint32_t a, uint32_t b, uint32_t& lo_out, uint32_t& hi_out, int) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  lo_out = r[0];
  hi_out = r[1];
}

// Split of a stream of L tokens: the last r = ((L - 1) mod R) + 1 stay in the
// residual window (r = 0 when L = 0).
__device__ __forceinline__ int resid_of(int L, int R) { return L > 0 ? ((L - 1) % R) + 1 : 0; }

// Work-groups past the encode blocks copy the last r tokens of each stream
// into the residual window (one group per (b, h), K or V).  Ragged prefill:
// r and the first copied token follow the row's length, and the group of
// (h = 0, K) writes the row's counters.
__device__ __forceinline__ void resid_copy(const EncodeArgs& a, int unit, int kv) {
  const int b = unit / a.H, h = unit % a.H;
  int t0 = a.rc_t0, r = a.rc_r;
  if (a.lens) {
    const int L = min(max(a.lens[b], 0), a.lens_max);
    r = resid_of(L, a.R);
    t0 = L - r;
    if (h == 0 && kv == 0 && threadIdx.x == 0) {
      a.out_quant[b] = t0;
      a.out_resid[b] = r;
    }
  }
  const uint16_t* src = a.src[kv] + (int64_t)b * a.sb + (int64_t)h * a.sh + (int64_t)t0 * a.st;
  uint16_t* dst = a.resid[kv] + (int64_t)unit * a.R * kDim;
  for (int i = threadIdx.x; i < r * 16; i += blockDim.x) {  // 16 x 8 halves per row
    const int t = i >> 4, c = (i & 15) * 8;
    *reinterpret_cast<uint4*>(dst + (int64_t)t * kDim + c) =
        *reinterpret_cast<const uint4*>(src + (int64_t)t * a.st + c);
  }
}

// Double-quantised format: bytes of one block's scales record (n2 fp16 per
// token, s1 4-bit codes, their (S, Z) pair, padding to 16) and mean record
// (4-bit codes of the 128 channels, (S, Z) per 32-channel group).
template <int R>
constexpr int dq_scales_bytes() { return ((2 * R + R / 2 + 4) + 15) / 16 * 16; }
constexpr int kDqMuBytes = 80;

// 4-bit round-to-nearest code of v in a group with fp16 zero Z and step S.
__device__ __forceinline__ float rtn4_code(float v, float Z, float S) {
  if (!(S > 0.f)) return 0.f;
  return fminf(fmaxf(rintf((v - Z) / S), 0.f), 15.f);
}

// Waves per encode work-group.  Exhaustive search: 8 x 64 lanes share one
// block's LDS staging, which lets 4 waves per SIMD stay resident (the 48 KB of
// LDS per group would otherwise cap a 4-wave group at 3).  Candidate-list
// search: 16 waves, one group per CU, since the block's sub-vector records
// and the boxes' operand tiles take ~150 KB of LDS.
template <int NT>
constexpr int enc_waves() { return NT ? 16 : 8; }

// B operand of the bias rows for a sub-vector: (|u|^2 hi, lo, 1, 1, 0, 0, 0, 0).
__device__ __forceinline__ half8_t bias_operand(uint32_t uu_pair) {
  return u32x4_to_half8(uu_pair, 0x3C003C00u, 0u, 0u);
}

// NT = 0: every codeword is compared.  NT = 2, 3 (2 bits): each sub-vector is
// compared with the first 32 NT entries of its orthant box's candidate list,
// or with the first 32 NT - 16 when HALF (the last tile's upper rows are not
// searched).
template <int SUB, int R, bool DQ, int NT, bool HALF>
__global__ __launch_bounds__(64 * enc_waves<NT>()) void encode_kernel(EncodeArgs a) {
  constexpr int NW = enc_waves<NT>();
  static_assert(NT == 0 || SUB == 4, "candidate lists exist for 4-element sub-vectors only");
  // work-groups past the encoding ones copy the residual tokens
  const int n_enc = NT ? a.n_enc : a.nblk * a.n_units;
  if ((int)blockIdx.x >= n_enc) {
    resid_copy(a, blockIdx.x - n_enc, blockIdx.y);
    return;
  }
  constexpr int S = kDim / SUB;      // slots = lanes per token
  constexpr int TPR = kWave / S;     // tokens per wave row
  constexpr int TPW = R / NW;        // tokens per wave
  constexpr int ROWS = TPW / TPR;    // rows per wave
  static_assert(ROWS * TPR * NW == R, "block split");

  __shared__ float red[NW][kDim];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int slot = lane % S;
  const int oslot = hslot(slot);  // the slot this lane holds after the transform
  const int tir = lane / S;
  const int kv = blockIdx.y;


  // ---- codebook operands (A side), per 32-codeword tile -------------------
  // Built once per group into LDS and re-read per row, which keeps ~40 VGPRs
  // free.  Exhaustive search: lane l of tile t holds codeword 32 t + (l % 32).
  // Candidate lists: tile t of box o holds list entries 32 t .. 32 t + 31, so
  // every operand read is a sequential, conflict-free 16-byte load.
  constexpr int NTILE = NT ? 16 * NT : 8;
  __shared__ half8_t sA1[NTILE][kWave];
  __shared__ half4_t sA2[SUB == 8 ? 8 : 1][kWave];
  for (int i = tid; i < NTILE * kWave; i += blockDim.x) {
    const int t = i / kWave, l = i % kWave;
    const int k = NT ? a.cand[(t / (NT ? NT : 1)) * 128 + 32 * (t % (NT ? NT : 1)) + (l & 31)] : 32 * t + (l & 31);
    const uint16_t* cb = a.codebook;
    float c[SUB];
    float nrm = 0.f;
#pragma unroll
    for (int e = 0; e < SUB; ++e) {
      c[e] = h2f(cb[k * SUB + e]);
      nrm = fmaf(c[e], c[e], nrm);
    }
    const float bsum = nrm + kDistEps;
    const half_t b_hi = (half_t)bsum;
    const half_t b_lo = (half_t)(bsum - (float)b_hi);
    half8_t av;
    if constexpr (SUB == 4) {
      if (l < 32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          av[e] = (half_t)(-2.f * c[e]);
          av[4 + e] = (half_t)(-2.f * c[e]);
        }
      } else {
        av[0] = (half_t)1.f; av[1] = (half_t)1.f; av[2] = b_hi; av[3] = b_lo;
        av[4] = (half_t)0.f; av[5] = (half_t)0.f; av[6] = (half_t)0.f; av[7] = (half_t)0.f;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) av[e] = (half_t)(-2.f * c[e]);
      sA2[t % 8][l] = half4_t{(half_t)1.f, (half_t)1.f, b_hi, b_lo};
    }
    sA1[t][l] = av;
  }

  // ---- candidate-list search state (NT > 0) -------------------------------
  // Per sub-vector i = token * S + slot: its fp16 hi/lo parts and |u|^2 pair
  // (plus one all-zero record for padding columns), its orthant box, later its
  // code; the box-sorted column order; the lists; per-box counts and offsets.
  constexpr int NSV = NT ? R * S : 1;     // sub-vectors of the block
  constexpr int kDummy = NSV;             // the all-zero record
  constexpr int kCols = NSV + 16 * 32;    // sorted columns, each box padded to 32
  __shared__ half8_t recs[NT ? NSV + 1 : 1];
  __shared__ uint32_t uus[NT ? NSV + 1 : 1];
  __shared__ __attribute__((aligned(16))) uint8_t boxc[NT ? NSV : 16];
  __shared__ uint16_t sidx[NT ? kCols : 1];
  __shared__ __attribute__((aligned(16))) uint8_t lst[NT ? 16 * 128 : 16];
  __shared__ uint8_t cbox[NT ? kCols / 32 : 1];
  __shared__ uint32_t whist[NT ? NW : 1][16];  // per wave and box: count, then first column
  __shared__ float n1t[NT ? R : 1], n2t[NT ? R : 1];
  if constexpr (NT > 0) {
    for (int i = tid; i < 128; i += blockDim.x)
      reinterpret_cast<uint4*>(lst)[i] = reinterpret_cast<const uint4*>(a.cand)[i];
    if (tid == 0) {
      recs[kDummy] = half8_t{};
      uus[kDummy] = 0u;
    }
  }
  // (visible after the first __syncthreads below)

  // One row = this lane's sub-vector of token `tok`: raw fp16 load, then
  // y = x / n1 with n1 = ||x|| / sqrt(d).  Pass 1 reads the block from HBM
  // once and keeps the raw fp16 rows in LDS; pass 2 recomputes y from there
  // instead of keeping R x 128 floats in registers.  (With candidate lists the
  // LDS holds the sub-vector records instead, and the rows stay in registers.)
  using raw_t = typename std::conditional<SUB == 4, uint2, uint4>::type;
  __shared__ raw_t xs[NT ? 1 : R * S];  // [token][slot], R x 256 bytes
  __shared__ float n1s[DQ ? R : 1];   // double quantisation: s1 per token
  __shared__ float n1hs[DQ ? R : 1];  // n1_hat per token
  __shared__ float mus[kDim];         // channel means of the block
  __shared__ float n1p[DQ ? 1 : R], invp[DQ ? 1 : R];  // pass 1's n1 and 1 / n1 per token
  // candidate lists: this lane's rows stay in registers from pass 1 to pass 2,
  // and the next block's rows are loaded under this block's products
  raw_t xr[NT ? ROWS : 1], xn[NT ? ROWS : 1];
  const int items = a.nblk * a.n_units;
  auto row_ptr = [&](int item) -> const uint16_t* {
    const int blk = item % a.nblk, unit = item / a.nblk;
    return a.src[kv] + (int64_t)(unit / a.H) * a.sb + (int64_t)(unit % a.H) * a.sh + (int64_t)blk * R * a.st +
           (int64_t)(wave * TPW + tir) * a.st + slot * SUB;
  };
  auto load_rows = [&](int item, raw_t (&dst)[NT ? ROWS : 1]) {
    const uint16_t* p = row_ptr(item);
#pragma unroll
    for (int r = 0; r < (NT ? ROWS : 1); ++r) dst[r] = *reinterpret_cast<const raw_t*>(p + (int64_t)r * TPR * a.st);
  };

  // Encode block `blk` of stream `unit` (b * H + h); `next` is the item whose
  // rows to prefetch (candidate lists), or past the end.  Returns whether the
  // prefetch was issued (false when the block is skipped).
  auto encode_block = [&](int blk, int unit, int next) -> bool {
  const int b = unit / a.H, h = unit % a.H;
  int dst0 = a.dst_tok0;  // first destination token of this launch's blocks
  if (a.lens) {           // ragged prefill: this row encodes L - r tokens
    const int L = min(max(a.lens[b], 0), a.lens_max);
    if (blk * R >= L - resid_of(L, R)) return false;
  } else if (a.fl_resid) {  // ragged flush: only full windows, each at its row's n_quant
    dst0 = a.fl_quant[b];
    if (a.fl_resid[b] != R || dst0 < 0 || dst0 % R != 0 || dst0 + R > a.cap) return false;
  }

  const uint16_t* src = a.src[kv] + (int64_t)b * a.sb + (int64_t)h * a.sh + (int64_t)blk * R * a.st;
  const int64_t tok_base = (int64_t)unit * a.cap + dst0 + (int64_t)blk * R;
  if constexpr (NT > 0) {
    if (tid < NW * 16) whist[tid / 16][tid % 16] = 0u;
  }
  auto load_raw = [&](int tok) -> raw_t {
    const raw_t v = *reinterpret_cast<const raw_t*>(src + (int64_t)tok * a.st + slot * SUB);
    if constexpr (NT == 0) xs[tok * S + slot] = v;
    return v;
  };
  auto lds_raw = [&](int tok) -> raw_t { return xs[NT ? 0 : tok * S + slot]; };
  auto fetch = [&](int r, int tok) -> raw_t {
    if constexpr (NT > 0) return xr[r];  // loaded ahead
    else return load_raw(tok);
  };
  auto row_raw = [&](int r, int tok) -> raw_t {
    if constexpr (NT > 0) return xr[r];
    else return lds_raw(tok);
  };
  auto norm_raw = [&](const raw_t& raw, float (&y)[SUB], float& n1, float& inv) {
    float v[SUB];
    v[0] = h2f(raw.x & 0xffff); v[1] = h2f(raw.x >> 16);
    v[2] = h2f(raw.y & 0xffff); v[3] = h2f(raw.y >> 16);
    if constexpr (SUB == 8) {
      v[4] = h2f(raw.z & 0xffff); v[5] = h2f(raw.z >> 16);
      v[6] = h2f(raw.w & 0xffff); v[7] = h2f(raw.w >> 16);
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < SUB; ++e) ss = fmaf(v[e], v[e], ss);
    ss = group_sum<S>(ss) * (1.0f / kDim);
    const float rs = __builtin_amdgcn_rsqf(ss);  // 1 / n1
    inv = ss > 0.f ? rs : 0.f;
    n1 = ss * inv;
#pragma unroll
    for (int e = 0; e < SUB; ++e) y[e] = v[e] * inv;
  };

  // ---- pass 1: channel sums of y over the block ---------------------------
  // Double-quantised format: s1 is first coded in 4 bits over the block and
  // tokens are divided by the stored value n1_hat (so the reconstruction from
  // stored values only carries the VQ error).
  constexpr int SR = dq_scales_bytes<R>();
  uint8_t* srec = reinterpret_cast<uint8_t*>(a.scales[kv]) + ((int64_t)unit * (a.cap / R) + dst0 / R + blk) * SR;
  uint8_t* mrec = reinterpret_cast<uint8_t*>(a.mu[kv]) + ((int64_t)unit * (a.cap / R) + dst0 / R + blk) * kDqMuBytes;
  float csum[SUB];
#pragma unroll
  for (int e = 0; e < SUB; ++e) csum[e] = 0.f;
  if constexpr (DQ) {
#pragma unroll 4
    for (int r = 0; r < ROWS; ++r) {
      const int tok = wave * TPW + r * TPR + tir;
      float y[SUB], n1, inv;
      norm_raw(fetch(r, tok), y, n1, inv);
      if (slot == 0) n1s[tok] = n1;
    }
    __syncthreads();
    float lo = INFINITY, hi = -INFINITY;
    for (int i = lane; i < R; i += kWave) {
      lo = fminf(lo, n1s[i]);
      hi = fmaxf(hi, n1s[i]);
    }
    lo = -group_max<kWave>(-lo);
    hi = group_max<kWave>(hi);
    const half_t Z1h = (half_t)lo, S1h = (half_t)((hi - lo) / 15.f);
    const float Z1 = (float)Z1h, S1 = (float)S1h;
    if (wave == 0) {
      for (int i = lane; i < R / 2; i += kWave) {
        const int q0 = (int)rtn4_code(n1s[2 * i], Z1, S1), q1 = (int)rtn4_code(n1s[2 * i + 1], Z1, S1);
        srec[2 * R + i] = (uint8_t)(q0 | (q1 << 4));
      }
      if (lane == 0) {
        *reinterpret_cast<uint32_t*>(srec + 2 * R + R / 2) = pack_h2(S1h, Z1h);
        for (int i = 2 * R + R / 2 + 4; i < SR; ++i) srec[i] = 0;
      }
    }
#pragma unroll 4
    for (int r = 0; r < ROWS; ++r) {
      const int tok = wave * TPW + r * TPR + tir;
      const float nh = fmaf(S1, rtn4_code(n1s[tok], Z1, S1), Z1);
      const float inv = nh > 0.f ? 1.f / nh : 0.f;
      const raw_t raw = row_raw(r, tok);
      float v[SUB];
      v[0] = h2f(raw.x & 0xffff); v[1] = h2f(raw.x >> 16);
      v[2] = h2f(raw.y & 0xffff); v[3] = h2f(raw.y >> 16);
      if constexpr (SUB == 8) {
        v[4] = h2f(raw.z & 0xffff); v[5] = h2f(raw.z >> 16);
        v[6] = h2f(raw.w & 0xffff); v[7] = h2f(raw.w >> 16);
      }
#pragma unroll
      for (int e = 0; e < SUB; ++e) csum[e] += v[e] * inv;
      if (slot == 0) n1hs[tok] = nh;
    }
  } else {
#pragma unroll 4
    for (int r = 0; r < ROWS; ++r) {
      const int tok = wave * TPW + r * TPR + tir;
      float y[SUB], n1, inv;
      norm_raw(fetch(r, tok), y, n1, inv);
      if (slot == 0) {
        n1p[tok] = n1;
        invp[tok] = inv;
      }
#pragma unroll
      for (int e = 0; e < SUB; ++e) csum[e] += y[e];
    }
  }
  // combine the TPR lanes holding the same channels, then the waves
#pragma unroll
  for (int e = 0; e < SUB; ++e) {
    if constexpr (S <= 16) csum[e] += xlane<16>(csum[e]);
    csum[e] += xlane<32>(csum[e]);
  }
  if (tir == 0) {
#pragma unroll
    for (int e = 0; e < SUB; ++e) red[wave][slot * SUB + e] = csum[e];
  }
  __syncthreads();
  // channel means: one thread per channel sums the waves' partials
  if (tid < kDim) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) sum += red[w][tid];
    mus[tid] = sum * (1.0f / R);
  }
  __syncthreads();
  float mu[SUB];
#pragma unroll
  for (int e = 0; e < SUB; ++e) mu[e] = mus[slot * SUB + e];
  if constexpr (DQ) {
    // 4-bit codes of the mean in groups of 32 channels (32 / SUB slots); the
    // pass below shifts by the stored mean mu_hat
    constexpr int GL = 32 / SUB;
    float lo = mu[0], hi = mu[0];
#pragma unroll
    for (int e = 1; e < SUB; ++e) {
      lo = fminf(lo, mu[e]);
      hi = fmaxf(hi, mu[e]);
    }
    lo = -group_max<GL>(-lo);
    hi = group_max<GL>(hi);
    const half_t Zh = (half_t)lo, Sh = (half_t)((hi - lo) / 15.f);
    const float Zm = (float)Zh, Sm = (float)Sh;
    int qm[SUB];
#pragma unroll
    for (int e = 0; e < SUB; ++e) {
      const float q = rtn4_code(mu[e], Zm, Sm);
      qm[e] = (int)q;
      mu[e] = fmaf(Sm, q, Zm);
    }
    if (wave == 0 && tir == 0) {
#pragma unroll
      for (int e = 0; e < SUB; e += 2) mrec[(slot * SUB + e) / 2] = (uint8_t)(qm[e] | (qm[e + 1] << 4));
      if (slot % GL == 0) *reinterpret_cast<uint32_t*>(mrec + 64 + 4 * (slot / GL)) = pack_h2(Sh, Zh);
    }
  } else if (wave == 0 && tir == 0) {
    uint16_t* pm = a.mu[kv] + ((int64_t)unit * (a.cap / R) + dst0 / R + blk) * kDim + slot * SUB;
#pragma unroll
    for (int e = 0; e < SUB; ++e) pm[e] = f2h(mu[e]);
  }

  uint8_t* codes = a.codes[kv];
  uint16_t* scales = a.scales[kv];
  // randomised Hadamard: u = H diag(s) w
  float sgn[SUB];
#pragma unroll
  for (int e = 0; e < SUB; ++e) sgn[e] = a.signs ? (float)a.signs[slot * SUB + e] : 1.f;
  const bool rht = a.signs != nullptr;

  // Shift, second normalisation and Hadamard transform of this lane's
  // sub-vector of token `tok`: n1, n2, and u before its final scale, which
  // is returned (sc u has norm sqrt(d) over the token).
  const float hscale = kInvSqrtD * hsign(slot);
  auto transform_u = [&](int tok, const raw_t& raw, float (&u)[SUB], float& n1, float& n2) -> float {
    if constexpr (DQ) {
      n1 = n1hs[tok];
    } else {  // pass 1's scales, so y is the same value without a second reduction
      n1 = n1p[tok];
    }
    const float inv = DQ ? (n1 > 0.f ? 1.f / n1 : 0.f) : invp[tok];
    // z = x / n1 - mu, one mixed-precision fma per element
    const uint32_t rw[4] = {raw.x, raw.y, SUB == 8 ? raw_hi(raw, 0) : 0u, SUB == 8 ? raw_hi(raw, 1) : 0u};
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < SUB; ++e) {
      u[e] = fmaf(h2f((e & 1) ? (rw[e >> 1] >> 16) : (rw[e >> 1] & 0xffff)), inv, -mu[e]);
      ss = fmaf(u[e], u[e], ss);
    }
    ss = group_sum<S>(ss) * (1.0f / kDim);
    // a token within 2^-12 (relative) of the block mean has no direction left:
    // store n2 = 0 and quantise w = 0 (reconstructed as n1 * mu)
    const float rs2 = __builtin_amdgcn_rsqf(ss);
    const bool live = ss >= kN2Floor * kN2Floor;
    const float inv2 = live ? rs2 : 0.f;
    n2 = ss * inv2;
    if (rht) {
#pragma unroll
      for (int e = 0; e < SUB; ++e) u[e] *= sgn[e];
    }
    // the transform is linear: the 1 / n2 scale goes after it, with 1 / sqrt(d)
    // and the lane's sign
    fwht_lanes<SUB>(u, slot);
    return inv2 * hscale;
  };
  auto transform = [&](int tok, const raw_t& raw, float (&u)[SUB], float& n1, float& n2) {
    const float sc = transform_u(tok, raw, u, n1, n2);
#pragma unroll
    for (int e = 0; e < SUB; ++e) u[e] *= sc;
  };
  // hi/lo fp16 split of u and the squared norm of this lane's sub-vector
  auto split = [&](const float (&u)[SUB], half_t (&hi)[SUB], half_t (&lo)[SUB], half_t& uu_hi, half_t& uu_lo,
                   float& uu) {
    uu = 0.f;
#pragma unroll
    for (int e = 0; e < SUB; ++e) {
      hi[e] = (half_t)u[e];
      lo[e] = (half_t)fmaf((float)hi[e], -1.f, u[e]);  // exact remainder, one mixed fma
      uu = fmaf(u[e], u[e], uu);
    }
    uu_hi = (half_t)uu;
    uu_lo = (half_t)fmaf((float)uu_hi, -1.f, uu);
  };
  // The record of sc u (4 channels): fp16 hi and lo parts, each from one
  // mixed-precision fma (lo = sc u - hi unrounded), and the pair
  // (|sc u|^2 hi, lo).
  auto split_scaled = [&](const float (&u)[SUB], float sc, uint32_t (&w)[4], uint32_t& uup) {
    float uu = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) uu = fmaf(u[e], u[e], uu);
    w[0] = mix_pair(u[0], u[1], sc);
    w[1] = mix_pair(u[2], u[3], sc);
    w[2] = mix_rem_pair(u[0], u[1], sc, w[0]);
    w[3] = mix_rem_pair(u[2], u[3], sc, w[1]);
    const float sc2 = sc * sc;
    uup = mix_rem_lo(uu, sc2, mix_lo(uu, sc2));
  };
  // the scales of token `tok` (slot-0 lane): (n1, n2) fp16, or n2 alone in
  // the double-quantised record
  auto store_scales = [&](int tok, float n1, float n2s) {
    if constexpr (DQ) {
      *reinterpret_cast<half_t*>(srec + 2 * tok) = (half_t)n2s;
    } else {
      *reinterpret_cast<uint32_t*>(scales + (tok_base + tok) * 2) = pack_h2((half_t)n1, (half_t)n2s);
    }
  };

  const uint32_t hbit = (uint32_t)(lane >> 5) << 2;

  if constexpr (NT == 0) {
    // ---- pass 2: per row: shift, second normalisation, Hadamard, VQ -------
#pragma unroll 1
    for (int r = 0; r < ROWS; ++r) {
      const int tok = wave * TPW + r * TPR + tir;
      float u[SUB], n1, n2;
      transform(tok, lds_raw(tok), u, n1, n2);
      half_t hi[SUB], lo[SUB], uu_hi, uu_lo;
      float uu;
      split(u, hi, lo, uu_hi, uu_lo, uu);

      // B operands of the two 32-column blocks (lanes 0-31 / 32-63 own data)
      half8_t B0, B1;
      half4_t Bb0, Bb1;
      if constexpr (SUB == 4) {
        const uint32_t P[4] = {pack_h2(hi[0], hi[1]), pack_h2(hi[2], hi[3]), pack_h2(lo[0], lo[1]),
                               pack_h2(lo[2], lo[3])};
        const uint32_t Q[4] = {pack_h2(uu_hi, uu_lo), pack_h2((half_t)1.f, (half_t)1.f), 0u, 0u};
        uint32_t b0[4], b1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) half_swap(P[i], Q[i], b0[i], b1[i], lane);
        B0 = u32x4_to_half8(b0[0], b0[1], b0[2], b0[3]);
        B1 = u32x4_to_half8(b1[0], b1[1], b1[2], b1[3]);
        Bb0 = Bb1 = half4_t{(half_t)0.f, (half_t)0.f, (half_t)0.f, (half_t)0.f};
      } else {
        const uint32_t P[4] = {pack_h2(hi[0], hi[1]), pack_h2(hi[2], hi[3]), pack_h2(hi[4], hi[5]),
                               pack_h2(hi[6], hi[7])};
        const uint32_t Q[4] = {pack_h2(lo[0], lo[1]), pack_h2(lo[2], lo[3]), pack_h2(lo[4], lo[5]),
                               pack_h2(lo[6], lo[7])};
        uint32_t b0[4], b1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) half_swap(P[i], Q[i], b0[i], b1[i], lane);
        B0 = u32x4_to_half8(b0[0], b0[1], b0[2], b0[3]);
        B1 = u32x4_to_half8(b1[0], b1[1], b1[2], b1[3]);
        const half4_t bias = {uu_hi, uu_lo, (half_t)1.f, (half_t)1.f};
        const half4_t zero4 = {(half_t)0.f, (half_t)0.f, (half_t)0.f, (half_t)0.f};
        Bb0 = lane < 32 ? bias : zero4;
        Bb1 = lane < 32 ? zero4 : bias;
      }

      uint32_t vmask;  // 0xffffff00 in a VGPR (opaque so it is not folded into a literal)
      asm("v_mov_b32 %0, %1" : "=v"(vmask) : "s"(0xffffff00u));
      uint32_t best0 = 0xffffffffu, best1 = 0xffffffffu;
      const float16_t zacc = {};
      // software pipeline: the products of tile t + 1 are issued before the keys
      // of tile t are formed, so the matrix core runs under the argmin
      auto tile = [&](int t, float16_t& acc0, float16_t& acc1) {
        const half8_t A1t = sA1[t][lane];
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A1t, B0, zacc, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A1t, B1, zacc, 0, 0, 0);
        if constexpr (SUB == 8) {
          const half4_t A2t = sA2[t][lane];
          acc0 = __builtin_amdgcn_mfma_f32_32x32x8f16(A2t, Bb0, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x8f16(A2t, Bb1, acc1, 0, 0, 0);
        }
      };
      // (at 1 bit the extra bias products would push the kernel past 168 VGPRs;
      // it keeps one tile in flight)
      constexpr bool kPipe = SUB == 4;
      float16_t cur0, cur1, nxt0, nxt1;
      if (kPipe) tile(0, cur0, cur1);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (!kPipe) tile(t, cur0, cur1);
        if (kPipe && t + 1 < 8) tile(t + 1, nxt0, nxt1);
#pragma unroll
        for (int q = 0; q < 16; q += 2) {
          // accumulator q holds codeword 32t + 8(q/4) + 4(lane/32) + q%4
          const uint32_t i0 = 32u * t + 8u * (q >> 2) + (q & 3);
          const uint32_t i1 = 32u * t + 8u * ((q + 1) >> 2) + ((q + 1) & 3);
          best0 = min(min(best0, make_key(cur0[q], vmask, i0)), make_key(cur0[q + 1], vmask, i1));
          best1 = min(min(best1, make_key(cur1[q], vmask, i0)), make_key(cur1[q + 1], vmask, i1));
        }
        if (kPipe && t + 1 < 8) {
          cur0 = nxt0;
          cur1 = nxt1;
        }
      }
      best0 |= hbit;
      best1 |= hbit;
      // column n of block 0 belongs to lane n, of block 1 to lane 32 + n: one
      // swap brings each column's other half next to it
      uint32_t klo, khi;
      half_swap(best0, best1, klo, khi, lane);  // klo = [b0 low, b1 low], khi = [b0 high, b1 high]
      const uint32_t mine = min(klo, khi);
      const uint32_t code = mine & 0xffu;
      codes[(tok_base + tok) * S + oslot] = (uint8_t)code;
      // Strategy-3 scale: alpha = |u|^2 / (u . c_hat), folded into n2
      float n2s = n2;
      if (a.scale_adjust) {
        // the codeword from the MFMA operand tiles: lanes < 32 of tile code/32
        // hold -2 c (exact in fp16)
        const half8_t cw = sA1[code >> 5][code & 31];
        float uc = 0.f;
#pragma unroll
        for (int e = 0; e < SUB; ++e) uc = fmaf(u[e], -0.5f * (float)cw[e], uc);
        uc = group_sum<S>(uc);
        const float utot = group_sum<S>(uu);
        if (uc > 0.f) n2s = n2 * (utot / uc);
      }
      if (slot == 0) store_scales(tok, n1, n2s);
    }
  } else {
    // ---- pass 2 with candidate lists (2 bits) -----------------------------
    static_assert(NW == 16, "wave w pads box w below: 16 waves for 16 boxes");
    // (a) per row: transform, hi/lo split, orthant box; the rank of the
    // sub-vector among its wave's sub-vectors of the same box
    uint32_t boxr[ROWS], rankr[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const int tok = wave * TPW + r * TPR + tir;
      float u[SUB], n1, n2;
      const float sc = transform_u(tok, xr[r], u, n1, n2);
      uint32_t w[4], uup;
      split_scaled(u, sc, w, uup);
      const int i = tok * S + oslot;
      recs[i] = u32x4_to_half8(w[0], w[1], w[2], w[3]);
      uus[i] = uup;
      // orthant box from the signs of the fp16 high parts (a zero part lies
      // on the boundary of both boxes, whose lists both hold its nearest)
      boxr[r] = ((w[0] >> 15) & 1u) | ((w[0] >> 30) & 2u) | ((w[1] >> 13) & 4u) | ((w[1] >> 28) & 8u);
      rankr[r] = atomicAdd(&whist[wave][boxr[r]], 1u);
      if (slot == 0) {
        if (a.scale_adjust) {
          n1t[tok] = n1;
          n2t[tok] = n2;
        } else {
          store_scales(tok, n1, n2);
        }
      }
    }
    __syncthreads();
    // (b) box offsets, computed by every wave for itself (no barrier): lane
    // `box` (< 16) sums the waves' counts of its box; each box's columns are
    // padded to a multiple of 32 (with the zero record).
    const int nblocks = [&] {
      const int box = lane & 15;
      uint32_t cnt = 0, mine = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const uint32_t c = whist[w][box];
        mine = (w == wave) ? cnt : mine;  // columns of the waves before this one
        cnt += c;
      }
      const uint32_t padded = (cnt + 31u) & ~31u;
      // inclusive prefix over the 16 boxes of each DPP row: row_shr adds,
      // lanes shifted in from outside the row read 0
      uint32_t incl = padded;
      incl += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x111, 0xF, 0xF, false);
      incl += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x112, 0xF, 0xF, false);
      incl += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x114, 0xF, 0xF, false);
      incl += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x118, 0xF, 0xF, false);
      const uint32_t st = incl - padded;
      // (c) box order: every sub-vector of this wave to its column
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const int tok = wave * TPW + r * TPR + tir;
        const uint32_t first = __shfl(st + mine, (int)boxr[r], kWave);
        sidx[first + rankr[r]] = (uint16_t)(tok * S + oslot);
      }
      // wave w pads box w with the zero record and labels its column blocks
      const uint32_t wst = __builtin_amdgcn_readlane(st, wave), wcnt = __builtin_amdgcn_readlane(cnt, wave);
      const uint32_t wpad = __builtin_amdgcn_readlane(padded, wave);
      if ((uint32_t)lane < wpad - wcnt) sidx[wst + wcnt + lane] = (uint16_t)kDummy;
      for (uint32_t q = lane; q < wpad / 32; q += kWave) cbox[wst / 32 + q] = (uint8_t)wave;  // up to R S / 32 blocks
      return (int)(__builtin_amdgcn_readlane(incl, 15) / 32);
    }();
    __syncthreads();
    if (next < items) load_rows(next, xn);
    // (d) distance products over the box's list, 32 sorted columns per MFMA;
    // lane n (< 32) holds column n's u parts, lane 32 + n its bias row; tile t
    // of a box holds its list entries 32 t .. 32 t + 31.  Each wave takes an
    // even share of the column blocks, two per step.
    const int n = lane & 31;
    const bool upper = lane >= 32;
    // B operand of sorted column `col` (both loads on every lane, then a select).
    // The bias row's K slots 12-15 meet zeros in every candidate tile, so the
    // upper lanes leave the record's (finite) low parts there.
    auto operand_b = [&](int col, int& idx) -> half8_t {
      idx = sidx[col];
      const uint4_t rv = __builtin_bit_cast(uint4_t, recs[idx]);
      const uint32_t q = uus[idx];
      const uint4_t w = {upper ? q : rv[0], upper ? 0x3C003C00u : rv[1], rv[2], rv[3]};
      return __builtin_bit_cast(half8_t, w);
    };
    auto search = [&](auto two, int c0) {
      constexpr bool TWO = decltype(two)::value;
      const int c1 = TWO ? c0 + NW : c0;
      const int o0 = cbox[c0], o1 = cbox[c1];
      int i0, i1 = 0;
      const half8_t B0 = operand_b(32 * c0 + n, i0);
      half8_t B1 = B0;
      if constexpr (TWO) B1 = operand_b(32 * c1 + n, i1);
      uint32_t vmask;  // 0xffffff00 in a VGPR (opaque so it is not folded into a literal)
      asm("v_mov_b32 %0, %1" : "=v"(vmask) : "s"(0xffffff00u));
      const float16_t zacc = {};
      uint32_t best0 = 0xffffffffu, best1 = 0xffffffffu;
      // where the registers allow (128 per lane for 4 waves per SIMD), the
      // next tile's candidate operands are read while this tile's distances
      // are reduced
      constexpr bool kPrefetchA = !DQ && (HALF || NT == 2);
      half8_t a0 = sA1[o0 * NT][lane], a1 = a0;
      if constexpr (TWO) a1 = sA1[o1 * NT][lane];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (!kPrefetchA && t > 0) {
          a0 = sA1[o0 * NT + t][lane];
          if constexpr (TWO) a1 = sA1[o1 * NT + t][lane];
        }
        float16_t cur0, cur1;
        cur0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, B0, zacc, 0, 0, 0);
        if constexpr (TWO) cur1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, B1, zacc, 0, 0, 0);
        if constexpr (kPrefetchA) {
          if (t + 1 < NT) {
            a0 = sA1[o0 * NT + t + 1][lane];
            if constexpr (TWO) a1 = sA1[o1 * NT + t + 1][lane];
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int q = 0; q < 16; q += 2) {
          // accumulator q holds list position 32t + 8(q/4) + 4(lane/32) + q%4:
          // rows 0-15 of the tile for q < 8
          if (HALF && t == NT - 1 && q >= 8) continue;
          const uint32_t p0 = 32u * t + 8u * (q >> 2) + (q & 3);
          const uint32_t p1 = 32u * t + 8u * ((q + 1) >> 2) + ((q + 1) & 3);
          best0 = min(min(best0, make_key(cur0[q], vmask, p0)), make_key(cur0[q + 1], vmask, p1));
          if constexpr (TWO)
            best1 = min(min(best1, make_key(cur1[q], vmask, p0)), make_key(cur1[q + 1], vmask, p1));
        }
      }
      best0 |= hbit;
      uint32_t mine;
      if constexpr (TWO) {
        best1 |= hbit;
        uint32_t klo, khi;
        half_swap(best0, best1, klo, khi, lane);  // lane n: block c0 column n; lane 32 + n: block c1 column n
        mine = min(klo, khi);
      } else {
        mine = min(best0, (uint32_t)__builtin_bit_cast(uint32_t, xlane<32>(__builtin_bit_cast(float, best0))));
      }
      const uint32_t pos = mine & 0xffu;
      const int idx = upper ? i1 : i0;
      // lists are ascending, so the lowest position of a tie is the lowest index
      if (idx != kDummy && (TWO || !upper)) boxc[idx] = lst[(upper ? o1 : o0) * 128 + pos];
    };
    // wave w takes blocks w, w + NW, w + 2 NW, ... two at a time
    for (int c0 = wave; c0 < nblocks; c0 += 2 * NW) {
      if (c0 + NW < nblocks) search(std::true_type{}, c0);
      else search(std::false_type{}, c0);
    }
    __syncthreads();
    // (e) codes (the block's R x S bytes are contiguous) and Strategy-3 scales
    for (int i = tid; i < NSV / 16; i += blockDim.x)
      reinterpret_cast<uint4*>(codes + tok_base * S)[i] = reinterpret_cast<const uint4*>(boxc)[i];
    if (a.scale_adjust) {
      for (int i = tid; i < NSV; i += blockDim.x) {  // a wave covers two whole tokens
        const int tok = i / S;
        const half8_t r8 = recs[i];
        const int code = boxc[i];
        const uint2 cw = *reinterpret_cast<const uint2*>(a.codebook + code * SUB);
        const float c[4] = {h2f(cw.x & 0xffff), h2f(cw.x >> 16), h2f(cw.y & 0xffff), h2f(cw.y >> 16)};
        float uc = 0.f;
#pragma unroll
        for (int e = 0; e < SUB; ++e) uc = fmaf((float)r8[e] + (float)r8[4 + e], c[e], uc);
        uc = group_sum<S>(uc);
        const uint32_t q = uus[i];
        const float utot = group_sum<S>(h2f(q & 0xffff) + h2f(q >> 16));
        if ((i % S) == 0) {
          float n2s = n2t[tok];
          if (uc > 0.f) n2s *= utot / uc;
          store_scales(tok, n1t[tok], n2s);
        }
      }
    }
    __syncthreads();  // the next block reuses the LDS records
  }
  return next < items;
  };

  if constexpr (NT == 0) {
    encode_block(blockIdx.x % a.nblk, blockIdx.x / a.nblk, items);
  } else {
    // persistent: work-group g encodes items g, g + n_enc, ...
    if ((int)blockIdx.x < items) load_rows(blockIdx.x, xr);
    for (int item = blockIdx.x; item < items; item += n_enc) {
      const int next = item + n_enc;
      const bool pre = encode_block(item % a.nblk, item / a.nblk, next);
      if (next < items) {
        if (pre) {
#pragma unroll
          for (int r = 0; r < (NT ? ROWS : 1); ++r) xr[r] = xn[r];
        } else {
          load_rows(next, xr);
        }
      }
    }
  }
}

// Append one token per row into the residual window (after any flush of the
// same step has run).  One group per row: every head's K and V row, then the
// row's counters.  Without a token (k_new null, ragged only) it just moves the
// counters of the rows that a flush has encoded.
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int b = blockIdx.x;
  int pos = a.pos;
  bool flushed = false;
  if (a.seq_resid) {
    pos = a.seq_resid[b];
    if (pos < 0 || pos > a.R) return;  // not a valid window position: the row is left as it is
    if (pos == a.R) {
      const int nq = a.seq_quant[b];
      if (nq < 0 || nq % a.R != 0 || nq + a.R > a.cap) return;  // no room: the row is left as it is
      flushed = true;
      pos = 0;
    }
  }
  if (!a.k_new) {
    if (a.seq_resid && flushed) {
      __syncthreads();
      if (threadIdx.x == 0) {
        a.seq_quant[b] += a.R;
        a.seq_resid[b] = 0;
      }
    }
    return;
  }
  for (int i = threadIdx.x; i < 2 * a.H * 16; i += blockDim.x) {  // 16 x 8 halves per row
    const int kv = i / (a.H * 16), h = (i / 16) % a.H, c = (i % 16) * 8;
    const int64_t unit = (int64_t)b * a.H + h;
    const uint16_t* src = (kv ? a.v_new : a.k_new) + unit * kDim + c;
    uint16_t* dst = (kv ? a.vresid : a.kresid) + (unit * a.R + pos) * kDim + c;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }
  if (a.seq_resid) {
    __syncthreads();
    if (threadIdx.x == 0) {
      if (flushed) a.seq_quant[b] += a.R;
      a.seq_resid[b] = pos + 1;
    }
  }
}

hipError_t launch_append(const AppendArgs& a, int B, hipStream_t stream) {
  hipLaunchKernelGGL(append_kernel, dim3(B), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// The list kernel searching `span` entries per list (16, 32, ... 96), or the
// exhaustive kernel.
template <int SUB, int R, bool DQ>
static hipError_t launch_encode_nt(const EncodeArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 b0(64 * enc_waves<0>()), b1(64 * enc_waves<1>());
  if constexpr (SUB == 4) {
    if (a.span > 0 && a.span <= 64) {
      hipLaunchKernelGGL((encode_kernel<4, R, DQ, 2, false>), grid, b1, 0, stream, a);
      return hipSuccess;
    }
    if (a.span > 64 && a.span <= 80) {
      hipLaunchKernelGGL((encode_kernel<4, R, DQ, 3, true>), grid, b1, 0, stream, a);
      return hipSuccess;
    }
    if (a.span > 80 && a.span <= 96) {
      hipLaunchKernelGGL((encode_kernel<4, R, DQ, 3, false>), grid, b1, 0, stream, a);
      return hipSuccess;
    }
  }
  // no table, or lists longer than 96 entries (their box tiles would not fit in LDS)
  hipLaunchKernelGGL((encode_kernel<SUB, R, DQ, 0, false>), grid, b0, 0, stream, a);
  return hipSuccess;
}

hipError_t launch_encode(const EncodeArgs& args, int sub, int R, hipStream_t stream) {
  EncodeArgs a = args;
  const bool rcopy = a.rc_r > 0 || a.lens != nullptr;
  const int items = a.nblk * a.n_units;
  int n_enc = items;
  if (sub == 4 && a.span > 0 && a.span <= 96) {
    // candidate lists: one persistent group per CU and K/V half
    int dev = 0, ncu = 0;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
      ncu = 256;
    n_enc = std::min(items, std::max(1, ncu / 2));
  }
  a.n_enc = n_enc;
  const dim3 grid(n_enc + (rcopy ? a.n_units : 0), 2);
  if (grid.x == 0) return hipSuccess;
  hipError_t e = hipErrorInvalidValue;
  if (a.dq) {
    if (sub == 4 && R == 128) e = launch_encode_nt<4, 128, true>(a, grid, stream);
    else if (sub == 4 && R == 64) e = launch_encode_nt<4, 64, true>(a, grid, stream);
    else if (sub == 8 && R == 128) e = launch_encode_nt<8, 128, true>(a, grid, stream);
    else if (sub == 8 && R == 64) e = launch_encode_nt<8, 64, true>(a, grid, stream);
  } else {
    if (sub == 4 && R == 128) e = launch_encode_nt<4, 128, false>(a, grid, stream);
    else if (sub == 4 && R == 64) e = launch_encode_nt<4, 64, false>(a, grid, stream);
    else if (sub == 8 && R == 128) e = launch_encode_nt<8, 128, false>(a, grid, stream);
    else if (sub == 8 && R == 64) e = launch_encode_nt<8, 64, false>(a, grid, stream);
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}


}  // namespace nsnq
