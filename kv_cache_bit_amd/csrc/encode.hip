// encode.hip -- fused NSN + Hadamard + VQ encode of R-token blocks (gfx950).
//
// One work-group (4 waves) encodes one block of R tokens of one (batch row,
// head) stream, K or V.  Each lane holds one sub-vector (s = SUB elements) of
// one token, so a token occupies S = 128/SUB consecutive lanes and a wave "row"
// covers 64/S tokens.
//
//  1. token-wise normalisation to norm sqrt(d) (n1), kept in registers;
//  2. channel mean over the block (wave partial sums, LDS across waves);
//  3. second normalisation (n2), w = z / n2;
//  4. Walsh-Hadamard transform across the S lanes of a token, scaled by
//     1/sqrt(d);
//  5. VQ: squared distances to all 256 codewords as an MFMA GEMM, then a
//     per-lane argmin on packed (distance | index) keys.
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

// Waves per encode work-group: 8 x 64 lanes share one block's LDS staging,
// which lets 4 waves per SIMD stay resident (the 48 KB of LDS per group would
// otherwise cap a 4-wave group at 3).
constexpr int kEncWaves = 8;

template <int SUB, int R, bool DQ>
__global__ __launch_bounds__(64 * kEncWaves) void encode_kernel(EncodeArgs a) {
  if ((int)blockIdx.x >= a.nblk * a.n_units) {
    resid_copy(a, blockIdx.x - a.nblk * a.n_units, blockIdx.y);
    return;
  }
  constexpr int S = kDim / SUB;      // slots = lanes per token
  constexpr int TPR = kWave / S;     // tokens per wave row
  constexpr int TPW = R / kEncWaves;  // tokens per wave
  constexpr int ROWS = TPW / TPR;    // rows per wave
  static_assert(ROWS * TPR * kEncWaves == R, "block split");

  __shared__ float red[kEncWaves][kDim];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slot = lane % S;
  const int tir = lane / S;

  const int blk = blockIdx.x % a.nblk;
  const int unit = blockIdx.x / a.nblk;  // b * H + h
  const int kv = blockIdx.y;
  const int b = unit / a.H, h = unit % a.H;
  int dst0 = a.dst_tok0;  // first destination token of this launch's blocks
  if (a.lens) {           // ragged prefill: this row encodes L - r tokens
    const int L = min(max(a.lens[b], 0), a.lens_max);
    if (blk * R >= L - resid_of(L, R)) return;
  } else if (a.fl_resid) {  // ragged flush: only full windows, each at its row's n_quant
    dst0 = a.fl_quant[b];
    if (a.fl_resid[b] != R || dst0 < 0 || dst0 % R != 0 || dst0 + R > a.cap) return;
  }

  const uint16_t* src = a.src[kv] + (int64_t)b * a.sb + (int64_t)h * a.sh + (int64_t)blk * R * a.st;
  const int64_t tok_base = (int64_t)unit * a.cap + dst0 + (int64_t)blk * R;

  // ---- codebook operands (A side), per 32-codeword tile -------------------
  // Built once per group into LDS (lane l of tile t holds codeword
  // 32 t + (l % 32)) and re-read per row, which keeps ~40 VGPRs free.
  __shared__ half8_t sA1[8][kWave];
  __shared__ half4_t sA2[8][kWave];
  for (int i = threadIdx.x; i < 8 * kWave; i += blockDim.x) {
    const int t = i / kWave, l = i % kWave;
    const int k = 32 * t + (l & 31);
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
    half4_t a2 = {(half_t)0.f, (half_t)0.f, (half_t)0.f, (half_t)0.f};
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
      a2 = half4_t{(half_t)1.f, (half_t)1.f, b_hi, b_lo};
    }
    sA1[t][l] = av;
    sA2[t][l] = a2;
  }
  // (visible after the first __syncthreads below)

  // One row = this lane's sub-vector of token `tok`: raw fp16 load, then
  // y = x / n1 with n1 = ||x|| / sqrt(d).  Pass 1 reads the block from HBM
  // once and keeps the raw fp16 rows in LDS; pass 2 recomputes y from there
  // instead of keeping R x 128 floats in registers.
  using raw_t = typename std::conditional<SUB == 4, uint2, uint4>::type;
  __shared__ raw_t xs[R * S];  // [token][slot], R x 256 bytes
  auto load_raw = [&](int tok) -> raw_t {
    const raw_t v = *reinterpret_cast<const raw_t*>(src + (int64_t)tok * a.st + slot * SUB);
    xs[tok * S + slot] = v;
    return v;
  };
  auto lds_raw = [&](int tok) -> raw_t { return xs[tok * S + slot]; };
  auto norm_raw = [&](const raw_t& raw, float (&y)[SUB], float& n1) {
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
    const float inv = ss > 0.f ? rs : 0.f;
    n1 = ss * inv;
#pragma unroll
    for (int e = 0; e < SUB; ++e) y[e] = v[e] * inv;
  };

  // ---- pass 1: channel sums of y over the block ---------------------------
  // Double-quantised format: s1 is first coded in 4 bits over the block and
  // tokens are divided by the stored value n1_hat (so the reconstruction from
  // stored values only carries the VQ error).
  constexpr int SR = dq_scales_bytes<R>();
  __shared__ float n1s[DQ ? R : 1];   // s1 per token
  __shared__ float n1hs[DQ ? R : 1];  // n1_hat per token
  uint8_t* srec = reinterpret_cast<uint8_t*>(a.scales[kv]) + ((int64_t)unit * (a.cap / R) + dst0 / R + blk) * SR;
  uint8_t* mrec = reinterpret_cast<uint8_t*>(a.mu[kv]) + ((int64_t)unit * (a.cap / R) + dst0 / R + blk) * kDqMuBytes;
  float csum[SUB];
#pragma unroll
  for (int e = 0; e < SUB; ++e) csum[e] = 0.f;
  if constexpr (DQ) {
#pragma unroll 4
    for (int r = 0; r < ROWS; ++r) {
      const int tok = wave * TPW + r * TPR + tir;
      float y[SUB], n1;
      norm_raw(load_raw(tok), y, n1);
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
      const raw_t raw = lds_raw(tok);
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
      float y[SUB], n1;
      norm_raw(load_raw(wave * TPW + r * TPR + tir), y, n1);
#pragma unroll
      for (int e = 0; e < SUB; ++e) csum[e] += y[e];
    }
  }
  // combine the TPR lanes holding the same channels, then the 4 waves
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
  float mu[SUB];
#pragma unroll
  for (int e = 0; e < SUB; ++e) {
    const int c = slot * SUB + e;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kEncWaves; ++w) sum += red[w][c];
    mu[e] = sum * (1.0f / R);
  }
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

  // ---- pass 2: per row: shift, second normalisation, Hadamard, VQ ---------
#pragma unroll 1
  for (int r = 0; r < ROWS; ++r) {
    const int tok = wave * TPW + r * TPR + tir;
    float u[SUB], n1;
    if constexpr (DQ) {
      n1 = n1hs[tok];
      const float inv = n1 > 0.f ? 1.f / n1 : 0.f;
      const raw_t raw = lds_raw(tok);
      u[0] = h2f(raw.x & 0xffff) * inv; u[1] = h2f(raw.x >> 16) * inv;
      u[2] = h2f(raw.y & 0xffff) * inv; u[3] = h2f(raw.y >> 16) * inv;
      if constexpr (SUB == 8) {
        u[4] = h2f(raw.z & 0xffff) * inv; u[5] = h2f(raw.z >> 16) * inv;
        u[6] = h2f(raw.w & 0xffff) * inv; u[7] = h2f(raw.w >> 16) * inv;
      }
    } else {
      norm_raw(lds_raw(tok), u, n1);
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < SUB; ++e) {
      u[e] -= mu[e];
      ss = fmaf(u[e], u[e], ss);
    }
    ss = group_sum<S>(ss) * (1.0f / kDim);
    // a token within 2^-12 (relative) of the block mean has no direction left:
    // store n2 = 0 and quantise w = 0 (reconstructed as n1 * mu)
    const float rs2 = __builtin_amdgcn_rsqf(ss);
    const bool live = ss >= kN2Floor * kN2Floor;
    const float inv2 = live ? rs2 : 0.f;
    const float n2 = ss * inv2;
#pragma unroll
    for (int e = 0; e < SUB; ++e) u[e] *= inv2 * sgn[e];
    fwht128<SUB>(u, lane);
#pragma unroll
    for (int e = 0; e < SUB; ++e) u[e] *= kInvSqrtD;

    // hi/lo split and squared norm of this lane's sub-vector
    half_t hi[SUB], lo[SUB];
    float uu = 0.f;
#pragma unroll
    for (int e = 0; e < SUB; ++e) {
      hi[e] = (half_t)u[e];
      lo[e] = (half_t)(u[e] - (float)hi[e]);
      uu = fmaf(u[e], u[e], uu);
    }
    const half_t uu_hi = (half_t)uu;
    const half_t uu_lo = (half_t)(uu - (float)uu_hi);

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
    const uint32_t hbit = (uint32_t)(lane >> 5) << 2;
    best0 |= hbit;
    best1 |= hbit;
    // column n of block 0 belongs to lane n, of block 1 to lane 32 + n: one
    // swap brings each column's other half next to it
    uint32_t klo, khi;
    half_swap(best0, best1, klo, khi, lane);  // klo = [b0 low, b1 low], khi = [b0 high, b1 high]
    const uint32_t mine = min(klo, khi);
    const uint32_t code = mine & 0xffu;
    codes[(tok_base + tok) * S + slot] = (uint8_t)code;
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
    if (slot == 0) {
      if constexpr (DQ) {
        *reinterpret_cast<half_t*>(srec + 2 * tok) = (half_t)n2s;
      } else {
        const uint32_t pk = pack_h2((half_t)n1, (half_t)n2s);
        *reinterpret_cast<uint32_t*>(scales + (tok_base + tok) * 2) = pk;
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

hipError_t launch_encode(const EncodeArgs& a, int sub, int R, hipStream_t stream) {
  const bool rcopy = a.rc_r > 0 || a.lens != nullptr;
  dim3 grid(a.nblk * a.n_units + (rcopy ? a.n_units : 0), 2), block(64 * kEncWaves);
  if (grid.x == 0) return hipSuccess;
  if (a.dq) {
    if (sub == 4 && R == 128) hipLaunchKernelGGL((encode_kernel<4, 128, true>), grid, block, 0, stream, a);
    else if (sub == 4 && R == 64) hipLaunchKernelGGL((encode_kernel<4, 64, true>), grid, block, 0, stream, a);
    else if (sub == 8 && R == 128) hipLaunchKernelGGL((encode_kernel<8, 128, true>), grid, block, 0, stream, a);
    else if (sub == 8 && R == 64) hipLaunchKernelGGL((encode_kernel<8, 64, true>), grid, block, 0, stream, a);
    else return hipErrorInvalidValue;
  } else {
    if (sub == 4 && R == 128) hipLaunchKernelGGL((encode_kernel<4, 128, false>), grid, block, 0, stream, a);
    else if (sub == 4 && R == 64) hipLaunchKernelGGL((encode_kernel<4, 64, false>), grid, block, 0, stream, a);
    else if (sub == 8 && R == 128) hipLaunchKernelGGL((encode_kernel<8, 128, false>), grid, block, 0, stream, a);
    else if (sub == 8 && R == 64) hipLaunchKernelGGL((encode_kernel<8, 64, false>), grid, block, 0, stream, a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}


}  // namespace nsnq
