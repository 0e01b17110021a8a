/*
 * nsnq_oracle.c -- plain, slow CPU reference of the NSNQuant hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, calls or
 * includes this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header, table or helper with the
 * GPU path: fp16 conversion, the Hadamard matrix, layouts and argmin are all
 * written out again here.
 *
 * Everything is computed in double precision with straightforward loops.  The
 * stored format (fp16 scalars, uint8 codes) is rounded with this file's own
 * round-to-nearest-even conversion.
 *
 * Sources (page title, then the section it falls in):
 *   [P2] "NSNQuant: A Double Normalization Approach for Calibration-Free Low-Bit
 *        Vector Quantization of KV Cache", research-map summary, "Approach".
 *   [P3] same title, technical summary ("Technische Samenvatting"), sections
 *        1 (NSN), 2 (Hadamard), 3 (VQ and codebook), 4 (implementation:
 *        residuals, attention).
 *   [P4] same title, machine review: "What carries the argument", referee
 *        minor comment 1 (paper Section 2, Eq. (1)), Lemma 1 (App. A.1).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- fp16 --- */

/* IEEE binary16 -> double, exact. */
double orc_h2d(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    v = ldexp((double)(m + 1024), e - 25); /* (1.m) * 2^(e-15) */
  }
  return sign ? -v : v;
}

/* double -> IEEE binary16, round to nearest, ties to even.  Works by scanning
 * the representable magnitudes: finds the two fp16 neighbours of |x| and picks
 * the nearer one (the even one on a tie).  Slow but plainly correct. */
uint16_t orc_d2h(double x) {
  if (isnan(x)) return 0x7e00;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  /* largest finite fp16 is 65504; values at or above 65520 round to inf */
  if (a >= 65520.0) return sign | 0x7c00;
  /* binary search over the 0x7c00 finite non-negative codes (monotone) */
  int lo = 0, hi = 0x7bff;
  if (a >= orc_h2d((uint16_t)hi)) return sign | (uint16_t)hi;
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (orc_h2d((uint16_t)mid) <= a) lo = mid; else hi = mid;
  }
  double dlo = a - orc_h2d((uint16_t)lo);
  double dhi = orc_h2d((uint16_t)hi) - a;
  int pick;
  if (dlo < dhi) pick = lo;
  else if (dhi < dlo) pick = hi;
  else pick = (lo % 2 == 0) ? lo : hi;
  return sign | (uint16_t)pick;
}

void orc_d2h_array(const double* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_d2h(x[i]);
}

void orc_h2d_array(const uint16_t* h, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_h2d(h[i]);
}

/* ------------------------------------------------------------ Hadamard --- */

static int popcount_int(int v) {
  int c = 0;
  while (v) { c += v & 1; v >>= 1; }
  return c;
}

/* The orthonormal Sylvester-ordered Hadamard matrix of size d (a power of 2):
 * H[i][j] = (-1)^popcount(i & j) / sqrt(d), written into Hm [d][d].
 * [P3 sec. 2; P4 "What carries the argument"]: after NSN the head vector is
 * rotated by a fixed (non-randomised) Hadamard transform.  H is symmetric and
 * its own inverse. */
void orc_hadamard_matrix(int d, double* Hm) {
  double scale = 1.0 / sqrt((double)d);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j)
      Hm[(size_t)i * d + j] = ((popcount_int(i & j) & 1) ? -1.0 : 1.0) * scale;
}

/* u = Hm w, plain matrix-vector product. */
static void matvec(const double* Hm, const double* w, double* u, int d) {
  for (int i = 0; i < d; ++i) {
    double acc = 0.0;
    for (int j = 0; j < d; ++j) acc += Hm[(size_t)i * d + j] * w[j];
    u[i] = acc;
  }
}

/* u = H w for one vector (builds H each call; for tests). */
void orc_hadamard(const double* w, double* u, int d) {
  double* Hm = (double*)malloc(sizeof(double) * (size_t)d * d);
  orc_hadamard_matrix(d, Hm);
  matvec(Hm, w, u, d);
  free(Hm);
}

/* ----------------------------------------------------------------- NSN --- */

/* Normalize-Shift-Normalize of one block of R tokens, x fp16 [R][d].
 * [P3 sec. 1; P4 "What carries the argument"; P2 "Approach"]:
 *   1. each token is rescaled to Euclidean norm sqrt(d); the factor is kept
 *      as n1 = ||x|| / sqrt(d) so that x = n1 * y;
 *   2. the channel-wise mean mu of the block is subtracted, z = y - mu;
 *   3. each token is rescaled to norm sqrt(d) again, n2 = ||z|| / sqrt(d),
 *      w = z / n2.
 * A zero token (n1 = 0) gives y = 0.  A token equal to the block mean has
 * z = 0 up to rounding noise; when n2 < 2^-12 the direction of z carries no
 * information (it is rounding noise in any finite precision), so n2 and w are
 * set to 0 and the token is reconstructed as N1 * MU, within 2^-12 of its norm.
 * The pages do not cover these cases; this is the reading under which the
 * stored values are the same at any working precision.
 * Any output pointer may be NULL. */
#define NSN_N2_FLOOR (1.0 / 4096.0)
void orc_nsn_block(const uint16_t* x, int R, int d,
                   double* n1_out, double* y_out, double* mu_out,
                   double* z_out, double* n2_out, double* w_out) {
  double* y = (double*)malloc(sizeof(double) * (size_t)R * d);
  double* mu = (double*)calloc((size_t)d, sizeof(double));
  double sqrt_d = sqrt((double)d);
  for (int t = 0; t < R; ++t) {
    double ss = 0.0;
    for (int c = 0; c < d; ++c) {
      double v = orc_h2d(x[(size_t)t * d + c]);
      ss += v * v;
    }
    double n1 = sqrt(ss) / sqrt_d;
    if (n1_out) n1_out[t] = n1;
    for (int c = 0; c < d; ++c) {
      double v = orc_h2d(x[(size_t)t * d + c]);
      y[(size_t)t * d + c] = (n1 > 0.0) ? v / n1 : 0.0;
    }
  }
  for (int c = 0; c < d; ++c) {
    double s = 0.0;
    for (int t = 0; t < R; ++t) s += y[(size_t)t * d + c];
    mu[c] = s / (double)R;
  }
  if (mu_out) memcpy(mu_out, mu, sizeof(double) * d);
  for (int t = 0; t < R; ++t) {
    double ss = 0.0;
    for (int c = 0; c < d; ++c) {
      double zc = y[(size_t)t * d + c] - mu[c];
      if (z_out) z_out[(size_t)t * d + c] = zc;
      ss += zc * zc;
    }
    double n2 = sqrt(ss) / sqrt_d;
    if (n2 < NSN_N2_FLOOR) n2 = 0.0;
    if (n2_out) n2_out[t] = n2;
    if (w_out) {
      for (int c = 0; c < d; ++c) {
        double zc = y[(size_t)t * d + c] - mu[c];
        w_out[(size_t)t * d + c] = (n2 > 0.0) ? zc / n2 : 0.0;
      }
    }
    if (y_out) memcpy(y_out + (size_t)t * d, y + (size_t)t * d, sizeof(double) * d);
  }
  free(y);
  free(mu);
}

/* ------------------------------------------------------------------ VQ --- */

/* Eq. (1) of the paper as given in [P4 referee minor comment 1] and [P3 sec. 3]:
 * the code of a sub-vector v (length s) is the index of the nearest codeword,
 * with D the squared Euclidean distance; equal distances go to the lowest
 * index.  Also returns the smallest distance and the relative gap between the
 * best and second-best distance, (D2 - D1) / D1 (+inf when D1 = 0 < D2). */
static int vq_dbl(const double* v, int s, const double* cbd, int ncw, double* dmin_out, double* gap_out) {
  int best = 0;
  double d1 = INFINITY, d2 = INFINITY;
  for (int k = 0; k < ncw; ++k) {
    double dist = 0.0;
    for (int i = 0; i < s; ++i) {
      double diff = v[i] - cbd[(size_t)k * s + i];
      dist += diff * diff;
    }
    if (dist < d1) {
      d2 = d1;
      d1 = dist;
      best = k;
    } else if (dist < d2) {
      d2 = dist;
    }
  }
  if (dmin_out) *dmin_out = d1;
  if (gap_out) {
    if (d1 > 0.0) *gap_out = (d2 - d1) / d1;
    else *gap_out = (d2 > 0.0) ? INFINITY : 0.0;
  }
  return best;
}

/* Same, with the fp16 codebook cb [ncw][s] taken exactly. */
int orc_vq(const double* v, int s, const uint16_t* cb, int ncw, double* dmin_out, double* gap_out) {
  double* cbd = (double*)malloc(sizeof(double) * (size_t)ncw * s);
  for (size_t e = 0; e < (size_t)ncw * s; ++e) cbd[e] = orc_h2d(cb[e]);
  int code = vq_dbl(v, s, cbd, ncw, dmin_out, gap_out);
  free(cbd);
  return code;
}

/* -------------------------------------------------------------- encode --- */

/* Number of tokens that stay in the fp16 residual window after a prefill of L
 * tokens with window R: r = ((L - 1) mod R) + 1 (0 when L = 0).  [P3 sec. 4,
 * residuals]: recent tokens are kept at full precision and the window is
 * quantised and appended only once it is full and another token arrives, so a
 * prefill leaves between 1 and R tokens in it. */
int orc_resid_count(int L, int R) {
  if (L <= 0) return 0;
  return ((L - 1) % R) + 1;
}

/* Encode one (batch row, head) stream, K or V, of L tokens x fp16 [L][d].
 * Outputs, for the nq = L - r flushed tokens, in blocks of R:
 *   codes  [nq][d/s]  uint8, slot j covers u[j*s .. j*s+s-1]
 *   scales [nq][2]    fp16 (n1, n2)
 *   mu     [nq/R][d]  fp16 channel mean of each block (original domain)
 *   gap    [nq][d/s]  relative best/second gap (may be NULL)
 *   u_out  [nq][d]    Hadamard output, before VQ (may be NULL)
 * and resid [R][d] fp16: the last r tokens, verbatim (rows >= r untouched).
 * signs: NULL for the plain Hadamard transform, or d values +1/-1 for the
 * randomised transform u = H diag(signs) w ([P3 sec. 2]).
 * scale_adjust: scale adjustment "Strategy 3" ([P3 sec. 3]): the quantised
 * vector c_hat (all slots' codewords) is scaled by alpha = |u|^2 / (u . c_hat)
 * so that its component along u equals u; alpha multiplies the stored n2
 * (alpha = 1 when u . c_hat <= 0).
 * Returns nq. */
int orc_encode_unit(const uint16_t* x, int L, int d, int R, int s,
                    const uint16_t* cb, int ncw, const double* signs, int scale_adjust,
                    uint8_t* codes, uint16_t* scales, uint16_t* mu_st,
                    uint16_t* resid, double* gap, double* u_out) {
  int r = orc_resid_count(L, R);
  int nq = L - r;
  int S = d / s;
  double* n1 = (double*)malloc(sizeof(double) * R);
  double* n2 = (double*)malloc(sizeof(double) * R);
  double* mu = (double*)malloc(sizeof(double) * d);
  double* w = (double*)malloc(sizeof(double) * (size_t)R * d);
  double* u = (double*)malloc(sizeof(double) * d);
  double* Hm = (double*)malloc(sizeof(double) * (size_t)d * d);
  double* cbd = (double*)malloc(sizeof(double) * (size_t)ncw * s);
  double* ws = (double*)malloc(sizeof(double) * d);
  orc_hadamard_matrix(d, Hm);
  for (size_t e = 0; e < (size_t)ncw * s; ++e) cbd[e] = orc_h2d(cb[e]);
  for (int blk = 0; blk < nq / R; ++blk) {
    const uint16_t* xb = x + (size_t)blk * R * d;
    orc_nsn_block(xb, R, d, n1, NULL, mu, NULL, n2, w);
    for (int c = 0; c < d; ++c) mu_st[(size_t)blk * d + c] = orc_d2h(mu[c]);
    for (int t = 0; t < R; ++t) {
      size_t tok = (size_t)blk * R + t;
      for (int c = 0; c < d; ++c) ws[c] = w[(size_t)t * d + c] * (signs ? signs[c] : 1.0);
      matvec(Hm, ws, u, d);
      if (u_out) memcpy(u_out + tok * d, u, sizeof(double) * d);
      double uu = 0.0, uc = 0.0;
      for (int j = 0; j < S; ++j) {
        double g;
        int code = vq_dbl(u + (size_t)j * s, s, cbd, ncw, NULL, &g);
        codes[tok * S + j] = (uint8_t)code;
        if (gap) gap[tok * S + j] = g;
        for (int e = 0; e < s; ++e) {
          uu += u[j * s + e] * u[j * s + e];
          uc += u[j * s + e] * cbd[(size_t)code * s + e];
        }
      }
      double alpha = 1.0;
      if (scale_adjust && uc > 0.0) alpha = uu / uc;
      scales[tok * 2 + 0] = orc_d2h(n1[t]);
      scales[tok * 2 + 1] = orc_d2h(n2[t] * alpha);
    }
  }
  for (int t = 0; t < r; ++t)
    memcpy(resid + (size_t)t * d, x + (size_t)(nq + t) * d, sizeof(uint16_t) * d);
  free(n1); free(n2); free(mu); free(w); free(u); free(Hm); free(cbd); free(ws);
  return nq;
}

/* Batched encode over n_units independent streams laid out back to back:
 * x [n_units][L][d]; outputs [n_units][...] with the per-unit shapes above
 * (codes/scales/gap/u sized for nq = L - r tokens per unit, mu for nq/R
 * blocks, resid for R rows).  OpenMP over units only. */
int orc_encode(const uint16_t* x, int64_t n_units, int L, int d, int R, int s,
               const uint16_t* cb, int ncw, const double* signs, int scale_adjust,
               uint8_t* codes, uint16_t* scales, uint16_t* mu_st, uint16_t* resid,
               double* gap, double* u_out) {
  int r = orc_resid_count(L, R);
  int nq = L - r;
  int S = d / s;
  int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
  for (i = 0; i < n_units; ++i) {
    orc_encode_unit(x + (size_t)i * L * d, L, d, R, s, cb, ncw, signs, scale_adjust,
                    codes + (size_t)i * nq * S, scales + (size_t)i * nq * 2,
                    mu_st + (size_t)i * (nq / R) * d, resid + (size_t)i * R * d,
                    gap ? gap + (size_t)i * nq * S : NULL,
                    u_out ? u_out + (size_t)i * nq * d : NULL);
  }
  return nq;
}

/* --------------------------------------------- double quantisation --- */

/* Double quantisation [P3 sec. 3, DQ: the NSN parameters (the mean o and the
 * scale s1) are stored in 4 bits; P4 implementation details: groups of 32
 * channels for o, of the residual size R for s1, round-to-nearest].  Reading
 * taken here: asymmetric min/max round-to-nearest per group,
 *   Z = fp16(min v), S = fp16((max v - min v) / 15),
 *   q_i = clamp(rint((v_i - Z) / S), 0, 15)   (S = 0: q_i = 0),
 *   v_hat_i = Z + S q_i,
 * and the stored (quantised) values are the ones the NSN forward pass uses:
 * tokens are divided by n1_hat and shifted by mu_hat, so the reconstruction
 * n1_hat (N2 H c_hat + mu_hat) differs from x only by the VQ error.  n2 stays
 * fp16.  margin_i = | frac((v_i - Z) / S) - 1/2 | is how far the rounding
 * decision is from a tie (in steps; 1/2 when S = 0). */
void orc_rtn4(const double* v, int n, uint16_t* Zb, uint16_t* Sb, uint8_t* q, double* vhat, double* margin) {
  double lo = v[0], hi = v[0];
  for (int i = 1; i < n; ++i) {
    if (v[i] < lo) lo = v[i];
    if (v[i] > hi) hi = v[i];
  }
  uint16_t zb = orc_d2h(lo), sb = orc_d2h((hi - lo) / 15.0);
  double Z = orc_h2d(zb), S = orc_h2d(sb);
  for (int i = 0; i < n; ++i) {
    double t = S > 0.0 ? (v[i] - Z) / S : 0.0;
    double k = rint(t);
    if (k < 0.0) k = 0.0;
    if (k > 15.0) k = 15.0;
    q[i] = (uint8_t)k;
    vhat[i] = Z + S * k;
    if (margin) margin[i] = S > 0.0 ? fabs(t - floor(t) - 0.5) : 0.5;
  }
  *Zb = zb;
  *Sb = sb;
}

/* Double quantisation of the codebook entries [P3 sec. 3, DQ: besides o and
 * s1, the codebook entries themselves are stored in 4 bits].  The pages give
 * no group for the codebook.  Reading taken here: the same asymmetric 4-bit
 * round-to-nearest as orc_rtn4, over groups of `group` consecutive entries of
 * the codebook in storage order (codeword-major [ncw][s]; the bench and tests
 * use 32, the group the pages give for o).  The codebook the encoder and the
 * attention use is then the read-back one, v_hat = Z + S q rounded to fp16
 * (S q and the sum are formed in double).
 *   cb        fp16 [n] (n = ncw * s, a multiple of group)
 *   record    out: n/2 bytes of 4-bit codes (entry i: byte i/2, low nibble for
 *             even i), then (S, Z) fp16 of each group (4 bytes per group)
 *   cb_hat    out: fp16 [n], the read-back codebook
 *   margin    out (may be NULL): per entry, the distance of its rounding
 *             decision from a tie (orc_rtn4). */
void orc_codebook_dq(const uint16_t* cb, int n, int group, uint8_t* record, uint16_t* cb_hat, double* margin) {
  double* v = (double*)malloc(sizeof(double) * (size_t)group);
  double* vh = (double*)malloc(sizeof(double) * (size_t)group);
  uint8_t* q = (uint8_t*)malloc((size_t)group);
  memset(record, 0, (size_t)n / 2);
  for (int g = 0; g * group < n; ++g) {
    for (int i = 0; i < group; ++i) v[i] = orc_h2d(cb[g * group + i]);
    uint16_t Zb, Sb;
    orc_rtn4(v, group, &Zb, &Sb, q, vh, margin ? margin + g * group : NULL);
    for (int i = 0; i < group; ++i) {
      const int e = g * group + i;
      record[e / 2] |= (uint8_t)(q[i] << (4 * (e & 1)));
      cb_hat[e] = orc_d2h(vh[i]);
    }
    uint8_t* sz = record + n / 2 + 4 * g;
    sz[0] = (uint8_t)(Sb & 0xff);
    sz[1] = (uint8_t)(Sb >> 8);
    sz[2] = (uint8_t)(Zb & 0xff);
    sz[3] = (uint8_t)(Zb >> 8);
  }
  free(v);
  free(vh);
  free(q);
}

/* Byte layout of one block of R tokens (per stream) in the double-quantised
 * format:
 *   scales record, orc_dq_scales_bytes(R) bytes:
 *     [0, 2R)            n2 fp16 per token
 *     [2R, 2R + R/2)     q1 nibbles (token t: byte t/2, low nibble for even t)
 *     next 4 bytes       S1, Z1 (fp16)
 *     zero padding to a multiple of 16
 *   mean record, 80 bytes:
 *     [0, 64)            mu nibbles (channel c: byte c/2, low nibble for even c)
 *     [64, 80)           (S, Z) fp16 pairs of the four 32-channel groups */
int orc_dq_scales_bytes(int R) { return ((2 * R + R / 2 + 4) + 15) / 16 * 16; }
#define ORC_DQ_MU_BYTES 80

static void put_h(uint8_t* p, uint16_t h) { p[0] = (uint8_t)(h & 0xff); p[1] = (uint8_t)(h >> 8); }
static uint16_t get_h(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static int get_nib(const uint8_t* p, int i) { return (p[i / 2] >> (4 * (i & 1))) & 15; }

/* Encode one stream in the double-quantised format (same split, NSN, Hadamard,
 * VQ and options as orc_encode_unit).  scales_rec: [nq/R][orc_dq_scales_bytes]
 * bytes, mu_rec: [nq/R][80] bytes.  Optional outputs per quantised token:
 * n1hat, m1 (margin of its q1); per block and channel: mmu (margin of its mu
 * code).  force_sr / force_mr (optional, laid out like scales_rec / mu_rec):
 * take every block's 4-bit decisions for s1 and the mean, (S, Z) and codes,
 * from these records instead of rounding, and run the rest of the encode from
 * their read-back values (a test compares another encoder's blocks whose
 * rounding decisions differ near a tie this way); their n2 bytes are ignored,
 * and m1 / mmu are 1/2.  Returns nq. */
int orc_encode_unit_dq(const uint16_t* x, int L, int d, int R, int s,
                       const uint16_t* cb, int ncw, const double* signs, int scale_adjust,
                       uint8_t* codes, uint8_t* scales_rec, uint8_t* mu_rec, uint16_t* resid,
                       double* gap, double* u_out, double* n1hat_out, double* m1_out, double* mmu_out,
                       const uint8_t* force_sr, const uint8_t* force_mr) {
  int r = orc_resid_count(L, R);
  int nq = L - r;
  int S = d / s;
  int SR = orc_dq_scales_bytes(R);
  double sqrt_d = sqrt((double)d);
  double* n1 = (double*)malloc(sizeof(double) * R);
  double* n1h = (double*)malloc(sizeof(double) * R);
  double* m1 = (double*)malloc(sizeof(double) * R);
  uint8_t* q1 = (uint8_t*)malloc(R);
  double* y = (double*)malloc(sizeof(double) * (size_t)R * d);
  double* mu = (double*)malloc(sizeof(double) * d);
  double* muh = (double*)malloc(sizeof(double) * d);
  double* mm = (double*)malloc(sizeof(double) * d);
  uint8_t* qm = (uint8_t*)malloc(d);
  double* w = (double*)malloc(sizeof(double) * d);
  double* u = (double*)malloc(sizeof(double) * d);
  double* Hm = (double*)malloc(sizeof(double) * (size_t)d * d);
  double* cbd = (double*)malloc(sizeof(double) * (size_t)ncw * s);
  orc_hadamard_matrix(d, Hm);
  for (size_t e = 0; e < (size_t)ncw * s; ++e) cbd[e] = orc_h2d(cb[e]);
  for (int blk = 0; blk < nq / R; ++blk) {
    const uint16_t* xb = x + (size_t)blk * R * d;
    uint8_t* sr = scales_rec + (size_t)blk * SR;
    uint8_t* mr = mu_rec + (size_t)blk * ORC_DQ_MU_BYTES;
    memset(sr, 0, SR);
    memset(mr, 0, ORC_DQ_MU_BYTES);
    /* s1 per token, then its 4-bit group over the block */
    for (int t = 0; t < R; ++t) {
      double ss = 0.0;
      for (int c = 0; c < d; ++c) {
        double v = orc_h2d(xb[(size_t)t * d + c]);
        ss += v * v;
      }
      n1[t] = sqrt(ss) / sqrt_d;
    }
    uint16_t Z1, S1;
    if (force_sr) {
      const uint8_t* fr = force_sr + (size_t)blk * SR;
      S1 = get_h(fr + 2 * R + R / 2);
      Z1 = get_h(fr + 2 * R + R / 2 + 2);
      for (int t = 0; t < R; ++t) {
        q1[t] = (uint8_t)get_nib(fr + 2 * R, t);
        n1h[t] = orc_h2d(Z1) + orc_h2d(S1) * (double)q1[t];
        m1[t] = 0.5;
      }
    } else {
      orc_rtn4(n1, R, &Z1, &S1, q1, n1h, m1);
    }
    for (int t = 0; t < R; ++t) sr[2 * R + t / 2] |= (uint8_t)(q1[t] << (4 * (t & 1)));
    put_h(sr + 2 * R + R / 2, S1);
    put_h(sr + 2 * R + R / 2 + 2, Z1);
    /* first normalisation by the stored s1, block mean, its 4-bit groups */
    for (int t = 0; t < R; ++t)
      for (int c = 0; c < d; ++c) {
        double v = orc_h2d(xb[(size_t)t * d + c]);
        y[(size_t)t * d + c] = n1h[t] > 0.0 ? v / n1h[t] : 0.0;
      }
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int t = 0; t < R; ++t) acc += y[(size_t)t * d + c];
      mu[c] = acc / (double)R;
    }
    for (int g = 0; g < d / 32; ++g) {
      uint16_t Zm, Sm;
      if (force_mr) {
        const uint8_t* fm = force_mr + (size_t)blk * ORC_DQ_MU_BYTES;
        Sm = get_h(fm + 64 + 4 * g);
        Zm = get_h(fm + 64 + 4 * g + 2);
        for (int c = 32 * g; c < 32 * g + 32; ++c) {
          qm[c] = (uint8_t)get_nib(fm, c);
          muh[c] = orc_h2d(Zm) + orc_h2d(Sm) * (double)qm[c];
          mm[c] = 0.5;
        }
      } else {
        orc_rtn4(mu + 32 * g, 32, &Zm, &Sm, qm + 32 * g, muh + 32 * g, mm + 32 * g);
      }
      put_h(mr + 64 + 4 * g, Sm);
      put_h(mr + 64 + 4 * g + 2, Zm);
    }
    for (int c = 0; c < d; ++c) mr[c / 2] |= (uint8_t)(qm[c] << (4 * (c & 1)));
    if (mmu_out) memcpy(mmu_out + (size_t)blk * d, mm, sizeof(double) * d);
    /* shift by the stored mean, second normalisation, Hadamard, VQ */
    for (int t = 0; t < R; ++t) {
      size_t tok = (size_t)blk * R + t;
      double ss = 0.0;
      for (int c = 0; c < d; ++c) {
        double zc = y[(size_t)t * d + c] - muh[c];
        ss += zc * zc;
      }
      double n2 = sqrt(ss) / sqrt_d;
      if (n2 < NSN_N2_FLOOR) n2 = 0.0;
      for (int c = 0; c < d; ++c) {
        double zc = y[(size_t)t * d + c] - muh[c];
        w[c] = (n2 > 0.0 ? zc / n2 : 0.0) * (signs ? signs[c] : 1.0);
      }
      matvec(Hm, w, u, d);
      if (u_out) memcpy(u_out + tok * d, u, sizeof(double) * d);
      double uu = 0.0, uc = 0.0;
      for (int j = 0; j < S; ++j) {
        double g;
        int code = vq_dbl(u + (size_t)j * s, s, cbd, ncw, NULL, &g);
        codes[tok * S + j] = (uint8_t)code;
        if (gap) gap[tok * S + j] = g;
        for (int e = 0; e < s; ++e) {
          uu += u[j * s + e] * u[j * s + e];
          uc += u[j * s + e] * cbd[(size_t)code * s + e];
        }
      }
      double alpha = (scale_adjust && uc > 0.0) ? uu / uc : 1.0;
      put_h(sr + 2 * t, orc_d2h(n2 * alpha));
      if (n1hat_out) n1hat_out[tok] = n1h[t];
      if (m1_out) m1_out[tok] = m1[t];
    }
  }
  for (int t = 0; t < r; ++t)
    memcpy(resid + (size_t)t * d, x + (size_t)(nq + t) * d, sizeof(uint16_t) * d);
  free(n1); free(n1h); free(m1); free(q1); free(y); free(mu); free(muh); free(mm); free(qm);
  free(w); free(u); free(Hm); free(cbd);
  return nq;
}

int orc_encode_dq(const uint16_t* x, int64_t n_units, int L, int d, int R, int s,
                  const uint16_t* cb, int ncw, const double* signs, int scale_adjust,
                  uint8_t* codes, uint8_t* scales_rec, uint8_t* mu_rec, uint16_t* resid,
                  double* gap, double* u_out, double* n1hat, double* m1, double* mmu,
                  const uint8_t* force_sr, const uint8_t* force_mr) {
  int r = orc_resid_count(L, R);
  int nq = L - r;
  int S = d / s;
  int SR = orc_dq_scales_bytes(R);
  int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
  for (i = 0; i < n_units; ++i) {
    orc_encode_unit_dq(x + (size_t)i * L * d, L, d, R, s, cb, ncw, signs, scale_adjust,
                       codes + (size_t)i * nq * S, scales_rec + (size_t)i * (nq / R) * SR,
                       mu_rec + (size_t)i * (nq / R) * ORC_DQ_MU_BYTES, resid + (size_t)i * R * d,
                       gap ? gap + (size_t)i * nq * S : NULL, u_out ? u_out + (size_t)i * nq * d : NULL,
                       n1hat ? n1hat + (size_t)i * nq : NULL, m1 ? m1 + (size_t)i * nq : NULL,
                       mmu ? mmu + (size_t)i * (nq / R) * d : NULL,
                       force_sr ? force_sr + (size_t)i * (nq / R) * SR : NULL,
                       force_mr ? force_mr + (size_t)i * (nq / R) * ORC_DQ_MU_BYTES : NULL);
  }
  return nq;
}

/* Reconstruct tokens [tok0, tok0 + ntok) of streams in the double-quantised
 * format (cap_tokens / R records each):
 *   x_hat = n1_hat (N2 diag(signs) H c_hat + mu_hat). */
void orc_dequant_dq(const uint8_t* codes, const uint8_t* scales_rec, const uint8_t* mu_rec,
                    int64_t n_units, int cap_tokens, int tok0, int ntok, int d, int R, int s,
                    const uint16_t* cb, const double* signs, double* out) {
  int S = d / s;
  int SR = orc_dq_scales_bytes(R);
  int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
  for (i = 0; i < n_units; ++i) {
    double* chat = (double*)malloc(sizeof(double) * d);
    double* rot = (double*)malloc(sizeof(double) * d);
    double* Hm = (double*)malloc(sizeof(double) * (size_t)d * d);
    orc_hadamard_matrix(d, Hm);
    const uint8_t* cu = codes + (size_t)i * cap_tokens * S;
    for (int k = 0; k < ntok; ++k) {
      int t = tok0 + k;
      const uint8_t* sr = scales_rec + ((size_t)i * (cap_tokens / R) + t / R) * SR;
      const uint8_t* mr = mu_rec + ((size_t)i * (cap_tokens / R) + t / R) * ORC_DQ_MU_BYTES;
      int tb = t % R;
      double n1h = orc_h2d(get_h(sr + 2 * R + R / 2 + 2)) +
                   orc_h2d(get_h(sr + 2 * R + R / 2)) * get_nib(sr + 2 * R, tb);
      double N2 = orc_h2d(get_h(sr + 2 * tb));
      for (int j = 0; j < S; ++j) {
        int code = cu[(size_t)t * S + j];
        for (int e = 0; e < s; ++e) chat[j * s + e] = orc_h2d(cb[(size_t)code * s + e]);
      }
      matvec(Hm, chat, rot, d);
      for (int c = 0; c < d; ++c) {
        int g = c / 32;
        double muh = orc_h2d(get_h(mr + 64 + 4 * g + 2)) + orc_h2d(get_h(mr + 64 + 4 * g)) * get_nib(mr, c);
        out[((size_t)i * ntok + k) * d + c] = n1h * (N2 * (signs ? signs[c] : 1.0) * rot[c] + muh);
      }
    }
    free(chat);
    free(rot);
    free(Hm);
  }
}

/* ------------------------------------------------------------- dequant --- */

/* Reconstruct tokens [tok0, tok0 + ntok) of one stream from stored values only:
 *   x_hat = N1 * (N2 * H^T c_hat + MU_block),  c_hat = concat_j C[code_j]
 * [P3 sec. 1: the byproducts (s1, o, s2) rebuild the tensor; sec. 4: dequant
 * kernel].  H^T = H for the Sylvester matrix; with signs, the inverse of
 * u = H diag(signs) w is w = diag(signs) H u. */
void orc_dequant_unit(const uint8_t* codes, const uint16_t* scales, const uint16_t* mu_st,
                      int tok0, int ntok, int d, int R, int s,
                      const uint16_t* cb, const double* signs, double* out) {
  int S = d / s;
  double* chat = (double*)malloc(sizeof(double) * d);
  double* rot = (double*)malloc(sizeof(double) * d);
  double* Hm = (double*)malloc(sizeof(double) * (size_t)d * d);
  orc_hadamard_matrix(d, Hm);
  for (int i = 0; i < ntok; ++i) {
    int t = tok0 + i;
    for (int j = 0; j < S; ++j) {
      int code = codes[(size_t)t * S + j];
      for (int e = 0; e < s; ++e) chat[j * s + e] = orc_h2d(cb[(size_t)code * s + e]);
    }
    matvec(Hm, chat, rot, d);
    double N1 = orc_h2d(scales[(size_t)t * 2 + 0]);
    double N2 = orc_h2d(scales[(size_t)t * 2 + 1]);
    const uint16_t* mub = mu_st + (size_t)(t / R) * d;
    for (int c = 0; c < d; ++c)
      out[(size_t)i * d + c] = N1 * (N2 * (signs ? signs[c] : 1.0) * rot[c] + orc_h2d(mub[c]));
  }
  free(chat);
  free(rot);
  free(Hm);
}

/* Batched dequant: streams back to back, each with cap_tokens rows of codes /
 * scales and cap_tokens/R rows of mu; out [n_units][ntok][d]. */
void orc_dequant(const uint8_t* codes, const uint16_t* scales, const uint16_t* mu_st,
                 int64_t n_units, int cap_tokens, int tok0, int ntok, int d, int R, int s,
                 const uint16_t* cb, const double* signs, double* out) {
  int S = d / s;
  int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
  for (i = 0; i < n_units; ++i) {
    orc_dequant_unit(codes + (size_t)i * cap_tokens * S, scales + (size_t)i * cap_tokens * 2,
                     mu_st + (size_t)i * (cap_tokens / R) * d, tok0, ntok, d, R, s, cb, signs,
                     out + (size_t)i * ntok * d);
  }
}

/* ---------------------------------------------------------------- RoPE --- */

/* Rotary position embedding of keys stored before RoPE [P3 sec. 4: NSN is
 * applied to keys before the rotary embedding]: rotate-half convention, pairs
 * (c, c + d/2) of token t rotated with the tables at position pos0 + t:
 *   k'[c]       = k[c] cos[p][c] - k[c + d/2] sin[p][c]
 *   k'[c + d/2] = k[c + d/2] cos[p][c] + k[c] sin[p][c].
 * k [n][T][d] in place; cos, sin fp32 [max_pos][d/2] (values taken exactly). */
void orc_rope(double* k, int64_t n, int T, int d, const float* cs, const float* sn, int pos0) {
  int h = d / 2;
  for (int64_t i = 0; i < n; ++i)
    for (int t = 0; t < T; ++t) {
      double* kt = k + ((size_t)i * T + t) * d;
      const float* cr = cs + (size_t)(pos0 + t) * h;
      const float* sr = sn + (size_t)(pos0 + t) * h;
      for (int c = 0; c < h; ++c) {
        double a = kt[c], b = kt[c + h];
        kt[c] = a * (double)cr[c] - b * (double)sr[c];
        kt[c + h] = b * (double)cr[c] + a * (double)sr[c];
      }
    }
}

/* ----------------------------------------------------------- attention --- */

/* Textbook single-query softmax attention, the plain definition the pages'
 * compressed-cache kernel computes [P3 sec. 4, attention: the score folds the
 * NSN byproducts in, which is an algebraic rewrite of attending over the
 * reconstructed cache].
 *   q   [B][Hq][d]  fp16
 *   k,v [B][Hkv][T][d] double (reconstructed tokens, then residual tokens)
 *   out [B][Hq][d]  double
 * Query head h reads KV head h / (Hq / Hkv).  scores = scale * q.k, softmax
 * with the maximum subtracted, out = sum_t p_t v_t. */
void orc_attention(const uint16_t* q, int B, int Hq, int Hkv, int d,
                   const double* k, const double* v, int T, double scale, double* out) {
  int G = Hq / Hkv;
  int64_t bh;
#pragma omp parallel for schedule(dynamic, 1)
  for (bh = 0; bh < (int64_t)B * Hq; ++bh) {
    int b = (int)(bh / Hq), h = (int)(bh % Hq);
    int hk = h / G;
    const double* kb = k + ((size_t)b * Hkv + hk) * (size_t)T * d;
    const double* vb = v + ((size_t)b * Hkv + hk) * (size_t)T * d;
    double* o = out + ((size_t)b * Hq + h) * d;
    double* sc = (double*)malloc(sizeof(double) * (T > 0 ? T : 1));
    double mx = -INFINITY;
    for (int t = 0; t < T; ++t) {
      double acc = 0.0;
      for (int c = 0; c < d; ++c) acc += orc_h2d(q[((size_t)b * Hq + h) * d + c]) * kb[(size_t)t * d + c];
      sc[t] = scale * acc;
      if (sc[t] > mx) mx = sc[t];
    }
    double l = 0.0;
    for (int t = 0; t < T; ++t) { sc[t] = exp(sc[t] - mx); l += sc[t]; }
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int t = 0; t < T; ++t) acc += sc[t] * vb[(size_t)t * d + c];
      o[c] = (T > 0) ? acc / l : 0.0;
    }
    free(sc);
  }
}

/* -------------------------------------------------------------- k-means --- */

/* Lloyd's k-means on samples [n][s] (fp32 values, taken exactly).
 * [P3 sec. 3, codebook construction; P2 "Approach"]: the codebook is fit once
 * with k-means on synthetic standard-normal (torch.randn) data.  The pages give
 * no initialisation, iteration count or empty-cluster rule; this oracle uses:
 *   init  = `init` if given, else the first ncw samples;
 *   each iteration: assign every sample to its nearest centroid (squared
 *   Euclidean, ties to the lowest index), record the mean squared error per
 *   element of that assignment in distortion[it], then move each centroid to
 *   the mean of its members (a centroid with no members stays where it is).
 * The final centroids are returned in double and rounded to fp16 (RNE). */
void orc_kmeans(const float* samples, int64_t n, int s, int ncw, int iters,
                const double* init, double* cent_out, uint16_t* cb_out, double* distortion) {
  double* c = (double*)malloc(sizeof(double) * (size_t)ncw * s);
  double* sum = (double*)malloc(sizeof(double) * (size_t)ncw * s);
  int64_t* cnt = (int64_t*)malloc(sizeof(int64_t) * ncw);
  int* assign = (int*)malloc(sizeof(int) * (size_t)n);
  double* dmin = (double*)malloc(sizeof(double) * (size_t)n);
  for (int k = 0; k < ncw; ++k)
    for (int i = 0; i < s; ++i)
      c[(size_t)k * s + i] = init ? init[(size_t)k * s + i] : (double)samples[(size_t)k * s + i];
  for (int it = 0; it < iters; ++it) {
    int64_t p;
#pragma omp parallel for schedule(static)
    for (p = 0; p < n; ++p) {
      int best = 0;
      double bd = INFINITY;
      for (int k = 0; k < ncw; ++k) {
        double dist = 0.0;
        for (int i = 0; i < s; ++i) {
          double diff = (double)samples[(size_t)p * s + i] - c[(size_t)k * s + i];
          dist += diff * diff;
        }
        if (dist < bd) { bd = dist; best = k; }
      }
      assign[p] = best;
      dmin[p] = bd;
    }
    double tot = 0.0;
    for (int64_t q = 0; q < n; ++q) tot += dmin[q];
    if (distortion) distortion[it] = tot / ((double)n * s);
    memset(sum, 0, sizeof(double) * (size_t)ncw * s);
    memset(cnt, 0, sizeof(int64_t) * ncw);
    for (int64_t q = 0; q < n; ++q) {
      int k = assign[q];
      cnt[k] += 1;
      for (int i = 0; i < s; ++i) sum[(size_t)k * s + i] += (double)samples[(size_t)q * s + i];
    }
    for (int k = 0; k < ncw; ++k)
      if (cnt[k] > 0)
        for (int i = 0; i < s; ++i) c[(size_t)k * s + i] = sum[(size_t)k * s + i] / (double)cnt[k];
  }
  for (size_t e = 0; e < (size_t)ncw * s; ++e) {
    if (cent_out) cent_out[e] = c[e];
    if (cb_out) cb_out[e] = orc_d2h(c[e]);
  }
  free(c); free(sum); free(cnt); free(assign); free(dmin);
}

/* ------------------------------------------------ cosine fine-tune --- */

/* Loss and gradient of the cosine objective of the codebook refinement
 * [P3 sec. 3, codebook construction: after k-means on torch.randn data the
 * codebook is refined to minimise the cosine distance between the original and
 * the quantised vectors].  Training vectors x [n][d] (fp32, taken exactly) are
 * head vectors of S = d / s sub-vectors; each sub-vector is assigned to its
 * nearest codeword (squared Euclidean, ties to the lowest index) and x_hat is
 * the concatenation of the assigned codewords.  Returns
 *   loss = mean over x of (1 - cos(x, x_hat)),
 * and grad [ncw][s] = d loss / d codebook with the assignment held fixed:
 *   d(1 - cos)/d x_hat = -( x / (|x| |x_hat|) - cos x_hat / |x_hat|^2 ),
 * added to the codeword each sub-vector is assigned to, then divided by n.
 * A vector with x = 0 or x_hat = 0 contributes 1 to the loss and nothing to
 * the gradient. */
double orc_cos_loss_grad(const float* x, int64_t n, int d, int s, const double* c, int ncw, double* grad) {
  int S = d / s;
  memset(grad, 0, sizeof(double) * (size_t)ncw * s);
  double loss = 0.0;
  int* code = (int*)malloc(sizeof(int) * S);
  double* xh = (double*)malloc(sizeof(double) * d);
  for (int64_t p = 0; p < n; ++p) {
    const float* xp = x + (size_t)p * d;
    for (int j = 0; j < S; ++j) {
      int best = 0;
      double bd = INFINITY;
      for (int k = 0; k < ncw; ++k) {
        double dist = 0.0;
        for (int e = 0; e < s; ++e) {
          double diff = (double)xp[j * s + e] - c[(size_t)k * s + e];
          dist += diff * diff;
        }
        if (dist < bd) { bd = dist; best = k; }
      }
      code[j] = best;
      for (int e = 0; e < s; ++e) xh[j * s + e] = c[(size_t)best * s + e];
    }
    double a = 0.0, xx = 0.0, hh = 0.0;
    for (int i = 0; i < d; ++i) {
      a += (double)xp[i] * xh[i];
      xx += (double)xp[i] * xp[i];
      hh += xh[i] * xh[i];
    }
    if (xx <= 0.0 || hh <= 0.0) {
      loss += 1.0;
      continue;
    }
    double nx = sqrt(xx), nh = sqrt(hh), cosv = a / (nx * nh);
    loss += 1.0 - cosv;
    for (int j = 0; j < S; ++j)
      for (int e = 0; e < s; ++e) {
        int i = j * s + e;
        grad[(size_t)code[j] * s + e] += -((double)xp[i] / (nx * nh) - cosv * xh[i] / hh);
      }
  }
  for (size_t e = 0; e < (size_t)ncw * s; ++e) grad[e] /= (double)n;
  free(code);
  free(xh);
  return loss / (double)n;
}

/* Full-batch gradient descent with a fixed step lr, `iters` steps from
 * cent_io (in: the k-means centroids; out: refined).  loss[it] is the loss of
 * step it's assignment, before the step.  cb_out: fp16 (RNE) of the result. */
void orc_finetune(const float* x, int64_t n, int d, int s, int ncw, int iters, double lr,
                  double* cent_io, uint16_t* cb_out, double* loss) {
  double* grad = (double*)malloc(sizeof(double) * (size_t)ncw * s);
  for (int it = 0; it < iters; ++it) {
    double l = orc_cos_loss_grad(x, n, d, s, cent_io, ncw, grad);
    if (loss) loss[it] = l;
    for (size_t e = 0; e < (size_t)ncw * s; ++e) cent_io[e] -= lr * grad[e];
  }
  if (cb_out)
    for (size_t e = 0; e < (size_t)ncw * s; ++e) cb_out[e] = orc_d2h(cent_io[e]);
  free(grad);
}

/* Number of OpenMP threads the batched routines use. */
int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Sets the number of OpenMP threads the batched routines use (n >= 1). */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
