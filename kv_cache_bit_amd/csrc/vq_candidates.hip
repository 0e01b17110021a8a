// vq_candidates.hip -- host-side candidate lists for the 2-bit VQ search.
//
// The encoder's vector quantiser looks for the codeword nearest to each
// 4-element sub-vector u of the Hadamard-domain vector (technical summary
// sec. 3, "Vector Quantization"; squared Euclidean distance, ties to the lowest
// index).  Exhaustive search compares all 256 codewords.  The search can be
// restricted, without changing its result, to the codewords whose Voronoi
// cell meets the region u can lie in.  u has norm sqrt(d) = 11.31, so every
// element lies in [-12, 12]; the region is split by the signs of the four
// elements into 16 orthant boxes.  For each orthant box O and codeword k a small
// linear programme decides whether some point of O is at least as close to
// c_k as to every other codeword:
//
//   t*(k, O) = min_{x in O} max_{j != k} [ 2 x . (c_j - c_k) - (|c_j|^2 - |c_k|^2) ]
//            = min_{x in O} max_{j != k} [ |x - c_k|^2 - |x - c_j|^2 ]
//
// k is a candidate for O iff t* <= 0 (up to a 1e-9 margin that only ever adds
// candidates).  If t* > 0, every point of O has a codeword closer than c_k, so
// c_k is never the nearest there.  The programme has four box-bounded
// variables and 259 constraints.  It is solved exactly in fp64 by a dense
// dictionary simplex with Bland's rule.

#include <math.h>
#include <string.h>

#include "../../include/nsnq.h"

namespace {

constexpr int kDimS = 4;          // sub-vector length at 2 bits
constexpr int kNcw = 256;         // codewords
constexpr double kBox = 12.0;     // |u_i| <= |u| = sqrt(128) < 12
constexpr double kMargin = 1e-9;  // t* within this of 0 counts as meeting O
constexpr int kListLen = 128;     // table entries per orthant

double half_to_double(uint16_t h) {
  const int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(m | 1024), e - 25);
  return s ? -v : v;
}

// Dictionary simplex, maximise z = sum_j c_j x_j subject to A x <= b with
// b >= 0 and x >= 0 (so the slack basis is feasible).  Basic variable i is
// rhs[i] - sum_j T[i][j] * (nonbasic j).  Variables 0..n-1 are structural,
// n..n+m-1 slacks; Bland's rule (lowest index enters and leaves) rules out
// cycling on the degenerate vertices these programmes have.
struct Simplex {
  static constexpr int kMaxRows = kNcw - 1 + kDimS;
  static constexpr int kCols = kDimS + 1;
  int m = 0;
  double T[kMaxRows][kCols];
  double rhs[kMaxRows];
  double c[kCols];
  double z0 = 0.0;
  int basic[kMaxRows];
  int nonbasic[kCols];

  // returns the optimum, or +inf if unbounded
  double run() {
    const double tol = 1e-12;
    for (int it = 0; it < 10000; ++it) {
      int e = -1;
      for (int j = 0; j < kCols; ++j)
        if (c[j] > tol && (e < 0 || nonbasic[j] < nonbasic[e])) e = j;
      if (e < 0) return z0;
      int l = -1;
      double best = 0.0;
      for (int i = 0; i < m; ++i) {
        if (T[i][e] <= tol) continue;
        const double r = rhs[i] / T[i][e];
        if (l < 0 || r < best - 1e-15 * (1.0 + fabs(best)) ||
            (r <= best + 1e-15 * (1.0 + fabs(best)) && basic[i] < basic[l])) {
          l = i;
          best = r;
        }
      }
      if (l < 0) return INFINITY;
      const double piv = T[l][e];
      rhs[l] /= piv;
      for (int j = 0; j < kCols; ++j) T[l][j] = (j == e) ? 1.0 / piv : T[l][j] / piv;
      for (int i = 0; i < m; ++i) {
        if (i == l) continue;
        const double f = T[i][e];
        if (f == 0.0) continue;
        rhs[i] -= f * rhs[l];
        if (rhs[i] < 0.0 && rhs[i] > -1e-12) rhs[i] = 0.0;
        for (int j = 0; j < kCols; ++j) T[i][j] = (j == e) ? -f * T[l][e] : T[i][j] - f * T[l][j];
      }
      const double ce = c[e];
      z0 += ce * rhs[l];
      for (int j = 0; j < kCols; ++j) c[j] = (j == e) ? -ce * T[l][e] : c[j] - ce * T[l][j];
      const int t = basic[l];
      basic[l] = nonbasic[e];
      nonbasic[e] = t;
    }
    return INFINITY;  // iteration cap (not reached in practice): keep the codeword
  }
};

// t*(k, O) as defined above; orthant bit i set = element i negative.
double cell_gap(const double (*C)[kDimS], const double* n2, int k, int orthant, Simplex& s) {
  double sg[kDimS];
  for (int i = 0; i < kDimS; ++i) sg[i] = ((orthant >> i) & 1) ? -1.0 : 1.0;
  // x_i = sg_i y_i with 0 <= y_i <= kBox; t = t0 - r with r >= 0, and
  // t0 = max_j (-delta_j) makes every right-hand side non-negative.
  double t0 = -INFINITY;
  for (int j = 0; j < kNcw; ++j)
    if (j != k) t0 = fmax(t0, -(n2[j] - n2[k]));
  s.m = 0;
  for (int j = 0; j < kNcw; ++j) {
    if (j == k) continue;
    for (int i = 0; i < kDimS; ++i) s.T[s.m][i] = 2.0 * sg[i] * (C[j][i] - C[k][i]);
    s.T[s.m][kDimS] = 1.0;
    s.rhs[s.m] = (n2[j] - n2[k]) + t0;
    if (s.rhs[s.m] < 0.0) s.rhs[s.m] = 0.0;
    ++s.m;
  }
  for (int i = 0; i < kDimS; ++i) {
    for (int j = 0; j < Simplex::kCols; ++j) s.T[s.m][j] = (j == i) ? 1.0 : 0.0;
    s.rhs[s.m] = kBox;
    ++s.m;
  }
  for (int j = 0; j < Simplex::kCols; ++j) {
    s.c[j] = (j == kDimS) ? 1.0 : 0.0;
    s.nonbasic[j] = j;
  }
  for (int i = 0; i < s.m; ++i) s.basic[i] = Simplex::kCols + i;
  s.z0 = 0.0;
  const double r = s.run();
  return t0 - r;
}

}  // namespace

extern "C" nsnq_status nsnq_vq_candidates(const nsnq_params* p, const uint16_t* codebook_host, uint8_t* table_host,
                                          int32_t* span) {
  if (!p || !codebook_host || !table_host || !span) return NSNQ_EINVAL;
  if (p->n_codewords != kNcw || p->head_dim != 128) return NSNQ_EINVAL;
  if (p->bits != 2) return NSNQ_EUNSUPPORTED;
  double C[kNcw][kDimS], n2[kNcw];
  for (int k = 0; k < kNcw; ++k) {
    n2[k] = 0.0;
    for (int i = 0; i < kDimS; ++i) {
      C[k][i] = half_to_double(codebook_host[k * kDimS + i]);
      if (!isfinite(C[k][i])) return NSNQ_EINVAL;
      n2[k] += C[k][i] * C[k][i];
    }
  }
  static thread_local Simplex s;
  int longest = 0;
  uint8_t lists[16][kListLen];
  for (int o = 0; o < 16; ++o) {
    int n = 0;
    for (int k = 0; k < kNcw; ++k) {
      if (cell_gap(C, n2, k, o, s) <= kMargin) {
        if (n == kListLen) return NSNQ_EUNSUPPORTED;  // no gain over the exhaustive search
        lists[o][n++] = (uint8_t)k;
      }
    }
    if (n == 0) return NSNQ_EINVAL;  // cannot happen for a finite codebook
    for (int q = n; q < kListLen; ++q) lists[o][q] = lists[o][n - 1];
    longest = n > longest ? n : longest;
  }
  static_assert(sizeof(lists) == NSNQ_VQ_TABLE_BYTES, "table layout");
  memcpy(table_host, lists, sizeof(lists));
  *span = (longest + 15) / 16 * 16;
  return NSNQ_OK;
}
