// codebook_dq.hip -- host-side 4-bit quantisation of the codebook entries.
//
// Double quantisation stores the NSN parameters and the codebook entries
// themselves in 4 bits (technical summary sec. 3, "Double Quantization").
// The codebook is shared by every cache and quantised once, on the host: the
// entries, in storage order ([256][s]), form groups of NSNQ_CODEBOOK_DQ_GROUP;
// a group keeps Z = fp16(min) and S = fp16((max - min) / 15) and each entry
// the 4-bit code q = clamp(rint((v - Z) / S), 0, 15) (0 when S = 0).  The
// codebook the encode and attention calls use is the read-back one,
// fp16(Z + S q).  Everything is formed in double and rounded to fp16 once.

#include <math.h>
#include <string.h>

#include "../../include/nsnq.h"

namespace {

double fp16_value(uint16_t h) {
  const int sgn = h >> 15, ex = (h >> 10) & 31, man = h & 1023;
  double v;
  if (ex == 0) v = ldexp((double)man, -24);
  else if (ex == 31) v = man ? NAN : INFINITY;
  else v = ldexp((double)(man | 1024), ex - 25);
  return sgn ? -v : v;
}

// Nearest fp16 to a finite double (ties to even), saturating to infinity
// beyond the fp16 range like any IEEE conversion.
uint16_t fp16_bits(double x) {
  const uint16_t sgn = signbit(x) ? 0x8000 : 0;
  const double a = fabs(x);
  if (a >= 65520.0) return sgn | 0x7c00;  // rounds past the largest finite value
  int e;
  frexp(a, &e);                 // a = f 2^e, f in [0.5, 1)
  const int exp16 = e - 1;      // a in [2^exp16, 2^(exp16+1))
  const int step_exp = exp16 < -14 ? -24 : exp16 - 10;  // spacing of fp16 values near a
  const double units = nearbyint(ldexp(a, -step_exp));  // current rounding mode: to nearest even
  const double r = ldexp(units, step_exp);
  if (r == 0.0) return sgn;
  int er;
  frexp(r, &er);
  const int ex16 = er - 1;
  if (ex16 < -14) return sgn | (uint16_t)units;  // subnormal: units of 2^-24
  const uint32_t man = (uint32_t)ldexp(r, 10 - ex16) - 1024u;
  return sgn | (uint16_t)((ex16 + 15) << 10) | (uint16_t)man;
}

}  // namespace

extern "C" nsnq_status nsnq_codebook_dq(const nsnq_params* p, const uint16_t* codebook_host, uint8_t* record_host,
                                        uint16_t* codebook_hat_host) {
  if (!p || !codebook_host || !record_host || !codebook_hat_host) return NSNQ_EINVAL;
  if (p->n_codewords != 256 || (p->bits != 1 && p->bits != 2)) return NSNQ_EINVAL;
  if (p->head_dim != 128) return NSNQ_EUNSUPPORTED;
  const int n = 256 * (p->bits == 2 ? 4 : 8);
  const int G = NSNQ_CODEBOOK_DQ_GROUP;
  for (int i = 0; i < n; ++i)
    if (!isfinite(fp16_value(codebook_host[i]))) return NSNQ_EINVAL;
  uint8_t* codes = record_host;
  uint8_t* params = record_host + n / 2;
  memset(codes, 0, (size_t)n / 2);
  for (int g = 0; g < n / G; ++g) {
    double lo = fp16_value(codebook_host[g * G]), hi = lo;
    for (int i = 1; i < G; ++i) {
      const double v = fp16_value(codebook_host[g * G + i]);
      lo = v < lo ? v : lo;
      hi = v > hi ? v : hi;
    }
    const uint16_t zb = fp16_bits(lo), sb = fp16_bits((hi - lo) / 15.0);
    const double Z = fp16_value(zb), S = fp16_value(sb);
    for (int i = 0; i < G; ++i) {
      const int e = g * G + i;
      int q = 0;
      if (S > 0.0) {
        const double t = nearbyint((fp16_value(codebook_host[e]) - Z) / S);
        q = t < 0.0 ? 0 : t > 15.0 ? 15 : (int)t;
      }
      codes[e >> 1] |= (uint8_t)(q << (4 * (e & 1)));
      codebook_hat_host[e] = fp16_bits(Z + S * (double)q);
    }
    params[4 * g + 0] = (uint8_t)(sb & 0xff);
    params[4 * g + 1] = (uint8_t)(sb >> 8);
    params[4 * g + 2] = (uint8_t)(zb & 0xff);
    params[4 * g + 3] = (uint8_t)(zb >> 8);
  }
  return NSNQ_OK;
}
