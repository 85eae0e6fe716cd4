// zk_gelu_exact.h -- GeLU(h) = h Phi(h) correctly rounded to binary32 by a
// double-double evaluation: the path the forward kernels take for the few
// arguments their binary64 table evaluation cannot round with certainty
// (a value near a binary32 rounding midpoint, a result below 2^-126, a
// negative argument beyond the table).
//
// GeLU is named by the Zero book (GPU chapter, element-wise section; GPT
// chapter, FFN) without a formula; the library computes the exact form
// h Phi(h), Phi the standard normal CDF, rounded once to binary32.
//
// A double-double (dd) value is hi + lo with |lo| <= ulp(hi) / 2; its
// operations keep about 104 significant bits (Dekker 1971, "A floating-point
// technique for extending the available precision"; Knuth's two-sum).  With
// x = |h| / sqrt2 and P = 2 Phi(h), so that GeLU(h) = (h / 2) P:
//   |h| < 2^-20 : P = 1 + sign(h) erf(x), erf from its Taylor series
//                 erf(x) = 2/sqrt(pi) sum_n (-1)^n x^(2n+1) / (n! (2n+1))
//                 (three terms; P keeps the tiny erf(x) in its low word);
//   up to the binary64 table's end (|h| <= 4.5 sqrt2): E = erfc(x) from the
//                 double-double piecewise polynomials of zk_gelu_dd_coeffs.h
//                 (the binary64 table's pieces, degree 16, fit error below
//                 2^-97), the high-degree terms in binary64 and the lowest
//                 few by compensated Horner steps (error below 2^-60 of E,
//                 see erfc_piece); GeLU(h) = h - (h / 2) E for h > 0 and
//                 (h / 2) E for h < 0;
//   beyond      : erfc(x) = exp(-x^2) / sqrt(pi) / K(x), K the Laplace
//                 continued fraction x + (1/2) / (x + 1 / (x + (3/2) / (x +
//                 ...))) taken backwards from depth 80 (below 2^-106 relative
//                 for x >= 3.5), exp(-x^2) = exp(-h^2 / 2) with h^2 / 2 exact
//                 in binary64 (Cody-Waite reduction by ln2, Taylor series of
//                 the remainder / 64, six squarings); P as above.
// The series and continued-fraction branches keep at least ~90 correct
// bits, the table branch at least ~60; either rounds like the exact value,
// since no binary32 argument of the table's range has a GeLU value within
// 2^-53.4 (relative) of a binary32 midpoint (exhaustive scan).
// Where h / 2 itself is a midpoint (h an odd multiple of 2^-149), y's low
// word carries the sign of the tiny term h^2 phi(0) that decides it.
//
// The functions are plain IEEE binary64 arithmetic with explicit fma (the
// library is built with -ffp-contract=off and correctly rounded division),
// so a host build computes the same bits; the CPU tests pin that build.
#pragma once

#include <math.h>
#include <stdint.h>

#include "zk_gelu_coeffs.h"
#include "zk_gelu_dd_coeffs.h"

#if defined(__HIPCC__)
#define ZK_HD __host__ __device__
// Loops of the rare path stay rolled or only partly unrolled: fully
// unrolled they would hoist all their coefficient loads into registers, and
// every kernel calling the path reserves the registers the path needs (the
// GeLU row kernel must stay within 64 VGPRs to keep 8 waves per SIMD).
#define ZK_PRAGMA(x) _Pragma(#x)
#define ZK_UNROLL(n) ZK_PRAGMA(unroll n)
#define ZK_ROLLED ZK_UNROLL(1)
#else
#define ZK_HD
#define ZK_UNROLL(n)
#define ZK_ROLLED
#endif

namespace zk {
namespace gx {

struct dd {
  double hi, lo;
};

// Mathematical constants as hi = RN64(c), lo = RN64(c - hi) (from mpmath at
// 300 bits).
constexpr double kInvSqrt2Hi = 0x1.6a09e667f3bcdp-1, kInvSqrt2Lo = -0x1.bdd3413b26456p-55;
constexpr double kTwoOverSqrtPiHi = 0x1.20dd750429b6dp+0, kTwoOverSqrtPiLo = 0x1.1ae3a914fed80p-56;
constexpr double kInvSqrtPiHi = 0x1.20dd750429b6dp-1, kInvSqrtPiLo = 0x1.1ae3a914fed80p-57;
// ln2 = L1 + L2 + L3, L1 with 40 significant bits (k * L1 is exact for the
// k <= 2^8 used here).
constexpr double kLn2Hi = 0x1.62e42fefa39efp-1;
constexpr double kLn2L1 = 0x1.62e42fefa2000p-1, kLn2L2 = 0x1.9ef35793c7673p-41,
                 kLn2L3 = 0x1.f97b57a079a19p-103;

ZK_HD inline dd two_sum(double a, double b) {
  const double s = a + b, bb = s - a;
  return dd{s, (a - (s - bb)) + (b - bb)};
}
ZK_HD inline dd fast_two_sum(double a, double b) {  // |a| >= |b| or a == 0
  const double s = a + b;
  return dd{s, b - (s - a)};
}
ZK_HD inline dd two_prod(double a, double b) {
  const double p = a * b;
  return dd{p, fma(a, b, -p)};
}
ZK_HD inline dd add(dd a, dd b) {
  dd s = two_sum(a.hi, b.hi);
  const dd t = two_sum(a.lo, b.lo);
  s.lo += t.hi;
  s = fast_two_sum(s.hi, s.lo);
  s.lo += t.lo;
  return fast_two_sum(s.hi, s.lo);
}
ZK_HD inline dd neg(dd a) { return dd{-a.hi, -a.lo}; }
ZK_HD inline dd mul(dd a, dd b) {
  dd p = two_prod(a.hi, b.hi);
  p.lo += a.hi * b.lo + a.lo * b.hi;
  return fast_two_sum(p.hi, p.lo);
}
ZK_HD inline dd mul_d(dd a, double b) {
  dd p = two_prod(a.hi, b);
  p.lo += a.lo * b;
  return fast_two_sum(p.hi, p.lo);
}
// a / b: three quotient digits with exact remainders.
ZK_HD inline dd div(dd a, dd b) {
  const double q1 = a.hi / b.hi;
  dd r = add(a, neg(mul_d(b, q1)));
  const double q2 = r.hi / b.hi;
  r = add(r, neg(mul_d(b, q2)));
  const double q3 = r.hi / b.hi;
  const dd q = fast_two_sum(q1, q2);
  return add(q, dd{q3, 0.0});
}
ZK_HD inline dd div_d(dd a, double b) {
  const double q1 = a.hi / b;
  const dd p = two_prod(q1, b);
  const double r = ((a.hi - p.hi) - p.lo) + a.lo;  // a - q1 b, nearly exact
  return fast_two_sum(q1, r / b);
}

// exp(-q) for 0 <= q <= 120 (q exact in binary64).
ZK_HD inline dd exp_neg(double q) {
  const double k = rint(q / kLn2Hi);
  // r = q - k ln2 in dd (k * L1 exact, the rest through exact products)
  dd r = two_sum(q, -k * kLn2L1);
  r = add(r, neg(two_prod(k, kLn2L2)));
  r = add(r, dd{-k * kLn2L3, 0.0});
  // exp(-r) = (exp(-r / 64))^64, |r / 64| <= 0.0055: Taylor to s^14 / 14!
  const dd s{-r.hi * 0.015625, -r.lo * 0.015625};
  dd p{1.0, 0.0};
  ZK_ROLLED
  for (int n = 14; n >= 1; --n) p = add(dd{1.0, 0.0}, div_d(mul(p, s), (double)n));
  ZK_ROLLED
  for (int j = 0; j < 6; ++j) p = mul(p, p);
  const int e = -(int)k;
  return dd{ldexp(p.hi, e), ldexp(p.lo, e)};
}

// Why ~60 bits suffice in the table's range: an exhaustive scan of every
// binary32 argument in [-10, 10] (the table covers |h| <= 6.37) finds no
// GeLU value closer than 2^-53.4 (relative) to a binary32 rounding midpoint.
// The path is kept short because a wave that meets a near tie waits for it,
// and the slowest wave decides when a kernel ends.

// erfc(a / sqrt2) for 2^-20 <= a, a^2 <= kGeluTabAmax2, as hi + lo, from
// a's double-double piece (ddtab: the rows of kGeluDDTab): the terms of
// degree kGeluDDSplit and up by binary64 Horner steps, the lower ones by
// compensated Horner steps (Graillat, Langlois and Louvet, "Compensated
// Horner scheme", 2005): each step's product and sum errors, found exactly
// by two-product and two-sum, go with the coefficient's low word into a
// second binary64 Horner sum, so only one product and one sum per step lie
// on the chain the result waits for.  That second sum is below 2^-50 of the
// first, so its own roundings cost ~2^-100; the binary64 terms' bound
// (2^-60, zk_gelu_dd_coeffs.h) dominates.
ZK_HD inline dd erfc_piece(double a, const double *ddtab) {
  // the piece of the binary64 table (a^2 is exact), its double-double twin
  int i = (int)(fma(a, kGeluTabK, a * a) * kGeluTabS);
  i = i < kGeluDDN - 1 ? i : kGeluDDN - 1;
  const double *row = ddtab + i * kGeluDDWidth;
  // d = a - mid is exact: it is a multiple of the finer of the two last
  // bits (a >= 2^-20 is a multiple of 2^-43; beyond the first piece a and
  // mid lie in the same or adjacent binades) and below 0.12, so below 2^53
  // of that unit
  const double d = a - row[0];
  double p = row[1 + 2 * kGeluDDDeg];
  ZK_UNROLL(6)
  for (int k = kGeluDDDeg - 1; k >= kGeluDDSplit; --k) p = fma(p, d, row[1 + 2 * k]);
  double e = 0.0;
  ZK_UNROLL(kGeluDDSplit)
  for (int k = kGeluDDSplit - 1; k >= 0; --k) {
    const dd m = two_prod(p, d);
    const dd s = two_sum(m.hi, row[1 + 2 * k]);
    e = fma(e, d, (m.lo + s.lo) + row[2 + 2 * k]);
    p = s.hi;
  }
  return fast_two_sum(p, e);
}

// 2 Phi(h) for a finite binary32 h with 0 < |h| < 15 outside the table's
// range (|h| < 2^-20 or h^2 > kGeluTabAmax2).
ZK_HD inline dd two_phi(float h) {
  const double a = fabs((double)h);
  const dd x = two_prod(a, kInvSqrt2Hi);
  const dd xs = add(x, dd{a * kInvSqrt2Lo, 0.0});  // x = |h| / sqrt2
  if (a < 0x1p-20) {
    const dd x2 = mul(xs, xs);
    dd t = xs, S = xs;
    ZK_ROLLED
    for (int n = 1; n <= 100; ++n) {
      t = div_d(mul(t, neg(x2)), (double)n);  // (-1)^n x^(2n+1) / n!
      const dd term = div_d(t, (double)(2 * n + 1));
      S = add(S, term);
      if (fabs(term.hi) < 0x1p-112 * fabs(S.hi)) break;
    }
    const dd erf = mul(S, dd{kTwoOverSqrtPiHi, kTwoOverSqrtPiLo});
    return add(dd{1.0, 0.0}, h > 0.f ? erf : neg(erf));
  }
  // Laplace continued fraction for erfc, evaluated from depth 80 upwards
  dd t = xs;
  ZK_ROLLED
  for (int k = 80; k >= 1; --k) t = add(xs, div(dd{0.5 * k, 0.0}, t));
  const double q = 0.5 * ((double)h * (double)h);  // h^2 / 2 = x^2, exact
  const dd erfc = div(mul(exp_neg(q), dd{kInvSqrtPiHi, kInvSqrtPiLo}), t);
  return h > 0.f ? add(dd{2.0, 0.0}, neg(erfc)) : erfc;
}

// hi + lo (|lo| <= ulp(hi) / 2) rounded to binary32, nearest-even.  Only a
// hi exactly on a binary32 midpoint can round otherwise than hi alone (the
// midpoints are binary64 numbers, and lo is below hi's last binary64 bit);
// there lo's sign decides.
ZK_HD inline float round_f32(dd y) {
  const float r = (float)y.hi;
  if ((double)r == y.hi || y.lo == 0.0) return r;
  const float r2 = nextafterf(r, y.hi > (double)r ? INFINITY : -INFINITY);
  const double mid = 0.5 * ((double)r + (double)r2);  // exact
  if (y.hi != mid) return r;
  return (y.lo > 0.0) == (r2 > r) ? r2 : r;
}

}  // namespace gx

// GeLU(h) = h Phi(h) correctly rounded to binary32, for every binary32 h:
// +inf -> +inf, -inf -> -0, NaN -> NaN, +-0 -> +-0, and -0 for h <= -15
// (|h Phi(h)| < 2^-160 there, below half the smallest subnormal).  ddtab
// as in erfc_piece.
ZK_HD inline float gelu32_exact(float h, const double *ddtab = kGeluDDTab) {
  if (h != h) return h;
  if (h == INFINITY) return h;
  if (h <= -15.0f) return -0.0f;
  if (h == 0.0f) return h * 0.5f;
  const double a = fabs((double)h);
  if (a * a <= kGeluTabAmax2 && a >= 0x1p-20) {
    // GeLU(h) = (h / 2) E for h < 0 and h - (h / 2) E for h > 0 (h / 2 exact)
    const gx::dd q = gx::mul_d(gx::erfc_piece(a, ddtab), 0.5 * (double)h);
    if (h < 0.f) return gx::round_f32(q);
    const gx::dd y = gx::two_sum((double)h, -q.hi);  // h - q.hi exactly
    return gx::round_f32(gx::fast_two_sum(y.hi, y.lo - q.lo));
  }
  const gx::dd P = gx::two_phi(h);
  return gx::round_f32(gx::mul_d(P, 0.5 * (double)h));  // (h / 2) * 2 Phi(h)
}

}  // namespace zk
