// zk_device.h -- device helpers shared by the gfx950 kernels: operator
// semantics, local gradient rules, GeLU, index math and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zk_gelu_coeffs.h"
#include "zk_kernels.h"

namespace zk {

// ------------------------------------------------------------ operators
// One IEEE binary32 operation, round-to-nearest-even (the library is built
// with -ffp-contract=off and the default correctly rounded division).
template <int OP>
__device__ __forceinline__ float op32(float x, float y) {
  if constexpr (OP == ZK_ADD) return x + y;
  else if constexpr (OP == ZK_SUB) return x - y;
  else if constexpr (OP == ZK_MUL) return x * y;
  else return x / y;
}

// Standard normal CDF in binary64 through the device libm erfc (accurate to
// a few binary64 ulps); the reference path of the forward GeLU.
__device__ __forceinline__ double phi_cdf(double h) {
  return 0.5 * erfc(-h * 0.70710678118654752440);
}

// GeLU through phi_cdf (the path taken near rounding ties).
__device__ __forceinline__ float gelu32_libm_inl(float h) {
  const double hd = (double)h;
  return (float)(hd * phi_cdf(hd));
}
// Out-of-line copy for kernels that would otherwise inline it many times.
__device__ __attribute__((noinline)) float gelu32_libm(float h) {
  return gelu32_libm_inl(h);
}

// a*b + c with c a wave-uniform binary64 constant held in scalar registers:
// one VOP3 v_fma_f64.  (Binary64 constants have no literal encoding; left
// to itself the compiler copies c into vector registers for every v_fmac.)
__device__ __forceinline__ double fma_s(double a, double b, double c) {
  double r;
  asm("v_fma_f64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(c));
  return r;
}

// Horner over W independent arguments: each coefficient is applied to all W
// before the next, so one scalar-register copy of it feeds W fused
// multiply-adds and the W dependency chains interleave.
template <int N, int W>
__device__ __forceinline__ void horner_w(const double (&c)[N], const double (&x)[W],
                                         double (&p)[W]) {
  double top[W];
#pragma unroll
  for (int k = 0; k < W; ++k) top[k] = c[N - 1];
#pragma unroll
  for (int k = 0; k < W; ++k) p[k] = fma_s(top[k], x[k], c[N - 2]);
#pragma unroll
  for (int j = N - 3; j >= 0; --j) {
#pragma unroll
    for (int k = 0; k < W; ++k) p[k] = fma_s(p[k], x[k], c[j]);
  }
}

// 1/d for d in a modest range (no scaling): hardware estimate and two
// Newton-Raphson steps.
__device__ __forceinline__ double rcp64(double d) {
  double r = __builtin_amdgcn_rcp(d);
  double e = fma(-d, r, 1.0);
  r = fma(r, e, r);
  e = fma(-d, r, 1.0);
  return fma(r, e, r);
}

// Phi(h) and exp(-h^2/2) for W finite arguments, branch-free binary64:
//   u = |h|/sqrt2, q = h^2/2 (exact: h is binary32),
//   exp(-q) = 2^-n exp(-r), n = rint(q/ln2), r = q - n ln2, polynomial in -r,
//   erfc(u) = erfcx(u) exp(-q), erfcx from the rational substitution
//   t = (u-K)/(u+K) (one reciprocal), Phi = erfc/2 or 1 - erfc/2.
// HI: relative error ~4e-13; LO: ~2e-8 (coefficients: zk_gelu_coeffs.h).
template <int W, bool HI>
__device__ __forceinline__ void phi_fast_w(const double (&hd)[W], double (&Phi)[W],
                                           double (&eq)[W]) {
  double u[W], n[W], mr[W], pe[W], s[W], rc[W], g[W];
#pragma unroll
  for (int k = 0; k < W; ++k) {
    u[k] = fmin(fabs(hd[k]) * 0.70710678118654752440, kErfcxUmax);
    const double q = fmin(0.5 * (hd[k] * hd[k]), 1000.0);
    n[k] = rint(q * 1.4426950408889634074);
    mr[k] = fma(n[k], 0.69314718055994530942, -q);  // -(q - n ln2)
  }
  if constexpr (HI) horner_w(kExpHI, mr, pe);
  else horner_w(kExpLO, mr, pe);
#pragma unroll
  for (int k = 0; k < W; ++k) {
    eq[k] = ldexp(pe[k], -(int)n[k]);
    rc[k] = rcp64(u[k] + kErfcxK);  // u + K in [3.75, 14.35]
    const double t = (u[k] - kErfcxK) * rc[k];
    s[k] = HI ? fma(t, kErfcxABHI[0], kErfcxABHI[1]) : fma(t, kErfcxABLO[0], kErfcxABLO[1]);
  }
  if constexpr (HI) horner_w(kErfcxHI, s, g);
  else horner_w(kErfcxLO, s, g);
#pragma unroll
  for (int k = 0; k < W; ++k) {
    const double E = (g[k] * rc[k]) * eq[k];
    Phi[k] = hd[k] < 0.0 ? 0.5 * E : fma(-0.5, E, 1.0);
  }
}

// Relative distance from a binary32 rounding boundary below which the fast
// forward value is not trusted: 2^-37 ~ 7.3e-12, about twenty times the HI
// error bound.  (Distances are measured in binary64 ulps of y, which are at
// most 2^-52 |y| and at least 2^-53 |y|.)
constexpr double kGeluTieMargin = 0x1p-37;

// GeLU(h) = h * Phi(h) rounded once to binary32.  The fast binary64 value is
// rounded when it lies farther than kGeluTieMargin (relative) from the
// midpoint between the two binary32 neighbours, which makes the result the
// correctly rounded exact value; otherwise the libm erfc path decides.
// Limits at +-inf are +inf and -0; NaN propagates.
// Fast part for W arguments: the rounded fast values, and bit k of *redo
// set when value k is too close to a rounding boundary to be trusted (the
// caller then recomputes it with gelu32_libm).
template <int W>
__device__ __forceinline__ void gelu32_fast_w(const float (&h)[W], float (&f)[W],
                                              uint32_t &redo) {
  double hd[W], Phi[W], eq[W];
#pragma unroll
  for (int k = 0; k < W; ++k) hd[k] = __builtin_isfinite(h[k]) ? (double)h[k] : 0.0;
  phi_fast_w<W, true>(hd, Phi, eq);
  redo = 0;
#pragma unroll
  for (int k = 0; k < W; ++k) {
    const double y = hd[k] * Phi[k];
    // Rounding y to binary32 discards the low 29 of its 52 mantissa bits;
    // a midpoint between binary32 neighbours has exactly 2^28 there.  y is
    // trusted when those bits are more than 2^15 units (2^-37 relative,
    // kGeluTieMargin) from 2^28.  Results below 2^-126 (binary32 subnormals
    // or zero) always take the libm path.
    const uint32_t lo = (uint32_t)__double_as_longlong(y);
    const uint32_t dist = (lo & 0x1fffffffu) - (0x10000000u - 0x8000u);
    uint32_t near = (uint32_t)(dist < 0x10000u || fabs(y) < 0x1p-126);
    float fy = (float)y;
    // Keep the fast value unconditional: left alone, the compiler turns the
    // select below into a branch per element around the whole evaluation,
    // which serialises the W independent chains.
    asm volatile("" : "+v"(fy), "+v"(near));
    const bool fin = __builtin_isfinite(h[k]);
    redo |= (fin ? near : 0u) << k;
    // limits: +inf -> +inf, -inf -> -0, NaN -> NaN
    f[k] = fin ? fy : (__builtin_isnan(h[k]) || h[k] > 0.f ? h[k] : -0.0f);
  }
}

__device__ __forceinline__ float gelu32(float h) {
  const float hv[1] = {h};
  float f[1];
  uint32_t redo;
  gelu32_fast_w<1>(hv, f, redo);
  return redo ? gelu32_libm(h) : f[0];
}

// Phi(h) and the density phi(h) at a binary32 h for the backward, whose
// tolerance is 2e-6 of the terms: a binary32 core (relative error ~1e-6)
// with the exponent scaling and the final products in binary64, so that
// nothing underflows before the binary64 terms are formed.
//   q = h^2/2 = qh + ql exactly (two-product); exp(-q) = 2^-n exp2(-r log2 e)
//   (1 - ql), n = rint(qh/ln2), r = qh - n ln2 (Cody-Waite: ln2 head with
//   10 significant bits, so n*head is exact); erfcx(u), u = |h|/sqrt2, from
//   the rational substitution with binary32 coefficients.
__device__ __forceinline__ void phi_pair_f32(float h, double &Phi, double &pdf) {
  if (!__builtin_isfinite(h)) {  // limits: Phi(+-inf) = 1 / 0, phi = 0
    Phi = h > 0.f ? 1.0 : (h < 0.f ? 0.0 : (double)h);
    pdf = h == h ? 0.0 : (double)h;
    return;
  }
  const float hh = 0.5f * h;
  const float qh = fminf(hh * h, 1000.0f);
  const float ql = fmaf(hh, h, -qh);  // exact remainder (0 once clamped: harmless)
  const float n = rintf(qh * 1.44269504f);
  float r = fmaf(-n, 0.693359375f, qh);  // exact
  r = fmaf(-n, -2.12194440e-4f, r);      // ln2 - head
  float e = __builtin_amdgcn_exp2f(-r * 1.44269504f);
  e = fmaf(-ql, e, e);  // exp(-ql) ~ 1 - ql, |ql| <= 2^-24 q
  const double eq = ldexp((double)e, -(int)n);
  const float u = fminf(fabsf(h) * 0.707106781f, (float)kErfcxUmax);
  const float rc = __builtin_amdgcn_rcpf(u + (float)kErfcxK);
  const float s = fmaf((u - (float)kErfcxK) * rc, kErfcxABF32[0], kErfcxABF32[1]);
  float g = kErfcxF32[9];
#pragma unroll
  for (int j = 8; j >= 0; --j) g = fmaf(g, s, kErfcxF32[j]);
  const double E = (double)(g * rc) * eq;
  Phi = h < 0.f ? 0.5 * E : fma(-0.5, E, 1.0);
  pdf = eq * 0.39894228040143267794;
}

// g * GeLU'(h) = g*Phi(h) + (g*h)*phi(h) entirely in binary32, valid for
// |h| <= kGeluGradFastMax, where exp(-h^2/2) >= 2^-60 and every intermediate
// is a normal binary32 number.  Same steps as phi_pair_f32: relative error
// of Phi and phi below ~8e-7, plus three binary32 roundings of the products,
// i.e. within ~1.1e-6 of the sum of the magnitudes of the two terms.
constexpr float kGeluGradFastMax = 9.0f;
__device__ __forceinline__ float gelu_grad_f32(float g, float h) {
  const float hh = 0.5f * h;
  const float qh = hh * h;
  const float ql = fmaf(hh, h, -qh);  // exact remainder of h^2/2
  const float n = rintf(qh * 1.44269504f);
  float r = fmaf(-n, 0.693359375f, qh);  // exact
  r = fmaf(-n, -2.12194440e-4f, r);      // ln2 - head
  float e = __builtin_amdgcn_exp2f(-r * 1.44269504f);
  e = fmaf(-ql, e, e);
  e = ldexpf(e, -(int)n);  // exp(-h^2/2)
  const float u = fabsf(h) * 0.707106781f;
  const float rc = __builtin_amdgcn_rcpf(u + (float)kErfcxK);
  const float sv = fmaf((u - (float)kErfcxK) * rc, kErfcxABF32[0], kErfcxABF32[1]);
  float gp = kErfcxF32[9];
#pragma unroll
  for (int j = 8; j >= 0; --j) gp = fmaf(gp, sv, kErfcxF32[j]);
  const float E = (gp * rc) * e;  // erfc(|h|/sqrt2)
  const float Phi = h < 0.f ? 0.5f * E : fmaf(-0.5f, E, 1.0f);
  const float pdf = e * 0.398942280f;
  return fmaf(g * h, pdf, g * Phi);
}

// Phi(h) and the density phi(h) for W arguments (LO accuracy, backward).
template <int W>
__device__ __forceinline__ void phi_pair_lo_w(const double (&h)[W], double (&Phi)[W],
                                              double (&pdf)[W]) {
  double hd[W], eq[W];
#pragma unroll
  for (int k = 0; k < W; ++k) hd[k] = __builtin_isfinite(h[k]) ? h[k] : 0.0;
  phi_fast_w<W, false>(hd, Phi, eq);
#pragma unroll
  for (int k = 0; k < W; ++k) {
    pdf[k] = eq[k] * 0.39894228040143267794;
    if (!__builtin_isfinite(h[k])) {  // limits: Phi(+-inf) = 1 / 0, phi = 0
      Phi[k] = h[k] > 0.0 ? 1.0 : (h[k] < 0.0 ? 0.0 : h[k]);
      pdf[k] = h[k] == h[k] ? 0.0 : h[k];
    }
  }
}

template <int OP, int EPI>
__device__ __forceinline__ float fwd32(float x, float y) {
  float h = op32<OP>(x, y);
  if constexpr (EPI == ZK_EPI_GELU) return gelu32(h);
  else return h;
}

// Four elements of a 128-bit vector: r = epi(x (op) y).  The rare libm redo
// of the GeLU is left to the caller (bit k of *redo), which batches it after
// its stores and so keeps that code out of the hot loop.
template <int OP, int EPI>
__device__ __forceinline__ void fwd4_fast(const float (&x)[4], const float (&y)[4],
                                          float (&r)[4], uint32_t &redo) {
  float h[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) h[k] = op32<OP>(x[k], y[k]);
  if constexpr (EPI == ZK_EPI_GELU) {
    gelu32_fast_w<4>(h, r, redo);
  } else {
    redo = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = h[k];
  }
}

// Upstream gradient seen by the operator for W elements: g itself, or
// g * GeLU'(h) with the epilogue, where GeLU'(h) = Phi(h) + h*phi(h) and
// h = x (op) y rounded to binary32 (binary64 results).
template <int OP, int EPI, int W>
__device__ __forceinline__ void gscale_w(const float (&g)[W], const float (&x)[W],
                                         const float (&y)[W], double (&gd)[W]) {
  if constexpr (EPI == ZK_EPI_GELU) {
    // binary32 for |h| <= kGeluGradFastMax; the rare larger, infinite or NaN
    // arguments take the binary64-scaled path afterwards
    float h[W];
    uint32_t slow = 0;
#pragma unroll
    for (int k = 0; k < W; ++k) {
      h[k] = op32<OP>(x[k], y[k]);
      slow |= (uint32_t)!(fabsf(h[k]) <= kGeluGradFastMax) << k;
      gd[k] = (double)gelu_grad_f32(g[k], h[k]);
    }
    if (slow) {
#pragma unroll
      for (int k = 0; k < W; ++k) {
        if ((slow >> k) & 1u) {
          double Phi, pdf;
          phi_pair_f32(h[k], Phi, pdf);
          const double gk = (double)g[k];
          gd[k] = gk * Phi + (gk * (double)h[k]) * pdf;
        }
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < W; ++k) gd[k] = (double)g[k];
  }
}

template <int OP, int EPI>
__device__ __forceinline__ double gscale(float g, float x, float y) {
  const float gv[1] = {g}, xv[1] = {x}, yv[1] = {y};
  double gd[1];
  gscale_w<OP, EPI, 1>(gv, xv, yv, gd);
  return gd[0];
}

// The operator's local rule for operand WHICH applied to a binary64
// upstream value gd.
template <int OP, int WHICH>
__device__ __forceinline__ double rule64(double gd, float x, float y) {
  if constexpr (OP == ZK_ADD) return gd;
  else if constexpr (OP == ZK_SUB) return WHICH ? -gd : gd;
  else if constexpr (OP == ZK_MUL) return WHICH ? gd * (double)x : gd * (double)y;
  else {
    double yd = (double)y;
    if constexpr (WHICH) return -(gd * (double)x) / (yd * yd);
    else return gd / yd;
  }
}

template <int OP, int EPI, int WHICH>
__device__ __forceinline__ double term64(float g, float x, float y) {
  return rule64<OP, WHICH>(gscale<OP, EPI>(g, x, y), x, y);
}

// The same local gradient rounded to binary32 for a full-shape gradient.
// Cheap single-precision forms where the rule is one product or quotient.
template <int OP, int EPI, int WHICH>
__device__ __forceinline__ float term32(float g, float x, float y) {
  if constexpr (EPI == ZK_EPI_GELU) {
    return (float)term64<OP, EPI, WHICH>(g, x, y);
  } else if constexpr (OP == ZK_ADD) {
    return g;
  } else if constexpr (OP == ZK_SUB) {
    return WHICH ? -g : g;
  } else if constexpr (OP == ZK_MUL) {
    return WHICH ? g * x : g * y;
  } else {
    if constexpr (WHICH) return (float)term64<OP, EPI, 1>(g, x, y);
    else return g / y;
  }
}

// Both local gradients at one element, sharing GeLU'(h): the reduced
// operand's term in binary64 (ts) and the full operand's in binary32 (tb).
// SMALL is the reduced operand (0: a, 1: b).
template <int OP, int EPI, int SMALL>
__device__ __forceinline__ void terms2(float g, float x, float y, double &ts,
                                       float &tb) {
  if constexpr (EPI == ZK_EPI_GELU) {
    const double gd = gscale<OP, EPI>(g, x, y);
    ts = rule64<OP, SMALL>(gd, x, y);
    tb = (float)rule64<OP, 1 - SMALL>(gd, x, y);
  } else {
    ts = term64<OP, EPI, SMALL>(g, x, y);
    tb = term32<OP, EPI, 1 - SMALL>(g, x, y);
  }
}

// terms2 for the W elements of a vector (GeLU' evaluated W-wide).
template <int OP, int EPI, int SMALL, int W>
__device__ __forceinline__ void terms2_w(const float (&g)[W], const float (&x)[W],
                                         const float (&y)[W], double (&ts)[W],
                                         float (&tb)[W]) {
  if constexpr (EPI == ZK_EPI_GELU) {
    double gd[W];
    gscale_w<OP, EPI, W>(g, x, y, gd);
#pragma unroll
    for (int k = 0; k < W; ++k) {
      ts[k] = rule64<OP, SMALL>(gd[k], x[k], y[k]);
      tb[k] = (float)rule64<OP, 1 - SMALL>(gd[k], x[k], y[k]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < W; ++k) terms2<OP, EPI, SMALL>(g[k], x[k], y[k], ts[k], tb[k]);
  }
}

// Both full-shape gradients at one element, sharing GeLU'(h).
template <int OP, int EPI>
__device__ __forceinline__ void terms_ab(float g, float x, float y, float &ta,
                                         float &tb) {
  if constexpr (EPI == ZK_EPI_GELU) {
    const double gd = gscale<OP, EPI>(g, x, y);
    ta = (float)rule64<OP, 0>(gd, x, y);
    tb = (float)rule64<OP, 1>(gd, x, y);
  } else {
    ta = term32<OP, EPI, 0>(g, x, y);
    tb = term32<OP, EPI, 1>(g, x, y);
  }
}

// Whether the rule for grad WHICH reads a (x) / b (y).
template <int OP, int EPI, int WHICH>
__host__ __device__ constexpr bool reads_x() {
  return EPI == ZK_EPI_GELU || ((OP == ZK_MUL || OP == ZK_DIV) && WHICH == 1);
}
template <int OP, int EPI, int WHICH>
__host__ __device__ constexpr bool reads_y() {
  return EPI == ZK_EPI_GELU || (OP == ZK_MUL && WHICH == 0) || OP == ZK_DIV;
}

// ------------------------------------------------------------ index math
__device__ __forceinline__ uint32_t fdiv(const FastDiv &f, uint32_t n) {
  return (__umulhi(n, f.m) + n) >> f.l;
}

// ------------------------------------------------------------ memory
__device__ __forceinline__ float4 ld4(const float *p) {
  return *reinterpret_cast<const float4 *>(p);
}
__device__ __forceinline__ void st4(float *p, float4 v) {
  *reinterpret_cast<float4 *>(p) = v;
}
typedef float v4f __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld4_nt(const float *p) {
  v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st4_nt(float *p, float4 v) {
  v4f w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<v4f *>(p));
}
__device__ __forceinline__ float &el(float4 &v, int k) {
  return reinterpret_cast<float *>(&v)[k];
}
__device__ __forceinline__ float el(const float4 &v, int k) {
  return reinterpret_cast<const float *>(&v)[k];
}

// ------------------------------------------------------------ reductions
// Butterfly sum over the 64 lanes of a wave; every lane ends with the same
// value, combined in an order that depends only on the lane layout.
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

}  // namespace zk
