// zk_device.h -- device helpers shared by the gfx950 kernels: operator
// semantics, local gradient rules, GeLU, index math and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zk_gelu_coeffs.h"
#include "zk_gelu_exact.h"
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

// GeLU correctly rounded through the double-double evaluation of
// zk_gelu_exact.h: the path taken near binary32 rounding midpoints, for
// results below 2^-126 and for arguments outside the table.  Out of line, so
// that the many kernels reaching it share one copy.
__device__ __attribute__((noinline)) float gelu32_slow(float h) { return gelu32_exact(h); }

// ------------------------------------------------------------- GeLU fwd
// GeLU(h) = h Phi(h) = max(h, 0) - |h E(|h|)|/2 with E(a) = erfc(a/sqrt2)
// (for h < 0, Phi(h) = E/2; for h >= 0, Phi(h) = 1 - E/2).  E comes from
// the piecewise polynomials of zk_gelu_coeffs.h, copied into LDS by each
// block: piece i = floor(a^2 + kGeluTabK a) of a = |h| (computed exactly in
// binary64; a piece stays accurate a little past its ends, so the rounding
// of the index does not matter), E = sum c_k d^k, d = a - mid_i, Horner in
// binary64.  Error of the binary64 result: fit ~9e-15 plus ~12 binary64
// roundings, below 2^-46 relative.
constexpr int kGeluTabLen = kGeluTabN * kGeluTabStride;

// Copies the table into the block's LDS; every thread of the block calls it.
__device__ __forceinline__ void gelu_tab_load(double *lds) {
  for (int j = threadIdx.x; j < kGeluTabLen; j += blockDim.x) lds[j] = kGeluTab[j];
  __syncthreads();
}

// GeLU(h) rounded once to binary32 for W arguments.  The binary64 value y
// is rounded when it lies farther than 2^-43 (relative, 2^3 times the error
// bound) from the midpoint between its two binary32 neighbours, which makes
// the result the correctly rounded exact value; otherwise bit k of *redo is
// set and the caller recomputes element k with gelu32_slow.  Also sent
// there: results below 2^-126 (binary32 subnormals or zero, including
// h = +-0) and negative h beyond the table.  Positive h beyond the table
// gives y = h exactly (GeLU(h) = h (1 - 1e-10) rounds to h); +inf gives
// +inf and NaN gives NaN; -inf is sent to the double-double path.
template <int W>
__device__ __forceinline__ void gelu32_fast_w(const double *tab, const float (&h)[W],
                                              float (&f)[W], uint32_t &redo) {
  // The W evaluations are interleaved step by step (table reads for all,
  // then each Horner step for all) so that their LDS reads and dependent
  // binary64 FMAs overlap instead of running one element after another.
  double hd[W], ad[W], d[W], e[W];
  bool beyond[W];
  const double *t[W];
#pragma unroll
  for (int k = 0; k < W; ++k) {
    hd[k] = (double)h[k];
    ad[k] = fabs(hd[k]);
    const double a2 = hd[k] * hd[k];  // exact
    beyond[k] = a2 > kGeluTabAmax2;
    int i = (int)(fma(ad[k], kGeluTabK, a2) * kGeluTabS);  // NaN -> 0, +inf -> INT_MAX
    i = i < kGeluTabN - 1 ? i : kGeluTabN - 1;
    t[k] = tab + i * kGeluTabStride;
  }
#pragma unroll
  for (int k = 0; k < W; ++k) {
    d[k] = ad[k] - t[k][0];
    e[k] = t[k][kGeluTabW - 1];
  }
#pragma unroll
  for (int j = kGeluTabW - 2; j >= 1; --j) {
#pragma unroll
    for (int k = 0; k < W; ++k) e[k] = fma(e[k], d[k], t[k][j]);
  }
  redo = 0;
#pragma unroll
  for (int k = 0; k < W; ++k) {
    double th = hd[k] * e[k];
    th = beyond[k] ? 0.0 : th;
    const double y = fma(-0.5, fabs(th), fmax(hd[k], 0.0));  // NaN: fmax gives 0, y NaN
    // Rounding y to binary32 discards the low 29 of its 52 mantissa bits; a
    // midpoint between binary32 neighbours has exactly 2^28 there.  y is
    // trusted when those bits are more than 2^9 units (2^-43 relative, about
    // 5x the error bound in those units) from 2^28.  Every element of the
    // rare path costs its wave the double-double evaluation, so the window
    // is kept narrow (on the [4096, 1024] forward: ~8 elements a call
    // instead of ~74 with 2^12 units, 10.4 -> 9.9 us).
    const uint32_t lo = (uint32_t)__double_as_longlong(y);
    const uint32_t dist = (lo & 0x1fffffffu) - (0x10000000u - 0x200u);
    uint32_t near = (uint32_t)(dist < 0x400u || fabs(y) < 0x1p-126);
    float fy = (float)y;
    // Keep the fast value unconditional: left alone, the compiler turns a
    // select on it into a branch per element around the whole evaluation.
    asm volatile("" : "+v"(fy), "+v"(near));
    redo |= near << k;
    f[k] = fy;
  }
}

// One element, with the rare double-double path.
__device__ __forceinline__ float gelu32(const double *tab, float h) {
  const float hv[1] = {h};
  float f[1];
  uint32_t redo;
  gelu32_fast_w<1>(tab, hv, f, redo);
  return redo ? gelu32_slow(h) : f[0];
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

// g * GeLU'(h) = g * (Phi(h) + h*phi(h)) entirely in binary32, valid for
// |h| <= kGeluGradFastMax, where exp(-h^2/2) >= 2^-60 and every intermediate
// is a normal binary32 number.  The erfcx step is phi_pair_f32's; the
// exponential takes the unreduced argument (below): relative error of Phi
// and phi below ~8e-7, plus two binary32 roundings of the combination,
// i.e. within ~1.1e-6 of the sum of the magnitudes of the two terms.
constexpr float kGeluGradFastMax = 9.0f;
__device__ __forceinline__ float gelu_grad_f32(float g, float h) {
  const float hh = 0.5f * h;
  const float qh = hh * h;
  const float ql = fmaf(hh, h, -qh);  // exact remainder of h^2/2
  // exp(-(qh + ql)) = 2^-p * exp(-t): p = qh*L1 rounded (L1 = log2(e) to
  // binary32), pe = qh*L1 - p exactly, and since log2(e)*ln2 = 1,
  // t = pe*ln2 + qh*(log2(e) - L1)*ln2 + ql, |t| < 5e-6, so exp(-t) = 1 - t
  // to 1e-11; 2^-p >= 2^-59 comes from the hardware exp2 over its whole
  // argument.
  const float p = qh * 1.44269502f;
  const float pe = fmaf(qh, 1.44269502f, -p);
  float t = fmaf(qh, 1.33497582e-8f, ql);
  t = fmaf(pe, 0.693147182f, t);
  float e = __builtin_amdgcn_exp2f(-p);
  e = fmaf(-t, e, e);  // exp(-h^2/2)
  const float u = fabsf(h) * 0.707106781f;
  const float rc = __builtin_amdgcn_rcpf(u + (float)kErfcxK);
  const float sv = fmaf((u - (float)kErfcxK) * rc, kErfcxABF32[0], kErfcxABF32[1]);
  float gp = kErfcxF32[9];
#pragma unroll
  for (int j = 8; j >= 0; --j) gp = fmaf(gp, sv, kErfcxF32[j]);
  const float E = (gp * rc) * e;  // erfc(|h|/sqrt2)
  const float Phi = h < 0.f ? 0.5f * E : fmaf(-0.5f, E, 1.0f);
  const float pdf = e * 0.398942280f;
  return g * fmaf(h, pdf, Phi);
}

// ReLU(h): h for h > 0, NaN for NaN (propagated), +0 otherwise.
__device__ __forceinline__ float relu32(float h) {
  return h > 0.f ? h : (h != h ? h : 0.f);
}

// r = epi(x (op) y); tab: the GeLU table in LDS (unused without GeLU).
template <int OP, int EPI>
__device__ __forceinline__ float fwd32(float x, float y, const double *tab) {
  float h = op32<OP>(x, y);
  if constexpr (EPI == ZK_EPI_GELU) return gelu32(tab, h);
  else if constexpr (EPI == ZK_EPI_RELU) return relu32(h);
  else return h;
}

// Four elements of a 128-bit vector: r = epi(x (op) y).  The rare slow-path redo
// of the GeLU is left to the caller (bit k of *redo), which batches it after
// its stores and so keeps that code out of the hot loop.
template <int OP, int EPI>
__device__ __forceinline__ void fwd4_fast(const float (&x)[4], const float (&y)[4],
                                          float (&r)[4], uint32_t &redo,
                                          const double *tab) {
  float h[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) h[k] = op32<OP>(x[k], y[k]);
  if constexpr (EPI == ZK_EPI_GELU) {
    gelu32_fast_w<4>(tab, h, r, redo);
  } else {
    redo = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = EPI == ZK_EPI_RELU ? relu32(h[k]) : h[k];
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
  } else if constexpr (EPI == ZK_EPI_RELU) {
    // ReLU'(h) = 1 for h > 0, else 0 (NaN included)
#pragma unroll
    for (int k = 0; k < W; ++k) gd[k] = op32<OP>(x[k], y[k]) > 0.f ? (double)g[k] : 0.0;
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
  if constexpr (EPI != ZK_EPI_NONE) {
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
  if constexpr (EPI != ZK_EPI_NONE) {
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
  if constexpr (EPI != ZK_EPI_NONE) {
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
  if constexpr (EPI != ZK_EPI_NONE) {
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
  return EPI != ZK_EPI_NONE || ((OP == ZK_MUL || OP == ZK_DIV) && WHICH == 1);
}
template <int OP, int EPI, int WHICH>
__host__ __device__ constexpr bool reads_y() {
  return EPI != ZK_EPI_NONE || (OP == ZK_MUL && WHICH == 0) || OP == ZK_DIV;
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
