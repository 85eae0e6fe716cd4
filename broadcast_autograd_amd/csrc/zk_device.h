// zk_device.h -- device helpers shared by the gfx950 kernels: operator
// semantics, local gradient rules, GeLU, index math and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Standard normal CDF / density in binary64 (device libm erfc / exp).
__device__ __forceinline__ double phi_cdf(double h) {
  return 0.5 * erfc(-h * 0.70710678118654752440);
}
__device__ __forceinline__ double phi_pdf(double h) {
  return exp(-0.5 * h * h) * 0.39894228040143267794;
}

// GeLU(h) = h * Phi(h) in binary64, rounded once to binary32; limits at
// +-inf are +inf and -0.
__device__ __forceinline__ float gelu32(float h) {
  if (__builtin_isinf(h)) return h > 0.f ? h : -0.0f;
  double hd = (double)h;
  return (float)(hd * phi_cdf(hd));
}

template <int OP, int EPI>
__device__ __forceinline__ float fwd32(float x, float y) {
  float h = op32<OP>(x, y);
  if constexpr (EPI == ZK_EPI_GELU) return gelu32(h);
  else return h;
}

// Local gradient of operand WHICH (0: a, 1: b) at one element, binary64.
// g is the upstream gradient, x the a value, y the b value.  With the GeLU
// epilogue g is first scaled by GeLU'(h) = Phi(h) + h*phi(h), h = x (op) y
// rounded to binary32.
template <int OP, int EPI, int WHICH>
__device__ __forceinline__ double term64(float g, float x, float y) {
  double gd = (double)g;
  if constexpr (EPI == ZK_EPI_GELU) {
    double h = (double)op32<OP>(x, y);
    gd = gd * phi_cdf(h) + (gd * h) * phi_pdf(h);
  }
  if constexpr (OP == ZK_ADD) return gd;
  else if constexpr (OP == ZK_SUB) return WHICH ? -gd : gd;
  else if constexpr (OP == ZK_MUL) return WHICH ? gd * (double)x : gd * (double)y;
  else {
    double yd = (double)y;
    if constexpr (WHICH) return -(gd * (double)x) / (yd * yd);
    else return gd / yd;
  }
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
