// zk_norm.hip -- global L2 norm of a list of gradients and the ClipGradNorm
// scaling, for gfx950 (wave64).
//
// The GPT chapter of the "Zero" book ("training loop") clips every parameter
// gradient by one common factor max_norm / (||g||_2 + 1e-6) when the L2 norm
// of all gradients together exceeds max_norm; the GPU chapter ("reduction")
// lists the gradient norm among the reductions that combine many inputs into
// few outputs.  Two launches for up to kNormTab tensors, no atomics, no host
// synchronisation:
//   norm_part  : a table of up to kNormTab dense tensors per launch; each
//                block squares and sums one chunk of kNormChunk elements of
//                one tensor in binary64 (squares of binary32 values are
//                exact) -> one binary64 partial per block in the workspace
//                (streaming loads: measured faster for the whole clip than
//                loads that leave the gradients in the last-level cache for
//                the scaling pass);
//   norm_final : (norm only) one block sums every partial in a fixed order
//                and takes the square root in binary64;
//   clip_scale : (clip) the same tables; every block first forms the norm
//                from the partials exactly as norm_final does, then, when it
//                exceeds max_norm, multiplies its chunk in place by the
//                binary32 factor max_norm / (norm + 1e-6).
// The partition depends on the element counts only, so the norm is the same
// bits on every call with the same counts, clipping or not.
#include "zk_device.h"

namespace zk {

constexpr int kNormBlk = 256;
// 128-bit loads in flight per lane (also in the in-place scaling, where
// issuing them 1, 2 or 4 at a time measured 24.4, 21.0 and 20.9 us against
// 20.7 us on the GPT gradient set)
constexpr int kNormU = 8;
constexpr int64_t kNormChunk = (int64_t)kNormBlk * 4 * kNormU;
constexpr int64_t kNormMaxGrid = (int64_t)1 << 22;

// Tensor of block b: the last t with b0[t] <= b (tables hold no empty
// tensor, so b0 is strictly increasing).
__device__ __forceinline__ int norm_find(const NormTab &tab, int64_t b) {
  int lo = 0, hi = tab.nt - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)tab.b0[mid] <= b) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(kNormBlk) void k_norm_part(NormTab tab, double *part) {
  __shared__ double sh[kNormBlk / 64];
  const int l = threadIdx.x;
  const int64_t nb = tab.b0[tab.nt];
  for (int64_t b = blockIdx.x; b < nb; b += gridDim.x) {
    const int t = norm_find(tab, b);
    const float *p = tab.p[t];
    const int64_t e0 = (b - (int64_t)tab.b0[t]) * kNormChunk;
    const int64_t rem = tab.n[t] - e0;
    double s = 0.0;
    if (rem >= kNormChunk && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
      float4 v[kNormU];
#pragma unroll
      for (int u = 0; u < kNormU; ++u) v[u] = ld4_nt(p + e0 + 4 * (l + kNormBlk * u));
#pragma unroll
      for (int u = 0; u < kNormU; ++u) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const double x = (double)el(v[u], q);
          s = __builtin_fma(x, x, s);  // the square is exact: same as s + x*x
        }
      }
    } else {
      // the ragged last chunk of a tensor, or a base that is not 16-byte
      // aligned: 32-bit loads
      const int64_t e1 = rem < kNormChunk ? rem : kNormChunk;
      for (int64_t i = l; i < e1; i += kNormBlk) {
        const double x = (double)p[e0 + i];
        s = __builtin_fma(x, x, s);
      }
    }
    s = wave_sum(s);
    if ((l & 63) == 0) sh[l >> 6] = s;
    __syncthreads();
    if (l == 0) part[b + tab.part0] = (sh[0] + sh[1]) + (sh[2] + sh[3]);
    __syncthreads();  // sh is rewritten by the next chunk
  }
}

// The square root of the sum of all P partials, in one fixed order (lane l
// sums partials l, l + 256, ...; then the wave and block trees).  Every
// block that calls it gets the same bits.  Called by all kNormBlk threads.
// A lane's loads are issued eight at a time and added in order (a missing
// one adds +0, which leaves the non-negative sum unchanged), so the clip's
// every block does not wait for them one by one.
__device__ __forceinline__ double norm_total(const double *part, int64_t P, double *sh) {
  const int l = threadIdx.x;
  double s = 0.0;
  for (int64_t i0 = l; i0 < P; i0 += 8 * kNormBlk) {
    double v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t i = i0 + (int64_t)k * kNormBlk;
      v[k] = i < P ? part[i] : 0.0;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) s += v[k];
  }
  s = wave_sum(s);
  if ((l & 63) == 0) sh[l >> 6] = s;
  __syncthreads();
  return sqrt((sh[0] + sh[1]) + (sh[2] + sh[3]));
}

__global__ __launch_bounds__(kNormBlk) void k_norm_final(const double *part, float *norm_out,
                                                         NormFinArgs fa) {
  __shared__ double sh[kNormBlk / 64];
  const double nrm = norm_total(part, fa.P, sh);
  if (threadIdx.x == 0) *norm_out = (float)nrm;
}

// ClipGradNorm's scaling.  Each block first forms the norm itself from the
// partials (the same bits in every block), so no separate launch has to
// publish it; the first launch's block 0 writes it out.
__global__ __launch_bounds__(kNormBlk) void k_clip_scale(NormTab tab, const double *part,
                                                         float *norm_out, NormFinArgs fa) {
  __shared__ double sh[kNormBlk / 64];
  const double nrm = norm_total(part, fa.P, sh);
  if (blockIdx.x == 0 && tab.part0 == 0 && threadIdx.x == 0) *norm_out = (float)nrm;
  if (!(nrm > fa.max_norm)) return;
  const float f = (float)(fa.max_norm / (nrm + 1e-6));
  const int l = threadIdx.x;
  const int64_t nb = tab.b0[tab.nt];
  for (int64_t b = blockIdx.x; b < nb; b += gridDim.x) {
    const int t = norm_find(tab, b);
    float *p = tab.p[t];
    const int64_t e0 = (b - (int64_t)tab.b0[t]) * kNormChunk;
    const int64_t rem = tab.n[t] - e0;
    if (rem >= kNormChunk && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
      float4 v[kNormU];
#pragma unroll
      for (int u = 0; u < kNormU; ++u) v[u] = ld4_nt(p + e0 + 4 * (l + kNormBlk * u));
#pragma unroll
      for (int u = 0; u < kNormU; ++u) {
#pragma unroll
        for (int q = 0; q < 4; ++q) el(v[u], q) = el(v[u], q) * f;
        st4_nt(p + e0 + 4 * (l + kNormBlk * u), v[u]);
      }
    } else {
      const int64_t e1 = rem < kNormChunk ? rem : kNormChunk;
      for (int64_t i = l; i < e1; i += kNormBlk) p[e0 + i] = p[e0 + i] * f;
    }
  }
}

// ------------------------------------------------------------------ host

static int64_t norm_blocks(int64_t n) { return (n + kNormChunk - 1) / kNormChunk; }

size_t norm_workspace(int count, const int64_t *numels) {
  int64_t P = 0;
  for (int t = 0; t < count; ++t) P += norm_blocks(numels[t]);
  return (size_t)(P > 0 ? P : 1) * sizeof(double);
}

// Walks the non-empty tensors in tables of up to kNormTab (and at most
// kNormMaxTableBlocks blocks), calling fn(tab) with each table's first
// partial index filled in.  Returns the number of tables through *ntab.
template <class Fn>
static hipError_t for_tables(int count, float *const *g, const int64_t *numels, Fn fn,
                             int *ntab = nullptr) {
  NormTab tab{};
  int64_t part0 = 0;
  int tables = 0;
  auto flush = [&]() -> hipError_t {
    if (tab.nt == 0) return hipSuccess;
    tab.part0 = part0;
    hipError_t e = fn(tab);
    part0 += tab.b0[tab.nt];
    tab = NormTab{};
    ++tables;
    return e;
  };
  for (int t = 0; t < count; ++t) {
    if (numels[t] == 0) continue;
    const int64_t nb = norm_blocks(numels[t]);
    if (tab.nt > 0 && (int64_t)tab.b0[tab.nt] + nb > kNormMaxTableBlocks) {
      hipError_t e = flush();
      if (e != hipSuccess) return e;
    }
    const int k = tab.nt;
    tab.p[k] = g[t];
    tab.n[k] = numels[t];
    tab.b0[k + 1] = (uint32_t)(tab.b0[k] + nb);
    tab.nt = k + 1;
    if (tab.nt == kNormTab) {
      hipError_t e = flush();
      if (e != hipSuccess) return e;
    }
  }
  hipError_t e = flush();
  if (ntab) *ntab = tables;
  return e;
}

static unsigned norm_grid(const NormTab &tab) {
  const int64_t nb = tab.b0[tab.nt];
  return (unsigned)(nb < kNormMaxGrid ? nb : kNormMaxGrid);
}

hipError_t launch_grad_norm(int count, float *const *g, const int64_t *numels, float *norm_out,
                            void *ws, bool clip, double max_norm, hipStream_t st) {
  double *part = static_cast<double *>(ws);
  int tables = 0;
  hipError_t e = for_tables(
      count, g, numels,
      [&](const NormTab &tab) {
        ProfScope prof(K_NORM_PART);
        ZK_LAUNCH(prof, k_norm_part, dim3(norm_grid(tab)), dim3(kNormBlk), 0, st, tab, part);
        return hipGetLastError();
      },
      &tables);
  if (e != hipSuccess) return e;
  NormFinArgs fa{};
  for (int t = 0; t < count; ++t) fa.P += norm_blocks(numels[t]);
  fa.max_norm = max_norm;
  if (!clip || tables == 0) {
    ProfScope prof(K_NORM_FINAL);
    ZK_LAUNCH(prof, k_norm_final, dim3(1), dim3(kNormBlk), 0, st, part, norm_out, fa);
    return hipGetLastError();
  }
  return for_tables(count, g, numels, [&](const NormTab &tab) {
    ProfScope prof(K_CLIP_SCALE);
    ZK_LAUNCH(prof, k_clip_scale, dim3(norm_grid(tab)), dim3(kNormBlk), 0, st, tab,
              static_cast<const double *>(part), norm_out, fa);
    return hipGetLastError();
  });
}

}  // namespace zk
