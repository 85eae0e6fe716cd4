// zk_rows.hip -- per-row statistics for gfx950 (wave64): the mean and
// variance a LayerNorm takes of each row, and the row max and sum of
// exponentials of a softmax.
//
// The GPU chapter of the "Zero" book ("reduction") lists mean, variance and
// softmax among the reductions that combine many inputs into few outputs;
// the Operator chapter ("fusion") computes the LayerNorm statistics inside
// one operator.  Here a wave owns whole rows: rows of up to 256*U elements
// are held in registers (U 128-bit vectors per lane, or 4U scalars when the
// rows are not 16-byte aligned; two or four short rows per wave at once), so
// the two passes each statistic needs (mean, then squared deviations; max,
// then exponentials) read HBM once; longer rows are streamed twice.  Sums are binary64 in a fixed order (lane
// accumulation, then the wave butterfly), rounded once.
#include <type_traits>

#include "zk_device.h"

namespace zk {

constexpr int kRowsBlk = 256;  // four rows per block

struct RowStatArgs {
  int64_t rows, cols, ld;
};

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// exp(d) for a binary64 d <= 0 that is the exact difference of two binary32
// values, or NaN: d below -746 is taken as -746 (exp is then below half the
// smallest binary64 subnormal either way, and -inf gives 0), NaN stays NaN.
// t = d log2(e) in binary64 (|t| <= 1077, error below 2^-42), t = n + f with
// n = rint(t) and |f| <= 1/2 exact, the hardware base-2 exponential of f in
// binary32 (f rounded to binary32 and the instruction's own error: relative
// error below 2e-7 together), scaled by 2^n in binary64.  The integer n is
// taken from max(n, -1100) so that a NaN converts to a defined value (the
// NaN still reaches the result through f).
__device__ __forceinline__ double exp_nonpos(double d) {
  d = d < -746.0 ? -746.0 : d;
  const double t = d * 1.4426950408889634;
  const double n = rint(t);
  const float e = __builtin_amdgcn_exp2f((float)(t - n));
  return ldexp((double)e, (int)fmax(n, -1100.0));
}

// MODE 0: o1 = mean, o2 = biased variance.  MODE 1: o1 = row max, o2 =
// sum exp(x - max).  U > 0: RPW rows per wave are held in registers at once
// (their loads all issued before any arithmetic; VEC: 128-bit loads, element
// 4(l + 64u) + q; else element l + 64i); U == 0: one row per wave, streamed.
// FULL (with VEC): the rows have exactly 256 U elements, so no element of a
// lane is out of range.
template <int MODE, int U, int RPW, bool VEC, bool FULL>
__global__ __launch_bounds__(kRowsBlk) void k_row_stats(const float *x, float *o1, float *o2,
                                                        RowStatArgs ra) {
  constexpr int WPB = kRowsBlk / 64;
  const int l = threadIdx.x & 63;
  const int64_t n = ra.cols;
  constexpr int NV = U > 0 ? 4 * U : 1;
  for (int64_t r0 = ((int64_t)blockIdx.x * WPB + (threadIdx.x >> 6)) * RPW; r0 < ra.rows;
       r0 += (int64_t)gridDim.x * WPB * RPW) {
    if constexpr (U > 0) {
      float v[RPW][NV];
      bool ok[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int64_t j = VEC ? 4 * ((int64_t)l + 64 * (i / 4)) + (i % 4) : (int64_t)l + 64 * i;
        ok[i] = FULL || j < n;
      }
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        const bool rok = r0 + rr < ra.rows;
        const float *row = x + (rok ? r0 + rr : r0) * ra.ld;
        if constexpr (VEC) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int64_t j = 4 * ((int64_t)l + 64 * u);
            float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
            if (rok && (FULL || j + 4 <= n)) {
              q = ld4_nt(row + j);
            } else if (rok) {
#pragma unroll
              for (int k = 0; k < 4; ++k)
                if (j + k < n) el(q, k) = row[j + k];
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) v[rr][4 * u + k] = el(q, k);
          }
        } else {
#pragma unroll
          for (int i = 0; i < NV; ++i) v[rr][i] = (rok && ok[i]) ? row[(int64_t)l + 64 * i] : 0.f;
        }
      }
      if constexpr (MODE == 0) {
        double s[RPW], q[RPW];
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) {
          s[rr] = 0.0;
#pragma unroll
          for (int i = 0; i < NV; ++i)
            if (ok[i]) s[rr] += (double)v[rr][i];
        }
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) s[rr] = wave_sum(s[rr]);
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) {
          const double mean = s[rr] / (double)n;
          q[rr] = 0.0;
#pragma unroll
          for (int i = 0; i < NV; ++i) {
            if (ok[i]) {
              const double d = (double)v[rr][i] - mean;
              q[rr] = fma(d, d, q[rr]);
            }
          }
        }
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) q[rr] = wave_sum(q[rr]);
        if (l == 0) {
#pragma unroll
          for (int rr = 0; rr < RPW; ++rr) {
            if (r0 + rr < ra.rows) {
              o1[r0 + rr] = (float)(s[rr] / (double)n);
              o2[r0 + rr] = (float)(q[rr] / (double)n);
            }
          }
        }
      } else {
        // The max ignores NaN.  With a finite max every d = x - max lies in
        // [-inf, 0] or is NaN, and a NaN element turns the sum into NaN,
        // which marks the row; a max of +-inf (a +inf element, or only -inf
        // and NaN elements, or an empty row) takes the rare branch, which
        // looks for NaN in the registers.  Both branches are wave-uniform.
        float m[RPW];
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) {
          m[rr] = -INFINITY;
#pragma unroll
          for (int i = 0; i < NV; ++i)
            if (ok[i]) m[rr] = fmaxf(m[rr], v[rr][i]);
        }
        double s[RPW];
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) {
          m[rr] = wave_max_f(m[rr]);
          if (__builtin_isfinite(m[rr])) {
            const double md = (double)m[rr];
            s[rr] = 0.0;
#pragma unroll
            for (int i = 0; i < NV; ++i)
              if (ok[i]) s[rr] += exp_nonpos((double)v[rr][i] - md);
            s[rr] = wave_sum(s[rr]);
            if (s[rr] != s[rr]) m[rr] = __builtin_nanf("");
          } else {
            bool nan = false;
#pragma unroll
            for (int i = 0; i < NV; ++i) nan = nan || (ok[i] && v[rr][i] != v[rr][i]);
            if (__any(nan)) m[rr] = __builtin_nanf("");
            // +inf - +inf, -inf - -inf and NaN - x are NaN: every term of a
            // non-empty row is NaN or the sum holds one
            s[rr] = n == 0 ? 0.0 : (double)__builtin_nanf("");
          }
        }
        if (l == 0) {
#pragma unroll
          for (int rr = 0; rr < RPW; ++rr) {
            if (r0 + rr < ra.rows) {
              o1[r0 + rr] = m[rr];
              o2[r0 + rr] = (float)s[rr];
            }
          }
        }
      }
    } else {
      // long rows: one row per wave, streamed twice
      const int64_t r = r0;
      const float *row = x + r * ra.ld;
      if constexpr (MODE == 0) {
        double s = 0.0;
        for (int64_t j = l; j < n; j += 64) s += (double)row[j];
        s = wave_sum(s);
        const double mean = s / (double)n;
        double q = 0.0;
        for (int64_t j = l; j < n; j += 64) {
          const double d = (double)row[j] - mean;
          q = fma(d, d, q);
        }
        q = wave_sum(q);
        if (l == 0) {
          o1[r] = (float)mean;
          o2[r] = (float)(q / (double)n);
        }
      } else {
        float m = -INFINITY;
        bool nan = false;
        for (int64_t j = l; j < n; j += 64) {
          const float e = row[j];
          nan = nan || e != e;
          m = fmaxf(m, e);
        }
        m = wave_max_f(m);
        if (__any(nan)) m = __builtin_nanf("");
        const double md = (double)m;
        double s = 0.0;
        for (int64_t j = l; j < n; j += 64) s += exp_nonpos((double)row[j] - md);
        s = wave_sum(s);
        if (l == 0) {
          o1[r] = m;
          o2[r] = (float)s;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ host

template <int MODE>
static hipError_t launch_rows_mode(const float *x, int64_t rows, int64_t cols, int64_t ld,
                                   float *o1, float *o2, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  RowStatArgs ra{rows, cols, ld};
  const bool vec = ((reinterpret_cast<uintptr_t>(x) & 15u) == 0) && (ld % 4 == 0);
  ProfScope prof(MODE == 0 ? K_ROW_MOMENTS : K_ROW_SOFTMAX);
  auto go = [&](auto Uc, auto Rc) -> hipError_t {
    constexpr int U = decltype(Uc)::value, RPW = decltype(Rc)::value;
    const int64_t per_block = (int64_t)(kRowsBlk / 64) * RPW;
    int64_t blocks = (rows + per_block - 1) / per_block;
    if (blocks > kMaxGridBlocks) blocks = kMaxGridBlocks;
    const dim3 grid((unsigned)blocks), blk(kRowsBlk);
    if (vec && U > 0 && cols == 256 * (int64_t)U)
      ZK_LAUNCH(prof, (k_row_stats<MODE, U, RPW, true, true>), grid, blk, 0, st, x, o1, o2, ra);
    else if (vec)
      ZK_LAUNCH(prof, (k_row_stats<MODE, U, RPW, true, false>), grid, blk, 0, st, x, o1, o2, ra);
    else
      ZK_LAUNCH(prof, (k_row_stats<MODE, U, RPW, false, false>), grid, blk, 0, st, x, o1, o2, ra);
    return hipGetLastError();
  };
  using std::integral_constant;
  // rows of up to 256: four per wave, so that each wave keeps >= 1 KB of
  // loads in flight (the GPT scores [98304, 256]: 28 us against 28-29 with
  // two and 32-33 with one); longer rows one per wave (the LayerNorm input
  // [16384, 384]: 8.3-8.6 us against 9.0-9.3 with two and 10.4-10.9 with
  // four)
  if (cols <= 256) return go(integral_constant<int, 1>{}, integral_constant<int, 4>{});
  if (cols <= 512) return go(integral_constant<int, 2>{}, integral_constant<int, 1>{});
  if (cols <= 1024) return go(integral_constant<int, 4>{}, integral_constant<int, 1>{});
  if (cols <= 2048) return go(integral_constant<int, 8>{}, integral_constant<int, 1>{});
  if (cols <= 4096) return go(integral_constant<int, 16>{}, integral_constant<int, 1>{});
  return go(integral_constant<int, 0>{}, integral_constant<int, 1>{});
}

hipError_t launch_row_stats(int mode, const float *x, int64_t rows, int64_t cols, int64_t ld,
                            float *o1, float *o2, hipStream_t st) {
  return mode == 0 ? launch_rows_mode<0>(x, rows, cols, ld, o1, o2, st)
                   : launch_rows_mode<1>(x, rows, cols, ld, o1, o2, st);
}

}  // namespace zk
