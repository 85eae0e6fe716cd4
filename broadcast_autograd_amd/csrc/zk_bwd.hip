// zk_bwd.hip -- backward kernels for gfx950 (wave64).
//
// Local rule per element, then the sum of each broadcast operand's gradient
// over the positions it was repeated into (Operator chapter of the "Zero"
// book, "broadcast").  The book's kernel adds into the small gradient with
// atomics; here the sum is split by the shapes alone into partials:
//   stage 1 (one fused kernel): stream the upstream grad and the operands the
//     rule needs, write the full-shape gradient, and accumulate the small
//     gradient's terms in binary64 per lane -> wave / LDS tree -> one binary64
//     partial per (workgroup tile, kept element) in the caller's workspace;
//   stage 2 (red_final): sum each kept element's partials in a fixed order,
//     add its acc, round once to binary32.
// No atomics, so every call on the same shapes returns the same bits.
//
// Stage-1 classes (canonical pattern, R = reduced dim, K = kept dim):
//   red_col     [R, K]             column sums; lanes own 4 columns
//   red_row     [R1, K, R0] / [K, R0] / [R0]  inner run reduced; a wave owns
//               one chunk of one row and reduces it with a butterfly
//   red_tile    [R, K] with the full-shape operand transposed; 64x64 tiles
//               of it are staged through LDS
//   red_generic any pattern, rank <= 8: one thread per (kept element,
//               partial), offsets decoded per term
#include <type_traits>

#include "zk_device.h"

namespace zk {

constexpr int kBlk = 256;

template <int V>
using IC = std::integral_constant<int, V>;

// Optional extra output of the fused two-operator backward: the gradient of
// the second operator's c, +-g (+ acc), written by the stage-1 kernel that
// streams g anyway.  p == nullptr: off.  Dense in the output layout.
struct GcOut {
  float *p;
  const float *acc;
  float sign;  // +1 (add) or -1 (sub): exact
};
__device__ __forceinline__ void gc_store4(const GcOut &o, int64_t i, float4 vg) {
  float4 v;
#pragma unroll
  for (int k = 0; k < 4; ++k) el(v, k) = o.sign * el(vg, k);
  if (o.acc) {
    const float4 x = ld4_nt(o.acc + i);
#pragma unroll
    for (int k = 0; k < 4; ++k) el(v, k) = el(x, k) + el(v, k);
  }
  st4_nt(o.p + i, v);
}
__device__ __forceinline__ void gc_store1(const GcOut &o, int64_t i, float g) {
  float v = o.sign * g;
  if (o.acc) v = o.acc[i] + v;
  o.p[i] = v;
}

template <typename Fn>
static hipError_t op_epi(zk_op op, zk_epi epi, Fn &&fn) {
  switch ((int)op * 3 + (int)epi) {
    case 0: return fn(IC<ZK_ADD>{}, IC<ZK_EPI_NONE>{});
    case 1: return fn(IC<ZK_ADD>{}, IC<ZK_EPI_GELU>{});
    case 2: return fn(IC<ZK_ADD>{}, IC<ZK_EPI_RELU>{});
    case 3: return fn(IC<ZK_SUB>{}, IC<ZK_EPI_NONE>{});
    case 4: return fn(IC<ZK_SUB>{}, IC<ZK_EPI_GELU>{});
    case 5: return fn(IC<ZK_SUB>{}, IC<ZK_EPI_RELU>{});
    case 6: return fn(IC<ZK_MUL>{}, IC<ZK_EPI_NONE>{});
    case 7: return fn(IC<ZK_MUL>{}, IC<ZK_EPI_GELU>{});
    case 8: return fn(IC<ZK_MUL>{}, IC<ZK_EPI_RELU>{});
    case 9: return fn(IC<ZK_DIV>{}, IC<ZK_EPI_NONE>{});
    case 10: return fn(IC<ZK_DIV>{}, IC<ZK_EPI_GELU>{});
    case 11: return fn(IC<ZK_DIV>{}, IC<ZK_EPI_RELU>{});
  }
  return hipErrorInvalidValue;
}

template <typename Fn>
static hipError_t side_acc(int side, int acc, Fn &&fn) {
  switch (side * 3 + acc) {
    case 0: return fn(IC<0>{}, IC<0>{});
    case 1: return fn(IC<0>{}, IC<1>{});
    case 2: return fn(IC<0>{}, IC<2>{});
    case 3: return fn(IC<1>{}, IC<0>{});
    case 4: return fn(IC<1>{}, IC<1>{});
    case 5: return fn(IC<1>{}, IC<2>{});
  }
  return hipErrorInvalidValue;
}

// Does the rule of either gradient read the a-role (x) / b-role (y) value?
template <int OP, int EPI>
constexpr bool any_x() { return reads_x<OP, EPI, 0>() || reads_x<OP, EPI, 1>(); }
template <int OP, int EPI>
constexpr bool any_y() { return reads_y<OP, EPI, 0>() || reads_y<OP, EPI, 1>(); }

// ---------------------------------------------------- element-wise, flat
// Both gradients have the full shape: no reduction.  acc modes: 0 none,
// 1 the upstream grad itself, 2 a separate buffer (or the gradient, in place).
// a_arg / b_arg: that operand is a host scalar passed by value (av / bv).
struct EwArgs {
  int64_t n;
  int32_t write_a, write_b, acc_a, acc_b, read_a, read_b;
  int32_t a_arg, b_arg;
  float av, bv;
};

template <int OP, int EPI>
__device__ __forceinline__ void ew_one(float gv, float x, float y, float aa,
                                       float ab, const EwArgs &ea, float &oa,
                                       float &ob) {
  if constexpr (EPI != ZK_EPI_NONE) {
    float ta, tb;
    terms_ab<OP, EPI>(gv, x, y, ta, tb);
    if (ea.write_a) oa = ea.acc_a == 1 ? gv + ta : (ea.acc_a == 2 ? aa + ta : ta);
    if (ea.write_b) ob = ea.acc_b == 1 ? gv + tb : (ea.acc_b == 2 ? ab + tb : tb);
  } else {
    if (ea.write_a) {
      float t = term32<OP, EPI, 0>(gv, x, y);
      oa = ea.acc_a == 1 ? gv + t : (ea.acc_a == 2 ? aa + t : t);
    }
    if (ea.write_b) {
      float t = term32<OP, EPI, 1>(gv, x, y);
      ob = ea.acc_b == 1 ? gv + t : (ea.acc_b == 2 ? ab + t : t);
    }
  }
}

template <int OP, int EPI, int VEC>
__global__ __launch_bounds__(kBlk) void k_bwd_ew_flat(
    const float *g, const float *a, const float *b, float *ga,
    const float *acc_a, float *gb, const float *acc_b, EwArgs ea, GcOut gco) {
  constexpr int U = 1;  // one vector per lane, one tile per block: streams best
  constexpr int64_t tile = (int64_t)kBlk * U * VEC;
  const int64_t ntiles = (ea.n + tile - 1) / tile;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    if constexpr (VEC == 4) {
      const int64_t base = t * tile + (int64_t)threadIdx.x * 4;
      float4 vg[U], va[U], vb[U], xa[U], xb[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int64_t i = base + (int64_t)u * kBlk * 4;
        if (i + 4 <= ea.n) {
          vg[u] = ld4_nt(g + i);
          if (ea.read_a)
            va[u] = ea.a_arg ? make_float4(ea.av, ea.av, ea.av, ea.av) : ld4_nt(a + i);
          if (ea.read_b)
            vb[u] = ea.b_arg ? make_float4(ea.bv, ea.bv, ea.bv, ea.bv) : ld4_nt(b + i);
          if (ea.acc_a == 2) xa[u] = ld4_nt(acc_a + i);
          if (ea.acc_b == 2) xb[u] = ld4_nt(acc_b + i);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int64_t i = base + (int64_t)u * kBlk * 4;
        if (i + 4 <= ea.n) {
          float4 oa, ob;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            ew_one<OP, EPI>(el(vg[u], k), ea.read_a ? el(va[u], k) : 0.f,
                            ea.read_b ? el(vb[u], k) : 0.f,
                            ea.acc_a == 2 ? el(xa[u], k) : 0.f,
                            ea.acc_b == 2 ? el(xb[u], k) : 0.f, ea, el(oa, k), el(ob, k));
          if (ea.write_a) st4_nt(ga + i, oa);
          if (ea.write_b) st4_nt(gb + i, ob);
          if (gco.p) gc_store4(gco, i, vg[u]);
        } else if (i < ea.n) {
          for (int64_t j = i; j < ea.n; ++j) {
            float oa = 0.f, ob = 0.f;
            ew_one<OP, EPI>(g[j], ea.read_a ? (ea.a_arg ? ea.av : a[j]) : 0.f,
                            ea.read_b ? (ea.b_arg ? ea.bv : b[j]) : 0.f,
                            ea.acc_a == 2 ? acc_a[j] : 0.f, ea.acc_b == 2 ? acc_b[j] : 0.f,
                            ea, oa, ob);
            if (ea.write_a) ga[j] = oa;
            if (ea.write_b) gb[j] = ob;
            if (gco.p) gc_store1(gco, j, g[j]);
          }
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int64_t j = t * tile + (int64_t)u * kBlk + threadIdx.x;
        if (j < ea.n) {
          float oa = 0.f, ob = 0.f;
          ew_one<OP, EPI>(g[j], ea.read_a ? (ea.a_arg ? ea.av : a[j]) : 0.f,
                          ea.read_b ? (ea.b_arg ? ea.bv : b[j]) : 0.f,
                          ea.acc_a == 2 ? acc_a[j] : 0.f, ea.acc_b == 2 ? acc_b[j] : 0.f,
                          ea, oa, ob);
          if (ea.write_a) ga[j] = oa;
          if (ea.write_b) gb[j] = ob;
          if (gco.p) gc_store1(gco, j, g[j]);
        }
      }
    }
  }
}

// ---------------------------------------------- pass-through gradients
// The gradient of both operands of add and of sub's first operand is g
// itself, of sub's second -g (the rules read neither operand).  With one
// such gradient requested, dense and 16-byte aligned, it is a copy (plus an
// accumulator buffer): out = (NEG ? -g : g) (+ acc), 32-bit indices, one
// 128-bit vector per lane.  The element-wise kernel's general form (two
// outputs, rule operands, run-time modes, 64-bit indices) streamed the
// 512 MiB grad_resid copy ~5% slower on MI355X.
template <bool NEG, bool ACC>
__global__ __launch_bounds__(kBlk) void k_bwd_pass(const float *g, const float *acc, float *out,
                                                  int32_t n) {
  for (int64_t j = ((int64_t)blockIdx.x * kBlk + threadIdx.x) * 4; j < (int64_t)n;
       j += (int64_t)gridDim.x * kBlk * 4) {
    const int32_t i = (int32_t)j;
    if (i + 4 <= n) {
      float4 v = ld4_nt(g + i);
      if constexpr (NEG) v = make_float4(-v.x, -v.y, -v.z, -v.w);
      if constexpr (ACC) {
        const float4 x = ld4_nt(acc + i);
        v = make_float4(x.x + v.x, x.y + v.y, x.z + v.z, x.w + v.w);
      }
      st4_nt(out + i, v);
    } else {
      for (int32_t k = i; k < n; ++k) {
        float v = NEG ? -g[k] : g[k];
        if constexpr (ACC) v = acc[k] + v;
        out[k] = v;
      }
    }
  }
}

// ------------------------------------------------- element-wise, generic
template <typename I>
__device__ __forceinline__ void offs_ab(const Space &sp, I i, I &oa, I &ob) {
  I rest = i;
  oa = 0;
  ob = 0;
#pragma unroll
  for (int k = kMaxDims - 1; k >= 1; --k) {
    if (k < sp.rank) {
      I q;
      if constexpr (sizeof(I) == 4) q = (I)fdiv(sp.fd[k], (uint32_t)rest);
      else q = rest / (I)sp.n[k];
      I c = rest - q * (I)sp.n[k];
      oa += c * (I)sp.s[1][k];
      ob += c * (I)sp.s[2][k];
      rest = q;
    }
  }
  oa += rest * (I)sp.s[1][0];
  ob += rest * (I)sp.s[2][0];
}

template <int OP, int EPI, typename I>
__global__ __launch_bounds__(kBlk) void k_bwd_ew_generic(
    const float *g, const float *a, const float *b, float *ga,
    const float *acc_a, float *gb, const float *acc_b, EwArgs ea, Space sp) {
  const I n = (I)ea.n;
  // 64-bit loop counter: i0 + stride may pass 2^31 even when n does not
  for (int64_t j0 = ((int64_t)blockIdx.x * kBlk + threadIdx.x) * 4; j0 < (int64_t)n;
       j0 += (int64_t)gridDim.x * kBlk * 4) {
    const I i0 = (I)j0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      I i = i0 + k;
      if (i < n) {
        I oa, ob;
        offs_ab<I>(sp, i, oa, ob);
        float o1 = 0.f, o2 = 0.f;
        ew_one<OP, EPI>(g[i], ea.read_a ? (ea.a_arg ? ea.av : a[oa]) : 0.f,
                        ea.read_b ? (ea.b_arg ? ea.bv : b[ob]) : 0.f,
                        ea.acc_a == 2 ? acc_a[i] : 0.f, ea.acc_b == 2 ? acc_b[i] : 0.f,
                        ea, o1, o2);
        if (ea.write_a) ga[i] = o1;
        if (ea.write_b) gb[i] = o2;
      }
    }
  }
}

// --------------------------------------------------------------- red_col
// g, the full operand and its gradient are dense [R, K]; the small operand
// is read at column c with stride ss.  Each wave owns 256 columns (4 per
// lane, 128-bit accesses) and walks rcw consecutive rows, keeping 4 binary64
// column sums per lane.  NW waves of a block share the same columns and
// consecutive row ranges; with NW > 1 their sums meet in LDS in wave order,
// so one partial covers NW * rcw rows.  (Finishing the sum in the last block
// to arrive, behind an atomic ticket, was measured 6-15x slower on MI355X:
// the device-scope fences it needs cost more than the second launch.)
struct ColArgs {
  int64_t R, K, rcw, ss, colblocks;
  int64_t bands;  // row bands (partials per fold copy): blocks = colblocks * bands
  int64_t kmod;   // the small operand's columns: column c reads element c % kmod
                  // (kmod == K, or a power of two below it for folded rows)
  int32_t write_big;
};

// One partial a column (short columns, DIRECT kernels): the kernel finishes
// each sum itself into out (negated when neg, plus acc, divided by div when
// has_div; rounded once) and no stage 2 runs.
struct ColDirect {
  float *out;
  const float *acc;
  int32_t neg, has_div;
  double div;
};

// The column's result from its one binary64 sum (the arithmetic of
// k_red_final for a single partial).
__device__ __forceinline__ float col_direct(const ColDirect &cd, int64_t c, double tot) {
  double v = cd.neg ? -tot : tot;
  if (cd.acc) v += (double)cd.acc[c];
  if (cd.has_div) v = v / cd.div;
  return (float)v;
}

// Interleaved rows (IL) for a 16-wave block that reads the full operand and
// writes its gradient with the plain rules other than division.
template <int OP, int EPI, int SIDE, int NW>
constexpr bool col_interleaved() {
  constexpr bool NEED_BIG = SIDE == 0 ? any_y<OP, EPI>() : any_x<OP, EPI>();
  return NW >= 16 && NEED_BIG && EPI == ZK_EPI_NONE && OP != ZK_DIV;
}

template <int OP, int EPI, int SIDE, int ACC, int NW, bool DIRECT, bool IL>
__global__ __launch_bounds__(64 * NW) void k_red_col(
    const float *g, const float *big, const float *small, float *gbig,
    const float *accbig, double *part, ColArgs ca, GcOut gco, ColDirect cd) {
  constexpr bool NEED_BIG = SIDE == 0 ? any_y<OP, EPI>() : any_x<OP, EPI>();
  constexpr bool NEED_SMALL = SIDE == 0 ? any_x<OP, EPI>() : any_y<OP, EPI>();
  // rows in flight per wave: two for the plain rules; one with the GeLU
  // epilogue, whose arithmetic is long enough per row (measured: the
  // [4096, 1024] GeLU step is ~10% faster than with two); four where the
  // 16-wave blocks of a long column sum (one block a CU) also read the full
  // operand (the [32768, 4096] multiply backward: 274-276 us against
  // 274-281, the fused one 391-399 against 391-411; a plain sum of g, which
  // reads one stream, is 3% slower with four).  Those blocks, when they also
  // write the full operand's gradient, walk their rows interleaved across
  // the grid (IL, also with a separate accumulator buffer; measured on
  // MI355X: [32768, 4096] 291 -> 283 us, [65536, 2048] 321 -> 274 us, the
  // fused [32768, 4096] backward 392-399 -> 380-385 us; plain sums, the
  // division backward and a multiply backward that only reads the full
  // operand were as fast or slower interleaved).
  // Within the 128 VGPRs of a 16-wave block division takes one row (two
  // spilled), ReLU and a separate accumulator buffer two.
  constexpr int U = (EPI == ZK_EPI_GELU || (NW >= 16 && OP == ZK_DIV)) ? 1
                    : (NW >= 16 && NEED_BIG && EPI == ZK_EPI_NONE && ACC != 2) ? 4 : 2;
  static_assert(!IL || col_interleaved<OP, EPI, SIDE, NW>(), "interleaved rows");
  const int w = NW > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
  const int l = threadIdx.x & 63;
  __shared__ double lds[NW > 1 ? NW : 1][4][64];
  // (band p, column group cb) blocks; one per workgroup up to the grid cap,
  // then with a grid stride (block-uniform, so the LDS barriers stay uniform)
  const int64_t blocks = ca.colblocks * ca.bands;
  for (int64_t it = blockIdx.x; it < blocks; it += gridDim.x) {
    const int64_t p = it / ca.colblocks;
    const int64_t cb = it - p * ca.colblocks;
    const int64_t c = cb * 256 + 4 * l;
    const bool active = c < ca.K;
    float sv[4] = {0.f, 0.f, 0.f, 0.f};
    if (NEED_SMALL && active) {
      // folded rows: kmod is a power of two dividing 256 and c a multiple of 4
      const int64_t cm = ca.kmod < ca.K ? (c & (ca.kmod - 1)) : c;
#pragma unroll
      for (int k = 0; k < 4; ++k) sv[k] = small[(cm + k) * ca.ss];
    }
    // Row walk of wave q = p * NW + w: rows q * rcw ... q * rcw + rcw - 1
    // (j runs over the rows themselves), or, interleaved (IL), rows q,
    // q + Q, q + 2Q, ... (Q = bands * NW walkers; j counts the wave's rcw
    // rows), so that the waves running together read one compact band of
    // rows of each array.
    const int64_t q = p * NW + w;
    const int64_t j0 = IL ? 0 : q * ca.rcw;
    const int64_t j1 = IL ? ca.rcw : (j0 + ca.rcw < ca.R ? j0 + ca.rcw : ca.R);
    const int64_t QQ = ca.bands * NW;
    double s[4] = {0.0, 0.0, 0.0, 0.0};
    if (active) {
      for (int64_t j = j0; j < j1; j += U) {
        float4 vg[U], vb[U], va[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t r = IL ? q + (j + u) * QQ : j + u;
          if (j + u < j1 && (!IL || r < ca.R)) {
            const int64_t i = r * ca.K + c;
            vg[u] = ld4_nt(g + i);
            if constexpr (NEED_BIG) vb[u] = ld4_nt(big + i);
            if constexpr (ACC == 2) va[u] = ld4_nt(accbig + i);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t r = IL ? q + (j + u) * QQ : j + u;
          if (j + u < j1 && (!IL || r < ca.R)) {
            const int64_t i = r * ca.K + c;
            float gv[4], x[4], y[4], tb[4];
            double ts[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              gv[k] = el(vg[u], k);
              const float bv = NEED_BIG ? el(vb[u], k) : 0.f;
              x[k] = SIDE == 0 ? sv[k] : bv;
              y[k] = SIDE == 0 ? bv : sv[k];
            }
            terms2_w<OP, EPI, SIDE, 4>(gv, x, y, ts, tb);
            float4 ob;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              s[k] += ts[k];
              float t = tb[k];
              if constexpr (ACC == 1) t = gv[k] + t;
              if constexpr (ACC == 2) t = el(va[u], k) + t;
              el(ob, k) = t;
            }
            if (ca.write_big) st4_nt(gbig + i, ob);
            if (gco.p) gc_store4(gco, i, vg[u]);
          }
        }
      }
    }
    if constexpr (NW == 1) {
      if (active) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if constexpr (DIRECT) cd.out[c + k] = col_direct(cd, c + k, s[k]);
          else part[p * ca.K + c + k] = s[k];
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) lds[w][k][l] = s[k];
      __syncthreads();
      if (w == 0 && active) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          double tot = lds[0][k][l];
#pragma unroll
          for (int ww = 1; ww < NW; ++ww) tot += lds[ww][k][l];
          if constexpr (DIRECT) cd.out[c + k] = col_direct(cd, c + k, tot);
          else part[p * ca.K + c + k] = tot;
        }
      }
      __syncthreads();  // lds is rewritten by the block's next (band, group)
    }
  }
}

// --------------------------------------------------------------- red_row
// Rows of R0 contiguous reduced elements; row = r1 * K + k.  Work item =
// (row, chunk of CL elements); one wave per item.
// Partials are kept-element major, part[k * P + r1 * NC + ch] (P = R1 * NC
// of them per kept element): the few kept elements of these sums (16 for the
// attention scale) each own thousands of partials, which stage 2 then reads
// in contiguous runs.  Blockwise (BW, for NC a multiple of 4): the four
// waves of a block take four consecutive chunks of one row and add their
// sums in LDS in wave order, one partial per block,
// part[k * P + r1 * (NC / 4) + ch / 4].
struct RowRedArgs {
  int64_t R0, K, NC, CL, items, ss, P;
  int32_t write_big;
};

// One wave's sum of the terms of work item `item` (not yet summed across
// lanes); writes the full operand's gradient on the way.
template <int OP, int EPI, int SIDE, int ACC>
__device__ __forceinline__ double row_item(const float *g, const float *big,
                                           const float *small, float *gbig,
                                           const float *accbig, const RowRedArgs &ra,
                                           const GcOut &gco, int64_t item, int l,
                                           int64_t &r1, int64_t &k, int64_t &ch) {
  constexpr bool NEED_BIG = SIDE == 0 ? any_y<OP, EPI>() : any_x<OP, EPI>();
  constexpr bool NEED_SMALL = SIDE == 0 ? any_x<OP, EPI>() : any_y<OP, EPI>();
  const int64_t row = item / ra.NC;
  ch = item - row * ra.NC;
  r1 = row / ra.K;
  k = row - r1 * ra.K;
  const float sv = NEED_SMALL ? small[k * ra.ss] : 0.f;
  const int64_t e0 = row * ra.R0 + ch * ra.CL;
  const int64_t lim = (ch + 1) * ra.CL < ra.R0 ? (ch + 1) * ra.CL : ra.R0;
  const int64_t e1 = row * ra.R0 + lim;
  double s = 0.0;
  // one vector per lane per trip over short chunks (many waves) streams best
  for (int64_t i = e0 + 4 * l; i < e1; i += 256) {
    const float4 vg = ld4_nt(g + i);
    float4 vb, va;
    if constexpr (NEED_BIG) vb = ld4_nt(big + i);
    if constexpr (ACC == 2) va = ld4_nt(accbig + i);
    float4 ob;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float gv = el(vg, q);
      const float bv = NEED_BIG ? el(vb, q) : 0.f;
      const float x = SIDE == 0 ? sv : bv;
      const float y = SIDE == 0 ? bv : sv;
      double ts;
      float tb;
      terms2<OP, EPI, SIDE>(gv, x, y, ts, tb);
      s += ts;
      if constexpr (ACC == 1) tb = gv + tb;
      if constexpr (ACC == 2) tb = el(va, q) + tb;
      el(ob, q) = tb;
    }
    if (ra.write_big) st4_nt(gbig + i, ob);
    if (gco.p) gc_store4(gco, i, vg);
  }
  return s;
}

template <int OP, int EPI, int SIDE, int ACC, bool BW>
__global__ __launch_bounds__(kBlk) void k_red_row(
    const float *g, const float *big, const float *small, float *gbig,
    const float *accbig, double *part, RowRedArgs ra, GcOut gco) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  int64_t r1, k, ch;
  if constexpr (!BW) {
    // items (row, chunk) item = 4 * blockIdx.x + w, then with a grid stride
    for (int64_t item = (int64_t)blockIdx.x * 4 + w; item < ra.items;
         item += (int64_t)gridDim.x * 4) {
      double s = row_item<OP, EPI, SIDE, ACC>(g, big, small, gbig, accbig, ra, gco, item, l,
                                              r1, k, ch);
      s = wave_sum(s);
      if (l == 0) part[k * ra.P + r1 * ra.NC + ch] = s;
    }
  } else {
    // items % 4 == 0: every wave of a block has an item, and the block's
    // trip count is uniform, so the barriers are too
    __shared__ double sh[4];
    for (int64_t bi = blockIdx.x; bi < ra.items / 4; bi += gridDim.x) {
      double s = row_item<OP, EPI, SIDE, ACC>(g, big, small, gbig, accbig, ra, gco, bi * 4 + w,
                                              l, r1, k, ch);
      s = wave_sum(s);
      if (l == 0) sh[w] = s;
      __syncthreads();
      if (threadIdx.x == 0)
        part[k * ra.P + r1 * (ra.NC / 4) + ch / 4] = ((sh[0] + sh[1]) + sh[2]) + sh[3];
      __syncthreads();  // sh is rewritten by the block's next trip
    }
  }
}

// ------------------------------------------------------------- red_rowd
// The [R1, K, R0] pattern of red_row in one pass when a kept element has
// few terms (T = R1 * R0, 2048..16384): block k owns kept element k, its
// 1024 lanes hold every term's loads at once (U vectors each), and the
// block's fixed-order sum is finished in place (sign, acc, divisor) and
// rounded once, so no partials and no stage-2 launch.
struct RowDirArgs {
  int64_t R0, K, T, ss;
  int32_t write_big;
  int32_t neg, has_div;
  double div;
};
constexpr int kDirBlk = 1024;

template <int OP, int EPI, int SIDE, int ACC, int U>
__global__ __launch_bounds__(kDirBlk) void k_red_rowd(
    const float *g, const float *big, const float *small, float *gbig,
    const float *accbig, float *out, const float *acc, RowDirArgs ra, GcOut gco) {
  constexpr bool NEED_BIG = SIDE == 0 ? any_y<OP, EPI>() : any_x<OP, EPI>();
  constexpr bool NEED_SMALL = SIDE == 0 ? any_x<OP, EPI>() : any_y<OP, EPI>();
  __shared__ double sh[kDirBlk / 64];
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int64_t k = blockIdx.x; k < ra.K; k += gridDim.x) {
    const float sv = NEED_SMALL ? small[k * ra.ss] : 0.f;
    double s = 0.0;
    for (int64_t t0 = 0; t0 < ra.T; t0 += (int64_t)kDirBlk * 4 * U) {
      float4 vg[U], vb[U], va[U];
      int64_t idx[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t t = t0 + 4 * ((int64_t)threadIdx.x + (int64_t)kDirBlk * u);
        idx[u] = -1;
        if (t < ra.T) {
          // R0 % 4 == 0, so the 4 terms t..t+3 lie in one row r1
          const int64_t r1 = t / ra.R0;
          const int64_t i = (r1 * ra.K + k) * ra.R0 + (t - r1 * ra.R0);
          idx[u] = i;
          vg[u] = ld4_nt(g + i);
          if constexpr (NEED_BIG) vb[u] = ld4_nt(big + i);
          if constexpr (ACC == 2) va[u] = ld4_nt(accbig + i);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (idx[u] >= 0) {
          const int64_t i = idx[u];
          float gv[4], x[4], y[4], tb[4];
          double ts[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            gv[q] = el(vg[u], q);
            const float bv = NEED_BIG ? el(vb[u], q) : 0.f;
            x[q] = SIDE == 0 ? sv : bv;
            y[q] = SIDE == 0 ? bv : sv;
          }
          terms2_w<OP, EPI, SIDE, 4>(gv, x, y, ts, tb);
          float4 ob;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            s += ts[q];
            float tq = tb[q];
            if constexpr (ACC == 1) tq = gv[q] + tq;
            if constexpr (ACC == 2) tq = el(va[u], q) + tq;
            el(ob, q) = tq;
          }
          if (ra.write_big) st4_nt(gbig + i, ob);
          if (gco.p) gc_store4(gco, i, vg[u]);
        }
      }
    }
    s = wave_sum(s);
    if (l == 0) sh[w] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
      double tot = 0.0;
#pragma unroll
      for (int j = 0; j < kDirBlk / 64; ++j) tot += sh[j];
      if (ra.neg) tot = -tot;
      if (acc) tot += (double)acc[k];
      if (ra.has_div) tot = tot / ra.div;
      out[k] = (float)tot;
    }
    __syncthreads();  // sh is rewritten for the next kept element
  }
}

// -------------------------------------------------------------- red_tile
// [R, K]; the full operand F[i, j] is at i + j*ld (transposed view); g and
// the full operand's gradient are dense [R, K].  Block = 64 columns x a
// chunk of rows walked in 64-row tiles.
struct TileRedArgs {
  int64_t R, K, ld, ss, rc, tiles_c, items;
  int32_t write_big;
  int32_t tv;  // the transposed operand's columns start 16-byte aligned
};

template <int OP, int EPI, int SIDE, int ACC>
__global__ __launch_bounds__(kBlk) void k_red_tile(
    const float *g, const float *big, const float *small, float *gbig,
    const float *accbig, double *part, TileRedArgs ta) {
  constexpr bool NEED_BIG = SIDE == 0 ? any_y<OP, EPI>() : any_x<OP, EPI>();
  constexpr bool NEED_SMALL = SIDE == 0 ? any_x<OP, EPI>() : any_y<OP, EPI>();
  __shared__ float tile[64][65];
  __shared__ double red[16][64];
  const int t = threadIdx.x;
  // (row chunk p, 64-column tile tj) items, one per block up to the grid cap
  for (int64_t bt = blockIdx.x; bt < ta.items; bt += gridDim.x) {
    // (Unlike the forward tile kernel, a diagonal order of the items
    // measured slower here: the row-major gradient streams dominate.)
    const int64_t p = bt / ta.tiles_c;
    const int64_t tj = bt - p * ta.tiles_c;
    const int64_t j0 = tj * 64;
    const int m = t & 15, q = t >> 4;
    const int64_t gj = j0 + 4 * m;
    const bool colok = gj < ta.K;  // K % 4 == 0, so all 4 columns are in range
    float sv[4] = {0.f, 0.f, 0.f, 0.f};
    if (NEED_SMALL && colok) {
#pragma unroll
      for (int k = 0; k < 4; ++k) sv[k] = small[(gj + k) * ta.ss];
    }
    const int64_t r0 = p * ta.rc;
    const int64_t r1 = r0 + ta.rc < ta.R ? r0 + ta.rc : ta.R;
    double s[4] = {0.0, 0.0, 0.0, 0.0};
    for (int64_t ti = r0; ti < r1; ti += 64) {
      // Issue every load of this tile first (the transposed operand's column
      // runs and the upstream gradient's row runs), so that both latencies
      // overlap; then stage the transposed operand through LDS.
      float4 av[4];
      float4 vg[4], va[4];
      // 128-bit loads down the transposed operand's columns when they start
      // 16-byte aligned: lane (t & 15) takes rows 4(t&15)..+3 of columns
      // t/16 + 16pp; else 32-bit loads, lane (t & 63) one row of columns
      // t/64 + 4k.
      const int i4 = ta.tv ? (t & 15) * 4 : (t & 63);
      const int jq = ta.tv ? t >> 4 : t >> 6;
      if constexpr (NEED_BIG) {
        const int64_t gi = ti + i4;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          av[pp] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (ta.tv) {
            const int64_t gj = j0 + jq + 16 * pp;
            if (gj < ta.K) {
              const float *src = big + gi + gj * ta.ld;
              if (gi + 3 < r1) {
                av[pp] = ld4_nt(src);
              } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                  if (gi + k < r1) el(av[pp], k) = src[k];
              }
            }
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int64_t gj = j0 + jq + 4 * (4 * pp + k);
              if (gi < r1 && gj < ta.K) el(av[pp], k) = big[gi + gj * ta.ld];
            }
          }
        }
      }
      if (colok) {
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int64_t gi = ti + q + 16 * pp;
          if (gi < r1) {
            const int64_t off = gi * ta.K + gj;
            vg[pp] = ld4_nt(g + off);
            if constexpr (ACC == 2) va[pp] = ld4_nt(accbig + off);
          }
        }
      }
      if constexpr (NEED_BIG) {
        if (ta.tv) {
#pragma unroll
          for (int pp = 0; pp < 4; ++pp)
#pragma unroll
            for (int k = 0; k < 4; ++k) tile[jq + 16 * pp][i4 + k] = el(av[pp], k);
        } else {
#pragma unroll
          for (int pp = 0; pp < 4; ++pp)
#pragma unroll
            for (int k = 0; k < 4; ++k) tile[jq + 4 * (4 * pp + k)][i4] = el(av[pp], k);
        }
        __syncthreads();
      }
      if (colok) {
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int i = q + 16 * pp;
          const int64_t gi = ti + i;
          if (gi < r1) {
            const int64_t off = gi * ta.K + gj;
            float4 ob;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const float gv = el(vg[pp], k);
              const float bv = NEED_BIG ? tile[4 * m + k][i] : 0.f;
              const float x = SIDE == 0 ? sv[k] : bv;
              const float y = SIDE == 0 ? bv : sv[k];
              double ts;
              float tb;
              terms2<OP, EPI, SIDE>(gv, x, y, ts, tb);
              s[k] += ts;
              if constexpr (ACC == 1) tb = gv + tb;
              if constexpr (ACC == 2) tb = el(va[pp], k) + tb;
              el(ob, k) = tb;
            }
            if (ta.write_big) st4_nt(gbig + off, ob);
          }
        }
      }
      if constexpr (NEED_BIG) __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) red[q][4 * m + k] = s[k];
    __syncthreads();
    if (t < 64 && j0 + t < ta.K) {
      double tot = 0.0;
#pragma unroll
      for (int qq = 0; qq < 16; ++qq) tot += red[qq][t];
      part[p * ta.K + j0 + t] = tot;
    }
    __syncthreads();  // red and tile are rewritten by the next item
  }
}

// ----------------------------------------------------------- red_generic
// One thread per (kept element k, partial p); p covers a contiguous range of
// the row-major flattening of the reduced dims.  IDENT: the term is the
// source value itself (reduce_to_shape).
struct GenArgs {
  int32_t nk, nr;
  int64_t kn[kMaxDims], rn[kMaxDims];
  int64_t ks[3][kMaxDims], rs[3][kMaxDims];  // strides of src/g, a, b
  FastDiv kfd[kMaxDims], rfd[kMaxDims];      // divisors kn / rn (32-bit indexing)
  int64_t K, P, chunk, red;
};

// q = n / d and the remainder for the gather decodes: magic-number division
// on the 32-bit index path (every index < 2^31), plain division otherwise.
template <typename I>
__device__ __forceinline__ I gen_div(I n, int64_t d, const FastDiv &f) {
  if constexpr (sizeof(I) == 4) return (I)fdiv(f, (uint32_t)n);
  else return n / (I)d;
}

template <int OP, int EPI, int WHICH, int IDENT, typename I>
__global__ __launch_bounds__(kBlk) void k_red_generic(const float *g,
                                                      const float *a,
                                                      const float *b,
                                                      double *part, GenArgs ga) {
  for (int64_t gid64 = (int64_t)blockIdx.x * kBlk + threadIdx.x; gid64 < ga.K * ga.P;
       gid64 += (int64_t)gridDim.x * kBlk) {
    const I gid = (I)gid64;
    const I k = gid % (I)ga.K, p = gid / (I)ga.K;
    I og = 0, oa = 0, ob = 0;
    {
      I rest = k;
#pragma unroll
      for (int d = kMaxDims - 1; d >= 0; --d) {
        if (d < ga.nk) {
          const I n = (I)ga.kn[d];
          const I q = gen_div<I>(rest, ga.kn[d], ga.kfd[d]), c = rest - q * n;
          og += c * (I)ga.ks[0][d];
          oa += c * (I)ga.ks[1][d];
          ob += c * (I)ga.ks[2][d];
          rest = q;
        }
      }
    }
    const I lo = p * (I)ga.chunk;
    const I hi = lo + (I)ga.chunk < (I)ga.red ? lo + (I)ga.chunk : (I)ga.red;
    double s = 0.0;
    for (I tt = lo; tt < hi; ++tt) {
      I rest = tt, dg = 0, da = 0, db = 0;
#pragma unroll
      for (int d = kMaxDims - 1; d >= 0; --d) {
        if (d < ga.nr) {
          const I n = (I)ga.rn[d];
          const I q = gen_div<I>(rest, ga.rn[d], ga.rfd[d]), c = rest - q * n;
          dg += c * (I)ga.rs[0][d];
          da += c * (I)ga.rs[1][d];
          db += c * (I)ga.rs[2][d];
          rest = q;
        }
      }
      const float gv = g[og + dg];
      if constexpr (IDENT) {
        s += (double)gv;
      } else {
        const float x = reads_x<OP, EPI, WHICH>() ? a[oa + da] : 0.f;
        const float y = reads_y<OP, EPI, WHICH>() ? b[ob + db] : 0.f;
        s += term64<OP, EPI, WHICH>(gv, x, y);
      }
    }
    part[p * (I)ga.K + k] = s;
  }
}

// ------------------------------------------------------------- red_final
// out[k] = RN32(sum_p part[p][k] + acc[k]).  tpk (a power of two) threads
// per kept element; thread q owns partials p = q + j*tpk, loads up to 8 of
// them at once and adds them as a fixed tree, then the tpk subtotals meet in
// an LDS tree.  Adjacent threads own adjacent k, so loads are coalesced.
struct FinArgs {
  int64_t K, P, per;  // per: partials per thread
  int64_t ps, ks;     // partial p of kept element k at part[p * ps + k * ks]
  int32_t tpk, kt, has_acc;
  int32_t neg;  // the terms are the negated partials (exact)
  int32_t has_div;
  double div;  // has_div: the result is the sum divided by div (a mean)
};

__global__ __launch_bounds__(kBlk) void k_red_final(const double *part,
                                                    const float *acc,
                                                    float *out, FinArgs fa) {
  __shared__ double sh[kBlk];
  const int t = threadIdx.x;
  const int kk = t % fa.kt, q = t / fa.kt;
  const int64_t groups = (fa.K + fa.kt - 1) / fa.kt;
  for (int64_t kg = blockIdx.x; kg < groups; kg += gridDim.x) {
    const int64_t k = kg * fa.kt + kk;
    const bool ok = k < fa.K;
    double s = 0.0;
    for (int64_t j0 = 0; j0 < fa.per; j0 += 8) {
      double v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t p = q + (j0 + j) * fa.tpk;
        v[j] = (ok && j0 + j < fa.per && p < fa.P) ? part[p * fa.ps + k * fa.ks] : 0.0;
      }
      s += ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    }
    sh[t] = s;
    __syncthreads();
    for (int off = fa.tpk >> 1; off >= 1; off >>= 1) {
      if (q < off) sh[t] += sh[t + off * fa.kt];
      __syncthreads();
    }
    if (q == 0 && ok) {
      double tot = fa.neg ? -sh[kk] : sh[kk];
      if (fa.has_acc) tot += (double)acc[k];
      if (fa.has_div) tot = tot / fa.div;
      out[k] = (float)tot;
    }
    __syncthreads();  // sh is rewritten by the next group
  }
}

// Stage 2 when a kept element owns C consecutive columns of every partial
// row ([R1, K, C] -> [K, 1] walked as column sums of [R1, K * C]): out[k] =
// RN32(sum over p < P, c < C of part[p][k * C + c] (+ acc[k])).  tpk threads
// (a power of two) per kept element walk its P * C values v = p * C + c
// (thread q takes v = q + j * tpk, so adjacent threads read adjacent
// columns), add them in a fixed tree of eight, and the subtotals meet in an
// LDS tree.
struct FinColsArgs {
  int64_t K, P, C, per;  // per: values per thread
  int32_t tpk, kt, has_acc, neg, has_div;
  double div;
};

__global__ __launch_bounds__(kBlk) void k_red_final_cols(const double *part,
                                                         const float *acc, float *out,
                                                         FinColsArgs fa) {
  __shared__ double sh[kBlk];
  const int t = threadIdx.x;
  const int q = t % fa.tpk, kk = t / fa.tpk;
  const int64_t groups = (fa.K + fa.kt - 1) / fa.kt;
  const uint32_t V = (uint32_t)(fa.P * fa.C), C = (uint32_t)fa.C;  // V < 2^31 (planner)
  const int64_t row = fa.K * fa.C;
  for (int64_t kg = blockIdx.x; kg < groups; kg += gridDim.x) {
    const int64_t k = kg * fa.kt + kk;
    const bool ok = k < fa.K;
    double s = 0.0;
    for (int64_t j0 = 0; j0 < fa.per; j0 += 8) {
      double v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t vi = q + (j0 + j) * fa.tpk;
        v[j] = 0.0;
        if (ok && j0 + j < fa.per && vi < (int64_t)V) {
          const uint32_t pp = (uint32_t)vi / C, cc = (uint32_t)vi - pp * C;
          v[j] = part[(int64_t)pp * row + k * fa.C + cc];
        }
      }
      s += ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    }
    sh[t] = s;
    __syncthreads();
    for (int off = fa.tpk >> 1; off >= 1; off >>= 1) {
      if (q < off) sh[t] += sh[t + off];
      __syncthreads();
    }
    if (q == 0 && ok) {
      double tot = fa.neg ? -sh[t] : sh[t];
      if (fa.has_acc) tot += (double)acc[k];
      if (fa.has_div) tot = tot / fa.div;
      out[k] = (float)tot;
    }
    __syncthreads();  // sh is rewritten by the next group
  }
}

// ------------------------------------------------------------ bwd_signed
// gc[i] = sign * g[i] (+ acc[i]) over the dense output layout: the gradient
// of the second operator's c when no stage-1 kernel streams g for it.
template <int VEC>
__global__ __launch_bounds__(kBlk) void k_bwd_signed(const float *g, GcOut gco, int64_t n) {
  constexpr int64_t tile = (int64_t)kBlk * VEC;
  const int64_t ntiles = (n + tile - 1) / tile;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    if constexpr (VEC == 4) {
      const int64_t i = t * tile + (int64_t)threadIdx.x * 4;
      if (i + 4 <= n) {
        gc_store4(gco, i, ld4_nt(g + i));
      } else {
        for (int64_t j = i; j < n; ++j) gc_store1(gco, j, g[j]);
      }
    } else {
      const int64_t j = t * tile + threadIdx.x;
      if (j < n) gc_store1(gco, j, g[j]);
    }
  }
}

// -------------------------------------------------------------- launchers
// Grids are capped (a dispatch counts work-items with 32 bits); kernels
// launched through gridn loop over their work with a grid stride.
constexpr int64_t kMaxGrid = (int64_t)1 << 22;
static inline unsigned gridn(int64_t n, int64_t per) {
  const int64_t g = (n + per - 1) / per;
  return (unsigned)(g < kMaxGrid ? g : kMaxGrid);
}

// red_col waves per block, as planned (kColWavesFew / kColWavesMany).
template <class Fn>
static hipError_t with_col_waves(int nw, bool direct, Fn fn) {
  // the planner gives short columns (one partial) kColWavesFew waves
  if (direct) {
    if (nw == kColWavesFew) return fn(IC<kColWavesFew>{}, std::true_type{});
    return hipErrorInvalidValue;
  }
  switch (nw) {
    case 1: return fn(IC<1>{}, std::false_type{});
    case 4: return fn(IC<4>{}, std::false_type{});
    case 16: return fn(IC<16>{}, std::false_type{});
    default: return hipErrorInvalidValue;
  }
}

// Short columns finish in stage 1 (k_red_col with DIRECT).
static bool col_direct_plan(const RedPlan &rp) {
  return rp.kernel == K_RED_COL && rp.partials == 1 && rp.nw == kColWavesFew && rp.csub == 1;
}

// red_col's arguments for its plan: the [rows, cols] matrix, folded.
static ColArgs col_args(const RedPlan &rp, int64_t ss, bool write_big) {
  ColArgs ca{};
  ca.R = rp.col_rows / rp.fold;
  ca.K = rp.col_cols * rp.fold;
  ca.kmod = rp.col_cols;
  ca.rcw = rp.chunk;
  ca.ss = ss;
  ca.colblocks = (ca.K + 255) / 256;
  ca.bands = rp.partials / rp.fold;
  ca.write_big = write_big ? 1 : 0;
  return ca;
}

// One-pass row reduction (red_rowd): stage 1 and the final rounding.
template <int OP, int EPI, int S, int A>
static hipError_t launch_rowd(const RedPlan &rp, const Canon &c, int sw, const float *g,
                              const float *big, const float *small, float *gbig,
                              const float *accbig, float *out, const float *acc,
                              bool write_big, bool neg, double mean_count, GcOut go,
                              hipStream_t st) {
  if (rp.kept == 0) return hipSuccess;
  RowDirArgs ra{};
  const int R = c.rank;
  ra.R0 = c.n[R - 1];
  ra.K = rp.kept;
  ra.T = rp.red;
  ra.ss = (R >= 2 && small) ? c.s[1 + sw][R - 2] : 0;
  ra.write_big = write_big ? 1 : 0;
  ra.neg = neg ? 1 : 0;
  ra.has_div = mean_count >= 0.0 ? 1 : 0;
  ra.div = mean_count;
  const unsigned grid = gridn(rp.kept, 1);
  ProfScope prof(K_RED_ROWD);
  switch (rp.chunk) {
    case 1:
      ZK_LAUNCH(prof, (k_red_rowd<OP, EPI, S, A, 1>), dim3(grid), dim3(kDirBlk), 0, st, g, big,
                small, gbig, accbig, out, acc, ra, go);
      break;
    case 2:
      ZK_LAUNCH(prof, (k_red_rowd<OP, EPI, S, A, 2>), dim3(grid), dim3(kDirBlk), 0, st, g, big,
                small, gbig, accbig, out, acc, ra, go);
      break;
    case 4:
      ZK_LAUNCH(prof, (k_red_rowd<OP, EPI, S, A, 4>), dim3(grid), dim3(kDirBlk), 0, st, g, big,
                small, gbig, accbig, out, acc, ra, go);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

static hipError_t launch_final(const RedPlan &rp, const double *part,
                               const float *acc, float *out, hipStream_t st,
                               bool neg = false, double mean_count = -1.0) {
  if (rp.kept == 0) return hipSuccess;
  if (rp.csub > 1) {
    FinColsArgs fc{};
    fc.K = rp.kept;
    fc.P = rp.partials;
    fc.C = rp.csub;
    const int64_t V = fc.P * fc.C;
    int tpk = 1;
    while (tpk < kBlk && V > 8 * (int64_t)tpk) tpk *= 2;
    fc.tpk = tpk;
    fc.kt = kBlk / tpk;
    fc.per = (V + tpk - 1) / tpk;
    fc.has_acc = acc != nullptr;
    fc.neg = neg ? 1 : 0;
    fc.has_div = mean_count >= 0.0;
    fc.div = mean_count;
    ProfScope prof(K_RED_FINAL);
    ZK_LAUNCH(prof, k_red_final_cols, dim3(gridn(rp.kept, fc.kt)), dim3(kBlk), 0, st, part,
              acc, out, fc);
    return hipGetLastError();
  }
  FinArgs fa{};
  fa.neg = neg ? 1 : 0;
  fa.K = rp.kept;
  fa.P = rp.partials;
  // red_row writes its partials kept-element major ([K][P]), every other
  // stage 1 partial major ([P][K]).
  const bool kmajor = rp.kernel == K_RED_ROW;
  fa.ps = kmajor ? 1 : rp.kept;
  fa.ks = kmajor ? rp.partials : 1;
  // Threads per kept element: enough that each loads about 8 partials, but
  // for [P][K] at most 16 once there are many kept elements, so that a wave
  // still reads runs of >= 16 consecutive k (128 B) from each partial row
  // ([K][P] runs are contiguous for any count).
  const int max_tpk = (kmajor || rp.kept < 1024) ? 256 : 16;
  int tpk = 1;
  while (tpk < max_tpk && rp.partials > 8 * (int64_t)tpk) tpk *= 2;
  fa.tpk = tpk;
  fa.kt = kBlk / tpk;
  fa.per = (rp.partials + tpk - 1) / tpk;
  fa.has_acc = acc != nullptr;
  fa.has_div = mean_count >= 0.0;
  fa.div = mean_count;
  ProfScope prof(K_RED_FINAL);
  ZK_LAUNCH(prof, k_red_final, dim3(gridn(rp.kept, fa.kt)), dim3(kBlk), 0, st,
            part, acc, out, fa);
  return hipGetLastError();
}

// Split the canonical dims into kept / reduced lists for the gather kernel.
// kept_op: stride set of the reduced gradient (0 where reduced).
// ------------------------------------------------------------- red_gend
// Any reduction pattern in one pass when a kept element has 32..4096 terms:
// WPK waves per kept element (one wave, or the whole 4-wave block beyond
// 1024 terms) walk its terms (thread j takes terms j, j + 64 WPK, ...), decoding
// offsets as red_generic does, write the full-shape operand's gradient at
// the elements they visit when asked (each element of the output space
// belongs to exactly one kept element), and finish the sum themselves
// (sign, acc, divisor; rounded once): no partials, no stage 2, no separate
// element-wise pass.

// Terms per lane and trip, their loads issued together (rank-8 workload,
// 384 terms a kept element: 10.0 us with 2, 10.6 with 4, 11.3 with 8).
constexpr int kGendU = 2;

struct GenDirArgs {
  GenArgs ga;
  int32_t write_big, big_acc;  // big_acc: 0 none, 1 acc is g, 2 a buffer
  int32_t neg, has_div;
  double div;
};

template <int OP, int EPI, int WHICH, int IDENT, int WPK, typename I>
__global__ __launch_bounds__(kBlk) void k_red_gend(const float *g, const float *a,
                                                   const float *b, float *gbig,
                                                   const float *accbig, float *out,
                                                   const float *acc, GenDirArgs da) {
  const GenArgs &ga = da.ga;
  // operands either rule reads (the full operand's gradient may be written)
  constexpr bool RA = !IDENT && (reads_x<OP, EPI, 0>() || reads_x<OP, EPI, 1>());
  constexpr bool RB = !IDENT && (reads_y<OP, EPI, 0>() || reads_y<OP, EPI, 1>());
  constexpr int KPB = (kBlk / 64) / WPK;  // kept elements per block
  constexpr int TPK = 64 * WPK;           // threads per kept element
  __shared__ double sh[kBlk / 64];
  const int w = threadIdx.x >> 6;
  const int j = threadIdx.x % TPK;  // thread within its kept element
  auto decode_r = [&](I tt, I &dg, I &dA, I &dB) {
    I rest = tt;
    dg = 0;
    dA = 0;
    dB = 0;
#pragma unroll
    for (int d = kMaxDims - 1; d >= 0; --d) {
      if (d < ga.nr) {
        const I n = (I)ga.rn[d];
        const I q = gen_div<I>(rest, ga.rn[d], ga.rfd[d]), c = rest - q * n;
        dg += c * (I)ga.rs[0][d];
        dA += c * (I)ga.rs[1][d];
        dB += c * (I)ga.rs[2][d];
        rest = q;
      }
    }
  };
  for (int64_t kb = (int64_t)blockIdx.x * KPB; kb < ga.K; kb += (int64_t)gridDim.x * KPB) {
    const int64_t k64 = kb + threadIdx.x / TPK;
    const bool kok = k64 < ga.K;
    const I k = (I)(kok ? k64 : 0);
    I og = 0, oa = 0, ob = 0;
    {
      I rest = k;
#pragma unroll
      for (int d = kMaxDims - 1; d >= 0; --d) {
        if (d < ga.nk) {
          const I n = (I)ga.kn[d];
          const I q = gen_div<I>(rest, ga.kn[d], ga.kfd[d]), c = rest - q * n;
          og += c * (I)ga.ks[0][d];
          oa += c * (I)ga.ks[1][d];
          ob += c * (I)ga.ks[2][d];
          rest = q;
        }
      }
    }
    double s = 0.0;
    // kGendU terms per trip, their loads issued together
    for (I t0 = (I)j; kok && t0 < (I)ga.red; t0 += kGendU * TPK) {
      I ig[kGendU], ia[kGendU], ib[kGendU];
      float gv[kGendU], x[kGendU], y[kGendU];
      bool ok[kGendU];
#pragma unroll
      for (int u = 0; u < kGendU; ++u) {
        const I tt = t0 + (I)(u * TPK);
        ok[u] = tt < (I)ga.red;
        I dg, dA, dB;
        decode_r(ok[u] ? tt : (I)0, dg, dA, dB);
        ig[u] = og + dg;
        ia[u] = oa + dA;
        ib[u] = ob + dB;
      }
#pragma unroll
      for (int u = 0; u < kGendU; ++u) {
        if (ok[u]) {
          gv[u] = g[ig[u]];
          x[u] = RA ? a[ia[u]] : 0.f;
          y[u] = RB ? b[ib[u]] : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < kGendU; ++u) {
        if (!ok[u]) continue;
        if constexpr (IDENT) {
          s += (double)gv[u];
        } else {
          double ts;
          float tb;
          terms2<OP, EPI, WHICH>(gv[u], x[u], y[u], ts, tb);
          s += ts;
          if (da.write_big) {
            if (da.big_acc == 1) tb = gv[u] + tb;
            else if (da.big_acc == 2) tb = accbig[ig[u]] + tb;
            gbig[ig[u]] = tb;
          }
        }
      }
    }
    s = wave_sum(s);
    if constexpr (WPK > 1) {
      if ((threadIdx.x & 63) == 0) sh[w] = s;
      __syncthreads();
      s = 0.0;
#pragma unroll
      for (int q = 0; q < WPK; ++q) s += sh[q];
      __syncthreads();  // sh is rewritten for the next kept element
    }
    if (j == 0 && kok) {
      double tot = da.neg ? -s : s;
      if (acc) tot += (double)acc[k];
      if (da.has_div) tot = tot / da.div;
      out[k] = (float)tot;
    }
  }
}

// ------------------------------------------------------------ red_rowseg
// Sums of the rows of a dense [K, C], C = 4 * lpr <= 256 (lpr a power of
// two): a wave reads 256 consecutive elements a trip (64 / lpr whole rows, lpr
// lanes a row, one 128-bit vector a lane), adds each lane's four in binary64
// in a fixed order, then a row's lanes in a butterfly (every lane of the row
// ends with the same bits); the row's first lane writes the result, negated
// when asked, plus acc, divided by div for a mean (as k_red_final), rounded
// once.  With `part` the row sums are binary64 partials instead (row
// r1 * K + k is partial r1 of kept element k) for k_red_final.
struct RowSegArgs {
  int64_t K, C;     // K: rows
  int32_t lpr, lg;  // lanes per row and its log2
  int32_t neg, has_div;
  double div;
};

__global__ __launch_bounds__(kBlk) void k_red_rowseg(const float *in, const float *acc,
                                                     float *out, double *part,
                                                     RowSegArgs ra) {
  const int l = threadIdx.x & 63;
  const int g = l >> ra.lg, q = l & (ra.lpr - 1);
  const int64_t rpt = 64 >> ra.lg;  // rows a trip
  const int64_t trips = (ra.K + rpt - 1) / rpt;
  const int64_t nwaves = ((int64_t)gridDim.x * kBlk) >> 6;
  for (int64_t t = ((int64_t)blockIdx.x * kBlk + threadIdx.x) >> 6; t < trips; t += nwaves) {
    const int64_t row = t * rpt + g;
    double s = 0.0;
    if (row < ra.K) {
      const float4 v = ld4_nt(in + row * ra.C + 4 * q);
      s = (((double)v.x + (double)v.y) + (double)v.z) + (double)v.w;
    }
    for (int m = 1; m < ra.lpr; m <<= 1) s += __shfl_xor(s, m, 64);
    if (q == 0 && row < ra.K) {
      if (part) {
        part[row] = s;
      } else {
        double v = ra.neg ? -s : s;
        if (acc) v += (double)acc[row];
        if (ra.has_div) v = v / ra.div;
        out[row] = (float)v;
      }
    }
  }
}

static GenArgs make_gen(const Canon &c, int kept_op, int src_op, int a_op,
                        int b_op, const RedPlan &rp) {
  GenArgs ga{};
  for (int d = 0; d < c.rank; ++d) {
    const int ops[3] = {src_op, a_op, b_op};
    const uint32_t d32 = c.n[d] < ((int64_t)1 << 31) ? (uint32_t)c.n[d] : 1u;
    if (c.s[kept_op][d] != 0) {
      ga.kn[ga.nk] = c.n[d];
      ga.kfd[ga.nk] = make_fastdiv(d32);
      for (int o = 0; o < 3; ++o) ga.ks[o][ga.nk] = ops[o] >= 0 ? c.s[ops[o]][d] : 0;
      ++ga.nk;
    } else {
      ga.rn[ga.nr] = c.n[d];
      ga.rfd[ga.nr] = make_fastdiv(d32);
      for (int o = 0; o < 3; ++o) ga.rs[o][ga.nr] = ops[o] >= 0 ? c.s[ops[o]][d] : 0;
      ++ga.nr;
    }
  }
  ga.K = rp.kept;
  ga.P = rp.partials;
  ga.chunk = rp.chunk;
  ga.red = rp.red;
  return ga;
}

// One-pass gather reduction (red_gend).
static hipError_t launch_gend(const RedPlan &rp, const Canon &c, bool idx64, int kept_op,
                              int a_op, int b_op, zk_op op, zk_epi epi, bool ident, int which,
                              const float *g, const float *a, const float *b, float *gbig,
                              const float *accbig, int big_acc, bool write_big, float *out,
                              const float *acc, bool neg, double mean_count, hipStream_t st) {
  if (rp.kept == 0) return hipSuccess;
  GenDirArgs da{};
  da.ga = make_gen(c, kept_op, 0, a_op, b_op, rp);
  da.write_big = write_big ? 1 : 0;
  da.big_acc = big_acc;
  da.neg = neg ? 1 : 0;
  da.has_div = mean_count >= 0.0 ? 1 : 0;
  da.div = mean_count;
  // a wave per kept element up to 1024 terms (16 per lane), else the whole
  // block (rank-8 workload, 384 terms: 10.0 us with a wave, 10.8 with a block)
  const bool whole = rp.red > 1024;
  const unsigned grid = gridn(rp.kept, whole ? 1 : kBlk / 64);
  ProfScope prof(K_RED_GEND);
  auto go = [&](auto OPc, auto EPIc, auto Wc, auto IDc) -> hipError_t {
    constexpr int OP = decltype(OPc)::value, EPI = decltype(EPIc)::value;
    constexpr int W = decltype(Wc)::value, ID = decltype(IDc)::value;
    if (idx64) {
      if (whole)
        ZK_LAUNCH(prof, (k_red_gend<OP, EPI, W, ID, kBlk / 64, int64_t>), dim3(grid),
                  dim3(kBlk), 0, st, g, a, b, gbig, accbig, out, acc, da);
      else
        ZK_LAUNCH(prof, (k_red_gend<OP, EPI, W, ID, 1, int64_t>), dim3(grid), dim3(kBlk), 0,
                  st, g, a, b, gbig, accbig, out, acc, da);
    } else {
      if (whole)
        ZK_LAUNCH(prof, (k_red_gend<OP, EPI, W, ID, kBlk / 64, int32_t>), dim3(grid),
                  dim3(kBlk), 0, st, g, a, b, gbig, accbig, out, acc, da);
      else
        ZK_LAUNCH(prof, (k_red_gend<OP, EPI, W, ID, 1, int32_t>), dim3(grid), dim3(kBlk), 0,
                  st, g, a, b, gbig, accbig, out, acc, da);
    }
    return hipGetLastError();
  };
  if (ident) return go(IC<ZK_ADD>{}, IC<ZK_EPI_NONE>{}, IC<1>{}, IC<1>{});
  return op_epi(op, epi, [&](auto OPc, auto EPIc) -> hipError_t {
    return which == 0 ? go(OPc, EPIc, IC<0>{}, IC<0>{}) : go(OPc, EPIc, IC<1>{}, IC<0>{});
  });
}

// -------------------------------------------------------------- red_run
// A reduction whose two innermost canonical dims form a short contiguous run
// (L = n0 * n1 elements, 64..256, any mix of kept and reduced) that the
// source and the full operand walk densely, e.g. the rank-8 pattern
// [2,3,4,5,6,7,8,9] -> [1,3,1,5,1,7,1,9] (run [8, 9]: 8 reduced x 9 kept).
// Block kb owns one combination of the outer kept dims and walks every
// combination of the outer reduced dims (a run each), 1024 / L runs at a time:
// lane j of a run slot reads element j of each of its runs, so every element
// is read once, in whole contiguous runs, and a lane always holds the same
// kept element (its run coordinates' kept part).  The block then adds, for
// each of its Kin kept elements, the lanes holding it in a fixed order (run
// coordinates within each slot, then the slots), finishes the sum (sign,
// acc, divisor; rounded once) and writes it: no partials, no stage 2.  The full operand's
// gradient is written at every element read.  32-bit offsets (numel < 2^31).
struct RunArgs {
  int32_t nk, nr;                                   // outer kept / reduced dims
  uint32_t kn[kMaxDims], rn[kMaxDims];              // (outer -> inner)
  FastDiv kfd[kMaxDims], rfd[kMaxDims];
  int32_t kg[kMaxDims], ksm[kMaxDims], kout[kMaxDims];  // kept dims: source, small, result strides
  int32_t rg[kMaxDims];                             // reduced dims: source strides
  int32_t n0, n1, k0, k1;                           // the run's dims, kept flags
  int32_t sm0, sm1, out0, out1;                     // small / result strides on the run
  int32_t blocks, runs, slots;
  int32_t write_big, big_acc;                       // big_acc: 0 none, 1 acc is g, 2 a buffer
  int32_t neg, has_div;
  double div;
};
constexpr int kRunU = 4;       // runs a lane has in flight
constexpr int kRunBlk = 1024;  // lanes a block: the rank-8 pattern's 48 runs of 72 in one
                               // round of loads (14 at once, 4 deep), 105 blocks

template <int OP, int EPI, int WHICH, int IDENT>
__global__ __launch_bounds__(kRunBlk) void k_red_run(const float *g, const float *a,
                                                  const float *b, float *gbig,
                                                  const float *accbig, float *out,
                                                  const float *acc, RunArgs ra) {
  constexpr bool RA = !IDENT && (reads_x<OP, EPI, 0>() || reads_x<OP, EPI, 1>());
  constexpr bool RB = !IDENT && (reads_y<OP, EPI, 0>() || reads_y<OP, EPI, 1>());
  constexpr bool R_SMALL = WHICH == 0 ? RA : RB;
  constexpr bool R_BIG = WHICH == 0 ? RB : RA;
  const float *small = WHICH == 0 ? a : b;
  const float *big = WHICH == 0 ? b : a;
  __shared__ double sh[kRunBlk];
  const int t = threadIdx.x;
  const int L = ra.n0 * ra.n1;
  const int slot = t / L, j = t - slot * L;
  const bool on = slot < ra.slots;
  const int j0 = j / ra.n1, j1 = j - j0 * ra.n1;
  const int kin = (ra.k0 ? ra.n0 : 1) * (ra.k1 ? ra.n1 : 1);
  for (int kb = blockIdx.x; kb < ra.blocks; kb += gridDim.x) {
    int og = 0, osm = 0, oout = 0;
    {
      uint32_t rest = (uint32_t)kb;
#pragma unroll
      for (int d = kMaxDims - 1; d >= 0; --d) {
        if (d < ra.nk) {
          const uint32_t q = fdiv(ra.kfd[d], rest), c = rest - q * ra.kn[d];
          og += (int)c * ra.kg[d];
          osm += (int)c * ra.ksm[d];
          oout += (int)c * ra.kout[d];
          rest = q;
        }
      }
    }
    float sv = 0.f;
    if (R_SMALL && on) sv = small[osm + j0 * ra.sm0 + j1 * ra.sm1];
    double s = 0.0;
    if (on) {
      for (int r0 = slot; r0 < ra.runs; r0 += ra.slots * kRunU) {
        int idx[kRunU];
        float gv[kRunU], bv[kRunU];
#pragma unroll
        for (int u = 0; u < kRunU; ++u) {
          const int r = r0 + u * ra.slots;
          idx[u] = -1;
          if (r < ra.runs) {
            uint32_t rest = (uint32_t)r;
            int off = og + j;  // the run is dense in the source
#pragma unroll
            for (int d = kMaxDims - 1; d >= 0; --d) {
              if (d < ra.nr) {
                const uint32_t q = fdiv(ra.rfd[d], rest), c = rest - q * ra.rn[d];
                off += (int)c * ra.rg[d];
                rest = q;
              }
            }
            idx[u] = off;
          }
        }
#pragma unroll
        for (int u = 0; u < kRunU; ++u) {
          if (idx[u] >= 0) {
            gv[u] = g[idx[u]];
            bv[u] = R_BIG ? big[idx[u]] : 0.f;
          }
        }
#pragma unroll
        for (int u = 0; u < kRunU; ++u) {
          if (idx[u] < 0) continue;
          if constexpr (IDENT) {
            s += (double)gv[u];
          } else {
            const float x = WHICH == 0 ? sv : bv[u];
            const float y = WHICH == 0 ? bv[u] : sv;
            double ts;
            float tb;
            terms2<OP, EPI, WHICH>(gv[u], x, y, ts, tb);
            s += ts;
            if (ra.write_big) {
              if (ra.big_acc == 1) tb = gv[u] + tb;
              else if (ra.big_acc == 2) tb = accbig[idx[u]] + tb;
              gbig[idx[u]] = tb;
            }
          }
        }
      }
    }
    sh[t] = s;
    __syncthreads();
    // Two fixed-order levels: lane (slot, kept element) adds the run lanes of
    // its slot holding that element, then one lane per kept element adds
    // the slots' subtotals in slot order.
    const int na = ra.slots * kin;
    double v = 0.0;
    int t0 = 0, t1 = 0;  // the kept element's run coordinates
    if (t < na) {
      const int sl = t / kin, tk = t - sl * kin;
      if (ra.k0 && ra.k1) {
        t0 = tk / ra.n1;
        t1 = tk - t0 * ra.n1;
      } else if (ra.k0) {
        t0 = tk;
      } else if (ra.k1) {
        t1 = tk;
      }
      const double *row = sh + sl * L;
      if (ra.k0 && ra.k1) {
        v = row[t0 * ra.n1 + t1];
      } else if (ra.k1) {
        for (int u0 = 0; u0 < ra.n0; ++u0) v += row[u0 * ra.n1 + t1];
      } else if (ra.k0) {
        for (int u1 = 0; u1 < ra.n1; ++u1) v += row[t0 * ra.n1 + u1];
      } else {
        for (int u = 0; u < L; ++u) v += row[u];
      }
    }
    __syncthreads();
    if (t < na) sh[t] = v;
    __syncthreads();
    if (t < kin) {
      double tot = 0.0;
      for (int sl = 0; sl < ra.slots; ++sl) tot += sh[sl * kin + t];
      const int k = oout + t0 * ra.out0 + t1 * ra.out1;
      if (ra.neg) tot = -tot;
      if (acc) tot += (double)acc[k];
      if (ra.has_div) tot = tot / ra.div;
      out[k] = (float)tot;
    }
    __syncthreads();  // sh is rewritten for the next block of kept elements
  }
}

// One-pass run reduction (red_run).  kept_op: the reduced gradient's stride
// set; small_op: the reduced operand's own strides (-1: none is read).
static hipError_t launch_run(const RedPlan &rp, const Canon &c, int kept_op, int small_op,
                             zk_op op, zk_epi epi, bool ident, int which, const float *g,
                             const float *a, const float *b, float *gbig, const float *accbig,
                             int big_acc, bool write_big, float *out, const float *acc,
                             bool neg, double mean_count, hipStream_t st) {
  if (rp.kept == 0) return hipSuccess;
  RunArgs ra{};
  const int R = c.rank;
  int64_t blocks = 1, runs = 1;
  for (int d = 0; d < R - 2; ++d) {
    const uint32_t n = (uint32_t)c.n[d];
    if (c.s[kept_op][d] != 0) {
      ra.kn[ra.nk] = n;
      ra.kfd[ra.nk] = make_fastdiv(n);
      ra.kg[ra.nk] = (int32_t)c.s[0][d];
      ra.ksm[ra.nk] = small_op >= 0 ? (int32_t)c.s[small_op][d] : 0;
      ra.kout[ra.nk] = (int32_t)c.s[kept_op][d];
      ++ra.nk;
      blocks *= n;
    } else {
      ra.rn[ra.nr] = n;
      ra.rfd[ra.nr] = make_fastdiv(n);
      ra.rg[ra.nr] = (int32_t)c.s[0][d];
      ++ra.nr;
      runs *= n;
    }
  }
  ra.n0 = (int32_t)c.n[R - 2];
  ra.n1 = (int32_t)c.n[R - 1];
  ra.k0 = c.s[kept_op][R - 2] != 0;
  ra.k1 = c.s[kept_op][R - 1] != 0;
  ra.sm0 = small_op >= 0 ? (int32_t)c.s[small_op][R - 2] : 0;
  ra.sm1 = small_op >= 0 ? (int32_t)c.s[small_op][R - 1] : 0;
  ra.out0 = (int32_t)c.s[kept_op][R - 2];
  ra.out1 = (int32_t)c.s[kept_op][R - 1];
  ra.blocks = (int32_t)blocks;
  ra.runs = (int32_t)runs;
  ra.slots = kRunBlk / (ra.n0 * ra.n1);
  if (ra.slots < 1 || c.s[0][R - 1] != 1 || c.s[0][R - 2] != ra.n1) return hipErrorInvalidValue;
  ra.write_big = write_big ? 1 : 0;
  ra.big_acc = big_acc;
  ra.neg = neg ? 1 : 0;
  ra.has_div = mean_count >= 0.0 ? 1 : 0;
  ra.div = mean_count;
  const unsigned grid = gridn(blocks, 1);
  ProfScope prof(K_RED_RUN);
  auto go = [&](auto OPc, auto EPIc, auto Wc, auto IDc) -> hipError_t {
    constexpr int OP = decltype(OPc)::value, EPI = decltype(EPIc)::value;
    constexpr int W = decltype(Wc)::value, ID = decltype(IDc)::value;
    ZK_LAUNCH(prof, (k_red_run<OP, EPI, W, ID>), dim3(grid), dim3(kRunBlk), 0, st, g, a, b, gbig,
              accbig, out, acc, ra);
    return hipGetLastError();
  };
  if (ident) return go(IC<ZK_ADD>{}, IC<ZK_EPI_NONE>{}, IC<1>{}, IC<1>{});
  return op_epi(op, epi, [&](auto OPc, auto EPIc) -> hipError_t {
    return which == 0 ? go(OPc, EPIc, IC<0>{}, IC<0>{}) : go(OPc, EPIc, IC<1>{}, IC<0>{});
  });
}

static int acc_mode(const float *acc, const float *g) {
  if (!acc) return 0;
  return acc == g ? 1 : 2;
}

static bool al16p(const void *q) { return ((uintptr_t)q & 15u) == 0; }

hipError_t launch_signed(const float *g, int64_t n, float *gc, const float *acc,
                         float sign, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const GcOut gco{gc, acc, sign};
  ProfScope prof(K_BWD_SIGNED);
  if (al16p(g) && al16p(gc) && al16p(acc))
    ZK_LAUNCH(prof, (k_bwd_signed<4>), dim3(gridn(n, kBlk * 4)), dim3(kBlk), 0, st, g, gco, n);
  else
    ZK_LAUNCH(prof, (k_bwd_signed<1>), dim3(gridn(n, kBlk)), dim3(kBlk), 0, st, g, gco, n);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdPlan &p, zk_op op, zk_epi epi, const float *g,
                      const float *a, const float *b, float *grad_a,
                      const float *acc_a, float *grad_b, const float *acc_b,
                      void *ws, hipStream_t st, float *grad_c, const float *acc_c,
                      float c_sign, const ScalarArg *sa) {
  const Canon &c = p.c;
  hipError_t e = hipSuccess;
  // The c gradient of the fused backward rides along with the first stage-1
  // kernel that streams all of g in the output layout with 128-bit accesses
  // (or any layout for the scalar element-wise kernel); otherwise it gets a
  // pass of its own at the end.
  bool gc_done = grad_c == nullptr;
  const bool gc_al = al16p(grad_c) && al16p(acc_c);
  // Element-wise gradients of full-shape operands.
  if (p.ew_kernel != K_NONE) {
    EwArgs ea{};
    ea.n = c.numel;
    ea.write_a = p.ew_write[0];
    ea.write_b = p.ew_write[1];
    ea.acc_a = ea.write_a ? acc_mode(acc_a, g) : 0;
    ea.acc_b = ea.write_b ? acc_mode(acc_b, g) : 0;
    ea.read_a = (ea.write_a && rule_reads_a(op, epi, 0)) || (ea.write_b && rule_reads_a(op, epi, 1));
    ea.read_b = (ea.write_a && rule_reads_b(op, epi, 0)) || (ea.write_b && rule_reads_b(op, epi, 1));
    if (sa) {
      ea.a_arg = sa->side == 0;
      ea.b_arg = sa->side == 1;
      ea.av = ea.bv = sa->value;
    }
    e = op_epi(op, epi, [&](auto OPc, auto EPIc) -> hipError_t {
      constexpr int OP = decltype(OPc)::value;
      constexpr int EPI = decltype(EPIc)::value;
      ProfScope prof(p.ew_kernel);
      if (p.ew_kernel == K_BWD_EW_FLAT) {
        GcOut go{nullptr, nullptr, c_sign};
        if (!gc_done && (p.vec == 1 || gc_al)) {
          go = GcOut{grad_c, acc_c, c_sign};
          gc_done = true;
        }
        if constexpr (EPI == ZK_EPI_NONE && (OP == ZK_ADD || OP == ZK_SUB)) {
          // one pass-through gradient: k_bwd_pass
          const bool wa = ea.write_a != 0;
          float *out = wa ? grad_a : grad_b;
          const float *acc = wa ? acc_a : acc_b;
          const int am = wa ? ea.acc_a : ea.acc_b;
          if (ea.write_a != ea.write_b && !sa && go.p == nullptr && am != 1 &&
              c.numel < ((int64_t)1 << 31) && al16p(g) && al16p(out) && (am == 0 || al16p(acc))) {
            const bool neg = OP == ZK_SUB && !wa;
            const dim3 grid(gridn(c.numel, kBlk * 4));
            const int32_t n = (int32_t)c.numel;
            if (neg && am == 2)
              ZK_LAUNCH(prof, (k_bwd_pass<true, true>), grid, dim3(kBlk), 0, st, g, acc, out, n);
            else if (neg)
              ZK_LAUNCH(prof, (k_bwd_pass<true, false>), grid, dim3(kBlk), 0, st, g, acc, out, n);
            else if (am == 2)
              ZK_LAUNCH(prof, (k_bwd_pass<false, true>), grid, dim3(kBlk), 0, st, g, acc, out, n);
            else
              ZK_LAUNCH(prof, (k_bwd_pass<false, false>), grid, dim3(kBlk), 0, st, g, acc, out, n);
            return hipGetLastError();
          }
        }
        if (p.vec == 4)
          ZK_LAUNCH(prof, (k_bwd_ew_flat<OP, EPI, 4>), dim3(gridn(c.numel, kBlk * 4)),
                    dim3(kBlk), 0, st, g, a, b, grad_a, acc_a, grad_b, acc_b, ea, go);
        else
          ZK_LAUNCH(prof, (k_bwd_ew_flat<OP, EPI, 1>), dim3(gridn(c.numel, kBlk)),
                    dim3(kBlk), 0, st, g, a, b, grad_a, acc_a, grad_b, acc_b, ea, go);
      } else {
        Space sp = make_space(c);
        if (p.idx64)
          ZK_LAUNCH(prof, (k_bwd_ew_generic<OP, EPI, int64_t>), dim3(gridn(c.numel, kBlk * 4)),
                    dim3(kBlk), 0, st, g, a, b, grad_a, acc_a, grad_b, acc_b, ea, sp);
        else
          ZK_LAUNCH(prof, (k_bwd_ew_generic<OP, EPI, int32_t>), dim3(gridn(c.numel, kBlk * 4)),
                    dim3(kBlk), 0, st, g, a, b, grad_a, acc_a, grad_b, acc_b, ea, sp);
      }
      return hipGetLastError();
    });
    if (e != hipSuccess) return e;
  }
  for (int ri = 0; ri < p.nred; ++ri) {
    const RedPlan &rp = p.red[ri];
    const int sw = rp.which, bw = 1 - rp.which;
    double *part = reinterpret_cast<double *>(static_cast<char *>(ws) + rp.ws_offset);
    const float *small = sw == 0 ? a : b;
    const float *big = sw == 0 ? b : a;
    float *gsmall = sw == 0 ? grad_a : grad_b;
    float *gbig = sw == 0 ? grad_b : grad_a;
    const float *accsmall = sw == 0 ? acc_a : acc_b;
    const float *accbig = sw == 0 ? acc_b : acc_a;
    const int amode = p.fused_big ? acc_mode(accbig, g) : 0;
    // red_col and red_row stream all of g in the output layout
    GcOut go{nullptr, nullptr, c_sign};
    if (!gc_done && gc_al &&
        ((rp.partials > 0 && (rp.kernel == K_RED_COL || rp.kernel == K_RED_ROW)) ||
         (rp.kernel == K_RED_ROWD && rp.kept > 0))) {
      go = GcOut{grad_c, acc_c, c_sign};
      gc_done = true;
    }
    if (rp.kernel == K_RED_RUN) {
      e = launch_run(rp, c, 3 + sw, 1 + sw, op, epi, false, sw, g, a, b, gbig, accbig,
                     p.fused_big ? acc_mode(accbig, g) : 0, p.fused_big, gsmall, accsmall, false,
                     -1.0, st);
      if (e != hipSuccess) return e;
      continue;
    }
    if (rp.kernel == K_RED_GEND) {
      e = launch_gend(rp, c, p.idx64, 3 + sw, 1, 2, op, epi, false, sw, g, a, b, gbig, accbig,
                      p.fused_big ? acc_mode(accbig, g) : 0, p.fused_big, gsmall, accsmall,
                      false, -1.0, st);
      if (e != hipSuccess) return e;
      continue;
    }
    if (rp.kernel == K_RED_ROWD) {
      e = op_epi(op, epi, [&](auto OPc, auto EPIc) -> hipError_t {
        constexpr int OP = decltype(OPc)::value;
        constexpr int EPI = decltype(EPIc)::value;
        return side_acc(sw, amode, [&](auto Sc, auto Ac) -> hipError_t {
          return launch_rowd<OP, EPI, decltype(Sc)::value, decltype(Ac)::value>(
              rp, c, sw, g, big, small, gbig, accbig, gsmall, accsmall, p.fused_big, false,
              -1.0, go, st);
        });
      });
      if (e != hipSuccess) return e;
      continue;
    }
    if (rp.partials > 0) {
      e = op_epi(op, epi, [&](auto OPc, auto EPIc) -> hipError_t {
        constexpr int OP = decltype(OPc)::value;
        constexpr int EPI = decltype(EPIc)::value;
        ProfScope prof(rp.kernel);
        switch (rp.kernel) {
          case K_RED_COL: {
            const ColArgs ca = col_args(rp, c.s[1 + sw][1], p.fused_big);
            ColDirect cd{gsmall, accsmall, 0, 0, 0.0};
            const unsigned grid = gridn(ca.colblocks * ca.bands, 1);
            return side_acc(sw, amode, [&](auto Sc, auto Ac) -> hipError_t {
              constexpr int S = decltype(Sc)::value, A = decltype(Ac)::value;
              return with_col_waves(rp.nw, col_direct_plan(rp), [&](auto Wc, auto Dc) {
                constexpr int NW = decltype(Wc)::value;
                constexpr bool D = decltype(Dc)::value;
                if constexpr (col_interleaved<OP, EPI, S, NW>()) {
                  if (ca.write_big) {
                    ZK_LAUNCH(prof, (k_red_col<OP, EPI, S, A, NW, D, true>), dim3(grid),
                              dim3(64 * NW), 0, st, g, big, small, gbig, accbig, part, ca, go, cd);
                    return hipGetLastError();
                  }
                }
                ZK_LAUNCH(prof, (k_red_col<OP, EPI, S, A, NW, D, false>), dim3(grid), dim3(64 * NW),
                          0, st, g, big, small, gbig, accbig, part, ca, go, cd);
                return hipGetLastError();
              });
            });
          }
          case K_RED_ROW: {
            RowRedArgs ra{};
            const int R = c.rank;
            ra.R0 = c.n[R - 1];
            ra.K = rp.kept;
            ra.CL = rp.chunk;
            ra.NC = (ra.R0 + ra.CL - 1) / ra.CL;
            ra.items = (c.numel / ra.R0) * ra.NC;
            ra.P = rp.partials;
            ra.ss = R >= 2 ? c.s[1 + sw][R - 2] : 0;
            ra.write_big = p.fused_big;
            // blockwise partials need four chunks a row (the planner's rule)
            if (rp.nw == 4 && ra.NC % 4 != 0) return hipErrorInvalidValue;
            unsigned grid = gridn(ra.items, 4);
            return side_acc(sw, amode, [&](auto Sc, auto Ac) -> hipError_t {
              constexpr int S = decltype(Sc)::value, A = decltype(Ac)::value;
              if (rp.nw == 4)
                ZK_LAUNCH(prof, (k_red_row<OP, EPI, S, A, true>), dim3(grid), dim3(kBlk), 0, st,
                          g, big, small, gbig, accbig, part, ra, go);
              else
                ZK_LAUNCH(prof, (k_red_row<OP, EPI, S, A, false>), dim3(grid), dim3(kBlk), 0, st,
                          g, big, small, gbig, accbig, part, ra, go);
              return hipGetLastError();
            });
          }
          case K_RED_TILE: {
            TileRedArgs ta{};
            ta.R = c.n[0];
            ta.K = c.n[1];
            ta.ld = c.s[1 + bw][1];
            ta.ss = c.s[1 + sw][1];
            ta.rc = rp.chunk;
            ta.tiles_c = (ta.K + 63) / 64;
            ta.items = ta.tiles_c * rp.partials;
            ta.write_big = p.fused_big;
            ta.tv = ta.ld % 4 == 0 && ((uintptr_t)big & 15u) == 0;
            unsigned grid = gridn(ta.items, 1);
            return side_acc(sw, amode, [&](auto Sc, auto Ac) -> hipError_t {
              ZK_LAUNCH(prof, (k_red_tile<OP, EPI, decltype(Sc)::value, decltype(Ac)::value>),
                        dim3(grid), dim3(kBlk), 0, st, g, big, small, gbig, accbig,
                        part, ta);
              return hipGetLastError();
            });
          }
          default: {
            GenArgs ga = make_gen(c, 3 + sw, 0, 1, 2, rp);
            unsigned grid = gridn(rp.kept * rp.partials, kBlk);
            if (sw == 0) {
              if (p.idx64)
                ZK_LAUNCH(prof, (k_red_generic<OP, EPI, 0, 0, int64_t>), dim3(grid), dim3(kBlk),
                          0, st, g, a, b, part, ga);
              else
                ZK_LAUNCH(prof, (k_red_generic<OP, EPI, 0, 0, int32_t>), dim3(grid), dim3(kBlk),
                          0, st, g, a, b, part, ga);
            } else {
              if (p.idx64)
                ZK_LAUNCH(prof, (k_red_generic<OP, EPI, 1, 0, int64_t>), dim3(grid), dim3(kBlk),
                          0, st, g, a, b, part, ga);
              else
                ZK_LAUNCH(prof, (k_red_generic<OP, EPI, 1, 0, int32_t>), dim3(grid), dim3(kBlk),
                          0, st, g, a, b, part, ga);
            }
            return hipGetLastError();
          }
        }
      });
      if (e != hipSuccess) return e;
    }
    if (col_direct_plan(rp)) continue;  // finished in stage 1
    e = launch_final(rp, part, accsmall, gsmall, st);
    if (e != hipSuccess) return e;
  }
  if (!gc_done) return launch_signed(g, c.numel, grad_c, acc_c, c_sign, st);
  return hipSuccess;
}

hipError_t launch_reduce(const BwdPlan &p, const float *in, float *out,
                         void *ws, hipStream_t st, const float *acc, bool neg,
                         double mean_count) {
  const GcOut none{nullptr, nullptr, 1.f};
  const Canon &c = p.c;
  for (int ri = 0; ri < p.nred; ++ri) {
    const RedPlan &rp = p.red[ri];
    double *part = reinterpret_cast<double *>(static_cast<char *>(ws) + rp.ws_offset);
    if (rp.kernel == K_RED_ROWSEG) {
      RowSegArgs ra{};
      ra.K = c.numel / rp.chunk;  // rows
      ra.C = rp.chunk;
      ra.lpr = (int32_t)(rp.chunk / 4);
      while ((1 << ra.lg) < ra.lpr) ++ra.lg;
      if ((1 << ra.lg) != ra.lpr || ra.lpr > 64) return hipErrorInvalidValue;
      ra.neg = neg ? 1 : 0;
      ra.has_div = mean_count >= 0.0 ? 1 : 0;
      ra.div = mean_count;
      const int64_t trips = (ra.K + (64 >> ra.lg) - 1) / (64 >> ra.lg);
      {
        ProfScope prof(K_RED_ROWSEG);
        ZK_LAUNCH(prof, k_red_rowseg, dim3(gridn(trips, kBlk / 64)), dim3(kBlk), 0, st, in,
                  acc, out, rp.partials > 0 ? part : nullptr, ra);
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      if (rp.partials > 0) {
        e = launch_final(rp, part, acc, out, st, neg, mean_count);
        if (e != hipSuccess) return e;
      }
      continue;
    }
    if (rp.kernel == K_RED_RUN) {
      hipError_t e = launch_run(rp, c, 4, -1, ZK_ADD, ZK_EPI_NONE, true, 1, in, nullptr, nullptr,
                                nullptr, nullptr, 0, false, out, acc, neg, mean_count, st);
      if (e != hipSuccess) return e;
      continue;
    }
    if (rp.kernel == K_RED_GEND) {
      hipError_t e = launch_gend(rp, c, p.idx64, 4, -1, -1, ZK_ADD, ZK_EPI_NONE, true, 1, in,
                                 nullptr, nullptr, nullptr, nullptr, 0, false, out, acc, neg,
                                 mean_count, st);
      if (e != hipSuccess) return e;
      continue;
    }
    if (rp.kernel == K_RED_ROWD) {
      hipError_t e = launch_rowd<ZK_ADD, ZK_EPI_NONE, 1, 0>(rp, c, 1, in, nullptr, nullptr,
                                                            nullptr, nullptr, out, acc, false,
                                                            neg, mean_count, none, st);
      if (e != hipSuccess) return e;
      continue;
    }
    if (rp.partials > 0) {
      ProfScope prof(rp.kernel);
      switch (rp.kernel) {
        case K_RED_COL: {
          const ColArgs ca = col_args(rp, 0, false);
          const ColDirect cd{out, acc, neg ? 1 : 0, mean_count >= 0.0 ? 1 : 0, mean_count};
          const unsigned grid = gridn(ca.colblocks * ca.bands, 1);
          hipError_t e = with_col_waves(rp.nw, col_direct_plan(rp), [&](auto Wc, auto Dc) {
            constexpr int NW = decltype(Wc)::value;
            constexpr bool D = decltype(Dc)::value;
            ZK_LAUNCH(prof, (k_red_col<ZK_ADD, ZK_EPI_NONE, 1, 0, NW, D, false>), dim3(grid),
                      dim3(64 * NW), 0, st, in, nullptr, nullptr, nullptr, nullptr, part, ca,
                      none, cd);
            return hipGetLastError();
          });
          if (e != hipSuccess) return e;
          break;
        }
        case K_RED_ROW: {
          RowRedArgs ra{};
          const int R = c.rank;
          ra.R0 = c.n[R - 1];
          ra.K = rp.kept;
          ra.CL = rp.chunk;
          ra.NC = (ra.R0 + ra.CL - 1) / ra.CL;
          ra.items = (c.numel / ra.R0) * ra.NC;
          ra.P = rp.partials;
          ra.ss = 0;
          ra.write_big = 0;
          ZK_LAUNCH(prof, (k_red_row<ZK_ADD, ZK_EPI_NONE, 1, 0, false>), dim3(gridn(ra.items, 4)),
                    dim3(kBlk), 0, st, in, nullptr, nullptr, nullptr, nullptr, part, ra, none);
          break;
        }
        default: {
          GenArgs ga = make_gen(c, 4, 0, -1, -1, rp);
          unsigned grid = gridn(rp.kept * rp.partials, kBlk);
          if (p.idx64)
            ZK_LAUNCH(prof, (k_red_generic<ZK_ADD, ZK_EPI_NONE, 1, 1, int64_t>), dim3(grid),
                      dim3(kBlk), 0, st, in, nullptr, nullptr, part, ga);
          else
            ZK_LAUNCH(prof, (k_red_generic<ZK_ADD, ZK_EPI_NONE, 1, 1, int32_t>), dim3(grid),
                      dim3(kBlk), 0, st, in, nullptr, nullptr, part, ga);
        }
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (col_direct_plan(rp)) continue;  // finished in stage 1
    hipError_t e = launch_final(rp, part, acc, out, st, neg, mean_count);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace zk
