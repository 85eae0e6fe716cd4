/*
 * oracle.c -- plain, slow CPU oracle for broadcasting binary operators and
 * their backward.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and
 * the benchmark's CPU-baseline leg call it; the product library never does.
 * It shares no code, header or constant with the HIP library.
 *
 * What it computes follows the "Zero" book (ismantic.github.io/zero):
 *   - strides count elements, offset = sum_k i_k * s_k
 *       (Tensor chapter, "shape and strides" section)
 *   - broadcast shape: right-align, each dim equal / one is 1 / one missing
 *       (Operator chapter, "broadcast" section)
 *   - broadcast forward: a size-1 input dim always reads coordinate 0
 *       (Operator chapter, "broadcast" section)
 *   - element-wise rules z = x*y -> (g*y, g*x); add passes g to both inputs
 *       (Autograd chapter, "chain rule"; GPU chapter, "OpAdd" walkthrough)
 *   - a broadcast input's gradient is the sum of the upstream gradient over
 *     every output position it was repeated into; a tensor reached along
 *     several paths gets the sum of the path gradients
 *       (Operator chapter, "broadcast"; Autograd chapter, "chain rule")
 * sub and div rules are not printed there; they are plain calculus.
 *   - a fused operator merges several operators into one unit without
 *     changing their math (Operator chapter, "fusion" section): the fused
 *     expression (a op1 b) op2 c is computed here as the two operators one
 *     after the other
 *   - the mean, and the global L2 norm of all parameter gradients with the
 *     ClipGradNorm scaling g <- g * c / (||g||_2 + 1e-6) applied when the
 *     norm exceeds c (GPU chapter, "reduction"; GPT chapter, "training loop")
 *
 * Precision (the pages fix none):
 *   forward  : one IEEE binary32 operation per element, round-to-nearest-even
 *              (built with -ffp-contract=off, SSE, no fast-math)
 *   GeLU     : exact function h*Phi(h), Phi(h) = erfc(-h/sqrt2)/2, correctly
 *              rounded to binary32: evaluated in binary64 with libm erfc, and
 *              again in binary128 (libquadmath) where the binary64 value cannot
 *              decide the rounding (near a binary32 midpoint, or a result
 *              below 2^-125)
 *   ReLU     : h for h > 0, NaN for NaN, +0 otherwise; derivative 1 for h > 0,
 *              else 0 (the pages name the activation without a formula)
 *   backward : every term in binary64 from the exact binary32 inputs, summed in
 *              binary64 in row-major index order, rounded once to binary32;
 *              the sum of |terms| is returned beside it for the tolerance.
 *   mean     : the binary64 sum divided by the count in binary64, rounded once;
 *              its gradient g / count is one binary32 division by the count
 *              rounded to binary32
 *   L2 norm  : squares summed in binary64 (exact squares), square root in
 *              binary64; the clip decision and factor are taken in binary64,
 *              the factor rounded once to binary32 and applied with one
 *              binary32 multiply per element.
 *
 * Loops are plain odometers over multi-indices.  OpenMP splits only the loop
 * over OUTPUT elements, so results do not depend on the thread count.
 */
#include <math.h>
#include <quadmath.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_MAX_DIMS 8

enum { OR_ADD = 0, OR_SUB = 1, OR_MUL = 2, OR_DIV = 3 };
enum { OR_EPI_NONE = 0, OR_EPI_GELU = 1, OR_EPI_RELU = 2 };
enum {
  OR_OK = 0,
  OR_ERR_BROADCAST = 1, /* shapes do not broadcast                   */
  OR_ERR_RANK = 2,      /* rank < 0 or > 8                           */
  OR_ERR_SIZE = 3,      /* negative size or stride                   */
  OR_ERR_ARG = 4        /* bad op / epilogue / target shape          */
};

typedef struct {
  int32_t rank;
  int64_t sizes[OR_MAX_DIMS];
  int64_t strides[OR_MAX_DIMS];
} or_desc;

static int g_threads = 1;

void or_set_threads(int n) { g_threads = n < 1 ? 1 : n; }
int or_get_threads(void) { return g_threads; }

/* ---------------------------------------------------------------- shapes */

/* Broadcast rule, compared from the last dim backwards.  A missing dim acts
 * as size 1.  Size 0 follows the same rule: 0 with 1 gives 0, 0 with n>1 is
 * incompatible. */
int or_broadcast_shape(int ra, const int64_t *na, int rb, const int64_t *nb,
                       int *ro, int64_t *no) {
  if (ra < 0 || rb < 0 || ra > OR_MAX_DIMS || rb > OR_MAX_DIMS) return OR_ERR_RANK;
  for (int k = 0; k < ra; ++k) if (na[k] < 0) return OR_ERR_SIZE;
  for (int k = 0; k < rb; ++k) if (nb[k] < 0) return OR_ERR_SIZE;
  int r = ra > rb ? ra : rb;
  int64_t tmp[OR_MAX_DIMS];
  for (int k = 0; k < r; ++k) {
    /* position counted from the right */
    int ka = ra - r + k, kb = rb - r + k;
    int64_t x = ka >= 0 ? na[ka] : 1;
    int64_t y = kb >= 0 ? nb[kb] : 1;
    if (x == y) tmp[k] = x;
    else if (x == 1) tmp[k] = y;
    else if (y == 1) tmp[k] = x;
    else return OR_ERR_BROADCAST;
  }
  *ro = r;
  for (int k = 0; k < r; ++k) no[k] = tmp[k];
  return OR_OK;
}

static int64_t numel(int r, const int64_t *n) {
  int64_t m = 1;
  for (int k = 0; k < r; ++k) m *= n[k];
  return m;
}

static int check_desc(const or_desc *d) {
  if (d->rank < 0 || d->rank > OR_MAX_DIMS) return OR_ERR_RANK;
  for (int k = 0; k < d->rank; ++k)
    if (d->sizes[k] < 0 || d->strides[k] < 0) return OR_ERR_SIZE;
  return OR_OK;
}

/* Offset of an operand element addressed by the OUTPUT multi-index idx
 * (rank r).  The operand is right-aligned; a size-1 operand dim reads
 * coordinate 0, which is what repeating it along that dim means. */
static int64_t operand_offset(const or_desc *d, int r, const int64_t *idx) {
  int64_t off = 0;
  for (int k = 0; k < d->rank; ++k) {
    int ko = r - d->rank + k;
    int64_t i = d->sizes[k] == 1 ? 0 : idx[ko];
    off += i * d->strides[k];
  }
  return off;
}

/* Row-major multi-index of flat position f in shape n (rank r). */
static void unflatten(int64_t f, int r, const int64_t *n, int64_t *idx) {
  for (int k = r - 1; k >= 0; --k) {
    int64_t m = n[k];
    idx[k] = m ? f % m : 0;
    f = m ? f / m : 0;
  }
}

/* ---------------------------------------------------------------- forward */

static float op32(int op, float x, float y) {
  switch (op) {
  case OR_ADD: return x + y;
  case OR_SUB: return x - y;
  case OR_MUL: return x * y;
  default:     return x / y;
  }
}

/* Standard normal CDF and density, binary64. */
double or_phi_cdf(double h) { return 0.5 * erfc(-h * M_SQRT1_2); }
double or_phi_pdf(double h) { return exp(-0.5 * h * h) / sqrt(2.0 * M_PI); }

/* GeLU in binary128 (113-bit significand; libquadmath erfq / erfcq, a few
 * units of 2^-113 relative), rounded once to binary32:
 *   h >= -1 : y = h/2 + d, d = (h/2) erf(h/sqrt2) > 0 for h != 0, since
 *             Phi(h) = (1 + erf(h/sqrt2)) / 2;
 *   h <  -1 : y = (h/2) erfc(|h|/sqrt2), Phi(h) = erfc(-h/sqrt2) / 2 (the
 *             sum would cancel there).
 * In the sum, h/2 is exact and the binary128 addition's own rounding error
 * e is recovered exactly (two-sum), so y = s + e.  When s is exactly a
 * binary32 midpoint -- as for h an odd multiple of 2^-149, where h/2 is the
 * midpoint and d lies far below the last bit of s -- the sign of e decides
 * the rounding; any other s rounds like y does. */
static float gelu32_q(float h) {
  const __float128 H = (__float128)h;
  const __float128 half = H * 0.5Q;
  __float128 s, e = 0;
  if (h >= -1.0f) {
    const __float128 d = half * erfq(H * M_SQRT1_2q);
    s = half + d;
    const __float128 dd = s - half;          /* two-sum (Knuth), exact */
    e = (half - (s - dd)) + (d - dd);
  } else {
    s = half * erfcq(-H * M_SQRT1_2q);
  }
  float r = (float)s;                        /* correctly rounded from s */
  if (e == 0 || (__float128)r == s) return r;
  const float r2 = nextafterf(r, s > (__float128)r ? INFINITY : -INFINITY);
  const __float128 mid = ((__float128)r + (__float128)r2) * 0.5Q;  /* exact */
  if (s != mid) return r;
  return (e > 0) == (r2 > r) ? r2 : r;       /* the neighbour on e's side */
}

/* y lies within rel * |y| of the midpoint between its binary32 neighbours. */
static int near_midpoint32(double y, double rel) {
  const float f = (float)y;
  if ((double)f == y) return 0;
  const double other = (double)nextafterf(f, y > (double)f ? INFINITY : -INFINITY);
  const double mid = 0.5 * ((double)f + other);  /* exact in binary64 */
  return fabs(y - mid) <= rel * fabs(y);
}

/* GeLU(h) = h * Phi(h) rounded once to binary32.  The binary64 evaluation
 * (libm erfc, relative error far below 1e-12) decides the rounding unless y
 * lies within 1e-12 of a binary32 midpoint or below 2^-125 (where h/2 itself
 * can be a midpoint); those go to the binary128 evaluation.  The limits at
 * +-inf are +inf and -0; GeLU(+-0) = +-0. */
float or_gelu32(float h) {
  if (isnan(h)) return h;
  if (isinf(h)) return h > 0 ? h : -0.0f;
  if (h == 0.0f) return h * 0.5f;
  const double hd = (double)h;
  const double y = hd * or_phi_cdf(hd);
  if (fabs(y) >= 0x1p-125 && !near_midpoint32(y, 1e-12)) return (float)y;
  return gelu32_q(h);
}

/* The binary128 evaluation alone (for the tests that pin it). */
float or_gelu32_q(float h) {
  if (isnan(h)) return h;
  if (isinf(h)) return h > 0 ? h : -0.0f;
  if (h == 0.0f) return h * 0.5f;
  return gelu32_q(h);
}

/* Binary32 arguments whose binary64 GeLU lies within rel of a binary32
 * midpoint: scans the bit patterns [lo, hi) of one sign (lo < hi, both in
 * the same sign half) and writes up to max of them to out, returning how
 * many were found (which may exceed max). */
int64_t or_gelu_tie_scan(uint32_t lo, uint32_t hi, double rel, uint32_t *out, int64_t max) {
  int64_t found = 0;
#pragma omp parallel for schedule(dynamic, 65536) num_threads(g_threads)
  for (int64_t u = lo; u < (int64_t)hi; ++u) {
    const uint32_t bits = (uint32_t)u;
    float h;
    memcpy(&h, &bits, 4);
    if (!isfinite(h) || h == 0.0f) continue;
    const double hd = (double)h;
    const double y = hd * or_phi_cdf(hd);
    if (fabs(y) < 0x1p-125 || !near_midpoint32(y, rel)) continue;
    int64_t k;
#pragma omp atomic capture
    k = found++;
    if (k < max) out[k] = bits;
  }
  return found;
}

/* ReLU(h): h for h > 0, NaN stays NaN, +0 otherwise. */
float or_relu32(float h) {
  if (isnan(h)) return h;
  return h > 0.0f ? h : 0.0f;
}

static float fwd_at(int op, int epi, const float *a, const or_desc *da,
                    const float *b, const or_desc *db, int r,
                    const int64_t *idx) {
  float x = a[operand_offset(da, r, idx)];
  float y = b[operand_offset(db, r, idx)];
  float h = op32(op, x, y);
  if (epi == OR_EPI_GELU) return or_gelu32(h);
  if (epi == OR_EPI_RELU) return or_relu32(h);
  return h;
}

int or_fwd(int op, int epi, const float *a, const or_desc *da, const float *b,
           const or_desc *db, float *out) {
  if (op < OR_ADD || op > OR_DIV || epi < 0 || epi > OR_EPI_RELU) return OR_ERR_ARG;
  int s;
  if ((s = check_desc(da)) || (s = check_desc(db))) return s;
  int r;
  int64_t n[OR_MAX_DIMS];
  if ((s = or_broadcast_shape(da->rank, da->sizes, db->rank, db->sizes, &r, n)))
    return s;
  int64_t total = numel(r, n);
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (int64_t f = 0; f < total; ++f) {
    int64_t idx[OR_MAX_DIMS];
    unflatten(f, r, n, idx);
    out[f] = fwd_at(op, epi, a, da, b, db, r, idx);
  }
  return OR_OK;
}

/* Forward at the listed flat output positions only (for spot checks of very
 * large outputs). */
int or_fwd_at(int op, int epi, const float *a, const or_desc *da,
              const float *b, const or_desc *db, int64_t count,
              const int64_t *pos, float *out) {
  if (op < OR_ADD || op > OR_DIV || epi < 0 || epi > OR_EPI_RELU) return OR_ERR_ARG;
  int s;
  if ((s = check_desc(da)) || (s = check_desc(db))) return s;
  int r;
  int64_t n[OR_MAX_DIMS];
  if ((s = or_broadcast_shape(da->rank, da->sizes, db->rank, db->sizes, &r, n)))
    return s;
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (int64_t t = 0; t < count; ++t) {
    int64_t idx[OR_MAX_DIMS];
    unflatten(pos[t], r, n, idx);
    out[t] = fwd_at(op, epi, a, da, b, db, r, idx);
  }
  return OR_OK;
}

/* --------------------------------------------------------------- backward */

/* Local gradient terms at one output position, binary64.
 * which = 0 -> d/da, 1 -> d/db.  Up to two pieces are returned (the GeLU
 * derivative Phi(h) + h*phi(h) is kept as two pieces so that the tolerance
 * base sum|pieces| does not collapse where GeLU' crosses zero). */
static int local_terms(int op, int epi, int which, double g, double x,
                       double y, float h32, double *piece) {
  int np = 1;
  double gg[2];
  gg[0] = g;
  if (epi == OR_EPI_GELU) {
    double h = (double)h32;
    gg[0] = g * or_phi_cdf(h);
    gg[1] = g * h * or_phi_pdf(h);
    np = 2;
  } else if (epi == OR_EPI_RELU) {
    gg[0] = h32 > 0.0f ? g : 0.0;
  }
  for (int p = 0; p < np; ++p) {
    double u = gg[p], t;
    switch (op) {
    case OR_ADD: t = u; break;
    case OR_SUB: t = which ? -u : u; break;
    case OR_MUL: t = which ? u * x : u * y; break;
    default:     t = which ? -u * x / (y * y) : u / y; break;
    }
    piece[p] = t;
  }
  return np;
}

/* Gradient of one operand at its dense row-major position j:
 *   sum over every output index i that reads element j (row-major order of i)
 * of the local terms, plus acc[j] when given.  Returns the binary64 sum and
 * the sum of absolute pieces through *absum. */
static double grad_at(int op, int epi, int which, const float *g,
                      const float *a, const or_desc *da, const float *b,
                      const or_desc *db, const float *acc, int r,
                      const int64_t *n, int64_t j, double *absum) {
  const or_desc *dx = which ? db : da;
  int64_t xidx[OR_MAX_DIMS];
  unflatten(j, dx->rank, dx->sizes, xidx);
  /* Fixed output coordinates come from x; the others are free. */
  int64_t lo[OR_MAX_DIMS], cnt[OR_MAX_DIMS];
  for (int k = 0; k < r; ++k) {
    int kx = k - (r - dx->rank);
    if (kx >= 0 && dx->sizes[kx] != 1) {
      lo[k] = xidx[kx];
      cnt[k] = 1;
    } else {
      lo[k] = 0;
      cnt[k] = n[k];
    }
  }
  double sum = 0.0, as = 0.0;
  if (acc) {
    sum = (double)acc[j];
    as = fabs(sum);
  }
  int64_t total = numel(r, cnt);
  int64_t idx[OR_MAX_DIMS], sub[OR_MAX_DIMS];
  int64_t gstr[OR_MAX_DIMS];
  {
    int64_t s = 1;
    for (int k = r - 1; k >= 0; --k) { gstr[k] = s; s *= n[k]; }
  }
  for (int64_t t = 0; t < total; ++t) {
    unflatten(t, r, cnt, sub);
    int64_t goff = 0;
    for (int k = 0; k < r; ++k) {
      idx[k] = lo[k] + sub[k];
      goff += idx[k] * gstr[k];
    }
    float xv = a[operand_offset(da, r, idx)];
    float yv = b[operand_offset(db, r, idx)];
    float h32 = epi != OR_EPI_NONE ? op32(op, xv, yv) : 0.0f;
    double piece[2];
    int np = local_terms(op, epi, which, (double)g[goff], (double)xv,
                         (double)yv, h32, piece);
    for (int p = 0; p < np; ++p) {
      sum += piece[p];
      as += fabs(piece[p]);
    }
  }
  *absum = as;
  return sum;
}

static int bwd_common(int op, int epi, const or_desc *da, const or_desc *db,
                      int *r, int64_t *n) {
  if (op < OR_ADD || op > OR_DIV || epi < 0 || epi > OR_EPI_RELU) return OR_ERR_ARG;
  int s;
  if ((s = check_desc(da)) || (s = check_desc(db))) return s;
  return or_broadcast_shape(da->rank, da->sizes, db->rank, db->sizes, r, n);
}

/* Full backward.  g is dense row-major in the broadcast shape; grad_a/grad_b
 * are dense row-major in a's / b's shape (NULL = not wanted); *_64 receive
 * the unrounded binary64 sums and abs_* the sums of |terms| (may be NULL). */
int or_bwd(int op, int epi, const float *g, const float *a, const or_desc *da,
           const float *b, const or_desc *db, const float *acc_a,
           const float *acc_b, float *grad_a, double *grad_a64, double *abs_a,
           float *grad_b, double *grad_b64, double *abs_b) {
  int r, s;
  int64_t n[OR_MAX_DIMS];
  if ((s = bwd_common(op, epi, da, db, &r, n))) return s;
  for (int which = 0; which < 2; ++which) {
    float *gx = which ? grad_b : grad_a;
    double *gx64 = which ? grad_b64 : grad_a64;
    double *ax = which ? abs_b : abs_a;
    const float *acc = which ? acc_b : acc_a;
    const or_desc *dx = which ? db : da;
    if (!gx && !gx64) continue;
    int64_t m = numel(dx->rank, dx->sizes);
#pragma omp parallel for schedule(dynamic, 64) num_threads(g_threads)
    for (int64_t j = 0; j < m; ++j) {
      double as;
      double v = grad_at(op, epi, which, g, a, da, b, db, acc, r, n, j, &as);
      if (gx) gx[j] = (float)v;
      if (gx64) gx64[j] = v;
      if (ax) ax[j] = as;
    }
  }
  return OR_OK;
}

/* Backward of one operand (which: 0 = a, 1 = b) at listed dense positions. */
int or_bwd_at(int op, int epi, int which, const float *g, const float *a,
              const or_desc *da, const float *b, const or_desc *db,
              const float *acc, int64_t count, const int64_t *pos, float *out,
              double *out64, double *absout) {
  int r, s;
  int64_t n[OR_MAX_DIMS];
  if ((s = bwd_common(op, epi, da, db, &r, n))) return s;
#pragma omp parallel for schedule(dynamic, 16) num_threads(g_threads)
  for (int64_t t = 0; t < count; ++t) {
    double as;
    double v = grad_at(op, epi, which, g, a, da, b, db, acc, r, n, pos[t], &as);
    if (out) out[t] = (float)v;
    if (out64) out64[t] = v;
    if (absout) absout[t] = as;
  }
  return OR_OK;
}

/* ------------------------------------------------------- reduce to shape */

/* out (dense, shape nout) = sum of `in` over every dim where the target is
 * 1 or missing; the target must broadcast to in's shape.  This is the
 * "sum back to the input shape" step of a broadcast backward. */
int or_reduce(const float *in, const or_desc *din, int rout,
              const int64_t *nout, float *out, double *out64, double *absout) {
  int s;
  if ((s = check_desc(din))) return s;
  if (rout < 0 || rout > OR_MAX_DIMS) return OR_ERR_RANK;
  for (int k = 0; k < rout; ++k) if (nout[k] < 0) return OR_ERR_SIZE;
  int r;
  int64_t n[OR_MAX_DIMS];
  if ((s = or_broadcast_shape(din->rank, din->sizes, rout, nout, &r, n))) return s;
  if (r != din->rank) return OR_ERR_ARG;
  for (int k = 0; k < r; ++k) if (n[k] != din->sizes[k]) return OR_ERR_ARG;
  int64_t m = numel(rout, nout);
#pragma omp parallel for schedule(dynamic, 64) num_threads(g_threads)
  for (int64_t j = 0; j < m; ++j) {
    int64_t oidx[OR_MAX_DIMS], lo[OR_MAX_DIMS], cnt[OR_MAX_DIMS];
    int64_t sub[OR_MAX_DIMS];
    unflatten(j, rout, nout, oidx);
    for (int k = 0; k < r; ++k) {
      int ko = k - (r - rout);
      if (ko >= 0 && nout[ko] != 1) { lo[k] = oidx[ko]; cnt[k] = 1; }
      else { lo[k] = 0; cnt[k] = n[k]; }
    }
    double sum = 0.0, as = 0.0;
    int64_t total = numel(r, cnt);
    for (int64_t t = 0; t < total; ++t) {
      unflatten(t, r, cnt, sub);
      int64_t off = 0;
      for (int k = 0; k < r; ++k) off += (lo[k] + sub[k]) * din->strides[k];
      double v = (double)in[off];
      sum += v;
      as += fabs(v);
    }
    if (out) out[j] = (float)sum;
    if (out64) out64[j] = sum;
    if (absout) absout[j] = as;
  }
  return OR_OK;
}

/* ------------------------------------------- fused two-operator expression */

static int check3(int op1, int op2, const or_desc *da, const or_desc *db,
                  const or_desc *dc, int *r, int64_t *n) {
  if (op1 < OR_ADD || op1 > OR_DIV || (op2 != OR_ADD && op2 != OR_SUB)) return OR_ERR_ARG;
  int s;
  if ((s = check_desc(da)) || (s = check_desc(db)) || (s = check_desc(dc))) return s;
  int r1;
  int64_t n1[OR_MAX_DIMS];
  if ((s = or_broadcast_shape(da->rank, da->sizes, db->rank, db->sizes, &r1, n1))) return s;
  return or_broadcast_shape(r1, n1, dc->rank, dc->sizes, r, n);
}

/* t = a (op1) b rounded to binary32, then t (op2) c rounded to binary32. */
static float fwd2_at(int op1, int op2, const float *a, const or_desc *da,
                     const float *b, const or_desc *db, const float *c,
                     const or_desc *dc, int r, const int64_t *idx) {
  float t = op32(op1, a[operand_offset(da, r, idx)], b[operand_offset(db, r, idx)]);
  return op32(op2, t, c[operand_offset(dc, r, idx)]);
}

/* out (dense, broadcast shape of a, b, c) = (a op1 b) op2 c. */
int or_fwd2(int op1, int op2, const float *a, const or_desc *da, const float *b,
            const or_desc *db, const float *c, const or_desc *dc, float *out) {
  int r, s;
  int64_t n[OR_MAX_DIMS];
  if ((s = check3(op1, op2, da, db, dc, &r, n))) return s;
  int64_t total = numel(r, n);
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (int64_t f = 0; f < total; ++f) {
    int64_t idx[OR_MAX_DIMS];
    unflatten(f, r, n, idx);
    out[f] = fwd2_at(op1, op2, a, da, b, db, c, dc, r, idx);
  }
  return OR_OK;
}

int or_fwd2_at(int op1, int op2, const float *a, const or_desc *da, const float *b,
               const or_desc *db, const float *c, const or_desc *dc, int64_t count,
               const int64_t *pos, float *out) {
  int r, s;
  int64_t n[OR_MAX_DIMS];
  if ((s = check3(op1, op2, da, db, dc, &r, n))) return s;
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (int64_t t = 0; t < count; ++t) {
    int64_t idx[OR_MAX_DIMS];
    unflatten(pos[t], r, n, idx);
    out[t] = fwd2_at(op1, op2, a, da, b, db, c, dc, r, idx);
  }
  return OR_OK;
}

/* Gradient of operand `which` (0 = a, 1 = b, 2 = c) of L = sum_i g_i out_i,
 * out = (a op1 b) op2 c, at its dense position j.  op2 (add or sub) hands
 * g_i to t = a op1 b and +-g_i to c (GPU chapter, "OpAdd"; sub by calculus);
 * op1's local rule turns the former into the terms of a and b.  Every
 * output position i reading element j contributes, in row-major order of i.
 * tie = which (0 or 1): c is the same tensor as this operand, and the c-path
 * term +-g_i of the same positions is added too (Autograd chapter: a tensor
 * reached along two paths gets the sum of the path gradients). */
static double grad2_at(int op1, int op2, int which, int tie, const float *g,
                       const float *a, const or_desc *da, const float *b,
                       const or_desc *db, const float *c, const or_desc *dc,
                       const float *acc, int r, const int64_t *n, int64_t j,
                       double *absum) {
  const or_desc *dx = which == 0 ? da : (which == 1 ? db : dc);
  int64_t xidx[OR_MAX_DIMS];
  unflatten(j, dx->rank, dx->sizes, xidx);
  int64_t lo[OR_MAX_DIMS], cnt[OR_MAX_DIMS];
  for (int k = 0; k < r; ++k) {
    int kx = k - (r - dx->rank);
    if (kx >= 0 && dx->sizes[kx] != 1) {
      lo[k] = xidx[kx];
      cnt[k] = 1;
    } else {
      lo[k] = 0;
      cnt[k] = n[k];
    }
  }
  double sum = 0.0, as = 0.0;
  if (acc) {
    sum = (double)acc[j];
    as = fabs(sum);
  }
  int64_t gstr[OR_MAX_DIMS];
  {
    int64_t s = 1;
    for (int k = r - 1; k >= 0; --k) { gstr[k] = s; s *= n[k]; }
  }
  int64_t total = numel(r, cnt);
  int64_t idx[OR_MAX_DIMS], sub[OR_MAX_DIMS];
  for (int64_t t = 0; t < total; ++t) {
    unflatten(t, r, cnt, sub);
    int64_t goff = 0;
    for (int k = 0; k < r; ++k) {
      idx[k] = lo[k] + sub[k];
      goff += idx[k] * gstr[k];
    }
    double gi = (double)g[goff];
    double cpath = op2 == OR_SUB ? -gi : gi;
    if (which == 2 || tie == which) {
      sum += cpath;
      as += fabs(cpath);
    }
    if (which < 2) {
      float xv = a[operand_offset(da, r, idx)];
      float yv = b[operand_offset(db, r, idx)];
      double piece[2];
      int np = local_terms(op1, OR_EPI_NONE, which, gi, (double)xv, (double)yv, 0.0f, piece);
      for (int p = 0; p < np; ++p) {
        sum += piece[p];
        as += fabs(piece[p]);
      }
    }
  }
  *absum = as;
  return sum;
}

/* Full backward of the fused expression; outputs as in or_bwd, three of
 * them (NULL = not wanted).  tie: -1, or 0 / 1 when c is the same tensor as
 * a / b (then grad_c is ignored and that operand's gradient has both paths). */
int or_bwd2(int op1, int op2, int tie, const float *g, const float *a,
            const or_desc *da, const float *b, const or_desc *db, const float *c,
            const or_desc *dc, const float *acc_a, const float *acc_b,
            const float *acc_c, float *grad_a, double *grad_a64, double *abs_a,
            float *grad_b, double *grad_b64, double *abs_b, float *grad_c,
            double *grad_c64, double *abs_c) {
  int r, s;
  int64_t n[OR_MAX_DIMS];
  if ((s = check3(op1, op2, da, db, dc, &r, n))) return s;
  if (tie < -1 || tie > 1) return OR_ERR_ARG;
  for (int which = 0; which < 3; ++which) {
    float *gx = which == 0 ? grad_a : (which == 1 ? grad_b : grad_c);
    double *gx64 = which == 0 ? grad_a64 : (which == 1 ? grad_b64 : grad_c64);
    double *ax = which == 0 ? abs_a : (which == 1 ? abs_b : abs_c);
    const float *acc = which == 0 ? acc_a : (which == 1 ? acc_b : acc_c);
    const or_desc *dx = which == 0 ? da : (which == 1 ? db : dc);
    if ((!gx && !gx64) || (which == 2 && tie >= 0)) continue;
    int64_t m = numel(dx->rank, dx->sizes);
#pragma omp parallel for schedule(dynamic, 64) num_threads(g_threads)
    for (int64_t j = 0; j < m; ++j) {
      double as;
      double v = grad2_at(op1, op2, which, tie, g, a, da, b, db, c, dc, acc, r, n, j, &as);
      if (gx) gx[j] = (float)v;
      if (gx64) gx64[j] = v;
      if (ax) ax[j] = as;
    }
  }
  return OR_OK;
}

/* One gradient of the fused expression at listed dense positions. */
int or_bwd2_at(int op1, int op2, int which, int tie, const float *g, const float *a,
               const or_desc *da, const float *b, const or_desc *db, const float *c,
               const or_desc *dc, const float *acc, int64_t count, const int64_t *pos,
               float *out, double *out64, double *absout) {
  int r, s;
  int64_t n[OR_MAX_DIMS];
  if ((s = check3(op1, op2, da, db, dc, &r, n))) return s;
  if (which < 0 || which > 2 || tie < -1 || tie > 1) return OR_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 16) num_threads(g_threads)
  for (int64_t t = 0; t < count; ++t) {
    double as;
    double v = grad2_at(op1, op2, which, tie, g, a, da, b, db, c, dc, acc, r, n, pos[t], &as);
    if (out) out[t] = (float)v;
    if (out64) out64[t] = v;
    if (absout) absout[t] = as;
  }
  return OR_OK;
}

/* ------------------------------------------------------------ materialise */

/* out (dense, shape nout) = in read through its strides, broadcast to nout
 * (Operator chapter, "view backward": a stride-aware copy into contiguous
 * storage).  nout must be the broadcast of in's shape with itself. */
int or_materialize(const float *in, const or_desc *din, int rout, const int64_t *nout,
                   float *out) {
  int s;
  if ((s = check_desc(din))) return s;
  if (rout < 0 || rout > OR_MAX_DIMS) return OR_ERR_RANK;
  for (int k = 0; k < rout; ++k) if (nout[k] < 0) return OR_ERR_SIZE;
  int r;
  int64_t n[OR_MAX_DIMS];
  if ((s = or_broadcast_shape(din->rank, din->sizes, rout, nout, &r, n))) return s;
  if (r != rout) return OR_ERR_ARG;
  for (int k = 0; k < r; ++k) if (n[k] != nout[k]) return OR_ERR_ARG;
  int64_t total = numel(r, n);
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (int64_t f = 0; f < total; ++f) {
    int64_t idx[OR_MAX_DIMS];
    unflatten(f, r, n, idx);
    out[f] = in[operand_offset(din, r, idx)];
  }
  return OR_OK;
}

/* ------------------------------------------------------- other reductions */

/* Mean back to a shape: out_j = RN32(S_j / count), S_j the binary64 sum in
 * index order of the `count` input elements that map to j (the elements
 * or_reduce sums), count the product of the input sizes over the reduced
 * dims.  An empty reduced dim gives count 0 and 0/0 = NaN.  out64 gets
 * S_j / count and absout sum|in_i| / count (the tolerance base). */
int or_mean(const float *in, const or_desc *din, int rout, const int64_t *nout,
            float *out, double *out64, double *absout) {
  int64_t m = numel(rout < 0 ? 0 : rout, nout);
  double *s64 = (double *)malloc(sizeof(double) * (size_t)(m > 0 ? m : 1));
  double *sab = (double *)malloc(sizeof(double) * (size_t)(m > 0 ? m : 1));
  int s = or_reduce(in, din, rout, nout, NULL, s64, sab);
  if (s == OR_OK) {
    int r = din->rank;
    int64_t count = 1;
    for (int k = 0; k < r; ++k) {
      int ko = k - (r - rout);
      if (ko < 0 || nout[ko] == 1) count *= din->sizes[k];
    }
    for (int64_t j = 0; j < m; ++j) {
      double v = s64[j] / (double)count;
      if (out) out[j] = (float)v;
      if (out64) out64[j] = v;
      if (absout) absout[j] = sab[j] / (double)count;
    }
  }
  free(s64);
  free(sab);
  return s;
}

/* Gradient of the mean: each input element (shape nin) receives the upstream
 * gradient of the output it was averaged into (g dense in shape nout, which
 * broadcasts to nin), divided by the count: grad_in_i = RN32(g_j /
 * RN32(count)), one binary32 division. */
int or_mean_bwd(const float *g, int rout, const int64_t *nout, int rin,
                const int64_t *nin, float *grad_in) {
  if (rout < 0 || rout > OR_MAX_DIMS || rin < 0 || rin > OR_MAX_DIMS) return OR_ERR_RANK;
  for (int k = 0; k < rout; ++k) if (nout[k] < 0) return OR_ERR_SIZE;
  for (int k = 0; k < rin; ++k) if (nin[k] < 0) return OR_ERR_SIZE;
  int r, s;
  int64_t n[OR_MAX_DIMS];
  if ((s = or_broadcast_shape(rin, nin, rout, nout, &r, n))) return s;
  if (r != rin) return OR_ERR_ARG;
  for (int k = 0; k < r; ++k) if (n[k] != nin[k]) return OR_ERR_ARG;
  int64_t count = 1;
  for (int k = 0; k < r; ++k) {
    int ko = k - (r - rout);
    if (ko < 0 || nout[ko] == 1) count *= nin[k];
  }
  const float c32 = (float)count;
  int64_t total = numel(r, nin);
  for (int64_t f = 0; f < total; ++f) {
    int64_t idx[OR_MAX_DIMS];
    unflatten(f, r, nin, idx);
    int64_t j = 0;
    for (int ko = 0; ko < rout; ++ko) {
      int k = ko + (r - rout);
      j = j * nout[ko] + (nout[ko] == 1 ? 0 : idx[k]);
    }
    grad_in[f] = g[j] / c32;
  }
  return OR_OK;
}

/* Global L2 norm of a list of dense gradients: the square root, in binary64,
 * of the binary64 sum of g^2 over every element of every tensor, in list
 * order then index order (each square of a binary32 value is exact). */
double or_grad_norm(int count, const float *const *g, const int64_t *n) {
  double s = 0.0;
  for (int t = 0; t < count; ++t)
    for (int64_t i = 0; i < n[t]; ++i) {
      double v = (double)g[t][i];
      s += v * v;
    }
  return sqrt(s);
}

/* ClipGradNorm: when the global norm exceeds c, every gradient element is
 * scaled by the one factor c / (norm + 1e-6).  The decision and the factor
 * are taken in binary64 from the binary64 norm; the factor is rounded once
 * to binary32 and each element becomes RN32(g * factor).  Scales in place;
 * returns the norm, and through the pointers whether it scaled and the
 * binary32 factor (1 when it did not). */
double or_clip_grad_norm(int count, float *const *g, const int64_t *n, double c,
                         int *clipped, float *factor) {
  double norm = or_grad_norm(count, (const float *const *)g, n);
  int clip = norm > c;
  float f = clip ? (float)(c / (norm + 1e-6)) : 1.0f;
  if (clip)
    for (int t = 0; t < count; ++t)
      for (int64_t i = 0; i < n[t]; ++i) g[t][i] = g[t][i] * f;
  if (clipped) *clipped = clip;
  if (factor) *factor = f;
  return norm;
}

/* ----------------------------------------------------- row statistics */

/* Per-row mean and (biased) variance, the statistics a LayerNorm takes of
 * each row (GPU chapter, "reduction": mean and variance are reductions;
 * Operator chapter, "fusion": LayerNorm computes them inside one operator).
 * Row r is x[r*ld .. r*ld + cols).  mean = sum x / cols and var = sum (x -
 * mean)^2 / cols, both in binary64 (two passes, index order), rounded once;
 * cols = 0 gives NaN.  abs_mean gets sum|x| / cols (the mean's tolerance
 * base); the variance's terms are its own squares. */
int or_row_moments(const float *x, int64_t rows, int64_t cols, int64_t ld, float *mean,
                   float *var, double *mean64, double *var64, double *abs_mean) {
  if (rows < 0 || cols < 0 || ld < cols) return OR_ERR_SIZE;
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (int64_t r = 0; r < rows; ++r) {
    const float *row = x + r * ld;
    double s = 0.0, a = 0.0;
    for (int64_t j = 0; j < cols; ++j) {
      s += (double)row[j];
      a += fabs((double)row[j]);
    }
    const double m = s / (double)cols;
    double q = 0.0;
    for (int64_t j = 0; j < cols; ++j) {
      const double d = (double)row[j] - m;
      q += d * d;
    }
    const double v = q / (double)cols;
    if (mean) mean[r] = (float)m;
    if (var) var[r] = (float)v;
    if (mean64) mean64[r] = m;
    if (var64) var64[r] = v;
    if (abs_mean) abs_mean[r] = a / (double)cols;
  }
  return OR_OK;
}

/* Per-row softmax statistics (GPU chapter, "reduction": Softmax is one of
 * the reductions; the GPT chapter's attention takes a softmax over each row
 * of the masked scores): rowmax = max_j x (exact; NaN if the row holds a
 * NaN, -inf for an empty row) and sumexp = sum_j exp(x - rowmax), each
 * exponent of the exact binary64 difference with libm exp, summed in
 * binary64 in index order and rounded once (0 for an empty row). */
int or_row_softmax_stats(const float *x, int64_t rows, int64_t cols, int64_t ld,
                         float *rowmax, float *sumexp, double *sumexp64) {
  if (rows < 0 || cols < 0 || ld < cols) return OR_ERR_SIZE;
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (int64_t r = 0; r < rows; ++r) {
    const float *row = x + r * ld;
    float m = -INFINITY;
    int nan = 0;
    for (int64_t j = 0; j < cols; ++j) {
      if (isnan(row[j])) nan = 1;
      else if (row[j] > m) m = row[j];
    }
    if (nan) m = NAN;
    double s = 0.0;
    for (int64_t j = 0; j < cols; ++j) s += exp((double)row[j] - (double)m);
    if (cols == 0) s = 0.0;
    if (rowmax) rowmax[r] = m;
    if (sumexp) sumexp[r] = (float)s;
    if (sumexp64) sumexp64[r] = s;
  }
  return OR_OK;
}
