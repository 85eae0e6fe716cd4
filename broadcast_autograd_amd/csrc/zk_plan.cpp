// zk_plan.cpp -- host-side canonicaliser and launch planner (see zk_plan.h).
#include "zk_plan.h"

#include <algorithm>
#include <cstring>

namespace zk {

const char *kernel_name(int32_t k) {
  static const char *names[K_COUNT] = {
      "fwd_flat",       "fwd_row",       "fwd_tile",   "fwd_generic",
      "bwd_ew_flat",    "bwd_ew_generic", "red_col",   "red_row",
      "red_tile",       "red_generic",   "red_final",  "fwd2_row",
      "fwd2_generic",   "bwd_signed",    "copy_row",   "copy_tile",
      "copy_generic",   "norm_part",     "norm_final", "clip_scale",
      "red_rowd",       "red_gend",      "row_moments", "row_softmax",
      "red_rowseg",     "red_run"};
  if (k < 0 || k >= K_COUNT) return "none";
  return names[k];
}

FastDiv make_fastdiv(uint32_t d) {
  FastDiv f{d, 0u, 0u};
  if (d <= 1) return f;  // m = 0, l = 0: q = n
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;  // l = ceil(log2 d)
  uint64_t m = ((((1ull << l) - d) << 32) / d) + 1;
  f.m = (uint32_t)m;
  f.l = l;
  return f;
}

static inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

zk_status check_desc(const zk_desc *d) {
  if (!d) return ZK_ERR_NULL;
  if (d->rank < 0 || d->rank > kMaxDims) return ZK_ERR_RANK;
  bool empty = false;
  for (int k = 0; k < d->rank; ++k) {
    if (d->sizes[k] < 0) return ZK_ERR_BAD_SIZE;
    empty = empty || d->sizes[k] == 0;
  }
  for (int k = 0; k < d->rank; ++k)
    if (d->strides[k] < 0) return ZK_ERR_BAD_STRIDE;
  if (empty) return ZK_OK;  // nothing is read or written
  // The element count and the largest element offset stay below kMaxExtent,
  // so every count, offset and byte extent formed from them fits in int64.
  int64_t numel = 1, last = 0;
  for (int k = 0; k < d->rank; ++k) {
    if (__builtin_mul_overflow(numel, d->sizes[k], &numel) || numel > kMaxExtent)
      return ZK_ERR_BAD_SIZE;
    int64_t span = 0;
    if (d->sizes[k] > 1 &&
        (__builtin_mul_overflow(d->sizes[k] - 1, d->strides[k], &span) ||
         __builtin_add_overflow(last, span, &last) || last > kMaxExtent))
      return ZK_ERR_BAD_STRIDE;
  }
  return ZK_OK;
}

zk_status broadcast_shape(int ra, const int64_t *na, int rb, const int64_t *nb,
                          int *ro, int64_t *no) {
  if (ra < 0 || rb < 0 || ra > kMaxDims || rb > kMaxDims) return ZK_ERR_RANK;
  if ((ra && !na) || (rb && !nb)) return ZK_ERR_NULL;
  for (int k = 0; k < ra; ++k) if (na[k] < 0) return ZK_ERR_BAD_SIZE;
  for (int k = 0; k < rb; ++k) if (nb[k] < 0) return ZK_ERR_BAD_SIZE;
  int r = std::max(ra, rb);
  int64_t tmp[kMaxDims];
  for (int k = 0; k < r; ++k) {
    int ka = k - (r - ra), kb = k - (r - rb);
    int64_t x = ka >= 0 ? na[ka] : 1, y = kb >= 0 ? nb[kb] : 1;
    if (x == y) tmp[k] = x;
    else if (x == 1) tmp[k] = y;
    else if (y == 1) tmp[k] = x;
    else return ZK_ERR_BROADCAST;
  }
  // the broadcast shape may hold more elements than either operand
  int64_t numel = 1;
  bool empty = false;
  for (int k = 0; k < r; ++k) empty = empty || tmp[k] == 0;
  for (int k = 0; k < r && !empty; ++k)
    if (__builtin_mul_overflow(numel, tmp[k], &numel) || numel > kMaxExtent)
      return ZK_ERR_BAD_SIZE;
  *ro = r;
  for (int k = 0; k < r; ++k) no[k] = tmp[k];
  return ZK_OK;
}

void align_strides(const zk_desc &d, int r, int64_t *st) {
  for (int k = 0; k < r; ++k) {
    int kx = k - (r - d.rank);
    st[k] = (kx < 0 || d.sizes[kx] == 1) ? 0 : d.strides[kx];
  }
}

void align_dense(const zk_desc &d, int r, int64_t *st) {
  int64_t dense[kMaxDims];
  int64_t s = 1;
  for (int k = d.rank - 1; k >= 0; --k) {
    dense[k] = s;
    s *= d.sizes[k];
  }
  for (int k = 0; k < r; ++k) {
    int kx = k - (r - d.rank);
    st[k] = (kx < 0 || d.sizes[kx] == 1) ? 0 : dense[kx];
  }
}

Canon canonicalise(int r, const int64_t *n, int nops,
                   const int64_t (*st)[kMaxDims]) {
  Canon c;
  c.nops = nops;
  int64_t numel = 1;
  for (int k = 0; k < r; ++k) numel *= n[k];
  c.numel = numel;
  if (numel == 0) {  // nothing to iterate: a single empty dim
    c.rank = 1;
    c.n[0] = 0;
    return c;
  }
  // Walk from the innermost dim outwards, keeping dims of size > 1 and
  // merging a dim into the current innermost kept one when every operand
  // steps over it contiguously.
  int64_t rn[kMaxDims], rs[kMaxOps][kMaxDims];
  int m = 0;  // kept dims, stored inner -> outer
  for (int k = r - 1; k >= 0; --k) {
    if (n[k] == 1) continue;
    if (m > 0) {
      bool merge = true;
      for (int o = 0; o < nops; ++o)
        if (st[o][k] != rs[o][m - 1] * rn[m - 1]) { merge = false; break; }
      if (merge) {
        rn[m - 1] *= n[k];
        continue;
      }
    }
    rn[m] = n[k];
    for (int o = 0; o < nops; ++o) rs[o][m] = st[o][k];
    ++m;
  }
  if (m == 0) {  // all dims of size 1 (or rank 0): one element
    c.rank = 1;
    c.n[0] = 1;
    for (int o = 0; o < nops; ++o) c.s[o][0] = 0;
    c.s[0][0] = 1;
    return c;
  }
  c.rank = m;
  for (int k = 0; k < m; ++k) {
    c.n[k] = rn[m - 1 - k];
    for (int o = 0; o < nops; ++o) c.s[o][k] = rs[o][m - 1 - k];
  }
  return c;
}

void byte_extent(const void *p, const zk_desc &d, uintptr_t *lo, uintptr_t *hi) {
  uintptr_t base = (uintptr_t)p;
  int64_t last = 0;
  for (int k = 0; k < d.rank; ++k) {
    if (d.sizes[k] == 0) { *lo = *hi = base; return; }
    last += (d.sizes[k] - 1) * d.strides[k];
  }
  *lo = base;
  *hi = base + (uintptr_t)(last + 1) * 4u;
}

void byte_extent_dense(const void *p, int64_t numel, uintptr_t *lo,
                       uintptr_t *hi) {
  *lo = (uintptr_t)p;
  *hi = (uintptr_t)p + (uintptr_t)numel * 4u;
}

bool overlaps(uintptr_t alo, uintptr_t ahi, uintptr_t blo, uintptr_t bhi) {
  if (alo == ahi || blo == bhi) return false;
  return alo < bhi && blo < ahi;
}

static int64_t numel_of(const zk_desc &d) {
  int64_t m = 1;
  for (int k = 0; k < d.rank; ++k) m *= d.sizes[k];
  return m;
}

static bool is_flat(const Canon &c, int o) {
  for (int k = 0; k < c.rank; ++k)
    if (c.s[o][k] != c.s[0][k]) return false;
  return true;
}

bool canon_is_flat(const Canon &c, int o) { return is_flat(c, o); }

static int64_t max_offset(const Canon &c, int o) {
  int64_t m = 0;
  for (int k = 0; k < c.rank; ++k)
    if (c.n[k] > 0) m += (c.n[k] - 1) * c.s[o][k];
  return m;
}

static bool needs_idx64(const Canon &c) {
  // margin: kernels form indices up to one tile past the end
  const int64_t lim = ((int64_t)1 << 31) - ((int64_t)1 << 20);
  if (c.numel >= lim) return true;
  for (int o = 0; o < c.nops; ++o)
    if (max_offset(c, o) >= lim) return true;
  return false;
}

static bool al16(uintptr_t p) { return (p & 15u) == 0; }

// Transposed rank-2 operand: x[i, j] at i * 1 + j * ld.
static bool is_transposed2(const Canon &c, int o) {
  return c.rank == 2 && c.s[o][0] == 1 && c.s[o][1] >= c.n[0];
}

bool rule_reads_a(zk_op op, zk_epi epi, int which) {
  if (epi != ZK_EPI_NONE) return true;
  if (op == ZK_MUL) return which == 1;
  if (op == ZK_DIV) return which == 1;
  return false;
}

bool rule_reads_b(zk_op op, zk_epi epi, int which) {
  if (epi != ZK_EPI_NONE) return true;
  if (op == ZK_MUL) return which == 0;
  if (op == ZK_DIV) return true;
  return false;
}

// ------------------------------------------------------------- forward
zk_status plan_fwd(zk_op op, zk_epi epi, const zk_desc &da, const zk_desc &db,
                   uintptr_t pa, uintptr_t pb, uintptr_t pout, FwdPlan *p) {
  (void)op;
  (void)epi;
  int r;
  int64_t n[kMaxDims];
  zk_status s = broadcast_shape(da.rank, da.sizes, db.rank, db.sizes, &r, n);
  if (s) return s;
  int64_t st[kMaxOps][kMaxDims];
  {
    int64_t d = 1;
    for (int k = r - 1; k >= 0; --k) { st[0][k] = d; d *= n[k]; }
  }
  align_strides(da, r, st[1]);
  align_strides(db, r, st[2]);
  p->c = canonicalise(r, n, 3, st);
  const Canon &c = p->c;
  if (c.numel == 0) {
    p->empty = true;
    p->kernel = K_NONE;
    return ZK_OK;
  }
  p->idx64 = needs_idx64(c);
  bool fa = is_flat(c, 1), fb = is_flat(c, 2);
  int64_t inner = c.n[c.rank - 1];
  if (fa && fb) {
    p->kernel = K_FWD_FLAT;
    p->vec = (al16(pa) && al16(pb) && al16(pout)) ? 4 : 1;
    return ZK_OK;
  }
  if ((fa || fb) && c.rank <= 3) {
    p->kernel = K_FWD_ROW;
    p->swap = !fa;  // swap: the dense operand is b
    int sm = p->swap ? 1 : 2;
    uintptr_t psmall = p->swap ? pa : pb, pbig = p->swap ? pb : pa;
    bool v4 = inner % 4 == 0 && al16(pbig) && al16(pout);
    p->vec = v4 ? 4 : 1;
    int64_t s0 = c.s[sm][c.rank - 1];
    if (s0 == 0) {
      p->small_mode = SM_BCAST;
    } else {
      bool contig = s0 == 1 && al16(psmall);
      for (int k = 0; k + 1 < c.rank; ++k)
        if (c.s[sm][k] % 4 != 0) contig = false;
      p->small_mode = contig ? SM_CONTIG : SM_GATHER;
    }
    return ZK_OK;
  }
  if (is_transposed2(c, 1) || is_transposed2(c, 2)) {
    p->kernel = K_FWD_TILE;
    p->swap = !is_transposed2(c, 1);
    p->vec = (c.n[1] % 4 == 0 && al16(pout)) ? 4 : 1;
    if (p->vec == 4) return ZK_OK;
  }
  p->kernel = K_FWD_GENERIC;
  p->swap = false;
  p->vec = (al16(pout) && (!fa || al16(pa)) && (!fb || al16(pb))) ? 4 : 1;
  return ZK_OK;
}

// ------------------------------------------------------- fused forward
zk_status broadcast_shape3(const zk_desc &da, const zk_desc &db, const zk_desc &dc,
                           int *r, int64_t *n) {
  int r1;
  int64_t n1[kMaxDims];
  zk_status s = broadcast_shape(da.rank, da.sizes, db.rank, db.sizes, &r1, n1);
  if (s) return s;
  return broadcast_shape(r1, n1, dc.rank, dc.sizes, r, n);
}

static bool same_view(const zk_desc &x, const zk_desc &y) {
  if (x.rank != y.rank) return false;
  for (int k = 0; k < x.rank; ++k)
    if (x.sizes[k] != y.sizes[k] || (x.sizes[k] != 1 && x.strides[k] != y.strides[k]))
      return false;
  return true;
}

zk_status plan_fwd2(const zk_desc &da, const zk_desc &db, const zk_desc &dc,
                    uintptr_t pa, uintptr_t pb, uintptr_t pc, uintptr_t pout,
                    Fwd2Plan *p) {
  int r;
  int64_t n[kMaxDims];
  zk_status s = broadcast_shape3(da, db, dc, &r, n);
  if (s) return s;
  int64_t st[kMaxOps][kMaxDims];
  {
    int64_t d = 1;
    for (int k = r - 1; k >= 0; --k) { st[0][k] = d; d *= n[k]; }
  }
  align_strides(da, r, st[1]);
  align_strides(db, r, st[2]);
  align_strides(dc, r, st[3]);
  p->c = canonicalise(r, n, 4, st);
  const Canon &c = p->c;
  if (c.numel == 0) {
    p->empty = true;
    p->kernel = K_NONE;
    return ZK_OK;
  }
  p->idx64 = needs_idx64(c);
  const int64_t inner = c.n[c.rank - 1];
  if (c.rank <= 3 && inner % 4 == 0 && al16(pout)) {
    p->kernel = K_FWD2_ROW;
    p->vec = 4;
    const uintptr_t ptr[3] = {pa, pb, pc};
    for (int x = 0; x < 3; ++x) {
      const int o = 1 + x;
      if (x == 2 && pc == pa && same_view(dc, da)) {
        p->mode[x] = IM_SAME_A;
      } else if (is_flat(c, o) && al16(ptr[x])) {
        p->mode[x] = IM_FLAT;
      } else if (c.s[o][c.rank - 1] == 0) {
        p->mode[x] = IM_BCAST;
      } else {
        bool contig = c.s[o][c.rank - 1] == 1 && al16(ptr[x]);
        for (int k = 0; k + 1 < c.rank; ++k)
          if (c.s[o][k] % 4 != 0) contig = false;
        p->mode[x] = contig ? IM_CONTIG : IM_GATHER;
      }
    }
    return ZK_OK;
  }
  p->kernel = K_FWD2_GENERIC;
  p->vec = al16(pout) ? 4 : 1;
  return ZK_OK;
}

// --------------------------------------------------------- materialise
zk_status plan_copy(const zk_desc &din, int rout, const int64_t *nout, uintptr_t pin,
                    uintptr_t pout, CopyPlan *p) {
  int r;
  int64_t n[kMaxDims];
  zk_status s = broadcast_shape(din.rank, din.sizes, rout, nout, &r, n);
  if (s == ZK_ERR_BROADCAST) return ZK_ERR_SHAPE;
  if (s) return s;
  // the result of the broadcast must be the target itself
  if (r != rout) return ZK_ERR_SHAPE;
  for (int k = 0; k < r; ++k)
    if (n[k] != nout[k]) return ZK_ERR_SHAPE;
  int64_t st[kMaxOps][kMaxDims];
  {
    int64_t d = 1;
    for (int k = r - 1; k >= 0; --k) { st[0][k] = d; d *= n[k]; }
  }
  align_strides(din, r, st[1]);
  p->c = canonicalise(r, n, 2, st);
  const Canon &c = p->c;
  if (c.numel == 0) {
    p->empty = true;
    return ZK_OK;
  }
  p->idx64 = needs_idx64(c);
  const int64_t inner = c.n[c.rank - 1];
  if (is_transposed2(c, 1) && c.n[1] % 4 == 0 && al16(pout)) {
    p->kernel = K_COPY_TILE;
    p->vec = 4;
    return ZK_OK;
  }
  if (c.rank <= 3 && inner % 4 == 0 && al16(pout)) {
    p->kernel = K_COPY_ROW;
    p->vec = 4;
    if (is_flat(c, 1) && al16(pin)) {
      p->mode = IM_FLAT;
    } else if (c.s[1][c.rank - 1] == 0) {
      p->mode = IM_BCAST;
    } else {
      bool contig = c.s[1][c.rank - 1] == 1 && al16(pin);
      for (int k = 0; k + 1 < c.rank; ++k)
        if (c.s[1][k] % 4 != 0) contig = false;
      p->mode = contig ? IM_CONTIG : IM_GATHER;
    }
    return ZK_OK;
  }
  p->kernel = K_COPY_GENERIC;
  p->vec = al16(pout) ? 4 : 1;
  return ZK_OK;
}

// ------------------------------------------------------- debug checks
zk_status check_ptr_records(const PtrRecord *r, int n, int stream_device) {
  if (stream_device < 0) return ZK_ERR_DEVICE;
  for (int i = 0; i < n; ++i) {
    if (!r[i].known) return ZK_ERR_DEVICE;
    if (r[i].mem_type == kMemManaged) continue;
    if (r[i].mem_type != kMemDevice || r[i].device != stream_device) return ZK_ERR_DEVICE;
  }
  return ZK_OK;
}

// ------------------------------------------------------------- backward

// Reduction pattern of operand stride set `o` over the canonical dims:
// bit k set when dim k is kept (stride != 0).
static unsigned kept_mask(const Canon &c, int o) {
  unsigned m = 0;
  for (int k = 0; k < c.rank; ++k)
    if (c.s[o][k] != 0) m |= 1u << k;
  return m;
}

static size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// Sizing of a generic (gather) reduction: K kept elements, `red` reduced
// elements each.  The split depends on the shapes only.
static void size_generic(RedPlan *rp, int64_t K, int64_t red) {
  rp->kernel = K_RED_GENERIC;
  rp->kept = K;
  rp->red = red;
  if (red <= 0) {
    rp->partials = 0;
    rp->chunk = 0;
    return;
  }
  int64_t P = std::max<int64_t>(1, ceil_div(65536, std::max<int64_t>(K, 1)));
  P = std::min<int64_t>(P, ceil_div(red, 8));
  P = std::max<int64_t>(P, 1);
  int64_t chunk = ceil_div(red, P);
  rp->chunk = chunk;
  rp->partials = ceil_div(red, chunk);
}

// The one-pass gather (red_gend) when each kept element has a moderate
// number of terms; false leaves rp alone.
static bool size_gend(RedPlan *rp, int64_t K, int64_t red) {
  if (K <= 0 || red < kGenDirMinTerms || red > kGenDirMaxTerms) return false;
  rp->kernel = K_RED_GEND;
  rp->kept = K;
  rp->red = red;
  rp->chunk = 0;
  rp->partials = 0;
  return true;
}

// Sizing of a red_col column sum over a dense [rows, cols] matrix (cols a
// multiple of 4): kept = cols, one partial per band of rows.
static void size_col(RedPlan *rp, int64_t rows, int64_t cols, bool col_il = false) {
  rp->kernel = K_RED_COL;
  rp->kept = cols;
  rp->red = rows;
  rp->col_rows = rows;
  rp->col_cols = cols;
  rp->csub = 1;
  // A wave owns 256 columns and walks rcw rows: enough waves to fill the
  // chip (~8192), between 4 and 64 rows each.  The waves of a block
  // combine their sums (kColWavesFew / kColWavesMany), so a partial covers
  // >= 16 rows and binary64 partials stay within a few % of the call's
  // bytes.  The number of blocks (column groups x partials) stays within
  // the dispatch limit where the rows allow it; the kernel walks its blocks
  // with a grid stride past that.
  // Narrow columns (cols < 256 dividing 256, e.g. [4194304, 32]): fold =
  // 256/cols consecutive rows of the dense operands form one row of 256
  // columns, so every lane of a wave stays busy; stage 2 then sums the fold
  // copies of each column along with the partials.
  int64_t fold = 1;
  if (cols < 256 && 256 % cols == 0 && rows % (256 / cols) == 0) fold = 256 / cols;
  const int64_t R0 = rows / fold;
  const int64_t colblocks = ceil_div(cols * fold, 256);
  int64_t rcw = std::min<int64_t>(kColRowsMany, std::max<int64_t>(4, R0 * colblocks / 8192));
  int nw = rcw >= kColRowsMany ? kColWavesMany : kColWavesFew;
  // Short columns (fewer rows than a block spans, e.g. [128, 1048576]):
  // kColWavesFew waves (one below that many rows) split the rows evenly,
  // one partial a column, rather than most waves of a block idling.
  if (R0 < nw * rcw) {
    nw = R0 >= kColWavesFew ? kColWavesFew : 1;
    rcw = std::max<int64_t>(1, ceil_div(R0, nw));
  }
  // Long columns whose pass reads the full operand and writes its gradient
  // with the interleaved column kernel (col_il): short row runs, 4 a wave
  // (all in flight at once) and 64 a partial, over many blocks (measured on
  // MI355X: the fused [32768, 4096] backward 380-385 us with 64 rows a wave,
  // 366-372 with 8, 338-343 with 4; the [32768, 4096] multiply backward's
  // two stages 274-277, 266-272, 262-265 us; [65536, 2048] 321, 301, 288;
  // with 2 rows 300-307 us.  The division and GeLU backwards, which walk
  // their rows in order, gained nothing or lost with 8).
  if (col_il && fold == 1 && nw == kColWavesMany && colblocks >= 8) rcw = kColRowsIL;
  // Longer row bands while the grid is above the dispatch limit, down to a
  // single band (more than 2^30 columns stay above it).
  while (colblocks * ceil_div(R0, nw * rcw) > kMaxGridBlocks && nw * rcw < R0) rcw *= 2;
  rp->chunk = rcw;
  rp->nw = nw;
  rp->fold = (int32_t)fold;
  rp->partials = ceil_div(R0, nw * rcw) * fold;
}

// red_col over [rows, cols] for a sum whose kept elements own C consecutive
// columns each: stage 2 indexes each kept element's partials * C values with
// 32 bits, so the plan is taken only below 2^31 of them.
static bool col_sub_fits(int64_t rows, int64_t cols, int64_t C, RedPlan *rp) {
  RedPlan q;
  size_col(&q, rows, cols);
  if (q.partials * C >= ((int64_t)1 << 31)) return false;
  *rp = q;
  return true;
}

// The one-pass run reduction (red_run) when the two innermost canonical dims
// form a run of kRunMinLen..kRunMaxLen elements that the source (op 0) and,
// when read, the full operand `big_op` walk densely, and the outer kept dims
// give at least kRunMinBlocks blocks; false leaves rp alone.  o: the reduced
// gradient's stride set (0 on reduced dims).
static bool size_run(const Canon &c, int o, int big_op, bool src_flat, bool idx64,
                     RedPlan *rp) {
  if (idx64 || !src_flat || c.rank < 3) return false;
  if (big_op >= 0 && !is_flat(c, big_op)) return false;
  const int R = c.rank;
  const int64_t L = c.n[R - 2] * c.n[R - 1];
  if (L < kRunMinLen || L > kRunMaxLen) return false;
  int64_t blocks = 1, runs = 1, kept = 1;
  for (int k = 0; k < R; ++k) {
    if (c.s[o][k] != 0) kept *= c.n[k];
    if (k < R - 2) (c.s[o][k] != 0 ? blocks : runs) *= c.n[k];
  }
  if (blocks < kRunMinBlocks || runs < 2) return false;
  rp->kernel = K_RED_RUN;
  rp->kept = kept;
  rp->red = c.numel / kept;
  rp->chunk = L;
  rp->partials = 0;
  return true;
}

// Try the fast stage-1 classes for the reduced operand stride set `o`
// (grad layout) with `big` the dense operand id (or -1 if none is read).
// Requires the source (op 0) to be dense.  `streams` counts the full-size
// arrays stage 1 moves (the upstream gradient, the full operand when read,
// its gradient when written).
static bool size_fast(const Canon &c, int o, int big_op, bool big_transposed,
                      bool src_flat, bool aligned, int streams, bool col_il, RedPlan *rp) {
  if (!src_flat || !aligned) return false;
  unsigned km = kept_mask(c, o);
  int R = c.rank;
  int64_t inner = c.n[R - 1];
  // [R, K] : column sums
  if (R == 2 && km == 2u && c.s[o][1] == 1) {
    if (big_transposed) {
      if (c.n[1] % 4 != 0) return false;
      rp->kernel = K_RED_TILE;
      rp->kept = c.n[1];
      rp->red = c.n[0];
      // two 64 x 64 tiles a block and partial, one below the other, while
      // that leaves at least 1024 blocks; else one (measured on MI355X, the
      // [4096, 4096] transposed multiply backward: 39.6-40.4 us with one
      // tile a block, 37.7-38.1 with two, 37.1-38.3 with four or eight,
      // 43.2-43.8 with sixteen, 256 blocks)
      const int64_t tiles_c = ceil_div(c.n[1], 64);
      rp->chunk = tiles_c * ceil_div(c.n[0], 128) >= 1024 ? 128 : 64;
      rp->partials = ceil_div(c.n[0], rp->chunk);
      return true;
    }
    if (big_op >= 0 && !is_flat(c, big_op)) return false;
    if (inner % 4 != 0) return false;
    size_col(rp, c.n[0], c.n[1], col_il);
    return true;
  }
  if (big_transposed) return false;
  if (big_op >= 0 && !is_flat(c, big_op)) return false;
  // [R0], [K, R0], [R1, K, R0] : inner dim reduced
  bool pat = (R == 1 && km == 0u) ||
             (R == 2 && km == 1u && c.s[o][0] == 1) ||
             (R == 3 && km == 2u && c.s[o][1] == 1);
  if (!pat || inner % 4 != 0 || inner < 256) return false;
  int64_t rows = c.numel / inner;               // (R1, K) rows
  int64_t K = (R == 1) ? 1 : c.n[R - 2];
  int64_t R1 = rows / K;
  // Chunks of 256..2048 elements (whole wave trips), about 8192 of them;
  // partials stay < 0.1% of bytes.  A pass that also reads or writes the
  // full operand streams best with chunks of 512 (two trips a wave), four
  // chunks of a row to a block and partial (measured on MI355X: the
  // [8, 16, 1048576] multiply backward 291 -> 266 us, the add backward
  // 202 -> 190 us; a plain sum is 2% slower that way and keeps 2048).
  const bool two_trips = streams >= kRowShortChunkStreams;
  const int64_t cmax = two_trips ? 512 : 2048;
  int64_t CL = std::min<int64_t>(cmax, std::max<int64_t>(256, c.numel / 8192));
  // at most 65536 partials per kept element, so that stage 2 stays short
  CL = std::max<int64_t>(CL, ceil_div(R1 * inner, 65536));
  CL = ceil_div(CL, 256) * 256;
  if (CL >= inner) CL = inner;
  int64_t NC = ceil_div(inner, CL);
  // Few terms per kept element: one block per kept element finishes its sum
  // itself (no partials, no stage-2 launch).  Plain row sums ([K, T], R1 = 1)
  // of many rows stream better through red_row's short chunks, where the
  // saved launch is small next to the data (measured: [65536, 2048] 242 ->
  // 81 us, [8192, 4096] 38 -> 25 us).
  const int64_t T = R1 * inner;
  if (T >= kDirMinTerms && T <= kDirMaxTerms && (R1 > 1 || c.numel <= kDirRowSumMaxElems)) {
    rp->kernel = K_RED_ROWD;
    rp->kept = K;
    rp->red = T;
    rp->chunk = T <= 4096 ? 1 : (T <= 8192 ? 2 : 4);  // vectors per lane
    rp->partials = 0;
    return true;
  }
  rp->kernel = K_RED_ROW;
  rp->kept = K;
  rp->red = R1 * inner;
  rp->chunk = CL;
  rp->nw = (two_trips && NC % 4 == 0) ? 4 : 1;  // waves sharing a partial
  rp->partials = R1 * NC / rp->nw;
  return true;
}

static void finish_workspace(BwdPlan *p) {
  size_t off = 0;
  for (int i = 0; i < p->nred; ++i) {
    p->red[i].ws_offset = off;
    off += round256((size_t)p->red[i].partials * (size_t)p->red[i].kept *
                    (size_t)p->red[i].csub * 8u);
  }
  p->workspace = off;
}

zk_status plan_bwd(zk_op op, zk_epi epi, const zk_desc &da, const zk_desc &db,
                   bool want_a, bool want_b, uintptr_t pg, uintptr_t pa,
                   uintptr_t pb, uintptr_t pga, uintptr_t pgb,
                   uintptr_t pacc_a, uintptr_t pacc_b, BwdPlan *p) {
  int r;
  int64_t n[kMaxDims];
  zk_status s = broadcast_shape(da.rank, da.sizes, db.rank, db.sizes, &r, n);
  if (s) return s;
  int64_t st[kMaxOps][kMaxDims];
  {
    int64_t d = 1;
    for (int k = r - 1; k >= 0; --k) { st[0][k] = d; d *= n[k]; }
  }
  align_strides(da, r, st[1]);
  align_strides(db, r, st[2]);
  align_dense(da, r, st[3]);
  align_dense(db, r, st[4]);
  p->c = canonicalise(r, n, 5, st);
  const Canon &c = p->c;
  p->want[0] = want_a;
  p->want[1] = want_b;
  int64_t ne[2] = {numel_of(da), numel_of(db)};
  p->nred = 0;
  if (c.numel == 0) {
    // Sums over nothing: a non-empty gradient is its acc (or zeros).
    p->empty_space = true;
    for (int w = 0; w < 2; ++w) {
      if (!p->want[w] || ne[w] == 0) continue;
      RedPlan &rp = p->red[p->nred++];
      size_generic(&rp, ne[w], 0);
      rp.which = w;
    }
    finish_workspace(p);
    return ZK_OK;
  }
  p->idx64 = needs_idx64(c);
  for (int w = 0; w < 2; ++w) p->full[w] = ne[w] == c.numel;
  bool reduced[2] = {want_a && !p->full[0], want_b && !p->full[1]};
  bool fa = is_flat(c, 1), fb = is_flat(c, 2);

  // Element-wise part: gradients of operands with the full shape.
  auto ew_kernel = [&](bool wa, bool wb) {
    bool ra = (wa && rule_reads_a(op, epi, 0)) || (wb && rule_reads_a(op, epi, 1));
    bool rb = (wa && rule_reads_b(op, epi, 0)) || (wb && rule_reads_b(op, epi, 1));
    bool flat = (!ra || fa) && (!rb || fb);
    bool al = al16(pg) && (!ra || al16(pa)) && (!rb || al16(pb)) &&
              (!wa || (al16(pga) && al16(pacc_a))) &&
              (!wb || (al16(pgb) && al16(pacc_b)));
    p->vec = al ? 4 : 1;
    return flat ? K_BWD_EW_FLAT : K_BWD_EW_GENERIC;
  };

  if (!reduced[0] && !reduced[1]) {
    if (want_a || want_b) {
      p->ew_kernel = ew_kernel(want_a, want_b);
      p->ew_write[0] = want_a;
      p->ew_write[1] = want_b;
    }
    finish_workspace(p);
    return ZK_OK;
  }

  if (reduced[0] != reduced[1]) {
    int sw = reduced[0] ? 0 : 1;  // reduced operand
    int bw = 1 - sw;              // the other (full, or not wanted)
    bool big_full = p->full[bw];
    bool big_read = rule_reads_a(op, epi, sw) && bw == 0;
    big_read = big_read || (rule_reads_b(op, epi, sw) && bw == 1);
    bool big_write = p->want[bw];
    if (big_write) {
      bool rd = (bw == 0) ? rule_reads_a(op, epi, 0) : rule_reads_b(op, epi, 1);
      big_read = big_read || rd;
    }
    // The fused classes need the other operand to have the full shape
    // (so its gradient and values walk with the upstream grad).
    if (big_full || (!big_read && !big_write)) {
      int big_op = (big_read && big_full) ? 1 + bw : -1;
      bool big_tr = big_read && big_full && is_transposed2(c, 1 + bw);
      uintptr_t pbig = bw == 0 ? pa : pb;
      uintptr_t pgbig = bw == 0 ? pga : pgb;
      uintptr_t paccbig = bw == 0 ? pacc_a : pacc_b;
      bool aligned = al16(pg) && (!big_read || big_tr || al16(pbig)) &&
                     (!big_write || (al16(pgbig) && al16(paccbig)));
      RedPlan rp;
      const int streams = 1 + (big_op >= 0) + big_write;
      // the column kernel's interleaved row walk: the full operand read and
      // its gradient written, no epilogue, not division
      const bool col_il = big_op >= 0 && big_write && epi == ZK_EPI_NONE && op != ZK_DIV;
      if (size_fast(c, 3 + sw, big_op, big_tr, true, aligned, streams, col_il, &rp)) {
        rp.which = sw;
        p->red[p->nred++] = rp;
        p->fused_big = big_write;
        p->vec = 4;
        finish_workspace(p);
        return ZK_OK;
      }
    }
    // A short contiguous inner run: one pass reading every element once, that
    // also writes the full operand's gradient.
    {
      RedPlan rr;
      const int run_big = big_read ? 1 + bw : -1;
      if ((!big_read || big_full) && (big_full || !big_write) &&
          size_run(c, 3 + sw, run_big, true, p->idx64, &rr)) {
        rr.which = sw;
        p->red[p->nred++] = rr;
        p->fused_big = big_write;
        finish_workspace(p);
        return ZK_OK;
      }
    }
    // Moderate term counts: one gather pass that also writes the full
    // operand's gradient.
    {
      RedPlan rd;
      if (size_gend(&rd, ne[sw], c.numel / ne[sw]) && (big_full || !big_write)) {
        rd.which = sw;
        p->red[p->nred++] = rd;
        p->fused_big = big_write;
        finish_workspace(p);
        return ZK_OK;
      }
    }
    // Fallback: generic gather for the reduced gradient, element-wise
    // kernel for the full one.
    RedPlan &rp = p->red[p->nred++];
    size_generic(&rp, ne[sw], c.numel / ne[sw]);
    rp.which = sw;
    if (big_write && big_full) {
      p->ew_kernel = ew_kernel(bw == 0, bw == 1);
      p->ew_write[bw] = true;
    } else if (big_write) {
      RedPlan &rq = p->red[p->nred++];
      size_generic(&rq, ne[bw], c.numel / ne[bw]);
      rq.which = bw;
    }
    finish_workspace(p);
    return ZK_OK;
  }
  // Both operands broadcast: one gather reduction each.
  for (int w = 0; w < 2; ++w) {
    RedPlan &rp = p->red[p->nred++];
    if (!size_gend(&rp, ne[w], c.numel / ne[w])) size_generic(&rp, ne[w], c.numel / ne[w]);
    rp.which = w;
  }
  finish_workspace(p);
  return ZK_OK;
}

zk_status plan_reduce(const zk_desc &din, int rout, const int64_t *nout,
                      uintptr_t pin, uintptr_t pout, BwdPlan *p) {
  (void)pout;
  int r;
  int64_t n[kMaxDims];
  zk_status s = broadcast_shape(din.rank, din.sizes, rout, nout, &r, n);
  if (s == ZK_ERR_BROADCAST) return ZK_ERR_SHAPE;
  if (s) return s;
  if (r != din.rank) return ZK_ERR_SHAPE;
  for (int k = 0; k < r; ++k)
    if (n[k] != din.sizes[k]) return ZK_ERR_SHAPE;
  zk_desc dt{};
  dt.rank = rout;
  for (int k = 0; k < rout; ++k) dt.sizes[k] = nout[k];
  int64_t st[kMaxOps][kMaxDims] = {};
  {
    int64_t d = 1;
    for (int k = r - 1; k >= 0; --k) { st[1][k] = d; d *= n[k]; }  // dense in
  }
  align_strides(din, r, st[0]);
  align_dense(dt, r, st[4]);
  // ops: 0 = input strides, 1 = dense layout of the input shape (to test
  // flatness), 2/3 unused, 4 = target.
  p->c = canonicalise(r, n, 5, st);
  const Canon &c = p->c;
  p->want[0] = false;
  p->want[1] = true;
  int64_t K = numel_of(dt);
  p->nred = 0;
  if (c.numel == 0) {
    p->empty_space = true;
    if (K > 0) {
      RedPlan &rp = p->red[p->nred++];
      size_generic(&rp, K, 0);
      rp.which = 1;
    }
    finish_workspace(p);
    return ZK_OK;
  }
  p->idx64 = needs_idx64(c);
  bool src_flat = true;
  for (int k = 0; k < c.rank; ++k)
    if (c.s[0][k] != c.s[1][k]) src_flat = false;
  RedPlan rp;
  // Short dense rows (C <= 256 dividing 256, aligned): a wave reads 256 / C
  // whole rows at a time (red_rowseg).  [K, C] to [K, 1]: each row sum is the
  // result (no partials).  [R1, K, C] to [K, 1] with R1 <= C: the row sums are
  // binary64 partials [R1, K] for stage 2 (at most kRowSegMaxPartials a kept
  // element, 2 / C of the input's bytes), unless red_rowd takes the whole sum
  // in one pass (R1 * C within its term range).  With R1 > C the same sum
  // walks the dense [R1, K * C] matrix as column sums (red_col), whose
  // partials cover bands of rows, and stage 2 adds each kept element's C
  // columns along with its partials.
  const int64_t C = c.n[c.rank - 1];
  const bool dense_al = K < c.numel && src_flat && al16(pin);
  const bool row2 = c.rank == 2 && kept_mask(c, 4) == 1u && c.s[4][0] == 1;
  const bool mid3 = c.rank == 3 && kept_mask(c, 4) == 2u && c.s[4][1] == 1;
  const bool short_rows = dense_al && C >= 4 && C <= 256 && 256 % C == 0;
  const bool rowd_range = c.rank == 3 && C == 256 && c.n[0] * C >= kDirMinTerms &&
                          c.n[0] * C <= kDirMaxTerms;  // red_rowd needs rows of >= 256
  const int64_t KC = mid3 ? c.n[1] * C : 0;
  if (short_rows && (row2 || (mid3 && !rowd_range && c.n[0] <= C))) {
    rp.kernel = K_RED_ROWSEG;
    rp.kept = c.n[c.rank - 2];
    rp.red = c.numel / rp.kept;
    rp.chunk = C;
    rp.partials = c.rank == 3 ? c.n[0] : 0;
    rp.which = 1;
    p->red[p->nred++] = rp;
    p->vec = 4;
  } else if (dense_al && mid3 && !rowd_range && C % 4 == 0 && C <= 256 &&
             (KC >= 256 || 256 % KC == 0) && col_sub_fits(c.n[0], KC, C, &rp)) {
    rp.kept = c.n[1];
    rp.csub = (int32_t)C;
    rp.red = c.n[0] * C;
    rp.which = 1;
    p->red[p->nred++] = rp;
    p->vec = 4;
  } else if (K < c.numel && size_fast(c, 4, -1, false, src_flat, al16(pin), 1, false, &rp)) {
    rp.which = 1;
    p->red[p->nred++] = rp;
    p->vec = 4;
  } else if (K < c.numel && size_run(c, 4, -1, src_flat, p->idx64, &rp)) {
    rp.which = 1;
    p->red[p->nred++] = rp;
  } else {
    RedPlan &q = p->red[p->nred++];
    if (!size_gend(&q, K, c.numel / K)) size_generic(&q, K, c.numel / K);
    q.which = 1;
  }
  finish_workspace(p);
  return ZK_OK;
}

}  // namespace zk
