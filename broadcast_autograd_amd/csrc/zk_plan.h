// zk_plan.h -- host-side shape/stride canonicaliser and launch planner.
//
// Pure C++ (no HIP): it validates descriptors, computes the broadcast shape,
// turns every operand into right-aligned strides over that shape (stride 0
// where an operand is repeated), drops size-1 dims, merges adjacent dims that
// every operand walks contiguously, and picks the kernel class for the
// resulting canonical form.  Nothing here touches a GPU.
#pragma once

#include <cstddef>
#include <cstdint>

#include "zk.h"

namespace zk {

constexpr int kMaxDims = ZK_MAX_DIMS;
constexpr int kMaxOps = 5;
// Largest grid the planner sizes a non-looping launch for: a dispatch counts
// work-items with 32 bits, and blocks have at most 1024 threads.
constexpr int64_t kMaxGridBlocks = (int64_t)1 << 22;
// Largest element count, and largest element offset, of any view (2^62).
constexpr int64_t kMaxExtent = (int64_t)1 << 62;

// Waves per red_col block (they combine their column sums in LDS): with
// fewer than kColRowsMany rows per wave, and with that many.  The kernel is
// instantiated for 1, 4 and 16.  Measured: on the [4096, 1024] GeLU
// backward, 4 waves x 4 rows 10.8-11.0 us against 12.1-15.2 us for 16 x 4
// (the larger blocks vary from one machine to the next); on the
// [32768, 4096] backward, 16 waves 270 us, 4 waves 289 us, 1 wave (no LDS
// combine) 296 us.
constexpr int kColRowsMany = 64;
constexpr int kColWavesFew = 4;
constexpr int kColWavesMany = 16;
// red_row: passes moving at least this many full-size arrays take 512-element chunks
constexpr int kRowShortChunkStreams = 2;
// red_col: rows a wave for long columns walked by the interleaved kernel
constexpr int kColRowsIL = 4;
// red_rowd: terms per kept element it takes (a 1024-lane block holds up to 4
// vectors per lane in flight).
constexpr int64_t kDirMinTerms = 2048;
constexpr int64_t kDirMaxTerms = 16384;
// red_rowd for plain row sums ([K, T]) only up to this many elements.
constexpr int64_t kDirRowSumMaxElems = (int64_t)1 << 24;
// red_gend: terms per kept element it takes (a wave walks them, 64 at a time).
constexpr int64_t kGenDirMinTerms = 32;
constexpr int64_t kGenDirMaxTerms = 4096;
// red_run: the run (the two innermost canonical dims) holds 64..256 elements
// (at least one whole run for each 256-lane block), and the outer kept dims
// give at least this many blocks.
constexpr int64_t kRunMinLen = 64;
constexpr int64_t kRunMaxLen = 256;
constexpr int64_t kRunMinBlocks = 32;

// Kernel classes (ids reported by zk_plan_describe).
enum KernelClass : int32_t {
  K_NONE = -1,
  K_FWD_FLAT = 0,     // every operand dense in the output layout
  K_FWD_ROW = 1,      // one dense operand, the other rank <= 3 strided
  K_FWD_TILE = 2,     // a transposed rank-2 operand, staged through LDS
  K_FWD_GENERIC = 3,  // anything (rank <= 8)
  K_BWD_EW_FLAT = 4,  // backward, no reduction, dense operands
  K_BWD_EW_GENERIC = 5,
  K_RED_COL = 6,      // fused backward stage 1, pattern [R, K]
  K_RED_ROW = 7,      // fused backward stage 1, pattern [.., K, R] (inner reduced)
  K_RED_TILE = 8,     // fused backward stage 1, [R, K] with a transposed operand
  K_RED_GENERIC = 9,  // gather stage 1, any pattern
  K_RED_FINAL = 10,   // stage 2: fixed-order sum of the partials
  K_FWD2_ROW = 11,    // fused (a op1 b) op2 c, rank <= 3, 128-bit output
  K_FWD2_GENERIC = 12,  // fused (a op1 b) op2 c, anything (rank <= 8)
  K_BWD_SIGNED = 13,  // +-g (+ acc) element-wise: the gradient of op2's c
  K_COPY_ROW = 14,    // materialise a view, rank <= 3, 128-bit output
  K_COPY_TILE = 15,   // materialise a transposed rank-2 view through LDS
  K_COPY_GENERIC = 16,  // materialise anything (rank <= 8)
  K_NORM_PART = 17,   // global L2 norm: binary64 partial sums of squares
  K_NORM_FINAL = 18,  // global L2 norm: fixed-order total, sqrt, clip factor
  K_CLIP_SCALE = 19,  // ClipGradNorm: in-place scaling by the factor
  K_RED_ROWD = 20,    // red_row's pattern in one pass: a block per kept element
  K_RED_GEND = 21,    // any pattern in one pass: a wave per kept element
  K_ROW_MOMENTS = 22,  // per-row mean and variance, a wave per row
  K_ROW_SOFTMAX = 23,  // per-row max and sum of exponentials, a wave per row
  K_RED_ROWSEG = 24,   // sums of short dense rows (C <= 256), 256/C rows a wave
  K_RED_RUN = 25,      // two innermost dims a short contiguous run: a block per
                       // outer kept combination, every element read once, one pass
  K_COUNT = 26
};

const char *kernel_name(int32_t k);

// Inner-dim access mode of a non-dense operand in the ROW classes.
// SM_ARG: the operand is a host scalar passed by value in the kernel arguments.
enum SmallMode : int32_t { SM_BCAST = 0, SM_CONTIG = 1, SM_GATHER = 2, SM_ARG = 3 };

// Magic-number division for 0 <= n < 2^31 and 1 <= d < 2^31
// (Granlund & Montgomery, "Division by invariant integers using
// multiplication", 1994, round-up variant):
//   l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1,
//   q = (umulhi(n, m) + n) >> l.
struct FastDiv {
  uint32_t d, m, l;
};
FastDiv make_fastdiv(uint32_t d);
inline uint32_t fastdiv_eval(const FastDiv &f, uint32_t n) {
  uint32_t hi = (uint32_t)(((uint64_t)n * f.m) >> 32);
  return (hi + n) >> f.l;
}

// A canonical iteration space: rank dims, sizes n, one stride set per
// operand (elements).  ops[0] is always the dense output / upstream grad.
struct Canon {
  int rank = 0;
  int nops = 0;
  int64_t n[kMaxDims] = {};
  int64_t s[kMaxOps][kMaxDims] = {};
  int64_t numel = 0;
};

// Right-aligns `d` to the rank-r shape `out`: stride 0 where d's dim is
// missing or has size 1.
void align_strides(const zk_desc &d, int r, int64_t *st);
// Dense row-major strides of d's own shape, right-aligned the same way.
void align_dense(const zk_desc &d, int r, int64_t *st);
// Drop size-1 dims and merge dim k into k+1 when every operand has
// s[k] == s[k+1] * n[k+1].  A zero-size or rank-0 space becomes rank 1.
Canon canonicalise(int r, const int64_t *n, int nops,
                   const int64_t (*st)[kMaxDims]);

zk_status check_desc(const zk_desc *d);
zk_status broadcast_shape(int ra, const int64_t *na, int rb, const int64_t *nb,
                          int *ro, int64_t *no);
// [lo, hi) byte extent an operand's elements span (hi == lo when empty).
void byte_extent(const void *p, const zk_desc &d, uintptr_t *lo, uintptr_t *hi);
void byte_extent_dense(const void *p, int64_t numel, uintptr_t *lo,
                       uintptr_t *hi);
bool overlaps(uintptr_t alo, uintptr_t ahi, uintptr_t blo, uintptr_t bhi);

// ---------------------------------------------------------------- forward
// Access mode of one input of the fused forward (K_FWD2_ROW).
enum InMode : int32_t {
  IM_FLAT = 0,    // walks the output's dense layout (128-bit, aligned)
  IM_BCAST = 1,   // decoded offset; inner dim repeated (stride 0)
  IM_CONTIG = 2,  // decoded offset; inner dim contiguous, 128-bit aligned
  IM_GATHER = 3,  // decoded offset; inner dim any stride
  IM_SAME_A = 4   // the same tensor as input a (read once)
};

struct FwdPlan {
  Canon c;            // ops: 0 out, 1 a, 2 b
  int32_t kernel = K_NONE;
  bool empty = false;
  bool idx64 = false;
  int vec = 1;
  bool swap = false;  // ROW/TILE: the dense / transposed operand is b
  int32_t small_mode = SM_GATHER;
};
zk_status plan_fwd(zk_op op, zk_epi epi, const zk_desc &da, const zk_desc &db,
                   uintptr_t pa, uintptr_t pb, uintptr_t pout, FwdPlan *p);

// Fused out = (a op1 b) op2 c.  Canon ops: 0 out, 1 a, 2 b, 3 c.
struct Fwd2Plan {
  Canon c;
  int32_t kernel = K_NONE;  // K_FWD2_ROW or K_FWD2_GENERIC
  bool empty = false;
  bool idx64 = false;
  int vec = 1;
  int32_t mode[3] = {IM_GATHER, IM_GATHER, IM_GATHER};  // a, b, c (ROW)
};
// Materialise a view into dense row-major storage of a target shape the
// view broadcasts to.  Canon ops: 0 out, 1 in.
struct CopyPlan {
  Canon c;
  int32_t kernel = K_NONE;  // K_COPY_ROW, K_COPY_TILE or K_COPY_GENERIC
  bool empty = false;
  bool idx64 = false;
  int vec = 1;
  int32_t mode = IM_GATHER;  // ROW: input access mode
};
zk_status plan_copy(const zk_desc &din, int rout, const int64_t *nout, uintptr_t pin,
                    uintptr_t pout, CopyPlan *p);

// Broadcast shape of three shapes (a with b, then with c).
zk_status broadcast_shape3(const zk_desc &da, const zk_desc &db, const zk_desc &dc,
                           int *r, int64_t *n);
zk_status plan_fwd2(const zk_desc &da, const zk_desc &db, const zk_desc &dc,
                    uintptr_t pa, uintptr_t pb, uintptr_t pc, uintptr_t pout,
                    Fwd2Plan *p);

// ------------------------------------------------------ debug checks
// One pointer as the HIP runtime describes it (hipPointerGetAttributes):
// known = 0 when the runtime could not describe it; mem_type holds the
// hipMemoryType value (kMemDevice, kMemManaged, ...), device the owner.
constexpr int32_t kMemUnregistered = 0, kMemHost = 1, kMemDevice = 2, kMemManaged = 3;
struct PtrRecord {
  int32_t known;
  int32_t mem_type;
  int32_t device;
};
// ZK_OK when the stream's device is known (stream_device >= 0) and every
// record is managed memory or device memory of stream_device; else
// ZK_ERR_DEVICE.
zk_status check_ptr_records(const PtrRecord *r, int n, int stream_device);

// --------------------------------------------------------------- backward
// One stage-1 reduction for one operand's gradient.
struct RedPlan {
  int32_t kernel = K_NONE;   // K_RED_*
  int which = -1;            // 0 = a, 1 = b (reduce_to_shape: 1 = target)
  int64_t kept = 0;          // K: elements of the reduced gradient
  int64_t partials = 0;      // P: partial sums per kept element
  int64_t chunk = 0;         // rows per wave (COL), rows (TILE) or elements
                             // (ROW/GENERIC) per partial
  int32_t nw = 1;            // COL, ROW: waves of a block that share one partial
  int32_t fold = 1;          // COL: rows of K < 256 columns read as one row of
                             // fold*K = 256 (stage 1 runs on [R/fold, 256];
                             // partials counts the fold copies too)
  int64_t col_rows = 0;      // COL: the [rows, cols] matrix stage 1 walks
  int64_t col_cols = 0;      //      (before folding)
  int32_t csub = 1;          // COL: consecutive columns per kept element
                             // ([R1, K, C] -> [K, 1] walks [R1, K*C]; stage 2
                             // sums each kept element's C columns too)
  int64_t red = 0;           // reduced elements per kept element
  size_t ws_offset = 0;      // byte offset of its partials in the workspace
};
// Rank-3 red_rowseg ([R1, K, C] -> [K, 1], row sums as stage-2 partials) is
// planned only for R1 <= C, so a kept element has at most this many partials
// and the partials hold at most 2 / C of the input's bytes.
constexpr int64_t kRowSegMaxPartials = 256;

struct BwdPlan {
  Canon c;                 // ops: 0 grad, 1 a, 2 b, 3 grad_a, 4 grad_b
  bool empty_space = false;  // broadcast shape has no elements
  bool want[2] = {false, false};
  bool full[2] = {false, false};   // operand has the full broadcast shape
  bool idx64 = false;
  int vec = 1;
  int32_t ew_kernel = K_NONE;      // element-wise kernel for full grads
  bool ew_write[2] = {false, false};
  int nred = 0;
  RedPlan red[2];
  size_t workspace = 0;
  // fused stage 1 writes the full operand's gradient too
  bool fused_big = false;
};
zk_status plan_bwd(zk_op op, zk_epi epi, const zk_desc &da, const zk_desc &db,
                   bool want_a, bool want_b, uintptr_t pg, uintptr_t pa,
                   uintptr_t pb, uintptr_t pga, uintptr_t pgb,
                   uintptr_t pacc_a, uintptr_t pacc_b, BwdPlan *p);

// reduce_to_shape: ops 0 = input (any strides), 1 = unused, 2 = unused,
// 3 = unused, 4 = target dense-aligned.  Reuses BwdPlan with which = 1.
zk_status plan_reduce(const zk_desc &din, int rout, const int64_t *nout,
                      uintptr_t pin, uintptr_t pout, BwdPlan *p);

// Operand o walks the canonical space exactly like the dense output (op 0).
bool canon_is_flat(const Canon &c, int o);

// Operands the local rule of `op` (with `epi`) reads for grad `which`.
bool rule_reads_a(zk_op op, zk_epi epi, int which);
bool rule_reads_b(zk_op op, zk_epi epi, int which);

}  // namespace zk
