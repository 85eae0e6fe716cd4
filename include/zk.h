/*
 * zk.h -- C ABI of the MI355X (gfx950) broadcasting binary-operator library.
 *
 * The library computes, on one GPU, the N-d strided broadcasting element-wise
 * operators add/sub/mul/div and their backward (the local gradient rule
 * followed by the sum back to each input's shape), as described by the "Zero"
 * book (ismantic.github.io/zero):
 *   - Tensor chapter, "shape and strides": sizes and strides per dim, strides
 *     counted in ELEMENTS, element offset = sum_k i_k * s_k.
 *   - Operator chapter, "element-wise operators": same-shape add/sub/mul/div
 *     and the mul rule dL/dx = g*y, dL/dy = g*x.
 *   - Operator chapter, "broadcast": the shape rule (compare from the last
 *     dim: equal, one is 1, or one missing) and the backward "repetition in
 *     the forward is a sum in the backward" (SumToSize).
 *   - GPU chapter, "kernel dispatch": at most 8 dims, passed by value.
 *   - GPU chapter, "OpAdd": add's backward hands g to both inputs.
 *   - GPU chapter, "asynchronous execution": work is queued on a stream and
 *     the caller is not synchronised.
 *
 * Conventions shared by every call:
 *   - Element type: IEEE binary32 (float) only.
 *   - Dims are listed outer -> inner (row-major order).  A descriptor's
 *     sizes and strides are int64 element counts; strides must be >= 0; a
 *     stride on a size-1 dim is ignored.  Rank 0 (a scalar) is allowed.
 *   - Every output is DENSE ROW-MAJOR: the forward result in the broadcast
 *     shape, each gradient in its operand's logical shape.
 *   - Pointers are device pointers on the device that owns `stream` (a
 *     hipStream_t passed as void*; NULL means the default stream).  Host
 *     arrays (sizes, descriptors) are read during the call only.  Inputs on
 *     another device lead to an illegal memory access (GPU chapter, "kernel
 *     dispatch": the devices of a call must match); with the environment
 *     variable ZK_DEBUG=1 (or zk_set_debug(1)) every call first asks the HIP
 *     runtime about each pointer it will touch and returns ZK_ERR_DEVICE,
 *     launching nothing, unless all of them are device (or managed) memory
 *     of the stream's device.
 *   - The library allocates nothing on the device, keeps no pointer after
 *     it returns and never synchronises: results are ready when the stream
 *     reaches them.
 *   - Every argument is validated before anything is launched; on an error
 *     nothing is launched and no output is written.
 *   - Forward results are one binary32 operation per element,
 *     round-to-nearest-even, subnormals kept, no fused multiply-add.
 *   - Backward reductions are deterministic: the same call on the same
 *     shapes returns the same bits, on any device of the same kind.
 */
#ifndef ZK_H_
#define ZK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Up to 8 dims per tensor (GPU chapter, "kernel dispatch"). */
#define ZK_MAX_DIMS 8

typedef enum {
  ZK_OK = 0,
  ZK_ERR_NULL = 1,        /* a required pointer is NULL                     */
  ZK_ERR_RANK = 2,        /* rank < 0 or > ZK_MAX_DIMS                      */
  ZK_ERR_BAD_SIZE = 3,    /* a size is negative, or a view, a broadcast     */
                          /* shape or a tensor holds more than 2^62 elements */
  ZK_ERR_BAD_STRIDE = 4,  /* a stride is negative, or a view's largest     */
                          /* element offset exceeds 2^62                   */
  ZK_ERR_BROADCAST = 5,   /* shapes do not broadcast                        */
  ZK_ERR_ALIAS = 6,       /* an output overlaps an input or another output  */
  ZK_ERR_WORKSPACE = 7,   /* workspace smaller than required, or not       */
                          /* 8-byte aligned                                */
  ZK_ERR_UNSUPPORTED = 8, /* unknown op / epilogue value                    */
  ZK_ERR_HIP = 9,         /* a kernel launch failed                         */
  ZK_ERR_SHAPE = 10,      /* reduce target does not broadcast to the input  */
  ZK_ERR_DEVICE = 11      /* (debug checks only) a pointer is not device or */
                          /* managed memory of the stream's device          */
} zk_status;

/* out = a (op) b.  Operator chapter, "element-wise operators". */
typedef enum { ZK_ADD = 0, ZK_SUB = 1, ZK_MUL = 2, ZK_DIV = 3 } zk_op;

/* Optional epilogue applied to the op's result h = a (op) b (itself rounded
 * to binary32 first):
 *   ZK_EPI_GELU: y = GeLU(h) = h * Phi(h), Phi the standard normal CDF (the
 *                activation the GPU chapter, "element-wise" section, and the
 *                GPT chapter's FFN name), correctly rounded to binary32 (a
 *                binary64 evaluation, redone in double-double where it cannot
 *                decide the rounding); GeLU' = Phi(h) + h*phi(h).
 *   ZK_EPI_RELU: y = ReLU(h) = h for h > 0, NaN for NaN, +0 otherwise (the
 *                activation of the Module chapter's example MLP); ReLU'(h) = 1 for
 *                h > 0, else 0. */
typedef enum { ZK_EPI_NONE = 0, ZK_EPI_GELU = 1, ZK_EPI_RELU = 2 } zk_epi;

/* A strided tensor view (Tensor chapter, "shape and strides").
 * sizes[k], strides[k] for k < rank; entries past rank are ignored. */
typedef struct {
  int32_t rank;
  int64_t sizes[ZK_MAX_DIMS];
  int64_t strides[ZK_MAX_DIMS];
} zk_desc;

/*
 * Broadcast shape of two shapes (Operator chapter, "broadcast"): align the
 * shapes at their last dim; per dim the sizes must be equal, or one is 1, or
 * one is missing (counts as 1).  Size 0 obeys the same rule (0 with 1 gives
 * 0; 0 with n > 1 is an error).
 *   rank_a, sizes_a / rank_b, sizes_b : the two shapes (host arrays)
 *   rank_out, sizes_out               : the result (host; ZK_MAX_DIMS slots)
 * Errors: ZK_ERR_NULL, ZK_ERR_RANK, ZK_ERR_BAD_SIZE, ZK_ERR_BROADCAST.
 * Pure host function: touches no GPU.
 */
zk_status zk_broadcast_shape(int32_t rank_a, const int64_t *sizes_a,
                             int32_t rank_b, const int64_t *sizes_b,
                             int32_t *rank_out,
                             int64_t sizes_out[ZK_MAX_DIMS]);

/*
 * Forward: out[i] = epi(a[off_a(i)] (op) b[off_b(i)]) for every i of the
 * broadcast shape (Operator chapter, "element-wise operators" and
 * "broadcast": a size-1 or missing operand dim always reads coordinate 0).
 *   a, da / b, db : inputs, any non-negative strides (views, stride 0 ok)
 *   out           : dense row-major, broadcast shape, caller-allocated
 *   stream        : hipStream_t or NULL
 * Aliasing: out may be exactly a (or b) when that operand is dense row-major
 * with the full broadcast shape (in-place); any other overlap of out with an
 * input is ZK_ERR_ALIAS.
 * An empty broadcast shape launches nothing and returns ZK_OK.
 * Errors: ZK_ERR_NULL, ZK_ERR_RANK, ZK_ERR_BAD_SIZE, ZK_ERR_BAD_STRIDE,
 *         ZK_ERR_BROADCAST, ZK_ERR_ALIAS, ZK_ERR_UNSUPPORTED, ZK_ERR_HIP.
 */
zk_status zk_binary_fwd(zk_op op, zk_epi epi, const float *a,
                        const zk_desc *da, const float *b, const zk_desc *db,
                        float *out, void *stream);

/*
 * Backward of y = epi(a (op) b) for the upstream gradient `grad` (dense
 * row-major, broadcast shape).  Local rules (Autograd chapter, "chain rule";
 * Operator chapter, "element-wise operators"; GPU chapter, "OpAdd"; sub and
 * div by calculus):
 *   add: (g, g)   sub: (g, -g)   mul: (g*b, g*a)   div: (g/b, -g*a/b^2)
 * With ZK_EPI_GELU, g is first replaced by g * GeLU'(h), h = a (op) b
 * recomputed in binary32, GeLU'(h) = Phi(h) + h*phi(h).
 * Each input's gradient is then summed over every output position its
 * elements were repeated into (Operator chapter, "broadcast"), and added to
 * the matching acc buffer (Autograd chapter: a tensor reached along several
 * paths gets the sum of the path gradients).
 *   grad_a, grad_b : dense row-major in a's / b's logical shape; NULL = skip
 *   acc_a, acc_b   : NULL (no accumulation), or a dense row-major buffer of
 *                    the gradient's shape; it may be exactly the gradient
 *                    pointer (in-place +=) or, when that operand has the full
 *                    broadcast shape, exactly `grad` (folds an identity path
 *                    without a copy)
 *   workspace      : device scratch owned by the caller.  Pass NULL to query:
 *                    the required size is written to *workspace_bytes and
 *                    nothing is launched.  Otherwise *workspace_bytes is the
 *                    size provided; too small, or a base that is not 8-byte
 *                    aligned (hipMalloc and torch allocations are), ->
 *                    ZK_ERR_WORKSPACE.  The size depends on the shapes only.
 *                    Contents need no initialisation and are garbage
 *                    afterwards.
 * Sums are accumulated in binary64 in an order fixed by the shapes and
 * rounded once to binary32 (bitwise reproducible run to run).
 * Aliasing: outputs may not overlap each other, `grad`, a, b or the
 * workspace, except an output equal to its own acc (ZK_ERR_ALIAS).
 * Errors: as zk_binary_fwd, plus ZK_ERR_WORKSPACE.
 */
zk_status zk_binary_bwd(zk_op op, zk_epi epi, const float *grad,
                        const float *a, const zk_desc *da, const float *b,
                        const zk_desc *db, float *grad_a, const float *acc_a,
                        float *grad_b, const float *acc_b, void *workspace,
                        size_t *workspace_bytes, void *stream);

/*
 * zk_binary_bwd without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The binary64 partial sums go to a device array the
 * library owns, ZK_SCRATCH_BYTES bytes on each GPU it runs on (held until the
 * process ends; its address is looked up on the first call on each device).
 * The call itself allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).
 *   Arguments, results, aliasing and errors as zk_binary_bwd, and:
 *   - a call whose workspace need (what zk_binary_bwd's query reports)
 *     exceeds ZK_SCRATCH_BYTES returns ZK_ERR_WORKSPACE, launching nothing;
 *   - `stream` must belong to the current device (else ZK_ERR_DEVICE).
 * Every call on one GPU shares that GPU's array, which keeps the last
 * call's contents: calls that overlap in time on one GPU (two streams, two
 * host threads) race and give wrong sums; serialise them.  Nothing needs
 * clearing between calls: every partial is written before it is read.
 */
#define ZK_SCRATCH_BYTES ((size_t)16 << 20)
zk_status zk_binary_bwd_noalloc(zk_op op, zk_epi epi, const float *grad,
                                const float *a, const zk_desc *da, const float *b,
                                const zk_desc *db, float *grad_a, const float *acc_a,
                                float *grad_b, const float *acc_b, void *stream);

/*
 * Sum `in` back to `sizes_out` (Operator chapter, "broadcast": SumToSize),
 * i.e. over every dim where the target is 1 or missing.  The target must
 * broadcast to in's shape with in's shape as the result (else ZK_ERR_SHAPE).
 *   in, din   : input view, any non-negative strides
 *   out       : dense row-major, target shape
 *   workspace : as in zk_binary_bwd (NULL queries *workspace_bytes)
 * An empty input writes zeros to a non-empty target.
 * Errors: ZK_ERR_NULL, ZK_ERR_RANK, ZK_ERR_BAD_SIZE, ZK_ERR_BAD_STRIDE,
 *         ZK_ERR_SHAPE, ZK_ERR_ALIAS, ZK_ERR_WORKSPACE, ZK_ERR_HIP.
 */
zk_status zk_reduce_to_shape(const float *in, const zk_desc *din,
                             int32_t rank_out, const int64_t *sizes_out,
                             float *out, void *workspace,
                             size_t *workspace_bytes, void *stream);

/*
 * A tensor and a host scalar (Operator chapter, "element-wise operators":
 * the same operators with one operand a constant):
 *   out = epi(t (op) s), or epi(s (op) t) when scalar_first != 0,
 * for every element of t; out is dense row-major in t's shape.  The
 * scalar travels by value in the kernel arguments (no device copy).
 *   t, dt : tensor, any non-negative strides
 * Aliasing: out may be exactly t when t is dense row-major; other overlaps
 * are ZK_ERR_ALIAS.  Errors: as zk_binary_fwd.
 */
zk_status zk_scalar_fwd(zk_op op, zk_epi epi, const float *t, const zk_desc *dt,
                        float s, int32_t scalar_first, float *out, void *stream);

/*
 * Backward of zk_scalar_fwd w.r.t. the tensor: grad_t = rule(g) (+ acc_t),
 * the operand-t rules of zk_binary_bwd with the scalar as the other operand.
 * A host scalar is a constant and gets no gradient (pass a rank-0 device
 * tensor to zk_binary_bwd when it needs one).  No reduction, no workspace.
 *   grad   : dense row-major, t's shape
 *   grad_t : dense row-major, t's shape; acc_t NULL, a buffer, exactly
 *            grad_t (in place) or exactly grad
 * Errors: as zk_binary_bwd (no ZK_ERR_WORKSPACE).
 */
zk_status zk_scalar_bwd(zk_op op, zk_epi epi, const float *grad, const float *t,
                        const zk_desc *dt, float s, int32_t scalar_first,
                        float *grad_t, const float *acc_t, void *stream);

/*
 * Stand-alone activation y = f(x), f = ZK_EPI_GELU or ZK_EPI_RELU (the
 * epilogues above applied to x itself), and its backward
 * grad_x = g * f'(x) (+ acc_x).  Computed as zk_scalar_fwd / _bwd of
 * x - 0, which is x for every binary32 x (-0, NaN and infinities included).
 * Errors: as zk_scalar_fwd / _bwd; f = ZK_EPI_NONE is ZK_ERR_UNSUPPORTED.
 */
zk_status zk_unary_fwd(zk_epi f, const float *x, const zk_desc *dx, float *out,
                       void *stream);
zk_status zk_unary_bwd(zk_epi f, const float *grad, const float *x,
                       const zk_desc *dx, float *grad_x, const float *acc_x,
                       void *stream);

/*
 * Stride-aware materialisation (Operator chapter, "view backward": the
 * broadcast-to copy that turns a view, e.g. a transposed gradient, into
 * contiguous storage; a View of a non-contiguous input first makes such a
 * row-major copy):
 *   out[i] = in[off(i)] for every i of the target shape (rank_out,
 *   sizes_out), with in broadcast to it (a size-1 or missing input dim
 *   repeats).  With the target equal to in's shape this is a contiguous copy.
 *   in, din : any non-negative strides
 *   out     : dense row-major, target shape, caller-allocated
 * No arithmetic: the copy is bit-exact.  The target must be the broadcast of
 * in's shape with itself, else ZK_ERR_SHAPE.  An empty target launches
 * nothing.  Any overlap of out with in is ZK_ERR_ALIAS.
 * Errors: ZK_ERR_NULL, ZK_ERR_RANK, ZK_ERR_BAD_SIZE, ZK_ERR_BAD_STRIDE,
 *         ZK_ERR_SHAPE, ZK_ERR_ALIAS, ZK_ERR_HIP.
 */
zk_status zk_materialize(const float *in, const zk_desc *din, int32_t rank_out,
                         const int64_t *sizes_out, float *out, void *stream);

/*
 * Fused two-operator expression (Operator chapter, "fusion": several small
 * element-wise operators merged into one execution unit, with the usual
 * forward/backward interface and without changing the math):
 *   out = (a (op1) b) (op2) c,  op1 in {add, sub, mul, div}, op2 in {add, sub}
 * over the broadcast shape of a, b and c (a with b, then with c).  Each
 * operator is still one binary32 operation with its own rounding (no fused
 * multiply-add), so the result equals zk_binary_fwd(op1, a, b) followed by
 * zk_binary_fwd(op2, ., c) bit for bit; the intermediate is never stored.
 *   a, da / b, db / c, dc : inputs, any non-negative strides; c may be the
 *                           same tensor as a (then read once)
 *   out                   : dense row-major, broadcast shape
 * Aliasing: out may be exactly an input that is dense row-major with the
 * full broadcast shape; any other overlap is ZK_ERR_ALIAS.
 * Errors: as zk_binary_fwd; op2 other than add or sub is
 * ZK_ERR_UNSUPPORTED.
 */
zk_status zk_binary2_fwd(zk_op op1, zk_op op2, const float *a,
                         const zk_desc *da, const float *b, const zk_desc *db,
                         const float *c, const zk_desc *dc, float *out,
                         void *stream);

/*
 * Backward of out = (a (op1) b) (op2) c for the upstream gradient `grad`
 * (dense row-major, broadcast shape).  op2 hands g to t = a (op1) b and +g
 * (add) or -g (sub) to c (GPU chapter, "OpAdd"; sub by calculus), so
 *   grad_a, grad_b : zk_binary_bwd's op1 rules applied to the gradient of t,
 *                    which is g summed to t's shape (g itself when t has the
 *                    full broadcast shape), then summed to a's / b's shape
 *   grad_c         : +-g summed to c's shape
 * Each requested gradient is added to its acc as in zk_binary_bwd; NULL
 * gradients are skipped.  When c's gradient has the full shape it is
 * written by the pass that streams g for a and b.
 * A tensor used twice (Autograd chapter, "chain rule", z = x*y + x): when c
 * is the same tensor as a (same pointer and descriptor) with the full
 * broadcast shape and op2 is add, grad_c may be exactly grad_a, with acc_a
 * and acc_c NULL; that buffer receives the sum of both paths.  Likewise for
 * b.  Any other shared gradient buffer is ZK_ERR_UNSUPPORTED (if it is
 * grad_a or grad_b) or ZK_ERR_ALIAS.
 * Workspace protocol as in zk_binary_bwd (NULL queries; size depends on the
 * shapes and on which gradients are requested).
 * Errors: as zk_binary_bwd; op2 other than add or sub is
 * ZK_ERR_UNSUPPORTED.
 */
zk_status zk_binary2_bwd(zk_op op1, zk_op op2, const float *grad,
                         const float *a, const zk_desc *da, const float *b,
                         const zk_desc *db, const float *c, const zk_desc *dc,
                         float *grad_a, const float *acc_a, float *grad_b,
                         const float *acc_b, float *grad_c, const float *acc_c,
                         void *workspace, size_t *workspace_bytes,
                         void *stream);

/*
 * Mean back to a shape (GPU chapter, "reduction": the mean is one of the
 * reductions that combine many inputs into few outputs; GPT chapter,
 * "training loop": the per-token loss is averaged over dim 0):
 *   out[j] = (sum of the in elements that map to j) / count,
 * count = the product of in's sizes over the dims where the target is 1 or
 * missing.  The sum is accumulated in binary64 in an order fixed by the
 * shapes, divided by the count in binary64 and rounded once to binary32.
 * An empty reduced dim gives NaN (0 / 0).  Arguments, workspace protocol
 * (the same size as zk_reduce_to_shape), aliasing and errors as
 * zk_reduce_to_shape.
 */
zk_status zk_mean_to_shape(const float *in, const zk_desc *din, int32_t rank_out,
                           const int64_t *sizes_out, float *out, void *workspace,
                           size_t *workspace_bytes, void *stream);

/*
 * Gradient of zk_mean_to_shape (Autograd chapter, "chain rule": upstream
 * gradient times the local derivative 1 / count):
 *   grad_in[i] = grad[j(i)] / count,
 * one binary32 division by the count rounded to binary32, j(i) the output
 * element that input element i is averaged into.
 *   grad    : dense row-major, shape (rank_out, sizes_out); that shape must
 *             broadcast to (rank_in, sizes_in) with the latter as the
 *             result, else ZK_ERR_SHAPE
 *   grad_in : dense row-major, shape (rank_in, sizes_in), caller-allocated
 * No workspace.  An empty grad_in launches nothing.  Any overlap of grad_in
 * with grad is ZK_ERR_ALIAS.
 * Errors: ZK_ERR_NULL, ZK_ERR_RANK, ZK_ERR_BAD_SIZE, ZK_ERR_SHAPE,
 *         ZK_ERR_ALIAS, ZK_ERR_HIP.
 */
zk_status zk_mean_bwd(const float *grad, int32_t rank_out, const int64_t *sizes_out,
                      int32_t rank_in, const int64_t *sizes_in, float *grad_in,
                      void *stream);

/*
 * Global L2 norm of a list of gradients (GPT chapter, "training loop": the
 * norm of all parameter gradients taken together), and ClipGradNorm: when
 * that norm exceeds max_norm, every gradient is multiplied by the one factor
 * max_norm / (norm + 1e-6), which keeps the overall direction.
 *   count     : number of tensors, >= 0
 *   grads     : host array of `count` device pointers, each a dense binary32
 *               tensor of numels[t] elements (any 4-byte alignment)
 *   numels    : host array of element counts, each >= 0
 *   norm_out  : device pointer to one float: the norm, rounded to binary32
 *   workspace : device scratch owned by the caller; NULL queries
 *               *workspace_bytes (the size depends on numels only; grads
 *               and norm_out are not read then), as in zk_binary_bwd
 * Squares are summed in binary64 in an order fixed by numels, the square
 * root taken in binary64 (bitwise reproducible).  zk_clip_grad_norm then
 * decides on the device, without a host synchronisation: if the binary64
 * norm is greater than max_norm, factor = max_norm / (norm + 1e-6) computed
 * in binary64 and rounded to binary32, and every element becomes
 * g * factor (one binary32 multiply) in place; otherwise nothing is
 * written to the gradients.
 * Aliasing: the tensors may not overlap each other, norm_out or the
 * workspace (ZK_ERR_ALIAS).
 * Errors: ZK_ERR_NULL, ZK_ERR_BAD_SIZE (negative count or numel, or more
 *         than 2^62 elements in all),
 *         ZK_ERR_ALIAS, ZK_ERR_WORKSPACE, ZK_ERR_HIP; zk_clip_grad_norm
 *         also ZK_ERR_UNSUPPORTED for a max_norm that is negative or NaN.
 */
zk_status zk_grad_norm(int32_t count, const float *const *grads, const int64_t *numels,
                       float *norm_out, void *workspace, size_t *workspace_bytes,
                       void *stream);
zk_status zk_clip_grad_norm(int32_t count, float *const *grads, const int64_t *numels,
                            float max_norm, float *norm_out, void *workspace,
                            size_t *workspace_bytes, void *stream);

/*
 * Per-row statistics of a [rows, cols] binary32 matrix whose row r starts at
 * x + r*ld (elements of a row contiguous, ld >= cols), reduced over each row
 * (GPU chapter, "reduction": mean, variance and softmax are reductions;
 * Operator chapter, "fusion": a LayerNorm computes its row statistics inside
 * one operator; GPT chapter, "attention": a softmax over each row of the
 * masked scores).
 * zk_row_moments:        mean[r] = sum_j x[r,j] / cols,
 *                        var[r]  = sum_j (x[r,j] - mean)^2 / cols (biased),
 *                        both in binary64 (two passes), rounded once; an empty
 *                        row gives NaN.
 * zk_row_softmax_stats:  rowmax[r] = max_j x[r,j] (exact; NaN if the row holds
 *                        a NaN; -inf for an empty row),
 *                        sumexp[r] = sum_j exp(x[r,j] - rowmax[r]), each term
 *                        with relative error below 2e-7, summed in binary64,
 *                        rounded once (0 for an empty row; NaN for a row of
 *                        -inf).
 * Outputs are dense float vectors of `rows` elements, caller-allocated.  Rows
 * of up to 4096 elements are read once, longer rows twice.  No workspace.
 * Aliasing: the outputs may not overlap each other or the extent of x
 * (ZK_ERR_ALIAS).  Errors: ZK_ERR_BAD_SIZE (negative rows or cols),
 * ZK_ERR_BAD_STRIDE (ld < cols, or (rows - 1) * ld + cols above 2^62),
 * ZK_ERR_NULL, ZK_ERR_ALIAS, ZK_ERR_HIP.
 */
zk_status zk_row_moments(const float *x, int64_t rows, int64_t cols, int64_t ld, float *mean,
                         float *var, void *stream);
zk_status zk_row_softmax_stats(const float *x, int64_t rows, int64_t cols, int64_t ld,
                               float *rowmax, float *sumexp, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *zk_status_string(zk_status s);

/*
 * Debug pointer checks (GPU chapter, "kernel dispatch": a call whose
 * tensors live on different devices faults).  mode 1 turns them on, 0 off,
 * -1 leaves them as they are; returns the mode in effect before the call.
 * Until the first zk_set_debug, the mode is 1 when the environment variable
 * ZK_DEBUG is "1" at the library's first call that consults it, else 0.
 * While on, every computing call (after validating its arguments) asks
 * hipPointerGetAttributes about each non-NULL pointer it would read or write
 * (the workspace too when the call needs one) and hipStreamGetDevice (or,
 * for the NULL stream, hipGetDevice) about the stream, and returns
 * ZK_ERR_DEVICE without launching anything unless every pointer is device
 * memory of the stream's device or managed memory.  Off, no check is made
 * and no runtime call is added.  Thread-safe (an atomic flag).
 */
int32_t zk_set_debug(int32_t mode);

/*
 * Host-only inspection of the launch plan a call would use, for tests and
 * tooling.  kind: 0 = zk_binary_fwd, 1 = zk_binary_bwd (both grads
 * requested), 2 = zk_reduce_to_shape (db holds the target shape, strides
 * ignored).  Fills *info; touches no GPU.
 */
typedef struct {
  int32_t kernel;              /* main kernel class, see zk_kernel_name   */
  int32_t kernel2;             /* second kernel class, -1 if none         */
  int32_t rank;                /* canonical rank after dropping/coalescing */
  int64_t sizes[ZK_MAX_DIMS];  /* canonical sizes                         */
  int64_t strides[3][ZK_MAX_DIMS]; /* canonical strides: [0] out/grad,
                                      [1] a (or reduce input), [2] b (or
                                      reduce target, dense, 0 = reduced)  */
  int32_t index64;             /* 1 when 64-bit index math is used        */
  int32_t vec;                 /* elements per vector access (4 or 1)     */
  int64_t partials;            /* partial sums per reduced element        */
  size_t workspace_bytes;      /* workspace the call needs                */
} zk_plan_info;

zk_status zk_plan_describe(int32_t kind, zk_op op, zk_epi epi,
                           const zk_desc *da, const zk_desc *db,
                           zk_plan_info *info);

/* Name of a kernel class id reported by zk_plan_describe. */
const char *zk_kernel_name(int32_t kernel);

/*
 * Optional per-kernel timing for measurement tools (off by default).
 * zk_profile_start(capacity) creates `capacity` pairs of HIP events on the
 * current device (a host call: make it before any timed or captured region)
 * and clears the log.  While started, every kernel the library launches is
 * bracketed by an event pair recorded on the kernel's own stream, until the
 * pairs run out.  zk_profile_stop() stops recording.  After the caller has
 * synchronised the streams, zk_profile_read() copies up to `max` records
 * (kernel class id and elapsed milliseconds, in launch order) and writes
 * their number to *count.  Not for concurrent use from several host threads
 * while started.  Errors: ZK_ERR_NULL, ZK_ERR_HIP.
 */
zk_status zk_profile_start(int32_t capacity);
zk_status zk_profile_stop(void);
zk_status zk_profile_read(int32_t max, int32_t *kernel_ids, float *ms,
                          int32_t *count);

#ifdef __cplusplus
}
#endif

#endif /* ZK_H_ */
