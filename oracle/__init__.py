"""Plain CPU oracle for broadcasting binary operators and their backward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does and
shares no code with it.  The arithmetic lives in ``oracle.c`` (plain C built
by gcc with -O2 -ffp-contract=off, no fast-math); this module only marshals
numpy arrays into it.

Descriptors are ``(storage, sizes, strides)`` with sizes/strides counted in
elements (the "Zero" book, Tensor chapter, "shape and strides" section).
A plain C-contiguous numpy array may be passed directly.
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SRC_PATH = os.path.join(HERE, "oracle.c")

ADD, SUB, MUL, DIV = 0, 1, 2, 3
EPI_NONE, EPI_GELU, EPI_RELU = 0, 1, 2
OPS = {"add": ADD, "sub": SUB, "mul": MUL, "div": DIV}

OK, ERR_BROADCAST, ERR_RANK, ERR_SIZE, ERR_ARG = 0, 1, 2, 3, 4
MAX_DIMS = 8


class OracleError(RuntimeError):
    def __init__(self, code):
        super().__init__(f"oracle status {code}")
        self.code = code


def build(force=True):
    """Compile liboracle.so with gcc (plain C, OpenMP over output elements)."""
    if not force and os.path.exists(LIB_PATH) and (
            os.path.getmtime(LIB_PATH) >= os.path.getmtime(SRC_PATH)):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-msse2", "-mfpmath=sse", "-fopenmp", "-fPIC", "-shared",
           "-D_GNU_SOURCE", SRC_PATH, "-o", tmp, "-lquadmath", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _Desc(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32),
                ("sizes", ctypes.c_int64 * MAX_DIMS),
                ("strides", ctypes.c_int64 * MAX_DIMS)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.or_broadcast_shape.argtypes = [ctypes.c_int, P, ctypes.c_int, P, P, P]
        L.or_fwd.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P, P, P]
        L.or_fwd_at.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P, P, I64, P, P]
        L.or_bwd.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P, P, P, P, P,
                             P, P, P, P, P, P]
        L.or_bwd_at.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P,
                                P, P, P, I64, P, P, P, P]
        L.or_reduce.argtypes = [P, P, ctypes.c_int, P, P, P, P]
        L.or_fwd2.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P, P, P, P, P]
        L.or_fwd2_at.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P, P, P, P, I64, P, P]
        L.or_bwd2.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P, P, P, P,
                              P, P, P, P, P, P, P, P, P, P, P, P, P]
        L.or_bwd2_at.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 P, P, P, P, P, P, P, P, I64, P, P, P, P]
        L.or_materialize.argtypes = [P, P, ctypes.c_int, P, P]
        L.or_mean.argtypes = [P, P, ctypes.c_int, P, P, P, P]
        L.or_mean_bwd.argtypes = [P, ctypes.c_int, P, ctypes.c_int, P, P]
        L.or_grad_norm.argtypes = [ctypes.c_int, P, P]
        L.or_grad_norm.restype = ctypes.c_double
        L.or_clip_grad_norm.argtypes = [ctypes.c_int, P, P, ctypes.c_double, P, P]
        L.or_clip_grad_norm.restype = ctypes.c_double
        L.or_row_moments.argtypes = [P, I64, I64, I64, P, P, P, P, P]
        L.or_row_softmax_stats.argtypes = [P, I64, I64, I64, P, P, P]
        L.or_relu32.argtypes = [ctypes.c_float]
        L.or_relu32.restype = ctypes.c_float
        L.or_gelu32.argtypes = [ctypes.c_float]
        L.or_gelu32.restype = ctypes.c_float
        L.or_gelu32_q.argtypes = [ctypes.c_float]
        L.or_gelu32_q.restype = ctypes.c_float
        L.or_gelu_tie_scan.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_double,
                                       P, I64]
        L.or_gelu_tie_scan.restype = I64
        L.or_phi_cdf.argtypes = [ctypes.c_double]
        L.or_phi_cdf.restype = ctypes.c_double
        L.or_phi_pdf.argtypes = [ctypes.c_double]
        L.or_phi_pdf.restype = ctypes.c_double
        L.or_set_threads.argtypes = [ctypes.c_int]
        L.or_get_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def set_threads(n):
    lib().or_set_threads(int(n))


def get_threads():
    return lib().or_get_threads()


class View:
    """A strided fp32 view: ``storage`` (1-D float32 array) read through
    ``sizes``/``strides`` (elements) from ``offset``."""

    def __init__(self, storage, sizes, strides, offset=0):
        self.storage = np.ascontiguousarray(storage, dtype=np.float32).reshape(-1)
        self.sizes = tuple(int(s) for s in sizes)
        self.strides = tuple(int(s) for s in strides)
        self.offset = int(offset)

    @property
    def shape(self):
        return self.sizes


def _as_view(x):
    if isinstance(x, View):
        return x
    x = np.asarray(x, dtype=np.float32)
    if not x.flags.c_contiguous:
        x = np.ascontiguousarray(x)
    st, s = [], 1
    for n in reversed(x.shape):
        st.append(s)
        s *= n
    return View(x.reshape(-1), x.shape, tuple(reversed(st)))


def _desc(v):
    d = _Desc()
    d.rank = len(v.sizes)
    for k, (n, s) in enumerate(zip(v.sizes, v.strides)):
        d.sizes[k] = n
        d.strides[k] = s
    return d


def _ptr(v):
    if v.storage.size == 0:
        return None
    return v.storage.ctypes.data + 4 * v.offset


def _i64(seq):
    arr = (ctypes.c_int64 * max(1, len(seq)))()
    for k, s in enumerate(seq):
        arr[k] = int(s)
    return arr


def _check(code):
    if code != OK:
        raise OracleError(code)


def broadcast_shape(sa, sb):
    ro = ctypes.c_int(0)
    no = (ctypes.c_int64 * MAX_DIMS)()
    code = lib().or_broadcast_shape(len(sa), _i64(sa), len(sb), _i64(sb),
                                    ctypes.byref(ro), no)
    _check(code)
    return tuple(no[k] for k in range(ro.value))


def _op(op):
    return OPS[op] if isinstance(op, str) else int(op)


def fwd(op, a, b, epi=EPI_NONE):
    """out = a (op) b in the broadcast shape, one binary32 op per element
    (optionally followed by GeLU)."""
    va, vb = _as_view(a), _as_view(b)
    shape = broadcast_shape(va.sizes, vb.sizes)
    out = np.empty(shape, dtype=np.float32)
    da, db = _desc(va), _desc(vb)
    _check(lib().or_fwd(_op(op), epi, _ptr(va), ctypes.byref(da), _ptr(vb),
                        ctypes.byref(db), out.ctypes.data if out.size else None))
    return out


def fwd_at(op, a, b, pos, epi=EPI_NONE):
    """Forward at flat output positions ``pos`` only."""
    va, vb = _as_view(a), _as_view(b)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    out = np.empty(pos.shape, dtype=np.float32)
    da, db = _desc(va), _desc(vb)
    _check(lib().or_fwd_at(_op(op), epi, _ptr(va), ctypes.byref(da), _ptr(vb),
                           ctypes.byref(db), pos.size, pos.ctypes.data,
                           out.ctypes.data))
    return out


class Grad:
    """Backward result of one operand: fp32 value, its binary64 sum and the
    sum of |terms| (the tolerance base)."""

    def __init__(self, f32, f64, absum):
        self.f32, self.f64, self.abs = f32, f64, absum


def bwd(op, g, a, b, acc_a=None, acc_b=None, want=(True, True), epi=EPI_NONE):
    """Gradients of sum(g * f(a, b)) w.r.t. a and b (dense, in a's / b's
    shape), each accumulated onto ``acc_*`` when given."""
    va, vb = _as_view(a), _as_view(b)
    g = np.ascontiguousarray(g, dtype=np.float32)
    da, db = _desc(va), _desc(vb)
    res = []
    bufs = []
    for k, (v, w) in enumerate(((va, want[0]), (vb, want[1]))):
        if not w:
            bufs.append((None, None, None))
            continue
        f32 = np.empty(v.sizes, dtype=np.float32)
        f64 = np.empty(v.sizes, dtype=np.float64)
        ab = np.empty(v.sizes, dtype=np.float64)
        bufs.append((f32, f64, ab))

    def p(x):
        return None if x is None or x.size == 0 else x.ctypes.data

    accs = [None if x is None else np.ascontiguousarray(x, dtype=np.float32)
            for x in (acc_a, acc_b)]
    _check(lib().or_bwd(_op(op), epi, p(g), _ptr(va), ctypes.byref(da), _ptr(vb),
                        ctypes.byref(db), p(accs[0]), p(accs[1]),
                        p(bufs[0][0]), p(bufs[0][1]), p(bufs[0][2]),
                        p(bufs[1][0]), p(bufs[1][1]), p(bufs[1][2])))
    for f32, f64, ab in bufs:
        res.append(None if f32 is None else Grad(f32, f64, ab))
    return res[0], res[1]


def bwd_at(op, which, g, a, b, pos, acc=None, epi=EPI_NONE):
    """Gradient of operand ``which`` (0 = a, 1 = b) at dense positions ``pos``."""
    va, vb = _as_view(a), _as_view(b)
    g = np.ascontiguousarray(g, dtype=np.float32)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    da, db = _desc(va), _desc(vb)
    f32 = np.empty(pos.shape, dtype=np.float32)
    f64 = np.empty(pos.shape, dtype=np.float64)
    ab = np.empty(pos.shape, dtype=np.float64)
    accp = None
    if acc is not None:
        acc = np.ascontiguousarray(acc, dtype=np.float32)
        accp = acc.ctypes.data
    _check(lib().or_bwd_at(_op(op), epi, which, g.ctypes.data, _ptr(va),
                           ctypes.byref(da), _ptr(vb), ctypes.byref(db), accp,
                           pos.size, pos.ctypes.data, f32.ctypes.data,
                           f64.ctypes.data, ab.ctypes.data))
    return Grad(f32, f64, ab)


def reduce_to_shape(x, shape):
    """Sum ``x`` back to ``shape`` (which must broadcast to x's shape)."""
    v = _as_view(x)
    d = _desc(v)
    shape = tuple(int(s) for s in shape)
    f32 = np.empty(shape, dtype=np.float32)
    f64 = np.empty(shape, dtype=np.float64)
    ab = np.empty(shape, dtype=np.float64)

    def p(z):
        return None if z.size == 0 else z.ctypes.data

    _check(lib().or_reduce(_ptr(v), ctypes.byref(d), len(shape), _i64(shape),
                           p(f32), p(f64), p(ab)))
    return Grad(f32, f64, ab)


def mean_to_shape(x, shape):
    """Mean of ``x`` over the dims where ``shape`` (which must broadcast to
    x's shape) is 1 or missing.  Returns a Grad: fp32 value, binary64 value
    and sum|x| / count (the tolerance base)."""
    v = _as_view(x)
    d = _desc(v)
    shape = tuple(int(s) for s in shape)
    f32 = np.empty(shape, dtype=np.float32)
    f64 = np.empty(shape, dtype=np.float64)
    ab = np.empty(shape, dtype=np.float64)

    def p(z):
        return None if z.size == 0 else z.ctypes.data

    _check(lib().or_mean(_ptr(v), ctypes.byref(d), len(shape), _i64(shape),
                         p(f32), p(f64), p(ab)))
    return Grad(f32, f64, ab)


def mean_bwd(g, shape_in):
    """Gradient of mean_to_shape: g (dense, the reduced shape) divided by the
    count and repeated over ``shape_in``."""
    g = np.array(g, dtype=np.float32, order="C")
    shape_in = tuple(int(s) for s in shape_in)
    out = np.empty(shape_in, dtype=np.float32)
    _check(lib().or_mean_bwd(g.ctypes.data if g.size else None, g.ndim, _i64(g.shape),
                             len(shape_in), _i64(shape_in),
                             out.ctypes.data if out.size else None))
    return out


def _tensor_list(gs):
    arrs = [np.array(x, dtype=np.float32, order="C") for x in gs]
    ptrs = (ctypes.c_void_p * max(1, len(arrs)))(
        *[a.ctypes.data if a.size else None for a in arrs])
    ns = _i64([a.size for a in arrs])
    return arrs, ptrs, ns


def grad_norm(gs):
    """Global L2 norm (binary64) of a list of gradients."""
    arrs, ptrs, ns = _tensor_list(gs)
    return float(lib().or_grad_norm(len(arrs), ptrs, ns))


def clip_grad_norm(gs, max_norm):
    """ClipGradNorm on copies of ``gs``: returns (scaled copies, norm as
    binary64, whether it scaled, the binary32 factor)."""
    arrs, ptrs, ns = _tensor_list(gs)
    arrs = [a.copy() for a in arrs]
    ptrs = (ctypes.c_void_p * max(1, len(arrs)))(
        *[a.ctypes.data if a.size else None for a in arrs])
    clipped = ctypes.c_int(0)
    factor = ctypes.c_float(0.0)
    norm = lib().or_clip_grad_norm(len(arrs), ptrs, ns, float(max_norm),
                                   ctypes.byref(clipped), ctypes.byref(factor))
    return arrs, float(norm), bool(clipped.value), np.float32(factor.value)


def _rows(x, cols=None, ld=None):
    """A [rows, cols] matrix given as 2-D array, or as flat storage with an
    explicit row pitch ``ld``."""
    x = np.array(x, dtype=np.float32, order="C")
    if ld is None:
        rows, cols = x.shape
        ld = cols
    else:
        rows = (x.size - cols) // ld + 1 if x.size else 0
    return x.reshape(-1), int(rows), int(cols), int(ld)


def row_moments(x, cols=None, ld=None):
    """Per-row mean and biased variance: (Grad of the mean with sum|x|/cols as
    its tolerance base, Grad of the variance with its own value as base)."""
    flat, rows, cols, ld = _rows(x, cols, ld)
    m32, v32 = np.empty(rows, np.float32), np.empty(rows, np.float32)
    m64, v64, am = np.empty(rows), np.empty(rows), np.empty(rows)

    def p(z):
        return z.ctypes.data if z.size else None

    _check(lib().or_row_moments(p(flat), rows, cols, ld, p(m32), p(v32), p(m64), p(v64),
                                p(am)))
    return Grad(m32, m64, am), Grad(v32, v64, v64.copy())


def row_softmax_stats(x, cols=None, ld=None):
    """Per-row max (binary32, exact) and Grad of sum exp(x - max) (its own
    value as the tolerance base: every term is positive)."""
    flat, rows, cols, ld = _rows(x, cols, ld)
    mx, s32, s64 = np.empty(rows, np.float32), np.empty(rows, np.float32), np.empty(rows)

    def p(z):
        return z.ctypes.data if z.size else None

    _check(lib().or_row_softmax_stats(p(flat), rows, cols, ld, p(mx), p(s32), p(s64)))
    return mx, Grad(s32, s64, s64.copy())


def materialize(x, shape=None):
    """Dense row-major copy of the view ``x`` broadcast to ``shape``."""
    v = _as_view(x)
    shape = tuple(v.sizes) if shape is None else tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float32)
    d = _desc(v)
    _check(lib().or_materialize(_ptr(v), ctypes.byref(d), len(shape), _i64(shape),
                                out.ctypes.data if out.size else None))
    return out


def broadcast_shape3(sa, sb, sc):
    return broadcast_shape(broadcast_shape(sa, sb), sc)


def fwd2(op1, op2, a, b, c):
    """out = (a (op1) b) (op2) c in the broadcast shape of a, b and c: the two
    operators one after the other, each one binary32 operation."""
    va, vb, vc = _as_view(a), _as_view(b), _as_view(c)
    shape = broadcast_shape3(va.sizes, vb.sizes, vc.sizes)
    out = np.empty(shape, dtype=np.float32)
    da, db, dc = _desc(va), _desc(vb), _desc(vc)
    _check(lib().or_fwd2(_op(op1), _op(op2), _ptr(va), ctypes.byref(da), _ptr(vb),
                         ctypes.byref(db), _ptr(vc), ctypes.byref(dc),
                         out.ctypes.data if out.size else None))
    return out


def fwd2_at(op1, op2, a, b, c, pos):
    """Fused forward at flat output positions ``pos`` only."""
    va, vb, vc = _as_view(a), _as_view(b), _as_view(c)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    out = np.empty(pos.shape, dtype=np.float32)
    da, db, dc = _desc(va), _desc(vb), _desc(vc)
    _check(lib().or_fwd2_at(_op(op1), _op(op2), _ptr(va), ctypes.byref(da), _ptr(vb),
                            ctypes.byref(db), _ptr(vc), ctypes.byref(dc), pos.size,
                            pos.ctypes.data, out.ctypes.data))
    return out


_TIE = {None: -1, "a": 0, "b": 1}


def bwd2(op1, op2, g, a, b, c, acc=(None, None, None), want=(True, True, True), tie=None):
    """Gradients of sum(g * ((a op1 b) op2 c)) w.r.t. a, b and c (dense, in
    each operand's shape), each accumulated onto its acc when given.  tie
    "a" / "b": c is the same tensor as a / b; that operand's gradient then
    has both paths and the c gradient is None."""
    va, vb, vc = _as_view(a), _as_view(b), _as_view(c)
    g = np.ascontiguousarray(g, dtype=np.float32)
    da, db, dc = _desc(va), _desc(vb), _desc(vc)
    t = _TIE[tie]
    bufs = []
    for k, (v, w) in enumerate(((va, want[0]), (vb, want[1]), (vc, want[2] and t < 0))):
        if not w:
            bufs.append((None, None, None))
            continue
        bufs.append((np.empty(v.sizes, dtype=np.float32), np.empty(v.sizes, dtype=np.float64),
                     np.empty(v.sizes, dtype=np.float64)))

    def p(x):
        return None if x is None or x.size == 0 else x.ctypes.data

    accs = [None if x is None else np.ascontiguousarray(x, dtype=np.float32) for x in acc]
    _check(lib().or_bwd2(_op(op1), _op(op2), t, p(g), _ptr(va), ctypes.byref(da), _ptr(vb),
                         ctypes.byref(db), _ptr(vc), ctypes.byref(dc), p(accs[0]),
                         p(accs[1]), p(accs[2]), *[p(x) for buf in bufs for x in buf]))
    return tuple(None if f32 is None else Grad(f32, f64, ab) for f32, f64, ab in bufs)


def bwd2_at(op1, op2, which, g, a, b, c, pos, acc=None, tie=None):
    """One gradient of the fused expression (which: 0 = a, 1 = b, 2 = c) at
    dense positions ``pos``."""
    va, vb, vc = _as_view(a), _as_view(b), _as_view(c)
    g = np.ascontiguousarray(g, dtype=np.float32)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    da, db, dc = _desc(va), _desc(vb), _desc(vc)
    f32 = np.empty(pos.shape, dtype=np.float32)
    f64 = np.empty(pos.shape, dtype=np.float64)
    ab = np.empty(pos.shape, dtype=np.float64)
    accp = None
    if acc is not None:
        acc = np.ascontiguousarray(acc, dtype=np.float32)
        accp = acc.ctypes.data
    _check(lib().or_bwd2_at(_op(op1), _op(op2), which, _TIE[tie], g.ctypes.data, _ptr(va),
                            ctypes.byref(da), _ptr(vb), ctypes.byref(db), _ptr(vc),
                            ctypes.byref(dc), accp, pos.size, pos.ctypes.data,
                            f32.ctypes.data, f64.ctypes.data, ab.ctypes.data))
    return Grad(f32, f64, ab)


def relu32(h):
    return np.float32(lib().or_relu32(float(h)))


def gelu32(h):
    return np.float32(lib().or_gelu32(float(h)))


def gelu32_q(h):
    """GeLU through the binary128 evaluation alone (the path the oracle takes
    where binary64 cannot decide the rounding)."""
    return np.float32(lib().or_gelu32_q(float(h)))


def gelu_tie_scan(lo_bits, hi_bits, rel, max_out=1 << 20):
    """Binary32 arguments (as uint32 bit patterns, bit patterns lo <= u < hi of
    one sign) whose binary64 GeLU lies within ``rel`` of a binary32 rounding
    midpoint; returns (patterns found, up to max_out; total count)."""
    out = np.empty(int(max_out), dtype=np.uint32)
    n = lib().or_gelu_tie_scan(int(lo_bits), int(hi_bits), float(rel), out.ctypes.data,
                               int(max_out))
    return np.sort(out[:min(n, max_out)]), int(n)


def phi_cdf(h):
    return lib().or_phi_cdf(float(h))


def phi_pdf(h):
    return lib().or_phi_pdf(float(h))
