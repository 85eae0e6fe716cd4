"""ctypes binding of libzk.so (include/zk.h).

Argument marshalling only: torch tensors supply device pointers, sizes and
strides (in elements) and the current HIP stream; outputs and workspaces are
allocated with torch when the caller does not pass them.  Every step of the
computation runs in the library's gfx950 kernels.  There is no fallback: if
libzk.so is missing, every call raises.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libzk.so")
MAX_DIMS = 8

OPS = {"add": 0, "sub": 1, "mul": 2, "div": 3}
EPIS = {"none": 0, "gelu": 1, "relu": 2}

STATUS = {0: "ZK_OK", 1: "ZK_ERR_NULL", 2: "ZK_ERR_RANK", 3: "ZK_ERR_BAD_SIZE",
          4: "ZK_ERR_BAD_STRIDE", 5: "ZK_ERR_BROADCAST", 6: "ZK_ERR_ALIAS",
          7: "ZK_ERR_WORKSPACE", 8: "ZK_ERR_UNSUPPORTED", 9: "ZK_ERR_HIP",
          10: "ZK_ERR_SHAPE", 11: "ZK_ERR_DEVICE"}
ERR = {v: k for k, v in STATUS.items()}

# exported symbols declared in include/zk.h
SYMBOLS = ("zk_broadcast_shape", "zk_binary_fwd", "zk_binary_bwd", "zk_binary_bwd_noalloc",
           "zk_reduce_to_shape", "zk_materialize", "zk_binary2_fwd", "zk_binary2_bwd",
           "zk_scalar_fwd", "zk_scalar_bwd", "zk_unary_fwd", "zk_unary_bwd",
           "zk_mean_to_shape", "zk_mean_bwd", "zk_grad_norm", "zk_clip_grad_norm",
           "zk_row_moments", "zk_row_softmax_stats",
           "zk_status_string", "zk_plan_describe", "zk_kernel_name", "zk_set_debug",
           "zk_profile_start", "zk_profile_stop", "zk_profile_read")


class ZkError(RuntimeError):
    def __init__(self, code, what=""):
        self.code = code
        self.name = STATUS.get(code, str(code))
        msg = f"{what}: {self.name}"
        try:
            msg += f" ({lib().zk_status_string(code).decode()})"
        except Exception:  # noqa: BLE001 - message only
            pass
        super().__init__(msg)


class Desc(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32),
                ("sizes", ctypes.c_int64 * MAX_DIMS),
                ("strides", ctypes.c_int64 * MAX_DIMS)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("kernel2", ctypes.c_int32),
                ("rank", ctypes.c_int32),
                ("sizes", ctypes.c_int64 * MAX_DIMS),
                ("strides", (ctypes.c_int64 * MAX_DIMS) * 3),
                ("index64", ctypes.c_int32), ("vec", ctypes.c_int32),
                ("partials", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_size_t)]


_lib = None


def lib():
    """Load libzk.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m broadcast_autograd_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I32 = ctypes.c_int32
        L.zk_broadcast_shape.argtypes = [I32, P, I32, P, P, P]
        L.zk_binary_fwd.argtypes = [I32, I32, P, P, P, P, P, P]
        L.zk_binary_bwd.argtypes = [I32, I32, P, P, P, P, P, P, P, P, P, P, P, P]
        L.zk_binary_bwd_noalloc.argtypes = [I32, I32, P, P, P, P, P, P, P, P, P, P]
        L.zk_reduce_to_shape.argtypes = [P, P, I32, P, P, P, P, P]
        L.zk_materialize.argtypes = [P, P, I32, P, P, P]
        F32 = ctypes.c_float
        L.zk_scalar_fwd.argtypes = [I32, I32, P, P, F32, I32, P, P]
        L.zk_scalar_bwd.argtypes = [I32, I32, P, P, P, F32, I32, P, P, P]
        L.zk_unary_fwd.argtypes = [I32, P, P, P, P]
        L.zk_unary_bwd.argtypes = [I32, P, P, P, P, P, P]
        L.zk_binary2_fwd.argtypes = [I32, I32, P, P, P, P, P, P, P, P]
        L.zk_binary2_bwd.argtypes = [I32, I32] + [P] * 16
        L.zk_mean_to_shape.argtypes = [P, P, I32, P, P, P, P, P]
        L.zk_mean_bwd.argtypes = [P, I32, P, I32, P, P, P]
        L.zk_grad_norm.argtypes = [I32, P, P, P, P, P, P]
        L.zk_clip_grad_norm.argtypes = [I32, P, P, F32, P, P, P, P]
        I64 = ctypes.c_int64
        L.zk_row_moments.argtypes = [P, I64, I64, I64, P, P, P]
        L.zk_row_softmax_stats.argtypes = [P, I64, I64, I64, P, P, P]
        L.zk_status_string.argtypes = [I32]
        L.zk_status_string.restype = ctypes.c_char_p
        L.zk_plan_describe.argtypes = [I32, I32, I32, P, P, P]
        L.zk_profile_start.argtypes = [I32]
        L.zk_profile_stop.argtypes = []
        L.zk_profile_read.argtypes = [I32, P, P, P]
        L.zk_kernel_name.argtypes = [I32]
        L.zk_set_debug.argtypes = [I32]
        L.zk_kernel_name.restype = ctypes.c_char_p
        for name in SYMBOLS:
            getattr(L, name).restype = getattr(L, name).restype or ctypes.c_int32
        L.zk_status_string.restype = ctypes.c_char_p
        L.zk_kernel_name.restype = ctypes.c_char_p
        _lib = L
    return _lib


def set_debug(mode):
    """Debug pointer checks: 1 on, 0 off, -1 unchanged; returns the previous
    mode (ZK_DEBUG=1 in the environment turns them on by default)."""
    return int(lib().zk_set_debug(int(mode)))


def _check(code, what):
    if code != 0:
        raise ZkError(code, what)


def make_desc(sizes, strides=None):
    """zk_desc from sizes and strides (elements); dense row-major if no
    strides are given."""
    sizes = [int(s) for s in sizes]
    if strides is None:
        strides, s = [], 1
        for n in reversed(sizes):
            strides.append(s)
            s *= n
        strides = list(reversed(strides))
    d = Desc()
    d.rank = len(sizes)
    for k, (n, s) in enumerate(zip(sizes, strides)):
        if k < MAX_DIMS:
            d.sizes[k] = n
            d.strides[k] = int(s)
    return d


def desc_of(t):
    return make_desc(t.shape, t.stride())


def _i64(seq):
    arr = (ctypes.c_int64 * max(1, len(seq)))()
    for k, s in enumerate(seq):
        arr[k] = int(s)
    return arr


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _keep(stream, *tensors):
    """Tensors this wrapper allocated come from torch's caching allocator on
    the current stream.  When the library runs on another stream, record that
    use, so that a block freed on return (a workspace) or later is not handed
    out again before that stream's kernels are done with it."""
    if stream is None:
        return
    import torch
    if stream == torch.cuda.current_stream(stream.device):
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _op(op):
    return OPS[op] if isinstance(op, str) else int(op)


def _epi(epi):
    return EPIS[epi] if isinstance(epi, str) else int(epi)


def broadcast_shape(sa, sb):
    ro = ctypes.c_int32(0)
    out = (ctypes.c_int64 * MAX_DIMS)()
    _check(lib().zk_broadcast_shape(len(sa), _i64(sa), len(sb), _i64(sb),
                                    ctypes.byref(ro), out), "zk_broadcast_shape")
    return tuple(out[k] for k in range(ro.value))


def binary_fwd(op, a, b, out=None, epi="none", stream=None):
    """out = epi(a (op) b) in the broadcast shape (dense row-major)."""
    import torch
    if out is None:
        shape = broadcast_shape(a.shape, b.shape)
        out = torch.empty(shape, dtype=torch.float32, device=a.device)
        _keep(stream, out)
    da, db = desc_of(a), desc_of(b)
    _check(lib().zk_binary_fwd(_op(op), _epi(epi), _ptr(a), ctypes.byref(da),
                               _ptr(b), ctypes.byref(db), _ptr(out),
                               _stream(stream)), "zk_binary_fwd")
    return out


def _workspace(nbytes, device):
    import torch
    return torch.empty(max(256, int(nbytes)), dtype=torch.uint8, device=device)


def bwd_workspace_bytes(op, a, b, need_a=True, need_b=True, epi="none"):
    """Workspace zk_binary_bwd needs for these operands (no launch)."""
    da, db = desc_of(a), desc_of(b)
    nbytes = ctypes.c_size_t(0)
    # Any non-NULL marker pointer requests the gradient in the query.
    mark = ctypes.c_void_p(16)
    _check(lib().zk_binary_bwd(_op(op), _epi(epi), mark, mark, ctypes.byref(da),
                               mark, ctypes.byref(db), mark if need_a else None,
                               None, mark if need_b else None, None, None,
                               ctypes.byref(nbytes), None), "zk_binary_bwd(query)")
    return nbytes.value


def binary_bwd(op, grad, a, b, need_a=True, need_b=True, grad_a=None,
               grad_b=None, acc_a=None, acc_b=None, epi="none", workspace=None,
               stream=None):
    """Gradients of epi(a (op) b) for the upstream ``grad``; returns
    (grad_a, grad_b), each dense in its operand's shape (None if not
    requested)."""
    import torch
    if need_a and grad_a is None:
        grad_a = torch.empty(a.shape, dtype=torch.float32, device=grad.device)
        _keep(stream, grad_a)
    if need_b and grad_b is None:
        grad_b = torch.empty(b.shape, dtype=torch.float32, device=grad.device)
        _keep(stream, grad_b)
    if not need_a:
        grad_a = None
    if not need_b:
        grad_b = None
    da, db = desc_of(a), desc_of(b)
    nbytes = ctypes.c_size_t(0)
    L = lib()
    args = (_op(op), _epi(epi), _ptr(grad), _ptr(a), ctypes.byref(da), _ptr(b),
            ctypes.byref(db), _ptr(grad_a), _ptr(acc_a), _ptr(grad_b), _ptr(acc_b))
    if workspace is None:
        _check(L.zk_binary_bwd(*args, None, ctypes.byref(nbytes), None),
               "zk_binary_bwd(query)")
        workspace = _workspace(nbytes.value, grad.device)
        _keep(stream, workspace)
    nbytes.value = workspace.numel() * workspace.element_size()
    _check(L.zk_binary_bwd(*args, _ptr(workspace), ctypes.byref(nbytes),
                           _stream(stream)), "zk_binary_bwd")
    return grad_a, grad_b


def scalar_fwd(op, t, s, scalar_first=False, out=None, epi="none", stream=None):
    """out = epi(t (op) s), or epi(s (op) t), s a host float (by value)."""
    import torch
    if out is None:
        out = torch.empty(tuple(t.shape), dtype=torch.float32, device=t.device)
        _keep(stream, out)
    d = desc_of(t)
    _check(lib().zk_scalar_fwd(_op(op), _epi(epi), _ptr(t), ctypes.byref(d), float(s),
                               1 if scalar_first else 0, _ptr(out), _stream(stream)),
           "zk_scalar_fwd")
    return out


def scalar_bwd(op, grad, t, s, scalar_first=False, grad_t=None, acc_t=None, epi="none",
               stream=None):
    """Gradient of epi(t (op) s) (or epi(s (op) t)) w.r.t. the tensor t."""
    import torch
    if grad_t is None:
        grad_t = torch.empty(tuple(t.shape), dtype=torch.float32, device=grad.device)
        _keep(stream, grad_t)
    d = desc_of(t)
    _check(lib().zk_scalar_bwd(_op(op), _epi(epi), _ptr(grad), _ptr(t), ctypes.byref(d),
                               float(s), 1 if scalar_first else 0, _ptr(grad_t), _ptr(acc_t),
                               _stream(stream)), "zk_scalar_bwd")
    return grad_t


def unary_fwd(f, x, out=None, stream=None):
    """out = f(x), f "gelu" or "relu"."""
    import torch
    if out is None:
        out = torch.empty(tuple(x.shape), dtype=torch.float32, device=x.device)
        _keep(stream, out)
    d = desc_of(x)
    _check(lib().zk_unary_fwd(_epi(f), _ptr(x), ctypes.byref(d), _ptr(out), _stream(stream)),
           "zk_unary_fwd")
    return out


def unary_bwd(f, grad, x, grad_x=None, acc_x=None, stream=None):
    """grad_x = grad * f'(x) (+ acc_x)."""
    import torch
    if grad_x is None:
        grad_x = torch.empty(tuple(x.shape), dtype=torch.float32, device=grad.device)
        _keep(stream, grad_x)
    d = desc_of(x)
    _check(lib().zk_unary_bwd(_epi(f), _ptr(grad), _ptr(x), ctypes.byref(d), _ptr(grad_x),
                              _ptr(acc_x), _stream(stream)), "zk_unary_bwd")
    return grad_x


def materialize(x, shape=None, out=None, stream=None):
    """Dense row-major copy of the view ``x``, broadcast to ``shape`` (default:
    x's own shape)."""
    import torch
    shape = tuple(x.shape) if shape is None else tuple(int(s) for s in shape)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=x.device)
        _keep(stream, out)
    d = desc_of(x)
    _check(lib().zk_materialize(_ptr(x), ctypes.byref(d), len(shape), _i64(shape), _ptr(out),
                                _stream(stream)), "zk_materialize")
    return out


def broadcast_shape3(sa, sb, sc):
    return broadcast_shape(broadcast_shape(sa, sb), sc)


def binary2_fwd(op1, op2, a, b, c, out=None, stream=None):
    """out = (a (op1) b) (op2) c in the broadcast shape of a, b and c, one
    pass, each operator rounded on its own (op2: "add" or "sub")."""
    import torch
    if out is None:
        shape = broadcast_shape3(a.shape, b.shape, c.shape)
        out = torch.empty(shape, dtype=torch.float32, device=a.device)
        _keep(stream, out)
    da, db, dc = desc_of(a), desc_of(b), desc_of(c)
    _check(lib().zk_binary2_fwd(_op(op1), _op(op2), _ptr(a), ctypes.byref(da), _ptr(b),
                                ctypes.byref(db), _ptr(c), ctypes.byref(dc), _ptr(out),
                                _stream(stream)), "zk_binary2_fwd")
    return out


def bwd2_workspace_bytes(op1, op2, a, b, c, need=(True, True, True), tie=None):
    """Workspace zk_binary2_bwd needs for these operands (no launch)."""
    da, db, dc = desc_of(a), desc_of(b), desc_of(c)
    nbytes = ctypes.c_size_t(0)
    m = [ctypes.c_void_p(16 + 64 * k) if need[k] else None for k in range(3)]
    if tie is not None:
        m[2] = m[0] if tie == "a" else m[1]
    mark = ctypes.c_void_p(16)
    cp = mark if tie is None else mark
    _check(lib().zk_binary2_bwd(_op(op1), _op(op2), mark, mark, ctypes.byref(da), mark,
                                ctypes.byref(db), cp, ctypes.byref(dc), m[0], None, m[1],
                                None, m[2], None, None, ctypes.byref(nbytes), None),
           "zk_binary2_bwd(query)")
    return nbytes.value


def binary2_bwd(op1, op2, grad, a, b, c, need=(True, True, True), grads=(None, None, None),
                accs=(None, None, None), tie=None, workspace=None, stream=None):
    """Gradients of (a (op1) b) (op2) c for the upstream ``grad``; returns
    (grad_a, grad_b, grad_c), each dense in its operand's shape (None if not
    requested).  tie "a" / "b": c is that same tensor and one buffer takes
    both paths (returned for that operand; grad_c is then None)."""
    import torch
    ops = (a, b, c)
    out = []
    for k in range(3):
        g = grads[k]
        if need[k] and g is None and not (k == 2 and tie is not None):
            g = torch.empty(ops[k].shape, dtype=torch.float32, device=grad.device)
            _keep(stream, g)
        out.append(g if need[k] else None)
    if tie is not None:
        out[2] = out[0] if tie == "a" else out[1]
    da, db, dc = desc_of(a), desc_of(b), desc_of(c)
    nbytes = ctypes.c_size_t(0)
    L = lib()
    args = (_op(op1), _op(op2), _ptr(grad), _ptr(a), ctypes.byref(da), _ptr(b),
            ctypes.byref(db), _ptr(c), ctypes.byref(dc), _ptr(out[0]), _ptr(accs[0]),
            _ptr(out[1]), _ptr(accs[1]), _ptr(out[2]), _ptr(accs[2]))
    if workspace is None:
        _check(L.zk_binary2_bwd(*args, None, ctypes.byref(nbytes), None),
               "zk_binary2_bwd(query)")
        workspace = _workspace(nbytes.value, grad.device)
        _keep(stream, workspace)
    nbytes.value = workspace.numel() * workspace.element_size()
    _check(L.zk_binary2_bwd(*args, _ptr(workspace), ctypes.byref(nbytes), _stream(stream)),
           "zk_binary2_bwd")
    if tie is not None:
        out[2] = None
    return tuple(out)


def reduce_workspace_bytes(x, shape):
    d = desc_of(x)
    nbytes = ctypes.c_size_t(0)
    _check(lib().zk_reduce_to_shape(ctypes.c_void_p(16), ctypes.byref(d), len(shape),
                                    _i64(shape), ctypes.c_void_p(16), None,
                                    ctypes.byref(nbytes), None),
           "zk_reduce_to_shape(query)")
    return nbytes.value


def reduce_to_shape(x, shape, out=None, workspace=None, stream=None):
    """Sum ``x`` back to ``shape`` (dense row-major)."""
    import torch
    shape = tuple(int(s) for s in shape)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=x.device)
        _keep(stream, out)
    d = desc_of(x)
    nbytes = ctypes.c_size_t(0)
    L = lib()
    if workspace is None:
        _check(L.zk_reduce_to_shape(_ptr(x), ctypes.byref(d), len(shape), _i64(shape),
                                    _ptr(out), None, ctypes.byref(nbytes), None),
               "zk_reduce_to_shape(query)")
        workspace = _workspace(nbytes.value, x.device)
        _keep(stream, workspace)
    nbytes.value = workspace.numel() * workspace.element_size()
    _check(L.zk_reduce_to_shape(_ptr(x), ctypes.byref(d), len(shape), _i64(shape),
                                _ptr(out), _ptr(workspace), ctypes.byref(nbytes),
                                _stream(stream)), "zk_reduce_to_shape")
    return out


def mean_to_shape(x, shape, out=None, workspace=None, stream=None):
    """Mean of ``x`` over the dims where ``shape`` is 1 or missing (dense
    row-major result); the workspace is the one reduce_to_shape needs."""
    import torch
    shape = tuple(int(s) for s in shape)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=x.device)
        _keep(stream, out)
    d = desc_of(x)
    nbytes = ctypes.c_size_t(0)
    L = lib()
    if workspace is None:
        workspace = _workspace(reduce_workspace_bytes(x, shape), x.device)
        _keep(stream, workspace)
    nbytes.value = workspace.numel() * workspace.element_size()
    _check(L.zk_mean_to_shape(_ptr(x), ctypes.byref(d), len(shape), _i64(shape),
                              _ptr(out), _ptr(workspace), ctypes.byref(nbytes),
                              _stream(stream)), "zk_mean_to_shape")
    return out


def mean_bwd(g, shape_in, out=None, stream=None):
    """Gradient of mean_to_shape: ``g`` (dense, the reduced shape) divided by
    the count and repeated over ``shape_in``."""
    import torch
    shape_in = tuple(int(s) for s in shape_in)
    if out is None:
        out = torch.empty(shape_in, dtype=torch.float32, device=g.device)
        _keep(stream, out)
    gs = tuple(g.shape)
    _check(lib().zk_mean_bwd(_ptr(g), len(gs), _i64(gs), len(shape_in), _i64(shape_in),
                             _ptr(out), _stream(stream)), "zk_mean_bwd")
    return out


def _grad_list(tensors):
    ptrs = (ctypes.c_void_p * max(1, len(tensors)))(
        *[t.data_ptr() if t.numel() else None for t in tensors])
    return ptrs, _i64([t.numel() for t in tensors])


def norm_workspace_bytes(numels):
    """Workspace zk_grad_norm / zk_clip_grad_norm need for these element
    counts (no launch)."""
    nbytes = ctypes.c_size_t(0)
    _check(lib().zk_grad_norm(len(numels), None, _i64(numels), None, None,
                              ctypes.byref(nbytes), None), "zk_grad_norm(query)")
    return nbytes.value


def _norm_call(tensors, clip, max_norm, norm_out, workspace, stream):
    import torch
    dev = tensors[0].device if tensors else torch.device("cuda")
    if norm_out is None:
        norm_out = torch.empty((), dtype=torch.float32, device=dev)
        _keep(stream, norm_out)
    if workspace is None:
        workspace = _workspace(norm_workspace_bytes([t.numel() for t in tensors]), dev)
        _keep(stream, workspace)
    ptrs, ns = _grad_list(tensors)
    nbytes = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    L = lib()
    if clip:
        _check(L.zk_clip_grad_norm(len(tensors), ptrs, ns, float(max_norm), _ptr(norm_out),
                                   _ptr(workspace), ctypes.byref(nbytes), _stream(stream)),
               "zk_clip_grad_norm")
    else:
        _check(L.zk_grad_norm(len(tensors), ptrs, ns, _ptr(norm_out), _ptr(workspace),
                              ctypes.byref(nbytes), _stream(stream)), "zk_grad_norm")
    return norm_out


def grad_norm(tensors, norm_out=None, workspace=None, stream=None):
    """Global L2 norm of dense fp32 tensors, as a 0-d device tensor."""
    return _norm_call(tensors, False, 0.0, norm_out, workspace, stream)


def clip_grad_norm(tensors, max_norm, norm_out=None, workspace=None, stream=None):
    """ClipGradNorm in place: scales every tensor by max_norm / (norm + 1e-6)
    when the global norm exceeds max_norm.  Returns the norm (0-d device
    tensor; nothing is synchronised)."""
    return _norm_call(tensors, True, max_norm, norm_out, workspace, stream)


def _row_view(x):
    """(rows, cols, ld) of a 2-D tensor whose rows are contiguous."""
    if x.dim() != 2 or (x.shape[1] > 1 and x.stride(1) != 1):
        raise ValueError("row statistics take a 2-D tensor with contiguous rows")
    rows, cols = x.shape
    ld = x.stride(0) if rows > 1 else max(cols, 1)
    return rows, cols, ld


def row_moments(x, mean=None, var=None, stream=None):
    """Per-row mean and biased variance of a 2-D tensor with contiguous rows."""
    import torch
    rows, cols, ld = _row_view(x)
    if mean is None:
        mean = torch.empty(rows, dtype=torch.float32, device=x.device)
        _keep(stream, mean)
    if var is None:
        var = torch.empty(rows, dtype=torch.float32, device=x.device)
        _keep(stream, var)
    _check(lib().zk_row_moments(_ptr(x), rows, cols, ld, _ptr(mean), _ptr(var),
                                _stream(stream)), "zk_row_moments")
    return mean, var


def row_softmax_stats(x, rowmax=None, sumexp=None, stream=None):
    """Per-row max and sum of exp(x - max) of a 2-D tensor with contiguous rows."""
    import torch
    rows, cols, ld = _row_view(x)
    if rowmax is None:
        rowmax = torch.empty(rows, dtype=torch.float32, device=x.device)
        _keep(stream, rowmax)
    if sumexp is None:
        sumexp = torch.empty(rows, dtype=torch.float32, device=x.device)
        _keep(stream, sumexp)
    _check(lib().zk_row_softmax_stats(_ptr(x), rows, cols, ld, _ptr(rowmax), _ptr(sumexp),
                                      _stream(stream)), "zk_row_softmax_stats")
    return rowmax, sumexp


def plan_describe(kind, op, da, db, epi="none"):
    """Launch plan a call would use (host only).  kind: "fwd", "bwd",
    "reduce" (db = target shape)."""
    info = PlanInfo()
    k = {"fwd": 0, "bwd": 1, "reduce": 2}[kind]
    _check(lib().zk_plan_describe(k, _op(op), _epi(epi), ctypes.byref(da),
                                  ctypes.byref(db), ctypes.byref(info)),
           "zk_plan_describe")
    r = info.rank
    return dict(kernel=lib().zk_kernel_name(info.kernel).decode(),
                kernel2=lib().zk_kernel_name(info.kernel2).decode(),
                rank=r, sizes=tuple(info.sizes[k] for k in range(r)),
                strides=tuple(tuple(info.strides[o][k] for k in range(r))
                              for o in range(3)),
                index64=bool(info.index64), vec=info.vec,
                partials=info.partials, workspace_bytes=info.workspace_bytes)


def profile_start(capacity):
    """Bracket every library kernel with HIP events (tooling; see zk.h)."""
    _check(lib().zk_profile_start(int(capacity)), "zk_profile_start")


def profile_stop():
    _check(lib().zk_profile_stop(), "zk_profile_stop")


def profile_read(max_records=1 << 16):
    """[(kernel class name, milliseconds)] in launch order (after a sync)."""
    ids = (ctypes.c_int32 * max_records)()
    ms = (ctypes.c_float * max_records)()
    n = ctypes.c_int32(0)
    _check(lib().zk_profile_read(max_records, ids, ms, ctypes.byref(n)), "zk_profile_read")
    L = lib()
    return [(L.zk_kernel_name(ids[i]).decode(), ms[i]) for i in range(n.value)]
