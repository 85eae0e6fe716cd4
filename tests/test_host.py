"""Host-side checks of libzk.so that need no GPU: exported symbols, the
broadcast shape rule, every validation error path (each returns before any
HIP call), the canonical form and kernel class chosen for each workload, and
the planner under ASan/UBSan."""
import ctypes
import itertools
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

from conftest import ROOT

zkmod = pytest.importorskip("broadcast_autograd_amd.zk")
zk = zkmod

HEADER = os.path.join(ROOT, "include", "zk.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(zk.LIB_PATH):
        from broadcast_autograd_amd import build
        build.build(verbose=False)
    return zk.lib()


def test_exports_every_declared_symbol(L):
    text = open(HEADER).read()
    declared = set(re.findall(r"^(?:zk_status|const char \*)\s*(zk_\w+)\(", text, re.M))
    assert {"zk_broadcast_shape", "zk_binary_fwd", "zk_binary_bwd",
            "zk_reduce_to_shape"} <= declared
    for name in declared:
        assert hasattr(L, name), name
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", zk.LIB_PATH],
                             capture_output=True, text=True).stdout
        for name in declared:
            assert re.search(rf"\bT {name}$", out, re.M), name


def test_header_is_plain_c(tmp_path):
    """include/zk.h compiles as C99 (and C++17): plain pointers, sizes and
    enums only, usable from any language with a C FFI."""
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("no gcc")
    src = tmp_path / "use.c"
    src.write_text('#include "zk.h"\nint main(void) { return (int)ZK_OK; }\n')
    for lang, std in (("c", "-std=c99"), ("c++", "-std=c++17")):
        r = subprocess.run([gcc, "-x", lang, std, "-Wall", "-Wextra", "-Werror",
                            "-I", os.path.dirname(HEADER), "-fsyntax-only", str(src)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_broadcast_shape_matches_oracle(L, orc):
    shapes = [s for r in range(4) for s in itertools.product((0, 1, 2, 3), repeat=r)]
    for sa in shapes:
        for sb in shapes:
            try:
                want = orc.broadcast_shape(sa, sb)
            except orc.OracleError:
                with pytest.raises(zk.ZkError) as e:
                    zk.broadcast_shape(sa, sb)
                assert e.value.name == "ZK_ERR_BROADCAST"
                continue
            assert zk.broadcast_shape(sa, sb) == want


def test_broadcast_shape_errors(L):
    with pytest.raises(zk.ZkError) as e:
        zk.broadcast_shape((1,) * 9, (1,))
    assert e.value.name == "ZK_ERR_RANK"
    with pytest.raises(zk.ZkError) as e:
        zk.broadcast_shape((-2,), (1,))
    assert e.value.name == "ZK_ERR_BAD_SIZE"
    with pytest.raises(zk.ZkError) as e:
        zk.broadcast_shape((2, 3, 4), (2, 4, 5))
    assert e.value.name == "ZK_ERR_BROADCAST"
    ro = ctypes.c_int32(0)
    assert L.zk_broadcast_shape(0, None, 0, None, ctypes.byref(ro), None) == zk.ERR["ZK_ERR_NULL"]


# Fake, distinct, 16-byte aligned device addresses: every call below fails
# validation, so none of them is ever dereferenced or launched.
FA, FB, FO, FG, FW = (ctypes.c_void_p(x) for x in (1 << 20, 2 << 20, 3 << 20, 4 << 20, 5 << 20))


def _fwd(op, da, db, a=FA, b=FB, out=FO, epi=0):
    return zk.STATUS[zk.lib().zk_binary_fwd(op, epi, a, ctypes.byref(da), b,
                                             ctypes.byref(db), out, None)]


def _bwd(op, da, db, ga=FO, gb=FW, acc_a=None, acc_b=None, g=FG, ws=None,
         wsb=1 << 30, epi=0, a=FA, b=FB):
    n = ctypes.c_size_t(wsb)
    return zk.STATUS[zk.lib().zk_binary_bwd(op, epi, g, a, ctypes.byref(da), b,
                                             ctypes.byref(db), ga, acc_a, gb, acc_b,
                                             ws, ctypes.byref(n), None)], n.value


def test_forward_validation_errors(L):
    d23 = zk.make_desc((2, 3))
    assert _fwd(7, d23, d23) == "ZK_ERR_UNSUPPORTED"
    assert _fwd(0, d23, d23, epi=5) == "ZK_ERR_UNSUPPORTED"
    bad = zk.make_desc((2, 3))
    bad.rank = 9
    assert _fwd(0, bad, d23) == "ZK_ERR_RANK"
    neg = zk.make_desc((2, -3))
    assert _fwd(0, neg, d23) == "ZK_ERR_BAD_SIZE"
    negs = zk.make_desc((2, 3), (-3, 1))
    assert _fwd(0, negs, d23) == "ZK_ERR_BAD_STRIDE"
    assert _fwd(0, zk.make_desc((2, 3, 4)), zk.make_desc((2, 4, 5))) == "ZK_ERR_BROADCAST"
    # int64 extents: element counts and largest offsets above 2^62 are refused
    huge = zk.make_desc((1 << 31, 1 << 32), (0, 0))
    assert _fwd(0, huge, zk.make_desc((1,))) == "ZK_ERR_BAD_SIZE"
    far = zk.make_desc((2, 3), (1 << 62, 1))
    assert _fwd(0, far, d23) == "ZK_ERR_BAD_STRIDE"
    wrap = zk.make_desc((3, 3), (1 << 62, 1 << 62))
    assert _fwd(0, wrap, zk.make_desc((3, 3))) == "ZK_ERR_BAD_STRIDE"
    col = zk.make_desc((1 << 31, 1), (1, 0))
    row = zk.make_desc((1, 1 << 32), (0, 1))
    assert _fwd(0, col, row) == "ZK_ERR_BAD_SIZE"  # each fits, their broadcast does not
    with pytest.raises(zk.ZkError) as e:
        zk.broadcast_shape((1 << 31, 1), (1, 1 << 32))
    assert e.value.name == "ZK_ERR_BAD_SIZE"
    # an empty view reads nothing: its strides may be anything non-negative
    empty = zk.make_desc((0, 3), (1 << 62, 1 << 62))
    assert _fwd(0, empty, zk.make_desc((3,))) == "ZK_OK"
    assert _fwd(0, d23, d23, a=None) == "ZK_ERR_NULL"
    assert _fwd(0, d23, d23, out=None) == "ZK_ERR_NULL"
    assert zk.STATUS[L.zk_binary_fwd(0, 0, FA, None, FB, ctypes.byref(d23), FO, None)] == "ZK_ERR_NULL"
    # out overlapping an input that is not the same dense full-shape buffer
    assert _fwd(0, d23, d23, out=ctypes.c_void_p(FA.value + 4)) == "ZK_ERR_ALIAS"
    assert _fwd(0, zk.make_desc((3,)), d23, out=FA) == "ZK_ERR_ALIAS"
    tr = zk.make_desc((2, 3), (1, 2))
    assert _fwd(0, tr, d23, out=FA) == "ZK_ERR_ALIAS"
    # an empty broadcast shape is a no-op even with NULL data pointers
    d0 = zk.make_desc((0, 3))
    assert _fwd(0, d0, zk.make_desc((1, 3)), a=None, b=None, out=None) == "ZK_OK"


def test_backward_validation_errors(L):
    da, db = zk.make_desc((4, 8)), zk.make_desc((8,))
    assert _bwd(9, da, db)[0] == "ZK_ERR_UNSUPPORTED"
    assert _bwd(2, da, zk.make_desc((5,)))[0] == "ZK_ERR_BROADCAST"
    # workspace query launches nothing and is a function of the shapes only
    st, need = _bwd(2, da, db, ws=None)
    assert st == "ZK_OK" and need > 0
    st2, need2 = _bwd(2, da, db, ws=None, g=ctypes.c_void_p(FG.value + 4),
                      a=ctypes.c_void_p(FA.value + 4))
    assert st2 == "ZK_OK" and need2 == need
    assert _bwd(2, da, db, ws=ctypes.c_void_p(6 << 20), wsb=need - 1)[0] == "ZK_ERR_WORKSPACE"
    # binary64 partials need an 8-byte aligned workspace
    assert _bwd(2, da, db, ws=ctypes.c_void_p((6 << 20) + 4), wsb=need + 8)[0] == "ZK_ERR_WORKSPACE"
    ws = ctypes.c_void_p(6 << 20)
    # outputs overlapping each other, the inputs, the upstream grad or the workspace
    assert _bwd(2, da, db, ws=ws, ga=FO, gb=ctypes.c_void_p(FO.value + 8))[0] == "ZK_ERR_ALIAS"
    assert _bwd(2, da, db, ws=ws, ga=FA)[0] == "ZK_ERR_ALIAS"
    assert _bwd(2, da, db, ws=ws, ga=FG)[0] == "ZK_ERR_ALIAS"
    assert _bwd(2, da, db, ws=ws, gb=ws)[0] == "ZK_ERR_ALIAS"
    # acc of one gradient overlapping the other gradient
    assert _bwd(2, da, db, ws=ws, acc_b=FO)[0] == "ZK_ERR_ALIAS"
    # missing data pointers
    assert _bwd(2, da, db, ws=ws, g=None)[0] == "ZK_ERR_NULL"
    n = ctypes.c_size_t(0)
    assert zk.STATUS[L.zk_binary_bwd(2, 0, FG, FA, ctypes.byref(da), FB, ctypes.byref(db),
                                     FO, None, FW, None, None, None, None)] == "ZK_ERR_NULL"


FC = ctypes.c_void_p(9 << 20)  # distinct from the addresses above


def _fwd2(op1, op2, da, db, dc, a=FA, b=FB, c=FC, out=FO):
    return zk.STATUS[zk.lib().zk_binary2_fwd(op1, op2, a, ctypes.byref(da), b,
                                              ctypes.byref(db), c, ctypes.byref(dc), out,
                                              None)]


def _bwd2(op1, op2, da, db, dc, ga=None, gb=None, gc=None, acc=(None, None, None),
          g=FG, a=FA, b=FB, c=FC, ws=None, wsb=1 << 30):
    n = ctypes.c_size_t(wsb)
    return zk.STATUS[zk.lib().zk_binary2_bwd(op1, op2, g, a, ctypes.byref(da), b,
                                              ctypes.byref(db), c, ctypes.byref(dc), ga,
                                              acc[0], gb, acc[1], gc, acc[2], ws,
                                              ctypes.byref(n), None)], n.value


def test_fused_validation_errors(L):
    d = zk.make_desc((4, 8))
    r = zk.make_desc((8,))
    assert _fwd2(2, 2, d, r, d) == "ZK_ERR_UNSUPPORTED"  # op2 must be add or sub
    assert _fwd2(5, 0, d, r, d) == "ZK_ERR_UNSUPPORTED"
    assert _fwd2(2, 0, d, r, zk.make_desc((5,))) == "ZK_ERR_BROADCAST"
    assert _fwd2(2, 0, d, r, d, c=None) == "ZK_ERR_NULL"
    assert _fwd2(2, 0, d, r, d, out=ctypes.c_void_p(FC.value + 4)) == "ZK_ERR_ALIAS"
    # the backward workspace query launches nothing
    st, need = _bwd2(2, 0, d, r, d, ga=FO, gb=FW, gc=ctypes.c_void_p(7 << 20))
    assert st == "ZK_OK" and need > 0
    ws = ctypes.c_void_p(6 << 20)
    gc = ctypes.c_void_p(7 << 20)
    assert _bwd2(2, 0, d, r, d, ga=FO, gb=FW, gc=gc, ws=ws, wsb=need - 1)[0] == "ZK_ERR_WORKSPACE"
    # shared gradient buffer: only grad_c == grad_a with c the same tensor as a
    assert _bwd2(2, 0, d, r, d, ga=FO, gc=FO, ws=ws)[0] == "ZK_ERR_UNSUPPORTED"   # c != a
    assert _bwd2(2, 1, d, r, d, ga=FO, gc=FO, c=FA, ws=ws)[0] == "ZK_ERR_UNSUPPORTED"  # sub
    assert _bwd2(2, 0, d, r, d, ga=FO, gc=FO, c=FA, ws=ws,
                 acc=(FW, None, None))[0] == "ZK_ERR_UNSUPPORTED"  # acc with a tie
    # grad_c overlapping another output, an input or the upstream gradient
    assert _bwd2(2, 0, d, r, d, ga=FO, gc=ctypes.c_void_p(FO.value + 8), ws=ws)[0] == "ZK_ERR_ALIAS"
    assert _bwd2(2, 0, d, r, d, gc=FA, ws=ws)[0] == "ZK_ERR_ALIAS"
    assert _bwd2(2, 0, d, r, d, gc=FG, ws=ws)[0] == "ZK_ERR_ALIAS"
    assert _bwd2(2, 0, d, r, d, gc=gc, acc=(None, None, FO), ga=FO, ws=ws)[0] == "ZK_ERR_ALIAS"


def test_materialize_validation_errors(L):
    def call(din, shape, inp=FA, out=FO):
        return zk.STATUS[L.zk_materialize(inp, ctypes.byref(din), len(shape),
                                          zk._i64(shape), out, None)]
    d = zk.make_desc((4, 8))
    assert call(d, (3, 8)) == "ZK_ERR_SHAPE"          # 4 does not broadcast to 3
    assert call(d, (8,)) == "ZK_ERR_SHAPE"            # the target must be the result
    assert call(d, (2, 4, 8), inp=None) == "ZK_ERR_NULL"
    assert call(d, (4, 8), out=ctypes.c_void_p(FA.value + 16)) == "ZK_ERR_ALIAS"
    bad = zk.make_desc((4, 8), (8, -1))
    assert call(bad, (4, 8)) == "ZK_ERR_BAD_STRIDE"
    d0 = zk.make_desc((0, 8))
    assert call(d0, (0, 8), inp=None, out=None) == "ZK_OK"  # empty: nothing launched


def test_reduce_validation_errors(L):
    d = zk.make_desc((4, 6))

    def red(shape, ws=None, wsb=1 << 30, inp=FA, out=FO):
        n = ctypes.c_size_t(wsb)
        arr = (ctypes.c_int64 * max(8, len(shape)))(*shape)
        return zk.STATUS[L.zk_reduce_to_shape(inp, ctypes.byref(d), len(shape), arr, out,
                                              ws, ctypes.byref(n), None)], n.value

    assert red((5,))[0] == "ZK_ERR_SHAPE"
    assert red((2, 4, 6))[0] == "ZK_ERR_SHAPE"   # broadcasts, but grows the shape
    assert red((1,) * 9)[0] == "ZK_ERR_RANK"
    assert red((-1,))[0] == "ZK_ERR_BAD_SIZE"
    st, need = red((6,))
    assert st == "ZK_OK" and need > 0
    assert red((6,), ws=FW, wsb=need - 1)[0] == "ZK_ERR_WORKSPACE"
    assert red((6,), ws=ctypes.c_void_p(FW.value + 4), wsb=need + 8)[0] == "ZK_ERR_WORKSPACE"
    assert red((6,), ws=FW, out=FA)[0] == "ZK_ERR_ALIAS"
    assert red((6,), ws=FW, out=ctypes.c_void_p(FW.value + 8))[0] == "ZK_ERR_ALIAS"


def test_mean_validation_errors(L):
    """zk_mean_to_shape shares zk_reduce_to_shape's checks and workspace size;
    zk_mean_bwd checks the shapes before anything is launched."""
    d = zk.make_desc((4, 6))

    def mean(shape, ws=None, wsb=1 << 30, out=FO):
        n = ctypes.c_size_t(wsb)
        arr = (ctypes.c_int64 * max(8, len(shape)))(*shape)
        return zk.STATUS[L.zk_mean_to_shape(FA, ctypes.byref(d), len(shape), arr, out,
                                            ws, ctypes.byref(n), None)], n.value

    assert mean((5,))[0] == "ZK_ERR_SHAPE"
    st, need = mean((6,))
    n2 = ctypes.c_size_t(0)
    L.zk_reduce_to_shape(FA, ctypes.byref(d), 1, zk._i64((6,)), FO, None, ctypes.byref(n2),
                         None)
    assert st == "ZK_OK" and need == n2.value
    assert mean((6,), ws=FW, wsb=need - 1)[0] == "ZK_ERR_WORKSPACE"
    assert mean((6,), ws=FW, out=FA)[0] == "ZK_ERR_ALIAS"

    def mbwd(sout, sin, g=FG, out=FO):
        return zk.STATUS[L.zk_mean_bwd(g, len(sout), zk._i64(sout), len(sin), zk._i64(sin),
                                       out, None)]

    assert mbwd((5,), (4, 6)) == "ZK_ERR_SHAPE"
    assert mbwd((2, 4, 6), (4, 6)) == "ZK_ERR_SHAPE"    # the target grows the shape
    assert mbwd((6,), (1,) * 9) == "ZK_ERR_RANK"
    assert mbwd((-1,), (4, 6)) == "ZK_ERR_BAD_SIZE"
    assert mbwd((6,), (4, 6), g=None) == "ZK_ERR_NULL"
    assert mbwd((6,), (4, 6), out=ctypes.c_void_p(FG.value + 8)) == "ZK_ERR_ALIAS"
    assert mbwd((6,), (0, 6), g=None, out=None) == "ZK_OK"  # empty: nothing launched


def test_grad_norm_validation_errors(L):
    """Queries need only the counts; every error returns before a launch."""
    def q(ns):
        n = ctypes.c_size_t(0)
        st = L.zk_grad_norm(len(ns), None, zk._i64(ns), None, None, ctypes.byref(n), None)
        return zk.STATUS[st], n.value

    st, need = q([12, 8192, 8193, 0])
    assert st == "ZK_OK" and need == 8 * 4
    assert q([])[1] == 8
    assert q([-1])[0] == "ZK_ERR_BAD_SIZE"
    assert q([1 << 62, 1])[0] == "ZK_ERR_BAD_SIZE"  # more than 2^62 elements in all
    assert q([(1 << 63) - 1])[0] == "ZK_ERR_BAD_SIZE"

    def call(ptrs, ns, ws=FW, wsb=1 << 30, norm=FO, clip=None):
        arr = (ctypes.c_void_p * max(1, len(ptrs)))(*[p.value if p else None for p in ptrs])
        n = ctypes.c_size_t(wsb)
        if clip is None:
            st = L.zk_grad_norm(len(ptrs), arr, zk._i64(ns), norm, ws, ctypes.byref(n), None)
        else:
            st = L.zk_clip_grad_norm(len(ptrs), arr, zk._i64(ns), clip, norm, ws,
                                     ctypes.byref(n), None)
        return zk.STATUS[st]

    assert call([FA, FB], [100, 100], wsb=8) == "ZK_ERR_WORKSPACE"
    assert call([FA, FB], [100, 100], ws=ctypes.c_void_p(FW.value + 4)) == "ZK_ERR_WORKSPACE"
    assert call([FA, None], [100, 100]) == "ZK_ERR_NULL"
    assert call([FA, FB], [100, 100], norm=None) == "ZK_ERR_NULL"
    # overlapping tensors, a tensor over the workspace or over norm_out
    assert call([FA, ctypes.c_void_p(FA.value + 396)], [100, 100]) == "ZK_ERR_ALIAS"
    assert call([FA, FB], [100, 100], ws=ctypes.c_void_p(FB.value + 64)) == "ZK_ERR_ALIAS"
    assert call([FA, FB], [100, 100], norm=ctypes.c_void_p(FA.value + 4)) == "ZK_ERR_ALIAS"
    assert call([FA, FB], [100, 100], clip=-1.0) == "ZK_ERR_UNSUPPORTED"
    assert call([FA, FB], [100, 100], clip=float("nan")) == "ZK_ERR_UNSUPPORTED"
    assert L.zk_grad_norm(-1, None, None, FO, FW, ctypes.byref(ctypes.c_size_t(1 << 20)),
                          None) == zk.ERR["ZK_ERR_BAD_SIZE"]


def test_row_stats_validation_errors(L):
    """Row statistics check sizes, pitch, pointers and overlaps before any
    launch; no rows launches nothing."""
    for fn in (L.zk_row_moments, L.zk_row_softmax_stats):
        def call(x=FA, rows=4, cols=8, ld=8, o1=FO, o2=FB):
            return zk.STATUS[fn(x, rows, cols, ld, o1, o2, None)]
        assert call(rows=-1) == "ZK_ERR_BAD_SIZE"
        assert call(cols=-1) == "ZK_ERR_BAD_SIZE"
        assert call(ld=7) == "ZK_ERR_BAD_STRIDE"
        assert call(rows=1 << 40, ld=1 << 30) == "ZK_ERR_BAD_STRIDE"  # offset above 2^62
        assert call(x=None) == "ZK_ERR_NULL"
        assert call(o2=None) == "ZK_ERR_NULL"
        assert call(o1=ctypes.c_void_p(FA.value + 64)) == "ZK_ERR_ALIAS"
        assert call(o2=ctypes.c_void_p(FO.value + 8)) == "ZK_ERR_ALIAS"
        assert call(rows=0, x=None, o1=None, o2=None) == "ZK_OK"


WORKLOAD_PLANS = [
    # (kind, op, epi, a (sizes, strides), b (sizes, strides), kernel, canonical sizes, b strides)
    ("fwd", "mul", "none", ((64, 128, 256), None), ((128, 1), None), "fwd_row",
     (64, 128, 256), (0, 1, 0)),
    ("fwd", "add", "none", ((64, 128, 256), None), ((64, 128, 256), None), "fwd_flat",
     (2097152,), (1,)),
    ("bwd", "mul", "none", ((64, 128, 256), None), ((128, 1), None), "red_rowd",
     (64, 128, 256), (0, 1, 0)),
    ("fwd", "add", "gelu", ((4096, 1024), None), ((1024,), None), "fwd_row",
     (4096, 1024), (0, 1)),
    ("bwd", "add", "gelu", ((4096, 1024), None), ((1024,), None), "red_col",
     (4096, 1024), (0, 1)),
    ("fwd", "mul", "none", ((8, 16, 1024, 1024), None), ((1, 16, 1, 1), None), "fwd_row",
     (8, 16, 1048576), (0, 1, 0)),
    ("fwd", "add", "none", ((8, 16, 1024, 1024), None), ((1, 1, 1024, 1024), None), "fwd_row",
     (128, 1048576), (0, 1)),
    ("bwd", "mul", "none", ((8, 16, 1024, 1024), None), ((1, 16, 1, 1), None), "red_row",
     (8, 16, 1048576), (0, 1, 0)),
    ("fwd", "mul", "none", ((4096, 4096), (1, 4096)), ((4096,), None), "fwd_tile",
     (4096, 4096), (0, 1)),
    ("bwd", "mul", "none", ((4096, 4096), (1, 4096)), ((4096,), None), "red_tile",
     (4096, 4096), (0, 1)),
    ("fwd", "div", "none", ((2, 3, 4, 5, 6, 7, 8, 9), None), ((1, 3, 1, 5, 1, 7, 1, 9), None),
     "fwd_generic", (2, 3, 4, 5, 6, 7, 8, 9), (0, 315, 0, 63, 0, 9, 0, 1)),
    ("bwd", "div", "none", ((2, 3, 4, 5, 6, 7, 8, 9), None), ((1, 3, 1, 5, 1, 7, 1, 9), None),
     "red_run", (2, 3, 4, 5, 6, 7, 8, 9), (0, 315, 0, 63, 0, 9, 0, 1)),
    ("fwd", "mul", "none", ((16, 2048, 4096), None), ((4096,), None), "fwd_row",
     (32768, 4096), (0, 1)),
    ("fwd", "add", "none", ((16, 2048, 4096), None), ((16, 2048, 4096), None), "fwd_flat",
     (134217728,), (1,)),
    ("bwd", "mul", "none", ((16, 2048, 4096), None), ((4096,), None), "red_col",
     (32768, 4096), (0, 1)),
]


@pytest.mark.parametrize("case", WORKLOAD_PLANS, ids=lambda c: f"{c[0]}-{c[1]}-{c[5]}")
def test_workload_canonical_forms(L, case):
    kind, op, epi, (sa, ta), (sb, tb), kernel, sizes, bstr = case
    info = zk.plan_describe(kind, op, zk.make_desc(sa, ta), zk.make_desc(sb, tb), epi=epi)
    assert info["kernel"] == kernel
    assert info["sizes"] == sizes
    assert info["strides"][2] == bstr
    assert not info["index64"]


@pytest.mark.parametrize("shape,target,kernel,partials,ws", [
    # short columns: one partial a column, finished by red_col (no workspace use)
    ((128, 1048576), (1048576,), "red_col", 1, None),
    # narrow columns fold 256/K rows into one: partials count the fold copies
    ((4194304, 32), (32,), "red_col", 512 * 8, 512 * 8 * 32 * 8),
    ((33554432, 4), (4,), "red_col", 512 * 64, 512 * 64 * 4 * 8),
    ((4001, 32), (32,), "red_col", None, None),          # rows not divisible: no fold
    # plain row sums: a block per row up to 2^24 elements, then red_row
    ((4096, 2048), (4096, 1), "red_rowd", 0, None),
    ((65536, 2048), (65536, 1), "red_row", 1, None),
    ((64, 128, 256), (128, 1), "red_rowd", 0, None),     # middle pattern stays one pass
    # short rows: 256 / C rows a wave
    ((1048576, 128), (1048576, 1), "red_rowseg", 0, None),
    ((16777216, 8), (16777216, 1), "red_rowseg", 0, None),
    # middle sums over more rows than the row length: column sums of
    # [R1, K * C], stage 2 adding each kept element's C columns
    ((256, 4096, 128), (4096, 1), "red_col", 1, 4096 * 128 * 8),
    ((1 << 22, 4, 4), (4, 1), "red_col", 2048 * 16, 2048 * 16 * 16 * 8),
    ((2, 4096, 128), (4096, 1), "red_rowseg", 2, 2 * 4096 * 8),  # R1 <= C: row sums
    ((10, 12), (10, 1), "red_generic", None, None),      # 12 does not divide 256
    ((524288, 256), (524288, 1), "red_rowseg", 0, None),
    ((2048, 256, 256), (256, 1), "red_col", 2, 2 * 65536 * 8),
    ((8, 64, 256), (64, 1), "red_rowd", 0, None),        # within red_rowd's one pass
    ((16, 1000, 128), (1000, 1), "red_rowseg", 16, None),  # rows too short for red_rowd
])
def test_reduce_plan_shapes(L, shape, target, kernel, partials, ws):
    """The planner's choice for the reduction shapes it treats specially."""
    info = zk.plan_describe("reduce", "add", zk.make_desc(shape), zk.make_desc(target))
    assert info["kernel"] == kernel
    if partials is not None:
        assert info["partials"] == partials
    if ws is not None:
        assert info["workspace_bytes"] == ws


def test_plans_beyond_the_grid_limit(L):
    """More than 2^30 kept columns (the column groups alone exceed the grid
    limit): planned with one band of rows and at least one partial, for the
    reduction and the multiply backward (host only, nothing allocated)."""
    big = 1 << 31
    info = zk.plan_describe("reduce", "add", zk.make_desc((2, big)), zk.make_desc((big,)))
    assert info["kernel"] == "red_col" and info["partials"] == 1
    assert info["workspace_bytes"] == big * 8
    info = zk.plan_describe("bwd", "mul", zk.make_desc((2, big)), zk.make_desc((big,)))
    assert info["kernel"] == "red_col" and info["partials"] == 1
    # [2^22, 4, 4] -> [4, 1]: bounded partials (was 2^22 row sums a kept element)
    info = zk.plan_describe("reduce", "add", zk.make_desc((1 << 22, 4, 4)),
                            zk.make_desc((4, 1)))
    assert info["partials"] <= 65536 and info["workspace_bytes"] <= (64 << 20) // 16


def test_reduce_plans(L):
    info = zk.plan_describe("reduce", "add", zk.make_desc((32768, 4096)), zk.make_desc((4096,)))
    assert info["kernel"] == "red_col" and info["sizes"] == (32768, 4096)
    info = zk.plan_describe("reduce", "add", zk.make_desc((8, 16, 1024, 1024)),
                            zk.make_desc((1, 16, 1, 1)))
    assert info["kernel"] == "red_row" and info["sizes"] == (8, 16, 1048576)
    info = zk.plan_describe("reduce", "add", zk.make_desc((8, 16, 1024, 1024)),
                            zk.make_desc((1, 1, 1024, 1024)))
    assert info["kernel"] == "red_col" and info["sizes"] == (128, 1048576)
    info = zk.plan_describe("reduce", "add", zk.make_desc((6, 4), (1, 6)), zk.make_desc((4,)))
    assert info["kernel"] == "red_generic"
    # 32..4096 terms per kept element on a gather pattern: one pass
    info = zk.plan_describe("reduce", "add", zk.make_desc((64, 4), (1, 64)), zk.make_desc((4,)))
    assert info["kernel"] == "red_gend" and info["partials"] == 0
    info = zk.plan_describe("reduce", "add", zk.make_desc((4097, 4), (1, 4097)),
                            zk.make_desc((4,)))
    assert info["kernel"] == "red_generic"
    # 2048..16384 terms per kept element: one pass, no partials
    for shape, target, kern in (((16384,), (), "red_rowd"), ((8192,), (), "red_rowd"),
                                ((4096,), (1,), "red_rowd"), ((2, 1024), (1, 1), "red_rowd"),
                                ((16, 1024), (16, 1), "red_row"),
                                ((32768,), (), "red_row"), ((7, 4, 4096), (1, 4, 1), "red_row")):
        info = zk.plan_describe("reduce", "add", zk.make_desc(shape), zk.make_desc(target))
        assert info["kernel"] == kern, (shape, target, info["kernel"])
        if kern == "red_rowd":
            assert info["partials"] == 0


# (op, epi, full shape, reduced shape, kernel, partials a kept element):
# a backward that reads the full operand and writes its gradient walks long
# columns interleaved, 4 rows a wave (64 a partial), and takes 512-element row
# chunks four to a partial; a plain sum, division, GeLU and folded narrow
# columns keep the longer runs.
STREAM_PLANS = [
    ("mul", "none", (32768, 4096), (4096,), "red_col", 512),
    ("div", "none", (32768, 4096), (4096,), "red_col", 32),
    ("add", "gelu", (32768, 4096), (4096,), "red_col", 32),
    ("mul", "none", (4194304, 32), (32,), "red_col", 4096),
    ("mul", "none", (2, 8, 262144), (8, 1), "red_row", 256),
    ("add", "none", (2, 8, 262144), (8, 1), "red_row", 256),
    ("mul", "none", (7, 3, 2600), (3, 1), "red_row", 77),
]


@pytest.mark.parametrize("op,epi,sa,sb,kernel,partials", STREAM_PLANS)
def test_stream_count_plans(L, op, epi, sa, sb, kernel, partials):
    info = zk.plan_describe("bwd", op, zk.make_desc(sa), zk.make_desc(sb), epi=epi)
    assert (info["kernel"], info["partials"]) == (kernel, partials), info
    # the same shapes summed alone (one stream) keep the longer runs
    red = zk.plan_describe("reduce", "add", zk.make_desc(sa), zk.make_desc(sb))
    assert red["kernel"] == kernel
    if (op, epi) == ("mul", "none") and len(sa) == 2 and sa[1] >= 2048:
        assert red["partials"] == 32
    if kernel == "red_row" and sa[-1] == 262144:
        assert red["partials"] == 1024


def test_index64_threshold(L):
    info = zk.plan_describe("fwd", "add", zk.make_desc((1 << 31,)), zk.make_desc((1,)))
    assert info["index64"]


def test_planner_under_sanitizers():
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("no g++")
    exe = os.path.join(ROOT, "_build", "plan_check")
    os.makedirs(os.path.dirname(exe), exist_ok=True)
    src = [os.path.join(ROOT, "tests", "host", "plan_check.cpp"),
           os.path.join(ROOT, "broadcast_autograd_amd", "csrc", "zk_plan.cpp")]
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "broadcast_autograd_amd", "csrc")] + src +
                   ["-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "OK" in r.stdout, r.stdout + r.stderr


def _gelu_exact_host():
    """The library's double-double GeLU (csrc/zk_gelu_exact.h) built for the
    host: the same IEEE binary64 operations the kernels run."""
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("no g++")
    exe = os.path.join(ROOT, "_build", "gelu_exact_check")
    os.makedirs(os.path.dirname(exe), exist_ok=True)
    subprocess.run([gxx, "-std=c++17", "-O2", "-ffp-contract=off", "-msse2", "-mfpmath=sse",
                    "-I", os.path.join(ROOT, "broadcast_autograd_amd", "csrc"),
                    os.path.join(ROOT, "tests", "host", "gelu_exact_check.cpp"), "-o", exe],
                   check=True)

    def run(hs):
        pats = np.asarray(hs, dtype=np.float32).view(np.uint32)
        r = subprocess.run([exe], input="\n".join(f"{u:08x}" for u in pats), text=True,
                           capture_output=True, timeout=600, check=True)
        return np.array([int(x, 16) for x in r.stdout.split()], dtype=np.uint32)
    return run


def test_gelu_exact_path_against_mpmath():
    """The kernels' double-double GeLU (their path wherever the binary64
    table cannot round with certainty) is h * Phi(h) correctly rounded: on
    every near-tie argument of [-10, 10], on constructed midpoint cases
    (odd multiples of 2^-149 and the like) and on random arguments down to
    -15, each against mpmath at 400 bits."""
    from gelu_cases import constructed_arguments, mp_gelu_f32, near_tie_arguments
    run = _gelu_exact_host()
    rng = np.random.default_rng(2024)
    hs = np.concatenate([near_tie_arguments(), constructed_arguments(),
                         rng.uniform(-15, 7, 400).astype(np.float32),
                         (rng.standard_normal(100) * 1e-20).astype(np.float32)])
    got = run(hs)
    want = np.array([mp_gelu_f32(h) for h in hs], dtype=np.float32).view(np.uint32)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(float(hs[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_gelu_exact_path_against_oracle(orc):
    """The same path against the oracle on 200k arguments spread over every
    binade the kernels send to it (tiny, ordinary, near -15, and the limits)."""
    run = _gelu_exact_host()
    rng = np.random.default_rng(2025)
    mags = 2.0 ** rng.uniform(-149, 4, 120000)
    hs = np.concatenate([(mags * rng.choice([-1, 1], mags.size)).astype(np.float32),
                         rng.uniform(-15, -6, 40000).astype(np.float32),
                         rng.uniform(-10, 10, 40000).astype(np.float32),
                         np.array([0.0, -0.0, np.inf, -np.inf, -15.0, -14.999], np.float32)])
    got = run(hs).view(np.float32)
    want = orc.fwd("sub", hs, np.zeros(1, np.float32), epi=orc.EPI_GELU)
    same = (got.view(np.uint32) == want.view(np.uint32))
    bad = np.flatnonzero(~same)
    assert bad.size == 0, [(float(hs[i]), float(got[i]), float(want[i])) for i in bad[:5]]


def test_debug_mode_from_environment():
    """ZK_DEBUG=1 turns the pointer checks on at the first consultation;
    zk_set_debug overrides it (a fresh process each, no GPU call)."""
    import sys
    code = ("from broadcast_autograd_amd import zk; L = zk.lib(); "
            "print(L.zk_set_debug(-1), L.zk_set_debug(0), L.zk_set_debug(-1), "
            "L.zk_set_debug(1), L.zk_set_debug(-1))")
    for env, want in (("1", "1 1 0 0 1"), ("0", "0 0 0 0 1"), (None, "0 0 0 0 1")):
        e = {k: v for k, v in os.environ.items() if k != "ZK_DEBUG"}
        if env is not None:
            e["ZK_DEBUG"] = env
        r = subprocess.run([sys.executable, "-c", code], env=e, cwd=ROOT, text=True,
                           capture_output=True, timeout=120, check=True)
        assert r.stdout.split() == want.split(), (env, r.stdout, r.stderr)


def test_debug_check_refuses_without_a_device(L):
    """With the checks on and no usable GPU (this host), a call is refused with
    ZK_ERR_DEVICE after validation and before any launch; validation errors
    still come first.  Skipped where a GPU is present: no test hands a host
    pointer to a call that could launch."""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    a = np.zeros(16, np.float32)
    d = zk.make_desc((16,))
    prev = zk.set_debug(1)
    try:
        p = a.ctypes.data
        rc = L.zk_binary_fwd(9, 0, p, ctypes.byref(d), p, ctypes.byref(d), p, None)
        assert rc == zk.ERR["ZK_ERR_UNSUPPORTED"]  # validation first
        out = np.zeros(16, np.float32)
        rc = L.zk_binary_fwd(0, 0, p, ctypes.byref(d), p, ctypes.byref(d), out.ctypes.data, None)
        assert rc == zk.ERR["ZK_ERR_DEVICE"]
        assert L.zk_status_string(rc).decode().startswith("a pointer is not device")
    finally:
        zk.set_debug(prev)


def test_noalloc_refusals_without_a_device(L):
    """zk_binary_bwd_noalloc on this GPU-less host: validation errors first,
    then a workspace need above ZK_SCRATCH_BYTES is ZK_ERR_WORKSPACE (decided
    from the shapes alone), and a call that fits is refused with ZK_ERR_DEVICE
    for want of a device.  Skipped where a GPU is present (no test hands a
    host pointer to a call that could launch)."""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    m = ctypes.c_void_p(1 << 20)  # non-NULL markers, never dereferenced here
    P = lambda k: ctypes.c_void_p(m.value + (k << 36))  # noqa: E731 (disjoint extents)
    # a transposed [131072, 4096] times [4096]: 1024 partials a column, 32 MiB
    da = zk.make_desc((131072, 4096), (1, 131072))
    db = zk.make_desc((4096,))
    rc = L.zk_binary_bwd_noalloc(9, 0, P(0), P(1), ctypes.byref(da), P(2), ctypes.byref(db),
                                 P(3), None, P(4), None, None)
    assert rc == zk.ERR["ZK_ERR_UNSUPPORTED"]
    rc = L.zk_binary_bwd_noalloc(2, 0, P(0), P(1), ctypes.byref(da), P(2), ctypes.byref(db),
                                 P(3), None, P(4), None, None)
    assert rc == zk.ERR["ZK_ERR_WORKSPACE"]
    ds, dsb = zk.make_desc((64, 256)), zk.make_desc((256,))
    rc = L.zk_binary_bwd_noalloc(2, 0, P(0), P(1), ctypes.byref(ds), P(2), ctypes.byref(dsb),
                                 P(3), None, P(4), None, None)
    assert rc == zk.ERR["ZK_ERR_DEVICE"]
