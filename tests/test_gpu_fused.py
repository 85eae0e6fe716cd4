"""GPU parity of the fused two-operator expression out = (a op1 b) op2 c
(Operator chapter, "fusion") against the CPU oracle, through the C ABI.

Forward: bit-exact (the same two binary32 roundings as the unfused pair).
Backward: |err| <= 2e-6 * sum|terms| (+ one binary32 subnormal step).
"""
import sys
import zlib

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from broadcast_autograd_amd import steps, workloads as W, zk  # noqa: E402
from gpu_util import assert_bitexact, assert_bwd, dev, host, strided_pair  # noqa: E402

OPS1 = ["add", "sub", "mul", "div"]
OPS2 = ["add", "sub"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _name(request):
    say(f"\n[gpu] {request.node.name}")
    yield
    torch.cuda.synchronize()


def _vals(rng, shape, lo=0.5, hi=2.0, signed=True):
    x = rng.uniform(lo, hi, shape).astype(np.float32)
    if signed:
        x *= np.where(rng.random(shape) < 0.5, -1, 1).astype(np.float32)
    return x


def check3(orc, op1, op2, a, b, c, ta, tb, tc, seed=0, need=(True, True, True), accs=None):
    want = orc.fwd2(op1, op2, a, b, c)
    got = host(zk.binary2_fwd(op1, op2, ta, tb, tc))
    assert_bitexact(got, want, f"fwd2 {op1},{op2}")
    g = np.random.default_rng(seed).standard_normal(want.shape).astype(np.float32)
    accs = accs or (None, None, None)
    dacc = tuple(None if x is None else dev(x) for x in accs)
    ga = zk.binary2_bwd(op1, op2, dev(g), ta, tb, tc, need=need, accs=dacc)
    ref = orc.bwd2(op1, op2, g, a, b, c, acc=accs, want=need)
    for k, name in enumerate("abc"):
        if need[k]:
            assert_bwd(host(ga[k]), ref[k], f"grad_{name} {op1},{op2}")


SHAPES = [
    ((64, 256), (256,), (64, 256)),          # residual-like, c dense
    ((4, 16, 64), (16, 1), (4, 16, 64)),     # x*y + z with y a column
    ((8, 4, 128), (1, 4, 1), (1, 1, 128)),   # attention-like: scale and mask
    ((32, 96), (96,), (1, 96)),              # c a broadcast row
    ((30, 70), (70,), (30, 1)),              # inner dim not a multiple of 4
    ((2, 3, 4, 5, 6), (1, 3, 1, 5, 1), (4, 5, 6)),  # rank 5: generic kernels
    ((3, 1), (1, 4), (2, 3, 4)),             # t repeated into out (split path)
    ((), (5,), (2, 5)),                      # scalar a
    ((5, 4096), (4096,), (5, 4096)),         # short columns: sums finished in stage 1
    ((6, 2048), (2048,), (1, 2048)),         # short columns, c a broadcast row
]


@pytest.mark.parametrize("shapes", SHAPES)
@pytest.mark.parametrize("op1", OPS1)
@pytest.mark.parametrize("op2", OPS2)
def test_fused_shapes(orc, shapes, op1, op2):
    sa, sb, sc = shapes
    rng = np.random.default_rng(zlib.crc32(repr((shapes, op1, op2)).encode()))
    a, b, c = _vals(rng, sa), _vals(rng, sb), _vals(rng, sc)
    check3(orc, op1, op2, a, b, c, dev(a), dev(b), dev(c), seed=3)


def test_fused_accumulate(orc):
    rng = np.random.default_rng(11)
    a, b, c = _vals(rng, (48, 64)), _vals(rng, (64,)), _vals(rng, (48, 64))
    accs = tuple(rng.standard_normal(s).astype(np.float32) for s in ((48, 64), (64,), (48, 64)))
    check3(orc, "mul", "sub", a, b, c, dev(a), dev(b), dev(c), seed=4, accs=accs)
    # c broadcast: its gradient is a (negated) sum plus acc
    c1 = _vals(rng, (1, 64))
    accs1 = (accs[0], accs[1], rng.standard_normal((1, 64)).astype(np.float32))
    check3(orc, "div", "sub", a, b, c1, dev(a), dev(b), dev(c1), seed=5, accs=accs1)


@pytest.mark.parametrize("need", [(True, False, True), (False, True, False),
                                  (False, False, True), (True, True, False)])
def test_fused_partial_requests(orc, need):
    rng = np.random.default_rng(12)
    a, b, c = _vals(rng, (16, 128)), _vals(rng, (128,)), _vals(rng, (16, 128))
    check3(orc, "mul", "add", a, b, c, dev(a), dev(b), dev(c), seed=6, need=need)


def test_fused_strided_views(orc):
    """Transposed and stride-0 views on every input (generic and gather
    paths of the fused kernels)."""
    rng = np.random.default_rng(13)
    s = rng.uniform(0.5, 2, 40 * 24).astype(np.float32)
    va, ta, _ = strided_pair(s, (24, 40), (1, 24))  # transposed
    b = _vals(rng, (40,))
    sc = rng.uniform(0.5, 2, 24 * 3).astype(np.float32)
    vc, tc, _ = strided_pair(sc, (24, 40), (3, 0))  # stride-0 inner
    for op1 in OPS1:
        check3(orc, op1, "add", va, b, vc, ta, dev(b), tc, seed=7)


def test_fused_tie_xy_plus_x(orc):
    """z = x*y + x (Autograd chapter worked example, config layout at a small
    size): x's two paths accumulate into one buffer."""
    h = W.xy_plus_x()
    x, y, g = h["x"][:4], h["y"], h["g"][:4]
    tx, ty = dev(x), dev(y)
    z = host(zk.binary2_fwd("mul", "add", tx, ty, tx))
    assert_bitexact(z, orc.fwd2("mul", "add", x, y, x), "fwd2 tie")
    gx, gy, gc = zk.binary2_bwd("mul", "add", dev(g), tx, ty, tx, tie="a")
    assert gc is None
    rx, ry, _ = orc.bwd2("mul", "add", g, x, y, x, tie="a")
    assert_bwd(host(gx), rx, "grad_x (both paths)")
    assert_bwd(host(gy), ry, "grad_y")
    # the worked example itself
    one = dev(np.array([1.0], np.float32))
    x3, y2 = dev(np.array([3.0], np.float32)), dev(np.array([2.0], np.float32))
    assert float(host(zk.binary2_fwd("mul", "add", x3, y2, x3))[0]) == 9.0
    gx, gy, _ = zk.binary2_bwd("mul", "add", one, x3, y2, x3, tie="a")
    assert float(host(gx)[0]) == 3.0 and float(host(gy)[0]) == 3.0


def test_fused_matches_unfused_pair_bitwise():
    """The fused forward equals zk_binary_fwd(op1) then zk_binary_fwd(op2)."""
    rng = np.random.default_rng(14)
    a, b, c = _vals(rng, (8, 16, 256)), _vals(rng, (16, 1)), _vals(rng, (8, 16, 256))
    ta, tb, tc = dev(a), dev(b), dev(c)
    for op1 in OPS1:
        for op2 in OPS2:
            t = zk.binary_fwd(op1, ta, tb)
            want = host(zk.binary_fwd(op2, t, tc))
            got = host(zk.binary2_fwd(op1, op2, ta, tb, tc))
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (op1, op2)


def test_fused_empty_and_zero_sizes(orc):
    a = np.zeros((3, 0), np.float32)
    b = np.ones((1,), np.float32)
    c = np.ones((3, 1), np.float32)
    out = zk.binary2_fwd("mul", "add", dev(a), dev(b), dev(c))
    assert tuple(out.shape) == (3, 0)
    # out is empty: every gradient is a sum over nothing (its acc, or 0)
    g = dev(np.zeros((3, 0), np.float32))
    acc_b = np.array([2.5], np.float32)
    ga, gb, gc = zk.binary2_bwd("mul", "add", g, dev(a), dev(b), dev(c),
                                accs=(None, dev(acc_b), None))
    assert host(gb)[0] == 2.5 and np.all(host(gc) == 0)


def test_fused_determinism():
    h = W.gpt_residual(b=2, t=128, c=4096)
    wl = steps.GPTResidualFused(host=h)
    outs = []
    for _ in range(2):
        wl.run()
        outs.append([host(getattr(wl, k)).copy() for k in ("out", "grad_h", "grad_gamma",
                                                            "grad_resid")])
    for x, y in zip(*outs):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


# ----------------------------------------- full sizes of the fused workloads
# Every element of every output against the oracle's full fused entry points.
@pytest.mark.parametrize("shapes", [
    ((2, 4, 65536), (1, 4, 1), (1, 1, 65536)),   # per-row scalar b, shared vector c (rank 3)
    ((4, 65536), (65536,), (4, 1)),              # shared vector b, per-row scalar c (rank 2)
    ((3, 65536), (1, 1), (65536,)),              # odd row count: the row kernel
    ((2, 4, 65532), (1, 4, 1), (1, 1, 65532)),   # rows below 65536 elements: the row kernel
])
@pytest.mark.parametrize("op1", ["add", "sub", "mul", "div"])
def test_fused_shared_row_vector(orc, shapes, op1):
    """(a op1 b) op2 c with one small operand a row vector every row shares
    and the other a scalar per row (the attention's scale and mask): the
    kernel that applies each piece of the vector to two rows, bit for bit
    against the oracle's two roundings, op2 add and sub."""
    rng = np.random.default_rng(zlib.crc32(repr((shapes, op1)).encode()))
    a = _vals(rng, shapes[0])
    b = _vals(rng, shapes[1])
    c = _vals(rng, shapes[2])
    for op2 in ("add", "sub"):
        got = host(zk.binary2_fwd(op1, op2, dev(a), dev(b), dev(c)))
        assert_bitexact(got, orc.fwd2(op1, op2, a, b, c), f"{op1} {op2} {shapes}")


def _check_fused(orc, wl, a, b, c, names, tie=None):
    h = wl.host
    say(f"  out: {wl.__dict__[names[3]].numel()} elements")
    assert_bitexact(host(getattr(wl, names[3])),
                    orc.fwd2("mul", "add", h[a], h[b], h[c]), names[3])
    want = tuple(n is not None for n in names[:3])
    refs = orc.bwd2("mul", "add", h["g"], h[a], h[b], h[c], want=want, tie=tie)
    for ref, name in zip(refs, names[:3]):
        if name is None:
            continue
        say(f"  {name}")
        m = assert_bwd(host(getattr(wl, name)), ref, name)
        say(f"    largest error / allowance {m:.3f}")


def test_full_size_fused_gpt_residual(orc):
    wl = steps.GPTResidualFused()
    wl.run()
    _check_fused(orc, wl, "h", "gamma", "resid", ("grad_h", "grad_gamma", "grad_resid", "out"))


def test_full_size_fused_attn_scale_mask(orc):
    wl = steps.AttnScaleMaskFused()
    wl.run()
    _check_fused(orc, wl, "scores", "scale", "mask", ("grad_scores", "grad_scale", None, "out"))


def test_full_size_fused_xy_plus_x(orc):
    wl = steps.XYPlusXFused()
    wl.run()
    _check_fused(orc, wl, "x", "y", "x", ("grad_x", "grad_y", None, "z"), tie="a")
