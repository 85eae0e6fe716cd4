"""GPU parity: the HIP path (through the C ABI) against the CPU oracle,
element by element, on seeded inputs.

Forward: bit-exact.  Backward: |err| <= 2e-6 * sum|terms| per element, plus one
binary32 subnormal step (2^-149) for results the format cannot resolve finer.
Every case, the full-size workloads included (the shapes and launch
configuration the benchmark times), is compared on every output element.
"""
import itertools
import math
import sys
import zlib

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from broadcast_autograd_amd import steps, workloads as W, zk  # noqa: E402
from gpu_util import (assert_bitexact, assert_bwd, assert_gelu_exact, dev,  # noqa: E402
                      host, strided_pair)

OPS = ["add", "sub", "mul", "div"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _name(request):
    say(f"\n[gpu] {request.node.name}")
    yield
    torch.cuda.synchronize()


def gpu_fwd(op, ta, tb, epi="none"):
    return host(zk.binary_fwd(op, ta, tb, epi=epi))


def check_pair(orc, op, va, ta, vb, tb, g_np=None, epi="none", acc=None,
               want=(True, True), seed=0):
    """Forward bit-exact and backward within tolerance for one operand pair."""
    e = orc.EPI_GELU if epi == "gelu" else orc.EPI_NONE
    want_f = orc.fwd(op, va, vb, epi=e)
    got_f = gpu_fwd(op, ta, tb, epi)
    if epi == "gelu":
        h = orc.fwd(op, va, vb)
        assert_gelu_exact(got_f, want_f, h)
    else:
        assert_bitexact(got_f, want_f, f"fwd {op}")
    if g_np is None:
        g_np = np.random.default_rng(seed).standard_normal(want_f.shape).astype(np.float32)
    g = dev(g_np)
    acc_a = acc_b = None
    acc_a_np = acc_b_np = None
    if acc is not None:
        acc_a_np, acc_b_np = acc
        acc_a = None if acc_a_np is None else dev(acc_a_np)
        acc_b = None if acc_b_np is None else dev(acc_b_np)
    ga, gb = zk.binary_bwd(op, g, ta, tb, need_a=want[0], need_b=want[1],
                           acc_a=acc_a, acc_b=acc_b, epi=epi)
    ra, rb = orc.bwd(op, g_np, va, vb, acc_a=acc_a_np, acc_b=acc_b_np, want=want, epi=e)
    if want[0]:
        assert_bwd(host(ga), ra, f"grad_a {op}")
    if want[1]:
        assert_bwd(host(gb), rb, f"grad_b {op}")


# ----------------------------------------------------------- worked examples
def test_chain_rule_worked_example_on_gpu(orc):
    """z = x*y + x at x=3, y=2: z = 9, dz/dx = 3, dz/dy = 3 (Autograd chapter)."""
    x = dev(np.array(3.0, np.float32))
    y = dev(np.array(2.0, np.float32))
    t = zk.binary_fwd("mul", x, y)
    z = zk.binary_fwd("add", t, x)
    assert float(host(z)) == 9.0
    g = dev(np.array(1.0, np.float32))
    g_t, g_x1 = zk.binary_bwd("add", g, t, x)
    g_x, g_y = zk.binary_bwd("mul", g_t, x, y, acc_a=g_x1)
    assert float(host(g_x)) == 3.0 and float(host(g_y)) == 3.0


def test_broadcast_worked_example_on_gpu():
    """[10,20,30] broadcast from [3] to [2,3]; its gradient sums to [2,2,2]."""
    v = dev(np.array([10, 20, 30], np.float32))
    z = dev(np.zeros((2, 3), np.float32))
    np.testing.assert_array_equal(host(zk.binary_fwd("add", z, v)),
                                  [[10, 20, 30], [10, 20, 30]])
    _, gb = zk.binary_bwd("add", dev(np.ones((2, 3), np.float32)), z, v)
    np.testing.assert_array_equal(host(gb), [2, 2, 2])


def test_strided_worked_example_on_gpu(orc):
    """Transposed view of [[1,2,3],[4,5,6]]: element (0,1) reads 4."""
    s = np.arange(1, 7, dtype=np.float32)
    v, t, _ = strided_pair(s, (3, 2), (1, 3))
    out = gpu_fwd("add", t, dev(np.zeros((3, 2), np.float32)))
    assert out[0, 1] == 4.0
    np.testing.assert_array_equal(out, [[1, 4], [2, 5], [3, 6]])


# ------------------------------------------- workloads at reduced sizes
def _rng_pair(shape_a, shape_b, seed, lo=0.5, hi=2.0, signed=True):
    rng = np.random.default_rng(seed)
    a = rng.uniform(lo, hi, shape_a).astype(np.float32)
    b = rng.uniform(lo, hi, shape_b).astype(np.float32)
    if signed:
        a *= np.where(rng.random(shape_a) < 0.5, -1, 1).astype(np.float32)
    return a, b


@pytest.mark.parametrize("shapes", [
    ((8, 128, 256), (128, 1)),        # config-1 layout, fewer batches
    ((7, 33, 260), (33, 1)),          # ragged rows and inner run
    ((3, 40, 1024), (40, 1)),
])
@pytest.mark.parametrize("op", OPS)
def test_row_scalar_broadcast(orc, shapes, op):
    a, b = _rng_pair(*shapes, seed=zlib.crc32(repr((shapes, op)).encode()))
    check_pair(orc, op, a, dev(a), b, dev(b), seed=1)
    # operand order swapped: the broadcast operand first
    check_pair(orc, op, b, dev(b), a, dev(a), seed=2)


@pytest.mark.parametrize("shapes", [
    ((512, 1024), (1024,)),           # config-2/5 layout
    ((300, 1000), (1000,)),           # ragged
    ((37, 4100), (4100,)),
    ((1, 4096), (4096,)),
])
@pytest.mark.parametrize("op", OPS)
def test_column_broadcast(orc, shapes, op):
    a, b = _rng_pair(*shapes, seed=zlib.crc32(repr((shapes, op)).encode()))
    check_pair(orc, op, a, dev(a), b, dev(b), seed=3)
    check_pair(orc, op, b, dev(b), a, dev(a), seed=4)


@pytest.mark.parametrize("shapes", [((512, 1024), (1024,)), ((300, 1000), (1000,)),
                                    ((64, 260), (64, 1))])
@pytest.mark.parametrize("op", OPS)
def test_gelu_epilogue(orc, shapes, op):
    rng = np.random.default_rng(5)
    a = rng.standard_normal(shapes[0]).astype(np.float32)
    b = (rng.standard_normal(shapes[1]) * 0.5 + (1.0 if op == "div" else 0.0)).astype(np.float32)
    check_pair(orc, op, a, dev(a), b, dev(b), epi="gelu", seed=6)


@pytest.mark.parametrize("rows,cols", [(2, 65536), (6, 70000), (7, 65536), (4, 262144),
                                       (6, 65532), (130, 4096), (1, 8)])
@pytest.mark.parametrize("epi", ["none", "relu"])
def test_shared_row_vector(orc, rows, cols, epi):
    """A dense [rows, cols] operand against one contiguous row vector that
    every row shares (the attention mask's pattern): an even row count with
    rows of at least 65536 elements takes the kernel that applies each
    16-byte piece of the vector to two rows; odd row counts and shorter rows
    the row kernel.  Both operand orders, every op, bit-exact."""
    rng = np.random.default_rng(zlib.crc32(repr((rows, cols, epi)).encode()))
    a = rng.standard_normal((rows, cols)).astype(np.float32)
    v = (rng.standard_normal(cols) + 2.0).astype(np.float32)
    e = orc.EPI_RELU if epi == "relu" else orc.EPI_NONE
    for op in OPS:
        for x, y in ((a, v), (v, a)):
            got = gpu_fwd(op, dev(x), dev(y), epi)
            assert_bitexact(got, orc.fwd(op, x, y, epi=e), f"{op} {x.shape} {y.shape} {epi}")


def test_mlp_bias_gelu_config_layout(orc):
    h = W.mlp_bias_gelu(rows=512)
    check_pair(orc, "add", h["act"], dev(h["act"]), h["bias"], dev(h["bias"]),
               g_np=h["g"], epi="gelu")


def test_attention_shaped_small(orc):
    h = W.attn_scale_mask(b=2, h=16, t=128)
    wl = steps.AttnScaleMask(host=h)
    wl.run()
    t = orc.fwd("mul", h["scores"], h["scale"])
    assert_bitexact(host(wl.t), t, "scores*scale")
    assert_bitexact(host(wl.out), orc.fwd("add", t, h["mask"]), "+mask")
    ra, rb = orc.bwd("mul", h["g"], h["scores"], h["scale"])
    assert_bwd(host(wl.grad_scores), ra, "grad_scores")
    assert_bwd(host(wl.grad_scale), rb, "grad_scale")
    # the mask's gradient would be g reduced to [1,1,T,T]
    mg = zk.reduce_to_shape(wl.g, (1, 1, 128, 128))
    assert_bwd(host(mg), orc.reduce_to_shape(h["g"], (1, 1, 128, 128)), "mask grad")


@pytest.mark.parametrize("n,m,ld,off", [(520, 392, 520, 0), (64, 64, 64, 0), (130, 260, 130, 0),
                                        (4096, 64, 4096, 0), (130, 260, 132, 0), (61, 128, 64, 0),
                                        (128, 96, 128, 1)])
@pytest.mark.parametrize("op", ["mul", "div", "sub"])
def test_transposed_operand(orc, n, m, ld, off, op):
    """a is a transposed view: sizes [n, m], strides [1, ld], storage offset
    off (column starts 16-byte aligned or not; rows a multiple of 4 or not)."""
    rng = np.random.default_rng(n * m + ld + off)
    s = rng.uniform(0.5, 2, off + ld * m).astype(np.float32)
    va, ta, _ = strided_pair(s, (n, m), (1, ld), off)
    b = rng.uniform(0.5, 2, (m,)).astype(np.float32)
    check_pair(orc, op, va, ta, b, dev(b), seed=7)
    check_pair(orc, op, b, dev(b), va, ta, seed=8)


def test_strided_transposed_config_layout(orc):
    h = W.strided_transposed(n=1024)
    wl = steps.StridedTransposed(host=h)
    wl.run()
    va = orc.View(h["a_storage"], h["a_sizes"], h["a_strides"])
    assert_bitexact(host(wl.out), orc.fwd("mul", va, h["b"]), "fwd")
    ra, rb = orc.bwd("mul", h["g"], va, h["b"])
    assert_bwd(host(wl.grad_a), ra, "grad_a")
    assert_bwd(host(wl.grad_b), rb, "grad_b")


def test_rank8_config_full(orc):
    h = W.rank8()
    wl = steps.Rank8(host=h)
    wl.run()
    assert_bitexact(host(wl.out), orc.fwd("div", h["a"], h["b"]), "fwd")
    ra, rb = orc.bwd("div", h["g"], h["a"], h["b"])
    assert_bwd(host(wl.grad_a), ra, "grad_a")
    assert_bwd(host(wl.grad_b), rb, "grad_b")


def test_xy_plus_x_small(orc):
    h = W.xy_plus_x(scale=0.125)
    wl = steps.XYPlusX(host=h)
    wl.run()
    t = orc.fwd("mul", h["x"], h["y"])
    assert_bitexact(host(wl.t), t, "x*y")
    assert_bitexact(host(wl.z), orc.fwd("add", t, h["x"]), "+x")
    # graph by hand: add hands g to t and x; mul adds x's second path
    rx, ry = orc.bwd("mul", h["g"], h["x"], h["y"], acc_a=h["g"])
    assert_bwd(host(wl.grad_x), rx, "grad_x")
    assert_bwd(host(wl.grad_y), ry, "grad_y")


def test_gpt_residual_small(orc):
    h = W.gpt_residual(b=2, t=64, c=4096)
    wl = steps.GPTResidual(host=h)
    wl.run()
    t = orc.fwd("mul", h["h"], h["gamma"])
    assert_bitexact(host(wl.t), t, "h*gamma")
    assert_bitexact(host(wl.out), orc.fwd("add", t, h["resid"]), "+resid")
    rh, rg = orc.bwd("mul", h["g"], h["h"], h["gamma"])
    assert_bwd(host(wl.grad_h), rh, "grad_h")
    assert_bwd(host(wl.grad_gamma), rg, "grad_gamma")
    _, rr = orc.bwd("add", h["g"], t, h["resid"], want=(False, True))
    assert_bwd(host(wl.grad_resid), rr, "grad_resid")


# ------------------------------------------------- brute force and fuzz
def _shapes(max_rank=3, sizes=(1, 2, 3)):
    for r in range(max_rank + 1):
        yield from itertools.product(sizes, repeat=r)


def test_bruteforce_small_shapes(orc):
    """Every shape pair of rank <= 3 with sizes in {1,2,3}, every op."""
    shapes = list(_shapes())
    rng = np.random.default_rng(21)
    count = 0
    for sa in shapes:
        for sb in shapes:
            try:
                np.broadcast_shapes(sa, sb)
            except ValueError:
                continue
            a = rng.uniform(0.5, 2, sa).astype(np.float32)
            b = rng.uniform(0.5, 2, sb).astype(np.float32)
            op = OPS[count % 4]
            check_pair(orc, op, a, dev(a), b, dev(b), seed=count)
            count += 1
    say(f"  {count} shape pairs")


def _random_view(rng, shape):
    """A random strided view with the given logical shape: permuted storage,
    stride-0 dims for size-1 dims, and a storage offset."""
    r = len(shape)
    perm = rng.permutation(r) if r else np.array([], int)
    # dense strides in a permuted storage order
    st = [0] * r
    s = 1
    for k in reversed(list(perm)):
        st[k] = s
        s *= max(shape[k], 1)
    for k in range(r):
        if shape[k] == 1 and rng.random() < 0.5:
            st[k] = 0
    off = int(rng.integers(0, 3))
    extent = off + sum((n - 1) * x for n, x in zip(shape, st)) + 1 if all(shape) else off + 1
    storage = rng.uniform(0.5, 2, max(extent, 1)).astype(np.float32)
    return strided_pair(storage, shape, st, off)


def test_fuzz_rank8_views(orc):
    """Seeded fuzz: rank <= 8, sizes 1-5, random broadcast masks, permuted
    views, zero strides, storage offsets (misaligned base pointers)."""
    rng = np.random.default_rng(77)
    for it in range(120):
        r = int(rng.integers(0, 9))
        out = [int(rng.integers(1, 6)) for _ in range(r)]
        if np.prod(out) > 20000:
            continue
        ra_ = int(rng.integers(0, r + 1))
        rb_ = int(rng.integers(0, r + 1))
        sa = [n if rng.random() < 0.6 else 1 for n in out[r - ra_:]]
        sb = [n if rng.random() < 0.6 else 1 for n in out[r - rb_:]]
        va, ta, _ = _random_view(rng, sa)
        vb, tb, _ = _random_view(rng, sb)
        op = OPS[it % 4]
        check_pair(orc, op, va, ta, vb, tb, seed=it)


def test_reduce_to_shape_cases(orc):
    rng = np.random.default_rng(31)
    cases = [((64, 1000), (1000,)), ((64, 1000), (64, 1)), ((64, 1000), ()),
             ((4, 5, 300), (5, 1)), ((4, 5, 300), (4, 1, 300)), ((3, 2048), (1, 1)),
             ((2, 3, 4, 5, 6, 7, 8, 9), (3, 1, 5, 1, 7, 1, 9)), ((16, 4096), (16, 4096)),
             ((0, 5), (5,)), ((6, 4096), (1,))]
    for sin, sout in cases:
        x = rng.standard_normal(sin).astype(np.float32)
        got = host(zk.reduce_to_shape(dev(x), sout))
        assert_bwd(got, orc.reduce_to_shape(x, sout), f"reduce {sin}->{sout}")
    # strided input
    s = rng.standard_normal(300 * 7).astype(np.float32)
    v, t, _ = strided_pair(s, (300, 7), (1, 300))
    assert_bwd(host(zk.reduce_to_shape(t, (7,))), orc.reduce_to_shape(v, (7,)), "strided")


def test_acc_modes(orc):
    rng = np.random.default_rng(41)
    a = rng.uniform(0.5, 2, (96, 512)).astype(np.float32)
    b = rng.uniform(0.5, 2, (512,)).astype(np.float32)
    g = rng.standard_normal((96, 512)).astype(np.float32)
    acc_a = rng.standard_normal((96, 512)).astype(np.float32)
    acc_b = rng.standard_normal((512,)).astype(np.float32)
    ta, tb, tg = dev(a), dev(b), dev(g)
    for op in OPS:
        # separate acc buffers
        ga, gb = zk.binary_bwd(op, tg, ta, tb, acc_a=dev(acc_a), acc_b=dev(acc_b))
        ra, rb = orc.bwd(op, g, a, b, acc_a=acc_a, acc_b=acc_b)
        assert_bwd(host(ga), ra, f"{op} acc_a")
        assert_bwd(host(gb), rb, f"{op} acc_b")
        # in place: acc == the gradient buffer
        xa, xb = dev(acc_a), dev(acc_b)
        zk.binary_bwd(op, tg, ta, tb, grad_a=xa, acc_a=xa, grad_b=xb, acc_b=xb)
        assert_bwd(host(xa), ra, f"{op} in-place a")
        assert_bwd(host(xb), rb, f"{op} in-place b")
        # acc == the upstream gradient itself
        ga, _ = zk.binary_bwd(op, tg, ta, tb, acc_a=tg)
        ra2, _ = orc.bwd(op, g, a, b, acc_a=g)
        assert_bwd(host(ga), ra2, f"{op} acc=grad")


@pytest.mark.parametrize("n", [4096, 1001, 3])
def test_pass_through_gradients(orc, n):
    """add's gradients and sub's are g and -g (the rules read no operand):
    one of them requested alone takes the plain copy kernel; with an
    accumulator buffer, in place, with the accumulator being g itself (the
    element-wise kernel), a ragged length (scalar tail) and a misaligned
    view (the element-wise kernel).  The result is exact: compared bit for
    bit with the oracle's rounded binary64 sum."""
    rng = np.random.default_rng(n)
    a = rng.standard_normal(n).astype(np.float32)
    b = rng.standard_normal(n).astype(np.float32)
    g = rng.standard_normal(n).astype(np.float32)
    acc = rng.standard_normal(n).astype(np.float32)
    ta, tb, tg = dev(a), dev(b), dev(g)
    for op in ("add", "sub"):
        for side in (0, 1):
            need = (side == 0, side == 1)
            kw = "acc_a" if side == 0 else "acc_b"
            gkw = "grad_a" if side == 0 else "grad_b"
            for mode in ("none", "buffer", "in_place", "g"):
                args = {}
                acc_np = None
                if mode == "buffer":
                    args[kw], acc_np = dev(acc), acc
                elif mode == "in_place":
                    x = dev(acc)
                    args[kw], args[gkw], acc_np = x, x, acc
                elif mode == "g":
                    args[kw], acc_np = tg, g
                got = zk.binary_bwd(op, tg, ta, tb, need_a=need[0], need_b=need[1], **args)[side]
                want = orc.bwd(op, g, a, b, want=need,
                               **({kw: acc_np} if acc_np is not None else {}))[side]
                assert_bitexact(host(got), want.f32, f"{op} side {side} acc {mode}")
    # a misaligned view of g: the element-wise kernel
    big = dev(np.concatenate([np.zeros(1, np.float32), g]))
    gv = big[1:]
    got = zk.binary_bwd("sub", gv, ta, tb, need_a=False)[1]
    want = orc.bwd("sub", g, a, b, want=(False, True))[1]
    assert_bitexact(host(got), want.f32, "sub side 1 misaligned")


def test_both_operands_broadcast(orc):
    rng = np.random.default_rng(51)
    for sa, sb in [((300, 1), (1, 200)), ((5, 1, 7), (1, 6, 1)), ((1, 64), (64, 1))]:
        for op in OPS:
            a, b = _rng_pair(sa, sb, seed=len(sa) * 7 + OPS.index(op))
            check_pair(orc, op, a, dev(a), b, dev(b), seed=3)


def test_edge_cases(orc):
    # rank 0 with rank 0, empty broadcast shapes, empty reduction
    for op in OPS:
        check_pair(orc, op, np.array(1.5, np.float32), dev(np.array(1.5, np.float32)),
                   np.array(0.75, np.float32), dev(np.array(0.75, np.float32)))
    e = dev(np.zeros((0, 4), np.float32))
    o = zk.binary_fwd("add", e, dev(np.ones((1, 4), np.float32)))
    assert tuple(o.shape) == (0, 4)
    _, gb = zk.binary_bwd("mul", dev(np.zeros((0, 4), np.float32)), e,
                          dev(np.ones((4,), np.float32)))
    np.testing.assert_array_equal(host(gb), np.zeros(4, np.float32))
    # special values: x/0, 0/0, inf - inf, subnormals, signed zeros
    a = np.array([1.0, 0.0, np.inf, 1e-40, -0.0, 3.0, -2.0, 1e38], np.float32)
    b = np.array([0.0, 0.0, np.inf, 3.0, 0.0, -0.0, 1e-39, 1e-2], np.float32)
    for op in OPS:
        assert_bitexact(gpu_fwd(op, dev(a), dev(b)), orc.fwd(op, a, b), f"special {op}")


def test_division_hard_cases(orc):
    """Correctly rounded binary32 division on awkward quotients."""
    rng = np.random.default_rng(61)
    n = 1 << 20
    a = (rng.standard_normal(n) * np.exp2(rng.integers(-126, 127, n))).astype(np.float32)
    b = (rng.standard_normal(n) * np.exp2(rng.integers(-126, 127, n))).astype(np.float32)
    b[::7] = np.exp2(rng.integers(-149, 128, b[::7].size).astype(np.float64)).astype(np.float32)
    b[b == 0] = 1.0
    assert_bitexact(gpu_fwd("div", dev(a), dev(b)), orc.fwd("div", a, b), "div")


def test_gelu_forward_dense_sweep(orc):
    """GeLU over 2^24 evenly spread binary32 values in [-12, 12]."""
    h = np.linspace(-12, 12, 1 << 24, dtype=np.float32)
    h[:16] = [0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45, 1e-38, -1e-38,
              -0.7518, -5.5, 5.5, -9.4, -13.0, 6.0, -6.0]
    z = np.zeros(1, np.float32)
    got = gpu_fwd("add", dev(h), dev(z), epi="gelu")
    want = orc.fwd("add", h, z, epi=orc.EPI_GELU)
    nties = assert_gelu_exact(got, want, h)
    say(f"  near-tie exceptions: {nties}")


def test_gelu_backward_dense_sweep(orc):
    """GeLU' over 2^20 evenly spread binary32 h in [-14, 14] (both sides of
    the kernels' binary32 range |h| <= 9) plus special values: the full-shape
    gradient and the gradient summed over 1024 rows."""
    n = 1 << 20
    h = np.linspace(-14, 14, n, dtype=np.float32)
    nine = np.float32(9.0)
    h[:14] = [0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45, nine, -nine,
              np.nextafter(nine, np.float32(10)), -np.nextafter(nine, np.float32(10)),
              -0.7518, 1e-38, -1e-38]
    act = h.reshape(1024, 1024)
    bias = np.zeros(1024, np.float32)
    g = np.random.default_rng(9).standard_normal((1024, 1024)).astype(np.float32)
    ga, gb = zk.binary_bwd("add", dev(g), dev(act), dev(bias), epi="gelu")
    ra, rb = orc.bwd("add", g, act, bias, epi=orc.EPI_GELU)
    ma = assert_bwd(host(ga), ra, "grad_act")
    mb = assert_bwd(host(gb), rb, "grad_bias")
    say(f"  largest error / allowance: grad_act {ma:.3f}, grad_bias {mb:.3f}")


def test_determinism(orc):
    """Two runs of the same backward give the same bits (no atomics)."""
    h = W.gpt_residual(b=2, t=256, c=4096)
    wl = steps.GPTResidual(host=h)
    outs = []
    for _ in range(2):
        wl.run()
        outs.append((host(wl.grad_h).copy(), host(wl.grad_gamma).copy()))
    for x, y in zip(*outs):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    wl2 = steps.AttnScaleMask(host=W.attn_scale_mask(b=2, h=16, t=256))
    r = []
    for _ in range(2):
        wl2.run()
        r.append(host(wl2.grad_scale).copy())
    assert np.array_equal(r[0].view(np.uint32), r[1].view(np.uint32))


@pytest.mark.parametrize("case", ["red_col", "red_col_interleaved", "red_row_blockwise",
                                  "red_col_gelu", "red_rowd"])
def test_determinism_concurrent_streams(orc, case):
    """The partition depends on the shapes only: a backward run alone and two
    copies of it running at once on two streams (other occupancy, other
    timing) give the same bits, within tolerance of the oracle."""
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    if case == "red_col":
        op, epi, sa, sb = "mul", "none", (2048, 4096), (4096,)
    elif case == "red_col_interleaved":
        op, epi, sa, sb = "mul", "none", (32768, 4096), (4096,)
    elif case == "red_row_blockwise":
        op, epi, sa, sb = "mul", "none", (2, 8, 262144), (8, 1)
    elif case == "red_col_gelu":
        op, epi, sa, sb = "add", "gelu", (1024, 1024), (1024,)
    else:
        op, epi, sa, sb = "mul", "none", (64, 128, 256), (128, 1)
    a_np = rng.standard_normal(sa).astype(np.float32)
    b_np = rng.standard_normal(sb).astype(np.float32)
    g_np = rng.standard_normal(sa).astype(np.float32)
    a, b, g = dev(a_np), dev(b_np), dev(g_np)
    nb = zk.bwd_workspace_bytes(op, a, b, epi=epi)
    outs = [(torch.empty_like(a), torch.empty_like(b), zk._workspace(nb, a.device))
            for _ in range(3)]
    torch.cuda.synchronize()
    zk.binary_bwd(op, g, a, b, grad_a=outs[0][0], grad_b=outs[0][1], workspace=outs[0][2],
                  epi=epi)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(2)]
    for s, o in zip(streams, outs[1:]):
        zk.binary_bwd(op, g, a, b, grad_a=o[0], grad_b=o[1], workspace=o[2], epi=epi,
                      stream=s)
    torch.cuda.synchronize()
    ref = [host(x).copy() for x in outs[0][:2]]
    for o in outs[1:]:
        for x, r in zip(o[:2], ref):
            assert np.array_equal(host(x).view(np.uint32), r.view(np.uint32))
    e = orc.EPI_GELU if epi == "gelu" else orc.EPI_NONE
    ra, rb = orc.bwd(op, g_np, a_np, b_np, epi=e)
    assert_bwd(ref[0], ra, "grad_a")
    assert_bwd(ref[1], rb, "grad_b")


def test_side_stream_allocations_outlive_their_kernels(orc, monkeypatch):
    """A backward on a side stream with the workspace and gradients left to
    the binding: those come from torch's allocator on the current stream, so
    the binding records their use on the side stream.  While that stream is
    still busy (a spin ahead of the call), a fresh allocation of the same size
    on the current stream must not get the workspace block back; a write
    there before synchronising leaves the result intact."""
    rng = np.random.default_rng(77)
    a_np = rng.standard_normal((1024, 1024)).astype(np.float32)
    b_np = rng.standard_normal(1024).astype(np.float32)
    g_np = rng.standard_normal((1024, 1024)).astype(np.float32)
    a, b, g = dev(a_np), dev(b_np), dev(g_np)
    seen = []
    real = zk._workspace

    def spy(nbytes, device):
        t = real(nbytes, device)
        seen.append((t.data_ptr(), t.numel()))
        return t

    monkeypatch.setattr(zk, "_workspace", spy)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        torch.cuda._sleep(int(2e8))     # keeps the side stream busy
    ga, gb = zk.binary_bwd("mul", g, a, b, stream=side)
    (wp, wn), = seen
    junk = torch.empty(wn, dtype=torch.uint8, device="cuda")
    assert junk.data_ptr() != wp, "workspace block reused while its kernels are queued"
    junk.fill_(0xFF)                    # NaN patterns, on the current stream
    torch.cuda.synchronize()
    ra, rb = orc.bwd("mul", g_np, a_np, b_np)
    assert_bwd(host(ga), ra, "grad_a")
    assert_bwd(host(gb), rb, "grad_b")


def test_debug_checks_accept_device_pointers(orc):
    """With the debug pointer checks on, every kind of call on device tensors
    of the current device, on the default stream and on a side stream, runs
    and returns the same bits as with the checks off."""
    rng = np.random.default_rng(81)
    a = dev(rng.standard_normal((256, 512)).astype(np.float32))
    b = dev(rng.standard_normal(512).astype(np.float32))
    c = dev(rng.standard_normal((256, 512)).astype(np.float32))
    g = dev(rng.standard_normal((256, 512)).astype(np.float32))

    def run(stream):
        gl = [c.clone(), g.clone()]     # clipped in place below
        if stream is not None:
            stream.wait_stream(torch.cuda.current_stream())
        out = [zk.binary_fwd("mul", a, b, epi="gelu", stream=stream)]
        out += zk.binary_bwd("mul", g, a, b, stream=stream)
        out.append(zk.reduce_to_shape(a, (1, 512), stream=stream))
        out.append(zk.mean_to_shape(a, (256, 1), stream=stream))
        out.append(zk.binary2_fwd("mul", "add", a, b, c, stream=stream))
        out += zk.binary2_bwd("mul", "add", g, a, b, c, stream=stream)
        out.append(zk.materialize(a.t(), stream=stream))
        out.append(zk.scalar_fwd("add", a, 2.5, stream=stream))
        out.append(zk.unary_bwd("gelu", g, a, stream=stream))
        out.append(zk.mean_bwd(b, (256, 512), stream=stream))
        out.append(zk.clip_grad_norm(gl, 1.0, stream=stream))
        out += gl
        out += zk.row_moments(a, stream=stream)
        out += zk.row_softmax_stats(a, stream=stream)
        return out

    torch.cuda.synchronize()
    ref = [host(x).copy() for x in run(None)]
    prev = zk.set_debug(1)
    try:
        for stream in (None, torch.cuda.Stream()):
            got = run(stream)
            torch.cuda.synchronize()
            for x, r in zip(got, ref):
                assert np.array_equal(host(x).view(np.uint32), r.view(np.uint32))
    finally:
        zk.set_debug(prev)


def test_mass_invariant_gpu():
    rng = np.random.default_rng(71)
    g = rng.standard_normal((64, 130, 64)).astype(np.float32)
    for tgt in [(130, 1), (1, 64), (64, 1, 1), ()]:
        r = host(zk.reduce_to_shape(dev(g), tgt)).astype(np.float64)
        exact = math.fsum(g.astype(np.float64).ravel())
        assert abs(r.sum() - exact) <= 2e-6 * np.abs(g).sum() + 1e-6 * r.size


# ------------------------------------ full sizes, every element checked
def _check_full_fwd(orc, op, a, b, got, what):
    """Every output element of a full-size forward against the oracle."""
    say(f"  {what}: {got.size} elements")
    assert_bitexact(got, orc.fwd(op, a, b), what)


def _check_full_bwd(orc, op, which, g, a, b, got, what, acc=None):
    """Every element of one full-size gradient against the oracle."""
    say(f"  {what}: {got.size} elements")
    want = (which == 0, which == 1)
    ra, rb = orc.bwd(op, g, a, b, acc_a=acc if which == 0 else None,
                     acc_b=acc if which == 1 else None, want=want)
    m = assert_bwd(got, ra if which == 0 else rb, what)
    say(f"    largest error / allowance {m:.3f}")


def test_full_size_xy_plus_x(orc):
    wl = steps.XYPlusX()
    h = wl.host
    wl.run()
    t = host(wl.t)
    _check_full_fwd(orc, "mul", h["x"], h["y"], t, "t = x * y")
    _check_full_fwd(orc, "add", t, h["x"], host(wl.z), "z = t + x")
    _check_full_bwd(orc, "mul", 0, h["g"], h["x"], h["y"], host(wl.grad_x), "grad_x",
                    acc=h["g"])
    _check_full_bwd(orc, "mul", 1, h["g"], h["x"], h["y"], host(wl.grad_y), "grad_y")


def test_full_size_mlp_bias_gelu(orc):
    wl = steps.MLPBiasGelu()
    h = wl.host
    wl.run()
    y = host(wl.y)
    want = orc.fwd("add", h["act"], h["bias"], epi=orc.EPI_GELU)
    assert_gelu_exact(y, want, orc.fwd("add", h["act"], h["bias"]))
    ra, rb = orc.bwd("add", h["g"], h["act"], h["bias"], epi=orc.EPI_GELU)
    ma = assert_bwd(host(wl.grad_act), ra, "grad_act")
    mb = assert_bwd(host(wl.grad_bias), rb, "grad_bias")
    say(f"  largest error / allowance: grad_act {ma:.3f}, grad_bias {mb:.3f}")


def test_full_size_attn_scale_mask(orc):
    wl = steps.AttnScaleMask()
    h = wl.host
    wl.run()
    t = host(wl.t)
    _check_full_fwd(orc, "mul", h["scores"], h["scale"], t, "t = scores * scale")
    _check_full_fwd(orc, "add", t, h["mask"], host(wl.out), "out = t + mask")
    del t
    _check_full_bwd(orc, "mul", 0, h["g"], h["scores"], h["scale"], host(wl.grad_scores),
                    "grad_scores")
    _check_full_bwd(orc, "mul", 1, h["g"], h["scores"], h["scale"], host(wl.grad_scale),
                    "grad_scale")


def test_full_size_attn_mask_grad(orc):
    """The benchmark's mask-gradient call: every one of the 1M outputs of
    g[8,16,1024,1024] summed to [1,1,1024,1024] against the oracle."""
    wl = steps.AttnMaskGrad()
    wl.run()
    ref = orc.reduce_to_shape(wl.host["g"], wl.target)
    m = assert_bwd(host(wl.grad_mask), ref, "grad_mask")
    say(f"  largest error / allowance: {m:.3f}")


@pytest.mark.parametrize("cols", [4, 8, 16, 32, 64, 128, 256])
@pytest.mark.parametrize("rows", [1, 63, 1001, 65537])
def test_short_rows(orc, rows, cols):
    """Row sums of short dense rows (256 / C rows a wave, a butterfly over a
    row's lanes), as sums and means, in rank 2 and as [rows, 1, C] -> [rows, 1, 1];
    a misaligned view takes the gather path."""
    rng = np.random.default_rng(zlib.crc32(repr((rows, cols)).encode()))
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    t = dev(x)
    ref = orc.reduce_to_shape(x, (rows, 1))
    assert_bwd(host(zk.reduce_to_shape(t, (rows, 1))), ref, f"sum {rows}x{cols}")
    assert_bwd(host(zk.mean_to_shape(t, (rows, 1))), orc.mean_to_shape(x, (rows, 1)), "mean")
    x3 = x.reshape(rows, 1, cols)
    assert_bwd(host(zk.reduce_to_shape(dev(x3), (rows, 1, 1))),
               orc.reduce_to_shape(x3, (rows, 1, 1)), "rank 3")
    if rows > 1:
        s = rng.standard_normal(rows * cols + 1).astype(np.float32)
        v, tv, _ = strided_pair(s, (rows, cols), (cols, 1), offset=1)
        assert_bwd(host(zk.reduce_to_shape(tv, (rows, 1))), orc.reduce_to_shape(v, (rows, 1)),
                   "misaligned")


@pytest.mark.parametrize("shape", [(3, 5, 8), (64, 1000, 4), (7, 33, 32), (256, 512, 128),
                                   (2, 4096, 64), (100, 30, 256), (8, 64, 256),
                                   (65536, 4, 4), (1000, 16, 16), (300, 100, 12),
                                   (4096, 3, 4), (513, 7, 12), (2049, 64, 256), (5, 300, 4)])
def test_short_rows_middle(orc, shape):
    """[R1, K, C] -> [K, 1] with short rows: with R1 <= C the row sums are
    binary64 partials of stage 2; with more rows the dense [R1, K * C] is
    summed by columns (folded below 256 columns) and stage 2 adds each kept
    element's C columns; other narrow shapes take the gather path (sums and
    means)."""
    rng = np.random.default_rng(zlib.crc32(repr(shape).encode()))
    x = rng.standard_normal(shape).astype(np.float32)
    t = dev(x)
    tgt = (shape[1], 1)
    assert_bwd(host(zk.reduce_to_shape(t, tgt)), orc.reduce_to_shape(x, tgt), f"sum {shape}")
    assert_bwd(host(zk.mean_to_shape(t, tgt)), orc.mean_to_shape(x, tgt), f"mean {shape}")


@pytest.mark.parametrize("rows,cols", [(4096, 4), (4096, 8), (8192, 32), (2048, 64), (1024, 128),
                                       (4000, 32), (4001, 32), (96, 128), (65536, 16)])
def test_narrow_columns(orc, rows, cols):
    """Column sums of fewer than 256 columns (rows folded into 256-wide ones
    when the row count allows): reduce, the multiply backward with the small
    operand's columns repeating across a folded row, GeLU, and acc in place."""
    rng = np.random.default_rng(zlib.crc32(repr((rows, cols)).encode()))
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    got = host(zk.reduce_to_shape(dev(x), (cols,)))
    assert_bwd(got, orc.reduce_to_shape(x, (cols,)), f"reduce {rows}x{cols}")
    b = rng.standard_normal(cols).astype(np.float32)
    g = rng.standard_normal((rows, cols)).astype(np.float32)
    ga, gb = zk.binary_bwd("mul", dev(g), dev(x), dev(b))
    ra, rb = orc.bwd("mul", g, x, b)
    assert_bwd(host(ga), ra, "grad_x")
    assert_bwd(host(gb), rb, "grad_b")
    bias = (0.02 * rng.standard_normal(cols)).astype(np.float32)
    ga, gb = zk.binary_bwd("add", dev(g), dev(x), dev(bias), epi="gelu")
    ra, rb = orc.bwd("add", g, x, bias, epi=orc.EPI_GELU)
    assert_bwd(host(ga), ra, "grad_act (gelu)")
    assert_bwd(host(gb), rb, "grad_bias (gelu)")
    prev = rng.standard_normal(cols).astype(np.float32)
    gb2 = dev(prev)
    zk.binary_bwd("mul", dev(g), dev(x), dev(b), need_a=False, grad_b=gb2, acc_b=gb2)
    _, rb2 = orc.bwd("mul", g, x, b, acc_b=prev, want=(False, True))
    assert_bwd(host(gb2), rb2, "grad_b += ")
    got = host(zk.mean_to_shape(dev(x), (cols,)))
    assert_bwd(got, orc.mean_to_shape(x, (cols,)), "mean")


@pytest.mark.parametrize("rows", [1, 2, 3, 4, 5, 7, 13, 100, 128, 257])
def test_short_columns(orc, rows):
    """Column sums over few rows of many columns (one partial a column, the
    rows split over the waves of a block), alone and fused with a rule."""
    rng = np.random.default_rng(1000 + rows)
    x = rng.standard_normal((rows, 8192)).astype(np.float32)
    got = host(zk.reduce_to_shape(dev(x), (8192,)))
    assert_bwd(got, orc.reduce_to_shape(x, (8192,)), f"reduce rows={rows}")
    b = rng.standard_normal(8192).astype(np.float32)
    g = rng.standard_normal((rows, 8192)).astype(np.float32)
    ga, gb = zk.binary_bwd("mul", dev(g), dev(x), dev(b))
    ra, rb = orc.bwd("mul", g, x, b)
    assert_bwd(host(ga), ra, "grad_x")
    assert_bwd(host(gb), rb, "grad_b")
    # accumulated in place onto an existing gradient, and the mean
    prev = rng.standard_normal(8192).astype(np.float32)
    gb2 = dev(prev)
    zk.binary_bwd("mul", dev(g), dev(x), dev(b), need_a=False, grad_b=gb2, acc_b=gb2)
    _, rb2 = orc.bwd("mul", g, x, b, acc_b=prev, want=(False, True))
    assert_bwd(host(gb2), rb2, "grad_b += ")
    got = host(zk.mean_to_shape(dev(x), (8192,)))
    assert_bwd(got, orc.mean_to_shape(x, (8192,)), f"mean rows={rows}")


def test_full_size_strided(orc):
    wl = steps.StridedTransposed()
    h = wl.host
    wl.run()
    va = orc.View(h["a_storage"], h["a_sizes"], h["a_strides"])
    _check_full_fwd(orc, "mul", va, h["b"], host(wl.out), "out = a^T * b")
    _check_full_bwd(orc, "mul", 0, h["g"], va, h["b"], host(wl.grad_a), "grad_a")
    _check_full_bwd(orc, "mul", 1, h["g"], va, h["b"], host(wl.grad_b), "grad_b")


def test_full_size_gpt_residual(orc):
    wl = steps.GPTResidual()
    h = wl.host
    wl.run()
    t = host(wl.t)
    _check_full_fwd(orc, "mul", h["h"], h["gamma"], t, "t = h * gamma")
    _check_full_fwd(orc, "add", t, h["resid"], host(wl.out), "out = t + resid")
    _check_full_bwd(orc, "mul", 0, h["g"], h["h"], h["gamma"], host(wl.grad_h), "grad_h")
    _check_full_bwd(orc, "mul", 1, h["g"], h["h"], h["gamma"], host(wl.grad_gamma),
                    "grad_gamma")
    _check_full_bwd(orc, "add", 1, h["g"], t, h["resid"], host(wl.grad_resid), "grad_resid")


def test_interleaved_column_sums_acc_modes(orc):
    """Long columns whose backward reads the full operand and writes its
    gradient: 16-wave blocks walk their rows interleaved across the grid, 4
    a wave.  A ragged row count (not a multiple of the 64 rows a partial
    covers), both sides, and every acc mode of the written gradient (none,
    acc == upstream grad, a separate buffer, in place)."""
    R, K = 32768 + 37, 4096
    info = zk.plan_describe("bwd", "mul", zk.make_desc((R, K)), zk.make_desc((K,)))
    assert info["kernel"] == "red_col" and info["partials"] == -(-R // 64), info
    rng = np.random.default_rng(83)
    a = rng.standard_normal((R, K)).astype(np.float32)
    b = rng.uniform(0.5, 2.0, K).astype(np.float32)
    g = rng.standard_normal((R, K)).astype(np.float32)
    acc = rng.standard_normal((R, K)).astype(np.float32)
    ta, tb, tg = dev(a), dev(b), dev(g)
    rb_ref = None
    for mode in ("none", "grad", "buffer", "inplace"):
        say(f"  acc mode {mode}")
        if mode == "none":
            ga, gb = zk.binary_bwd("mul", tg, ta, tb)
            want = orc.bwd("mul", g, a, b)
        elif mode == "grad":
            ga, gb = zk.binary_bwd("mul", tg, ta, tb, acc_a=tg)
            want = orc.bwd("mul", g, a, b, acc_a=g)
        elif mode == "buffer":
            ga, gb = zk.binary_bwd("mul", tg, ta, tb, acc_a=dev(acc))
            want = orc.bwd("mul", g, a, b, acc_a=acc)
        else:
            ga = dev(acc)
            _, gb = zk.binary_bwd("mul", tg, ta, tb, grad_a=ga, acc_a=ga)
            want = orc.bwd("mul", g, a, b, acc_a=acc)
        assert_bwd(host(ga), want[0], f"grad_a acc {mode}")
        assert_bwd(host(gb), want[1], f"grad_b acc {mode}")
        # the reduced gradient does not depend on the other gradient's acc
        got_b = host(gb)
        if rb_ref is None:
            rb_ref = got_b
        assert np.array_equal(got_b.view(np.int32), rb_ref.view(np.int32)), mode
        del ga, gb
    # the small operand first: b's gradient written in full, a's reduced
    ga, gb = zk.binary_bwd("mul", tg, tb, ta)
    want = orc.bwd("mul", g, b, a)
    assert_bwd(host(ga), want[0], "swapped grad_a")
    assert_bwd(host(gb), want[1], "swapped grad_b")


def test_interleaved_narrow_columns(orc):
    """The interleaved walk over folded rows: 32 columns read as rows of 256
    (8 rows each), 524,296 folded rows over 16-wave blocks (a ragged last
    band), the multiply backward writing the full gradient, with and without
    acc == upstream grad."""
    R, K = 4194304 + 64, 32
    info = zk.plan_describe("bwd", "mul", zk.make_desc((R, K)), zk.make_desc((K,)))
    assert info["kernel"] == "red_col" and info["partials"] == 8 * -(-(R // 8) // 1024), info
    rng = np.random.default_rng(89)
    a = rng.standard_normal((R, K)).astype(np.float32)
    b = rng.uniform(0.5, 2.0, K).astype(np.float32)
    g = rng.standard_normal((R, K)).astype(np.float32)
    ta, tb, tg = dev(a), dev(b), dev(g)
    for acc in (None, g):
        ga, gb = zk.binary_bwd("mul", tg, ta, tb, acc_a=None if acc is None else tg)
        ra, rb = orc.bwd("mul", g, a, b, acc_a=acc)
        assert_bwd(host(ga), ra, f"grad_a acc {acc is not None}")
        assert_bwd(host(gb), rb, f"grad_b acc {acc is not None}")


# One-pass row reductions (2048..16384 terms per kept element): a block per
# kept element finishes the sum itself.  Term counts at and between the
# limits of 1, 2 and 4 vectors per lane, ragged last vectors, every op with
# and without GeLU, the acc modes, and the plain reduction.
ROWD_SHAPES = [((64, 128, 256), (128, 1)),   # the x*y + x workload's y: T = 16384
               ((2, 7, 1024), (7, 1)),       # T = 2048, U = 1
               ((4096,), ()),                # T = 4096: one kept element
               ((3, 5, 1372), (5, 1)),       # T = 4116: U = 2, ragged vectors
               ((31, 2, 264), (2, 1)),       # T = 8184: U = 2
               ((4, 9, 2052), (9, 1)),       # T = 8208: U = 4
               ((16384,), (1,))]             # T = 16384, rank 1


@pytest.mark.parametrize("shapes", ROWD_SHAPES)
@pytest.mark.parametrize("op", OPS)
def test_one_pass_row_reduction(orc, shapes, op):
    sa, sb = shapes
    info = zk.plan_describe("bwd", op, zk.make_desc(sa), zk.make_desc(sb))
    assert info["kernel"] == "red_rowd", info
    a, b = _rng_pair(sa, sb, seed=sum(sa) + OPS.index(op))
    check_pair(orc, op, a, dev(a), b, dev(b), seed=5)
    if op in ("add", "mul"):
        check_pair(orc, op, a, dev(a), b, dev(b), seed=6, epi="gelu")
    rng = np.random.default_rng(sum(sa))
    g = rng.standard_normal(sa).astype(np.float32)
    acc_b = rng.standard_normal(sb).astype(np.float32)
    ga, gb = zk.binary_bwd(op, dev(g), dev(a), dev(b), acc_a=dev(g), acc_b=dev(acc_b))
    ra, rb = orc.bwd(op, g, a, b, acc_a=g, acc_b=acc_b)
    assert_bwd(host(ga), ra, f"{op} acc_a=g")
    assert_bwd(host(gb), rb, f"{op} acc_b")
    x = rng.standard_normal(sa).astype(np.float32)
    assert_bwd(host(zk.reduce_to_shape(dev(x), sb)), orc.reduce_to_shape(x, sb), "reduce")
    m = host(zk.mean_to_shape(dev(x), sb))
    assert_bwd(m, orc.mean_to_shape(x, sb), "mean")


@pytest.mark.parametrize("op2", ["add", "sub"])
def test_one_pass_row_reduction_fused(orc, op2):
    """The fused expression's c gradient through the one-pass kernels: c with
    the full shape (written beside a's gradient) and c broadcast (a signed
    one-pass reduction of g)."""
    rng = np.random.default_rng(61)
    a = rng.standard_normal((16, 96, 256)).astype(np.float32)
    b = rng.uniform(0.5, 2.0, (96, 1)).astype(np.float32)
    g = rng.standard_normal((16, 96, 256)).astype(np.float32)
    for c in (rng.standard_normal((16, 96, 256)).astype(np.float32),
              rng.standard_normal((96, 1)).astype(np.float32)):
        grads = zk.binary2_bwd("mul", op2, dev(g), dev(a), dev(b), dev(c))
        want = orc.bwd2("mul", op2, g, a, b, c)
        for got, ref, name in zip(grads, want, "abc"):
            assert_bwd(host(got), ref, f"fused {op2} grad_{name} c{c.shape}")


# Streaming row reductions whose pass also reads or writes the full operand:
# four chunks of a row to a block, their sums met in LDS (one partial per
# block) when a row's chunk count divides by 4; else one partial a wave.
# (shapes, partials per kept element): ragged last chunks, rank 2 and 3,
# 256- and 512-element chunks.
ROWB_SHAPES = [(((9, 5, 2000), (5, 1)), 18),      # 8 chunks of 256 a row, last 208
               (((5, 3, 4000), (3, 1)), 20),      # 16 chunks, last 160
               (((3, 20480), (3, 1)), 20),        # rank 2, 80 chunks
               (((7, 3, 2600), (3, 1)), 77),      # 11 chunks a row: one partial a wave
               (((2, 8, 262144), (8, 1)), 256)]   # 512-element chunks


@pytest.mark.parametrize("shapes,parts", ROWB_SHAPES, ids=[str(s[0][0]) for s in ROWB_SHAPES])
@pytest.mark.parametrize("op", OPS)
def test_row_reduction_blockwise(orc, shapes, parts, op):
    sa, sb = shapes
    info = zk.plan_describe("bwd", op, zk.make_desc(sa), zk.make_desc(sb))
    assert info["kernel"] == "red_row" and info["partials"] == parts, info
    a, b = _rng_pair(sa, sb, seed=sum(sa) + OPS.index(op))
    check_pair(orc, op, a, dev(a), b, dev(b), seed=9)
    if op in ("add", "mul"):
        check_pair(orc, op, a, dev(a), b, dev(b), seed=10, epi="gelu")
    rng = np.random.default_rng(sum(sa) + 1)
    g = rng.standard_normal(sa).astype(np.float32)
    acc_a = rng.standard_normal(sa).astype(np.float32)
    acc_b = rng.standard_normal(sb).astype(np.float32)
    # separate acc buffers (a third full-size read)
    ga, gb = zk.binary_bwd(op, dev(g), dev(a), dev(b), acc_a=dev(acc_a), acc_b=dev(acc_b))
    ra, rb = orc.bwd(op, g, a, b, acc_a=acc_a, acc_b=acc_b)
    assert_bwd(host(ga), ra, f"{op} acc_a")
    assert_bwd(host(gb), rb, f"{op} acc_b")
    # the reduced gradient alone (the full operand read, not written)
    _, gb = zk.binary_bwd(op, dev(g), dev(a), dev(b), need_a=False)
    assert_bwd(host(gb), orc.bwd(op, g, a, b)[1], f"{op} grad_b alone")


# One-pass gather reductions (32..4096 terms per kept element on patterns
# the streaming classes do not take): a wave per kept element, also writing
# the full operand's gradient.
GEND_SHAPES = [((40, 3, 7), (1, 3, 1)),       # T = 280, inner dim reduced but short
               ((5, 64, 3), (5, 1, 3)),       # middle dim reduced: T = 64
               ((4096, 3), (1, 3)),           # T = 4096, inner 3
               ((33, 5), (1, 5))]             # T = 33


@pytest.mark.parametrize("shapes", GEND_SHAPES)
@pytest.mark.parametrize("op", OPS)
def test_one_pass_gather_reduction(orc, shapes, op):
    sa, sb = shapes
    info = zk.plan_describe("bwd", op, zk.make_desc(sa), zk.make_desc(sb))
    assert info["kernel"] == "red_gend", info
    a, b = _rng_pair(sa, sb, seed=sum(sa) + OPS.index(op))
    check_pair(orc, op, a, dev(a), b, dev(b), seed=7)
    if op in ("add", "mul"):
        check_pair(orc, op, a, dev(a), b, dev(b), seed=8, epi="gelu")
    rng = np.random.default_rng(sum(sa) + 1)
    g = rng.standard_normal(sa).astype(np.float32)
    acc_a = rng.standard_normal(sa).astype(np.float32)
    acc_b = rng.standard_normal(sb).astype(np.float32)
    # acc == g for the full gradient, a separate acc for the reduced one
    ga, gb = zk.binary_bwd(op, dev(g), dev(a), dev(b), acc_a=dev(g), acc_b=dev(acc_b))
    ra, rb = orc.bwd(op, g, a, b, acc_a=g, acc_b=acc_b)
    assert_bwd(host(ga), ra, f"{op} acc_a=g")
    assert_bwd(host(gb), rb, f"{op} acc_b")
    # separate acc buffers, in place
    xa, xb = dev(acc_a), dev(acc_b)
    zk.binary_bwd(op, dev(g), dev(a), dev(b), grad_a=xa, acc_a=xa, grad_b=xb, acc_b=xb)
    ra, rb = orc.bwd(op, g, a, b, acc_a=acc_a, acc_b=acc_b)
    assert_bwd(host(xa), ra, f"{op} in-place a")
    assert_bwd(host(xb), rb, f"{op} in-place b")
    # only the reduced gradient
    _, gb = zk.binary_bwd(op, dev(g), dev(a), dev(b), need_a=False)
    _, rb = orc.bwd(op, g, a, b, want=(False, True))
    assert_bwd(host(gb), rb, f"{op} b only")


# One-pass run reductions: the two innermost canonical dims form a short
# contiguous run ([reduced, kept] or [kept, reduced], 64..256 elements), a
# block per combination of the outer kept dims reading every element once.
RUN_SHAPES = [((2, 3, 4, 5, 6, 7, 8, 9), (1, 3, 1, 5, 1, 7, 1, 9)),  # the rank-8 workload: run [8, 9]
              ((4, 40, 6, 12), (1, 40, 1, 12)),          # run [6 reduced, 12 kept]
              ((2, 33, 3, 4, 16), (1, 33, 1, 4, 1)),     # run [4 kept, 16 reduced]
              ((6, 40, 3, 8, 8), (1, 40, 1, 8, 8))]      # run [3 reduced, 64 kept] (8 x 8 merged)


@pytest.mark.parametrize("shapes", RUN_SHAPES)
@pytest.mark.parametrize("op", OPS)
def test_one_pass_run_reduction(orc, shapes, op):
    sa, sb = shapes
    info = zk.plan_describe("bwd", op, zk.make_desc(sa), zk.make_desc(sb))
    assert info["kernel"] == "red_run", info
    a, b = _rng_pair(sa, sb, seed=sum(sa) + OPS.index(op) + 7)
    check_pair(orc, op, a, dev(a), b, dev(b), seed=17)
    if op in ("add", "mul"):
        check_pair(orc, op, a, dev(a), b, dev(b), seed=18, epi="gelu")
    rng = np.random.default_rng(sum(sa) + 3)
    g = rng.standard_normal(sa).astype(np.float32)
    acc_a = rng.standard_normal(sa).astype(np.float32)
    acc_b = rng.standard_normal(sb).astype(np.float32)
    ga, gb = zk.binary_bwd(op, dev(g), dev(a), dev(b), acc_a=dev(g), acc_b=dev(acc_b))
    ra, rb = orc.bwd(op, g, a, b, acc_a=g, acc_b=acc_b)
    assert_bwd(host(ga), ra, f"{op} acc_a=g")
    assert_bwd(host(gb), rb, f"{op} acc_b")
    xa, xb = dev(acc_a), dev(acc_b)
    zk.binary_bwd(op, dev(g), dev(a), dev(b), grad_a=xa, acc_a=xa, grad_b=xb, acc_b=xb)
    ra, rb = orc.bwd(op, g, a, b, acc_a=acc_a, acc_b=acc_b)
    assert_bwd(host(xa), ra, f"{op} in-place a")
    assert_bwd(host(xb), rb, f"{op} in-place b")
    _, gb = zk.binary_bwd(op, dev(g), dev(a), dev(b), need_a=False)
    _, rb = orc.bwd(op, g, a, b, want=(False, True))
    assert_bwd(host(gb), rb, f"{op} b only")
    # the same pattern with a as the broadcast operand
    ga, gb = zk.binary_bwd(op, dev(g), dev(b), dev(a))
    ra, rb = orc.bwd(op, g, b, a)
    assert_bwd(host(ga), ra, f"{op} swapped grad_a")
    assert_bwd(host(gb), rb, f"{op} swapped grad_b")
    # reduce and mean through the same class, and twice for determinism
    info = zk.plan_describe("reduce", "add", zk.make_desc(sa), zk.make_desc(sb))
    assert info["kernel"] == "red_run", info
    r1 = host(zk.reduce_to_shape(dev(g), sb))
    assert_bwd(r1, orc.reduce_to_shape(g, sb), "reduce")
    assert np.array_equal(r1.view(np.uint32), host(zk.reduce_to_shape(dev(g), sb)).view(np.uint32))
    assert_bwd(host(zk.mean_to_shape(dev(g), sb)), orc.mean_to_shape(g, sb), "mean")


def test_one_pass_gather_reduce_mean_and_fused(orc):
    rng = np.random.default_rng(71)
    # transposed views reduced and averaged
    for sizes, strides, target in (((300, 7), (1, 300), (7,)), ((64, 40), (1, 64), (1, 40)),
                                   ((9, 10, 11), (110, 1, 10), (1, 10, 1))):
        span = sum((n - 1) * st for n, st in zip(sizes, strides)) + 1
        stor = rng.standard_normal(span).astype(np.float32)
        v, t, _ = strided_pair(stor, sizes, strides)
        info = zk.plan_describe("reduce", "add", zk.desc_of(t), zk.make_desc(target))
        assert info["kernel"] == "red_gend", info
        assert_bwd(host(zk.reduce_to_shape(t, target)), orc.reduce_to_shape(v, target),
                   f"reduce {sizes}")
        assert_bwd(host(zk.mean_to_shape(t, target)), orc.mean_to_shape(v, target),
                   f"mean {sizes}")
    # both operands broadcast
    for sa, sb in (((300, 1), (1, 200)), ((40, 1, 7), (1, 30, 1))):
        for op in OPS:
            a, b = _rng_pair(sa, sb, seed=len(sa) + OPS.index(op))
            check_pair(orc, op, a, dev(a), b, dev(b), seed=9)
    # fused expression whose c is reduced on a gather pattern, with a sign
    a = rng.standard_normal((40, 3, 7)).astype(np.float32)
    b = rng.uniform(0.5, 2.0, (1, 3, 1)).astype(np.float32)
    c = rng.standard_normal((1, 3, 7)).astype(np.float32)
    g = rng.standard_normal((40, 3, 7)).astype(np.float32)
    for op2 in ("add", "sub"):
        grads = zk.binary2_bwd("mul", op2, dev(g), dev(a), dev(b), dev(c))
        want = orc.bwd2("mul", op2, g, a, b, c)
        for got, ref, name in zip(grads, want, "abc"):
            assert_bwd(host(got), ref, f"fused {op2} grad_{name}")
