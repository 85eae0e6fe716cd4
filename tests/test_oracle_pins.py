"""Pins for the CPU oracle: facts fixed by the "Zero" book's worked examples,
by calculus and by IEEE-754, checked independently of the oracle's own code.

Each test names what it pins; together they are chosen so that a dropped term,
a wrong sign, a wrong index or a transposed operand in the oracle fails one.
"""
import ast
import itertools
import math
import os
import re
import zlib

import numpy as np
import pytest

from conftest import GOLDEN

F32 = np.float32


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def _kv(lines):
    out = {}
    for ln in lines:
        k, v = ln.split("=")
        out[k.strip()] = float(v)
    return out


def _scalar(v):
    return np.array(v, dtype=np.float32)


# --------------------------------------------------------------- P1 -------
def test_chain_rule_worked_example(orc):
    """Autograd chapter, "computation graph": z = x*y + x at x=3, y=2."""
    v = _kv(_golden("chain_rule_example.txt"))
    x, y = _scalar(v["x"]), _scalar(v["y"])
    t = orc.fwd("mul", x, y)
    z = orc.fwd("add", t, x)
    assert float(t) == v["xy"] and float(z) == v["z"]
    # backward, root gradient 1: Add passes it to both inputs ...
    g = _scalar(v["dz_dz"])
    g_t, g_x_add = orc.bwd("add", g, t, x)
    # ... Mul's rule then gives x the second path, accumulated on the first.
    g_x, g_y = orc.bwd("mul", g_t.f32, x, y, acc_a=g_x_add.f32)
    assert float(g_x.f32) == v["dz_dx"]
    assert float(g_y.f32) == v["dz_dy"]
    # dropping the accumulated path gives y = 2, not 3
    g_x_only, _ = orc.bwd("mul", g_t.f32, x, y)
    assert float(g_x_only.f32) == 2.0


# ----------------------------------------------------------- P2, P3, P4 ---
def test_broadcast_worked_examples(orc):
    """Operator chapter, "broadcast": shape rule, [3]->[2,3] and its sum."""
    for ln in _golden("broadcast_examples.txt"):
        if ln.startswith("shape"):
            m = re.match(r"shape (\[.*\]) & (\[.*\]) -> (.*)", ln)
            sa, sb = ast.literal_eval(m.group(1)), ast.literal_eval(m.group(2))
            res = m.group(3).strip()
            if res == "incompatible":
                with pytest.raises(orc.OracleError) as e:
                    orc.broadcast_shape(sa, sb)
                assert e.value.code == orc.ERR_BROADCAST
                with pytest.raises(orc.OracleError):
                    orc.broadcast_shape(sb, sa)
            else:
                assert orc.broadcast_shape(sa, sb) == tuple(ast.literal_eval(res))
                assert orc.broadcast_shape(sb, sa) == tuple(ast.literal_eval(res))
        elif ln.startswith("expand"):
            m = re.match(r"expand (\[.*\]) : (\[.*\]) -> (\[.*\]) = (.*)", ln)
            vec = np.array(ast.literal_eval(m.group(1)), dtype=np.float32)
            tgt = ast.literal_eval(m.group(3))
            want = np.array(ast.literal_eval(m.group(4)), dtype=np.float32)
            got = orc.fwd("add", np.zeros(tgt, np.float32), vec)
            assert got.shape == tuple(tgt)
            np.testing.assert_array_equal(got, want)
        elif ln.startswith("reduce"):
            m = re.match(r"reduce ones(\[.*\]) -> (\[.*\]) = (.*)", ln)
            big = ast.literal_eval(m.group(1))
            small = ast.literal_eval(m.group(2))
            want = np.array(ast.literal_eval(m.group(3)), dtype=np.float32)
            g = np.ones(big, np.float32)
            _, gb = orc.bwd("add", g, np.zeros(big, np.float32),
                            np.zeros(small, np.float32))
            np.testing.assert_array_equal(gb.f32, want)
            np.testing.assert_array_equal(orc.reduce_to_shape(g, small).f32, want)


def test_broadcast_shape_edges(orc):
    """Right alignment, missing dims, size 0 and the rank limit of 8."""
    assert orc.broadcast_shape((), ()) == ()
    assert orc.broadcast_shape((), (2, 3)) == (2, 3)
    assert orc.broadcast_shape((3, 1), (1, 4)) == (3, 4)
    assert orc.broadcast_shape((5, 1, 4), (3, 1)) == (5, 3, 4)
    assert orc.broadcast_shape((0,), (1,)) == (0,)
    assert orc.broadcast_shape((2, 0), (2, 1)) == (2, 0)
    with pytest.raises(orc.OracleError):
        orc.broadcast_shape((0,), (2,))
    with pytest.raises(orc.OracleError):
        orc.broadcast_shape((3,), (4,))
    with pytest.raises(orc.OracleError) as e:
        orc.broadcast_shape((1,) * 9, (1,))
    assert e.value.code == orc.ERR_RANK
    with pytest.raises(orc.OracleError) as e:
        orc.broadcast_shape((-1,), (1,))
    assert e.value.code == orc.ERR_SIZE


# ------------------------------------------------------------------ P5 ----
def test_strided_reads_worked_examples(orc):
    """Tensor chapter, "shape and strides" / "zero-copy view"."""
    lines = _golden("strides_examples.txt")
    storage = np.array(ast.literal_eval(lines[0].split("=")[1]), np.float32)
    for ln in lines[1:]:
        if ln.startswith("view"):
            m = re.match(r"view sizes=(\[.*\]) strides=(\[.*\]) at=(\(.*\)) "
                         r"offset=(\d+) value=(\S+)", ln)
            sizes = ast.literal_eval(m.group(1))
            strides = ast.literal_eval(m.group(2))
            at = ast.literal_eval(m.group(3))
            assert sum(i * s for i, s in zip(at, strides)) == int(m.group(4))
            v = orc.View(storage, sizes, strides)
            out = orc.fwd("add", v, np.zeros(sizes, np.float32))
            assert out[at] == float(m.group(5))
            # the whole view agrees with an independent strided read
            ref = np.lib.stride_tricks.as_strided(
                storage, shape=sizes, strides=[4 * s for s in strides])
            np.testing.assert_array_equal(out, ref)
        elif ln.startswith("init_strides"):
            m = re.match(r"init_strides (\[.*\]) = (\[.*\])", ln)
            shape = ast.literal_eval(m.group(1))
            want = ast.literal_eval(m.group(2))
            arr = np.arange(np.prod(shape), dtype=np.float32)
            # explicit row-major strides read the storage in flat order
            out = orc.fwd("add", orc.View(arr, shape, want),
                          np.zeros(shape, np.float32))
            np.testing.assert_array_equal(out.reshape(-1), arr)
            assert [s // 4 for s in arr.reshape(shape).strides] == want


def test_transposed_operand_is_not_swapped(orc):
    """A transposed view of a non-square matrix must read (i,j) at i*1+j*R."""
    rng = np.random.default_rng(7)
    s = rng.standard_normal(6, dtype=np.float32)  # 2x3 storage
    t = orc.View(s, (3, 2), (1, 3))
    b = rng.standard_normal((2,), dtype=np.float32)
    out = orc.fwd("sub", t, b)
    want = s.reshape(2, 3).T - b
    np.testing.assert_array_equal(out, want)


# ------------------------------------------------------------------ P6 ----
def test_ieee_identities(orc):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((4, 5), dtype=np.float32) * np.float32(1e3)
    x[0, 0] = np.float32(1e-40)  # subnormal survives
    np.testing.assert_array_equal(orc.fwd("add", x, np.zeros(1, np.float32)), x)
    np.testing.assert_array_equal(orc.fwd("mul", x, np.ones(1, np.float32)), x)
    np.testing.assert_array_equal(orc.fwd("div", x, np.ones((4, 1), np.float32)), x)
    np.testing.assert_array_equal(orc.fwd("mul", x, np.full(5, 8.0, np.float32)),
                                  x * np.float32(8))
    np.testing.assert_array_equal(orc.fwd("div", x, np.full(5, 0.25, np.float32)),
                                  x * np.float32(4))
    d = orc.fwd("sub", x, x)
    assert np.all(d == 0) and not np.any(np.signbit(d))
    # reduce to the same shape is a bitwise copy; a size-1 dim likewise
    np.testing.assert_array_equal(orc.reduce_to_shape(x, x.shape).f32, x)
    x1 = x.reshape(4, 1, 5)
    np.testing.assert_array_equal(orc.reduce_to_shape(x1, (4, 1, 5)).f32, x1)
    np.testing.assert_array_equal(
        orc.reduce_to_shape(x.reshape(1, 4, 5), (4, 5)).f32, x)


def test_division_is_correctly_rounded(orc):
    one = np.ones(1, np.float32)
    three = np.full(1, 3.0, np.float32)
    q = orc.fwd("div", one, three)
    assert q.view(np.uint32)[0] == 0x3EAAAAAB  # RN(1/3)
    rng = np.random.default_rng(5)
    a = rng.standard_normal(4096, dtype=np.float32)
    b = rng.standard_normal(4096, dtype=np.float32)
    a[:8] = [1e-38, 3e-39, 1.0, 3.4e38, 7.0, -0.0, 1e-45, 2.0]
    b[:8] = [10.0, 3.0, 1e-39, 0.5, 2.0 ** -120, 5.0, 2.0, 3.0]
    got = orc.fwd("div", a, b)
    # exact quotient of two binary32 values, rounded once: float64 division
    # of binary32 inputs followed by RN to binary32 is correctly rounded
    # (53 >= 2*24+2), so it is an independent reference.
    with np.errstate(over="ignore"):
        want = (a.astype(np.float64) / b.astype(np.float64)).astype(np.float32)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


# ------------------------------------------------------------ P7, P8 ------
def test_mass_invariant(orc):
    rng = np.random.default_rng(3)
    g = rng.standard_normal((7, 5, 6), dtype=np.float32)
    x = rng.standard_normal((7, 5, 6), dtype=np.float32)
    for tgt in [(5, 1), (1, 6), (7, 1, 1), (), (5, 6), (7, 5, 1)]:
        r = orc.reduce_to_shape(g, tgt)
        exact = math.fsum(g.astype(np.float64).ravel())
        assert abs(math.fsum(r.f64.ravel()) - exact) <= 2e-6 * np.abs(g).sum()
    # for mul, the small gradient carries sum(g * x)
    y = rng.standard_normal((5, 1), dtype=np.float32)
    _, gy = orc.bwd("mul", g, x, y)
    exact = math.fsum((g.astype(np.float64) * x.astype(np.float64)).ravel())
    assert abs(float(gy.f64.sum()) - exact) <= 2e-6 * float(gy.abs.sum())


def test_reduce_special_cases(orc):
    rng = np.random.default_rng(4)
    G = rng.standard_normal((33, 17), dtype=np.float32)
    G64 = G.astype(np.float64)
    # to [] : the total, i.e. RN32 of the exact sum (within rounding of the
    # binary64 accumulation)
    tot = orc.reduce_to_shape(G, ())
    exact = math.fsum(G64.ravel())
    assert abs(tot.f64 - exact) <= 1e-13 * np.abs(G64).sum()
    # [R,K] -> [K] : column sums, ones^T G
    col = orc.reduce_to_shape(G, (17,))
    np.testing.assert_allclose(col.f64, np.ones(33) @ G64, rtol=0, atol=1e-12)
    # [K,R] -> [K,1] : row sums
    row = orc.reduce_to_shape(G, (33, 1))
    np.testing.assert_allclose(row.f64, G64 @ np.ones((17, 1)), rtol=0, atol=1e-12)
    # summing a reduced axis of a broadcast is the multiplicity
    ones = np.ones((4, 3), np.float32)
    np.testing.assert_array_equal(orc.reduce_to_shape(ones, (3,)).f32, [4, 4, 4])
    # strided input: a transposed view reduced to its columns
    s = rng.standard_normal(12, dtype=np.float32)
    v = orc.View(s, (4, 3), (1, 4))
    want = s.reshape(3, 4).astype(np.float64).sum(axis=1)
    np.testing.assert_allclose(orc.reduce_to_shape(v, (3,)).f64, want, atol=1e-12)
    # empty reduction gives zeros
    e = orc.reduce_to_shape(np.zeros((0, 3), np.float32), (3,))
    np.testing.assert_array_equal(e.f32, [0, 0, 0])


# ------------------------------------------------------------------ P9 ----
def _f64(op, a, b):
    return {"add": a + b, "sub": a - b, "mul": a * b, "div": a / b}[op]


def _gelu64(h):
    return h * 0.5 * np.vectorize(math.erfc)(-h / math.sqrt(2.0))


@pytest.mark.parametrize("op", ["add", "sub", "mul", "div"])
@pytest.mark.parametrize("gelu", [False, True])
@pytest.mark.parametrize("shapes", [((2, 3), (3,)), ((3, 1), (1, 4)),
                                    ((2, 1, 3), (2, 3))])
def test_backward_rules_finite_differences(orc, op, gelu, shapes):
    """Central differences of L = sum(g * f(a, b)) in binary64."""
    sa, sb = shapes
    rng = np.random.default_rng(zlib.crc32(repr((op, gelu, shapes)).encode()))
    a = rng.uniform(0.5, 2.0, sa).astype(np.float32)
    b = rng.uniform(0.5, 2.0, sb).astype(np.float32)
    if op in ("add", "sub", "mul"):
        a *= np.where(rng.random(sa) < 0.5, -1, 1).astype(np.float32)
    out_shape = np.broadcast_shapes(sa, sb)
    g = rng.standard_normal(out_shape).astype(np.float32)
    epi = orc.EPI_GELU if gelu else orc.EPI_NONE
    ga, gb = orc.bwd(op, g, a, b, epi=epi)

    def L(a64, b64):
        f = _f64(op, a64, b64)
        if gelu:
            f = _gelu64(f)
        return math.fsum((g.astype(np.float64) * f).ravel())

    for which, x, gx in ((0, a, ga), (1, b, gb)):
        x64 = x.astype(np.float64)
        for j in np.ndindex(x.shape):
            h = 1e-4 * max(1.0, abs(x64[j]))
            xp, xm = x64.copy(), x64.copy()
            xp[j] += h
            xm[j] -= h
            if which == 0:
                fd = (L(xp, b.astype(np.float64)) - L(xm, b.astype(np.float64))) / (2 * h)
            else:
                fd = (L(a.astype(np.float64), xp) - L(a.astype(np.float64), xm)) / (2 * h)
            # bilinear rules are exact up to rounding; div and GeLU are O(h^2)
            tol = 1e-6 * max(1.0, gx.abs[j]) if (op != "div" and not gelu) \
                else 2e-5 * max(1.0, gx.abs[j])
            assert abs(fd - gx.f64[j]) <= tol, (op, gelu, which, j, fd, gx.f64[j])


def test_backward_sign_and_operand_roles(orc):
    """Asymmetric ops must not swap roles: d(a-b)/db = -1, d(a/b)/da = 1/b."""
    a = np.array([6.0], np.float32)
    b = np.array([2.0], np.float32)
    g = np.array([1.0], np.float32)
    ga, gb = orc.bwd("sub", g, a, b)
    assert ga.f64[0] == 1.0 and gb.f64[0] == -1.0
    ga, gb = orc.bwd("div", g, a, b)
    assert ga.f64[0] == 0.5 and gb.f64[0] == -1.5
    ga, gb = orc.bwd("mul", g, a, b)
    assert ga.f64[0] == 2.0 and gb.f64[0] == 6.0


# ---------------------------------------------------- P10 (oracle side) ---
def _all_shapes(max_rank=3, sizes=(1, 2, 3)):
    for r in range(max_rank + 1):
        for s in itertools.product(sizes, repeat=r):
            yield s


def test_forward_bruteforce_against_numpy(orc):
    """Every shape pair of rank <= 3, sizes in {1,2,3}: numpy's float32
    broadcasting ops (one IEEE op per element) agree bit for bit."""
    rng = np.random.default_rng(9)
    shapes = list(_all_shapes())
    n = 0
    for sa in shapes:
        for sb in shapes:
            try:
                out_shape = np.broadcast_shapes(sa, sb)
            except ValueError:
                with pytest.raises(orc.OracleError):
                    orc.broadcast_shape(sa, sb)
                continue
            a = rng.uniform(0.5, 2, sa).astype(np.float32)
            b = rng.uniform(0.5, 2, sb).astype(np.float32)
            for op, f in (("add", np.add), ("sub", np.subtract),
                          ("mul", np.multiply), ("div", np.divide)):
                got = orc.fwd(op, a, b)
                want = f(a, b)
                assert got.shape == out_shape
                np.testing.assert_array_equal(got.view(np.uint32),
                                              np.asarray(want).view(np.uint32))
            n += 1
    assert n > 300


def test_reduce_bruteforce_against_numpy(orc):
    rng = np.random.default_rng(10)
    for sb in _all_shapes():
        for st in _all_shapes():
            try:
                if np.broadcast_shapes(sb, st) != sb:
                    continue
            except ValueError:
                continue
            x = rng.standard_normal(sb).astype(np.float32)
            # numpy: sum the leading extra dims, then the size-1 target dims
            lead = len(sb) - len(st)
            ref = x.astype(np.float64).sum(axis=tuple(range(lead)))
            axes = tuple(k for k, n in enumerate(st) if n == 1 and ref.shape[k] != 1)
            ref = ref.sum(axis=axes, keepdims=True).reshape(st)
            got = orc.reduce_to_shape(x, st)
            np.testing.assert_allclose(got.f64, ref, rtol=0, atol=1e-12)


# ----------------------------------------------------------------- P12 ----
def test_gelu_pins(orc):
    # closed forms and textbook values of the standard normal CDF
    assert orc.gelu32(0.0) == 0.0
    assert abs(orc.phi_pdf(0.0) - 1 / math.sqrt(2 * math.pi)) < 1e-17
    table = {1.0: 0.8413447460685429, -1.0: 0.15865525393145707,
             1.959963984540054: 0.975, -3.0: 0.0013498980316300946,
             0.5: 0.6914624612740131}
    for h, p in table.items():
        assert abs(orc.phi_cdf(h) - p) <= 1e-15 * max(1, p / 1e-3), h
    # symmetry Phi(h) + Phi(-h) = 1, hence GeLU(h) - GeLU(-h) = h
    for h in np.linspace(-8, 8, 161):
        assert abs(orc.phi_cdf(h) + orc.phi_cdf(-h) - 1) < 1e-15
    # Phi against Simpson integration of the density from -12
    for h in (-6.0, -2.5, -0.7518, 0.0, 0.3, 1.7, 4.0):
        xs = np.linspace(-12.0, h, 20001)
        ys = np.exp(-0.5 * xs * xs) / math.sqrt(2 * math.pi)
        w = np.ones_like(xs)
        w[1:-1:2], w[2:-1:2] = 4, 2
        simp = (xs[1] - xs[0]) / 3 * np.dot(w, ys)
        assert abs(orc.phi_cdf(h) - simp) <= 1e-11 * max(simp, 1e-9), h
    # gelu32 is the correctly rounded value of h*Phi(h) away from ties
    rng = np.random.default_rng(12)
    for h in rng.uniform(-10, 10, 2000).astype(np.float32):
        v = float(h) * orc.phi_cdf(float(h))
        got = float(orc.gelu32(h))
        up = np.nextafter(np.float32(got), np.float32(np.inf))
        dn = np.nextafter(np.float32(got), np.float32(-np.inf))
        assert abs(v - got) <= 0.5 * (float(up) - float(dn)) / 2 + 1e-45
    # limits
    assert orc.gelu32(np.inf) == np.inf
    z = orc.gelu32(-np.inf)
    assert z == 0 and np.signbit(z)
    assert np.isnan(orc.gelu32(np.nan))
    # derivative pieces: Phi(h) + h*phi(h) equals the slope of h*Phi(h)
    for h in (-3.0, -0.7518, 0.0, 0.4, 2.2):
        d = 1e-5
        fd = ((h + d) * orc.phi_cdf(h + d) - (h - d) * orc.phi_cdf(h - d)) / (2 * d)
        assert abs(fd - (orc.phi_cdf(h) + h * orc.phi_pdf(h))) < 1e-9


def _check_gelu_exact(orc, hs, what):
    from gelu_cases import mp_gelu_f32
    for h in hs:
        h = F32(h)
        want = mp_gelu_f32(h)
        for name, fn in (("gelu32", orc.gelu32), ("binary128", orc.gelu32_q)):
            got = fn(h)
            assert got.view(np.uint32) == want.view(np.uint32), \
                (what, name, float(h), float(got), float(want))


def test_gelu_near_ties_correctly_rounded(orc):
    """Every binary32 h in [-10, 10] whose binary64 GeLU lies within 1e-14 of
    a binary32 midpoint (tests/golden/gelu_near_ties.txt, an exhaustive scan):
    the oracle's result equals mpmath's h * Phi(h) correctly rounded."""
    from gelu_cases import near_tie_arguments
    hs = near_tie_arguments()
    assert hs.size > 100 and np.all(np.abs(hs) <= 10)
    _check_gelu_exact(orc, hs, "near tie")


def test_gelu_constructed_hard_cases(orc):
    """Arguments built to sit on or next to binary32 midpoints (see
    gelu_cases.constructed_arguments), and a spread of ordinary ones, each
    against mpmath."""
    from gelu_cases import constructed_arguments
    _check_gelu_exact(orc, constructed_arguments(), "constructed")
    rng = np.random.default_rng(121)
    _check_gelu_exact(orc, rng.uniform(-10, 10, 300).astype(np.float32), "random")


def test_gelu_odd_subnormal_examples(orc):
    """Closed forms at the smallest arguments: GeLU(2^-149) = 2^-149 (the exact
    value 2^-150 + 2^-298 phi(0) lies above the midpoint 2^-150), while
    GeLU(-2^-149) = -0 (the exact value -2^-150 + 2^-298 phi(0) is closer to 0),
    and GeLU(3 * 2^-149) = 2 * 2^-149."""
    t = F32(2.0 ** -149)
    assert orc.gelu32(t) == t
    z = orc.gelu32(-t)
    assert z == 0 and np.signbit(z)
    assert orc.gelu32(F32(3) * t) == F32(2) * t


@pytest.mark.parametrize("op1", ["add", "sub", "mul", "div"])
@pytest.mark.parametrize("op2", ["add", "sub"])
@pytest.mark.parametrize("tie", [None, "a", "b"])
@pytest.mark.parametrize("with_acc", [False, True])
def test_fused_sampled_paths_agree_with_full(orc, op1, op2, tie, with_acc):
    """The fused point-wise entry points (or_fwd2_at, or_bwd2_at, which the
    full-size fused GPU checks use) return, at every position and in a
    shuffled order, the same binary32 value, binary64 sum and sum of |terms|
    as the full fused entry points, which the fused finite-difference and
    worked-example pins fix: for each gradient (a, b, c), each tie and with
    or without acc."""
    rng = np.random.default_rng(zlib.crc32(repr((op1, op2, tie, with_acc)).encode()))
    full = (4, 5, 6)
    if tie == "b":
        sa, sb = (5, 1), full
    else:
        sa, sb = full, (5, 1)
    sc = {None: (1, 6), "a": sa, "b": sb}[tie]
    a = rng.uniform(0.5, 2, sa).astype(np.float32)
    b = rng.uniform(0.5, 2, sb).astype(np.float32)
    c = a if tie == "a" else (b if tie == "b" else rng.standard_normal(sc).astype(np.float32))
    g = rng.standard_normal(full).astype(np.float32)
    out = orc.fwd2(op1, op2, a, b, c)
    pos = rng.permutation(out.size).astype(np.int64)
    got = orc.fwd2_at(op1, op2, a, b, c, pos)
    np.testing.assert_array_equal(got.view(np.uint32), out.reshape(-1)[pos].view(np.uint32))
    shapes = (sa, sb, sc)
    accs = tuple(rng.standard_normal(sh).astype(np.float32) if with_acc else None
                 for sh in shapes)
    grads = orc.bwd2(op1, op2, g, a, b, c, acc=accs, tie=tie)
    for which in range(3):
        if which == 2 and tie is not None:
            assert grads[2] is None
            continue
        ref = grads[which]
        n = int(np.prod(shapes[which]))
        pos = rng.permutation(n).astype(np.int64)
        s = orc.bwd2_at(op1, op2, which, g, a, b, c, pos, acc=accs[which], tie=tie)
        for field in ("f32", "f64", "abs"):
            want = getattr(ref, field).reshape(-1)[pos]
            have = getattr(s, field)
            assert np.array_equal(have.view(np.uint8), want.view(np.uint8)), (which, field)


def test_sampled_paths_agree_with_full(orc):
    """The point-wise entry points compute the same values as the full ones."""
    rng = np.random.default_rng(13)
    a = rng.standard_normal((6, 5, 4), dtype=np.float32)
    b = rng.uniform(0.5, 2, (5, 1)).astype(np.float32)
    g = rng.standard_normal((6, 5, 4), dtype=np.float32)
    full = orc.fwd("div", a, b)
    pos = np.array([0, 7, 33, 119], np.int64)
    np.testing.assert_array_equal(orc.fwd_at("div", a, b, pos), full.reshape(-1)[pos])
    ga, gb = orc.bwd("div", g, a, b)
    pb = np.arange(5, dtype=np.int64)
    s = orc.bwd_at("div", 1, g, a, b, pb)
    np.testing.assert_array_equal(s.f64, gb.f64.reshape(-1))
    s = orc.bwd_at("div", 0, g, a, b, pos)
    np.testing.assert_array_equal(s.f32, ga.f32.reshape(-1)[pos])


# ------------------------------------------ fused (a op1 b) op2 c (f1) -----
def test_fused_chain_rule_worked_example(orc):
    """Autograd chapter, "computation graph": z = x*y + x at x=3, y=2, as one
    fused expression with x used twice (both paths into one gradient)."""
    v = _kv(_golden("chain_rule_example.txt"))
    x, y = _scalar([v["x"]]), _scalar([v["y"]])
    z = orc.fwd2("mul", "add", x, y, x)
    assert float(z[0]) == v["z"]
    g = _scalar([v["dz_dz"]])
    gx, gy, gc = orc.bwd2("mul", "add", g, x, y, x, tie="a")
    assert gc is None
    assert float(gx.f32[0]) == v["dz_dx"] and float(gy.f32[0]) == v["dz_dy"]
    # without the tie the two paths stay apart: 2 through x*y, 1 through + x
    ga, gb, gc = orc.bwd2("mul", "add", g, x, y, x)
    assert float(ga.f32[0]) == 2.0 and float(gc.f32[0]) == 1.0 and float(gb.f32[0]) == 3.0


@pytest.mark.parametrize("op1", ["add", "sub", "mul", "div"])
@pytest.mark.parametrize("op2", ["add", "sub"])
@pytest.mark.parametrize("shapes", [((2, 3), (3,), (2, 3)), ((3, 1), (1, 4), (4,)),
                                    ((2, 1, 3), (2, 3), (1, 2, 1))])
def test_fused_backward_finite_differences(orc, op1, op2, shapes):
    """Central differences of L = sum(g * ((a op1 b) op2 c)) in binary64 pin
    every rule, sign and broadcast sum of the fused backward, c included."""
    sa, sb, sc = shapes
    rng = np.random.default_rng(zlib.crc32(repr((op1, op2, shapes)).encode()))
    a = rng.uniform(0.5, 2.0, sa).astype(np.float32)
    b = rng.uniform(0.5, 2.0, sb).astype(np.float32)
    c = rng.uniform(-2.0, 2.0, sc).astype(np.float32)
    if op1 in ("add", "sub", "mul"):
        a *= np.where(rng.random(sa) < 0.5, -1, 1).astype(np.float32)
    out_shape = np.broadcast_shapes(sa, sb, sc)
    g = rng.standard_normal(out_shape).astype(np.float32)
    grads = orc.bwd2(op1, op2, g, a, b, c)

    def L(a64, b64, c64):
        f = _f64(op2, _f64(op1, a64, b64), c64)
        return math.fsum((g.astype(np.float64) * f).ravel())

    xs = [a.astype(np.float64), b.astype(np.float64), c.astype(np.float64)]
    for which in range(3):
        gx = grads[which]
        for j in np.ndindex(xs[which].shape):
            h = 1e-4 * max(1.0, abs(xs[which][j]))
            xp = [x.copy() for x in xs]
            xm = [x.copy() for x in xs]
            xp[which][j] += h
            xm[which][j] -= h
            fd = (L(*xp) - L(*xm)) / (2 * h)
            tol = (2e-5 if op1 == "div" else 1e-6) * max(1.0, gx.abs[j])
            assert abs(fd - gx.f64[j]) <= tol, (op1, op2, which, j, fd, gx.f64[j])


def test_fused_forward_is_two_roundings(orc):
    """The fused forward rounds after each operator: it equals the unfused
    pair of forwards bit for bit, and differs from a single rounding of the
    exact a*b + c on inputs chosen so that the two disagree."""
    rng = np.random.default_rng(31)
    a = rng.standard_normal((5, 7)).astype(np.float32)
    b = rng.standard_normal((7,)).astype(np.float32)
    c = rng.standard_normal((5, 1)).astype(np.float32)
    for op1 in ("add", "sub", "mul", "div"):
        for op2 in ("add", "sub"):
            want = orc.fwd(op2, orc.fwd(op1, a, b), c)
            got = orc.fwd2(op1, op2, a, b, c)
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # (1 + 2^-23) * (1 - 2^-23) = 1 - 2^-46 rounds to 1; minus 1 gives 0,
    # while a fused multiply-add would give -2^-46.
    x = np.array([1 + 2.0 ** -23], np.float32)
    y = np.array([1 - 2.0 ** -23], np.float32)
    one = np.array([1.0], np.float32)
    assert orc.fwd2("mul", "sub", x, y, one)[0] == 0.0


def test_fused_mass_and_tie_identities(orc):
    """sum(grad_c) = +-sum(g) (Operator chapter, "broadcast": a repeated
    operand's gradient is the sum); a tied gradient is the sum of the two
    untied path gradients (Autograd chapter, "chain rule")."""
    rng = np.random.default_rng(5)
    a = rng.standard_normal((6, 8)).astype(np.float32)
    b = rng.standard_normal((8,)).astype(np.float32)
    c = rng.standard_normal((1, 8)).astype(np.float32)
    g = rng.standard_normal((6, 8)).astype(np.float32)
    exact = math.fsum(g.astype(np.float64).ravel())
    for op2, sgn in (("add", 1.0), ("sub", -1.0)):
        _, _, gc = orc.bwd2("mul", op2, g, a, b, c)
        assert abs(math.fsum(gc.f64.ravel()) - sgn * exact) <= 1e-12 * np.abs(g).sum()
    ga, gb, gc = orc.bwd2("mul", "add", g, a, b, a)
    gt, gbt, none = orc.bwd2("mul", "add", g, a, b, a, tie="a")
    assert none is None
    assert np.allclose(gt.f64, ga.f64 + gc.f64, rtol=0, atol=1e-12)
    assert np.array_equal(gbt.f64, gb.f64)


# ------------------------------------------------ materialise a view (f2) --
def test_materialize_worked_examples(orc):
    """Tensor chapter, "zero-copy view": the transposed view of
    [[1,2,3],[4,5,6]] (sizes [3,2], strides [1,3]) made contiguous is the
    transpose; Operator chapter, "broadcast": [10,20,30] broadcast to [2,3]."""
    storage = np.arange(1, 7, dtype=np.float32)
    tv = orc.View(storage, (3, 2), (1, 3))
    got = orc.materialize(tv)
    assert got.tolist() == [[1, 4], [2, 5], [3, 6]]
    assert orc.materialize(tv)[0, 1] == 4  # element (0,1) of the view is storage[3]
    b = np.array([10, 20, 30], np.float32)
    assert orc.materialize(b, (2, 3)).tolist() == [[10, 20, 30], [10, 20, 30]]


def test_materialize_against_numpy(orc):
    """Random strided views (transposes, stride-0 repeats, offsets) against
    numpy's as_strided + broadcast_to + ascontiguousarray, bit for bit."""
    rng = np.random.default_rng(17)
    for trial in range(60):
        r = int(rng.integers(0, 5))
        sizes = tuple(int(x) for x in rng.integers(1, 5, r))
        strides = tuple(int(x) for x in rng.integers(0, 7, r))
        off = int(rng.integers(0, 4))
        span = off + sum((n - 1) * s for n, s in zip(sizes, strides)) + 1
        st = rng.standard_normal(span).astype(np.float32)
        v = orc.View(st, sizes, strides, off)
        lead = tuple(int(x) for x in rng.integers(1, 3, int(rng.integers(0, 2))))
        shape = lead + tuple(n if rng.random() < 0.7 or n != 1 else int(rng.integers(1, 4))
                             for n in sizes)
        ref = np.lib.stride_tricks.as_strided(st[off:], sizes, tuple(4 * s for s in strides))
        want = np.array(np.broadcast_to(ref, shape), order="C")  # keeps 0-d arrays 0-d
        got = orc.materialize(v, shape)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (sizes, strides, shape)
    with pytest.raises(orc.OracleError):
        orc.materialize(np.ones((2, 3), np.float32), (3, 3))


# ------------------------------------------- ReLU epilogue, scalars (f3) --
def test_relu_pins(orc):
    """ReLU(h) = h for h > 0, NaN for NaN, +0 otherwise (the reading for the
    activation the Module chapter's example MLP uses); numpy.maximum agrees
    away from -0 and NaN."""
    assert orc.relu32(2.5) == np.float32(2.5)
    assert orc.relu32(-3.0) == 0.0
    z = orc.relu32(-0.0)
    assert z == 0.0 and not np.signbit(z)
    assert orc.relu32(np.inf) == np.inf and orc.relu32(-np.inf) == 0.0
    assert np.isnan(orc.relu32(np.nan))
    x = np.random.default_rng(3).standard_normal(1000).astype(np.float32)
    y = orc.fwd("add", x, np.zeros((), np.float32), epi=orc.EPI_RELU)
    assert np.array_equal(y, np.maximum(x, np.float32(0)))


@pytest.mark.parametrize("op", ["add", "sub", "mul", "div"])
def test_relu_backward_finite_differences(orc, op):
    """d/dx of sum(g * ReLU(a op b)) by central differences at points away
    from the kink; at h exactly 0 the rule gives 0 (subgradient, reading)."""
    rng = np.random.default_rng(zlib.crc32(repr(op).encode()))
    a = rng.uniform(0.5, 2.0, (3, 4)).astype(np.float32)
    a *= np.where(rng.random((3, 4)) < 0.5, -1, 1).astype(np.float32)
    b = rng.uniform(0.5, 2.0, (4,)).astype(np.float32)
    g = rng.standard_normal((3, 4)).astype(np.float32)
    ga, gb = orc.bwd(op, g, a, b, epi=orc.EPI_RELU)

    def L(a64, b64):
        return math.fsum((g.astype(np.float64) * np.maximum(_f64(op, a64, b64), 0.0)).ravel())

    for which, x, gx in ((0, a, ga), (1, b, gb)):
        x64 = x.astype(np.float64)
        for j in np.ndindex(x.shape):
            h = 1e-4 * max(1.0, abs(x64[j]))
            xp, xm = x64.copy(), x64.copy()
            xp[j] += h
            xm[j] -= h
            if which == 0:
                fd = (L(xp, b.astype(np.float64)) - L(xm, b.astype(np.float64))) / (2 * h)
            else:
                fd = (L(a.astype(np.float64), xp) - L(a.astype(np.float64), xm)) / (2 * h)
            tol = (2e-5 if op == "div" else 1e-6) * max(1.0, gx.abs[j])
            assert abs(fd - gx.f64[j]) <= tol, (op, which, j, fd, gx.f64[j])
    zero = np.zeros((2,), np.float32)
    gz, _ = orc.bwd("add", np.ones(2, np.float32), zero, zero, epi=orc.EPI_RELU)
    assert np.all(gz.f64 == 0.0)


def test_scalar_operand_is_rank0_broadcast(orc):
    """A scalar operand is the rank-0 case of the broadcast rule (Operator
    chapter, "broadcast"): t op s reads s at every position; s op t too."""
    t = np.array([[1.0, -2.0, 3.0], [4.0, 0.5, -6.0]], np.float32)
    s = np.array(2.0, np.float32)
    assert orc.fwd("sub", t, s).tolist() == [[-1.0, -4.0, 1.0], [2.0, -1.5, -8.0]]
    assert orc.fwd("sub", s, t).tolist() == [[1.0, 4.0, -1.0], [-2.0, 1.5, 8.0]]
    # operand roles of div against numpy's correctly rounded binary32 division
    assert np.array_equal(orc.fwd("div", s, t), np.float32(2.0) / t)
    assert np.array_equal(orc.fwd("div", t, s), t / np.float32(2.0))
    g = np.ones((2, 3), np.float32)
    gt, gs = orc.bwd("div", g, s, t)
    # d(s/t)/dt = -s/t^2
    assert np.allclose(gs.f64, -2.0 / t.astype(np.float64) ** 2, rtol=1e-15, atol=0)
    assert gt.f64 == pytest.approx(float(np.sum(1.0 / t.astype(np.float64))), rel=1e-15)


# ------------------------------------------------------- other reductions
# The mean and the global gradient norm are the reductions the pages list
# beside the sum (GPU chapter, "reduction"); the training loop averages the
# per-token loss over dim 0 and clips the gradients to a global L2 norm of
# 1.0 with g <- g * c / (||g||_2 + 1e-6) (GPT chapter, "training loop").


def test_mean_closed_forms(orc):
    """Mean of a constant is that constant (bitwise); the mean of
    x[i, j] = 10 i + j over i is j + 5 (R - 1), over j it is 10 i + (K - 1)/2."""
    R, K = 7, 6
    v = np.float32(0.3)
    c = np.full((R, K), v, np.float32)
    for shape in ((), (K,), (R, 1), (1, K)):
        got = orc.mean_to_shape(c, shape).f32
        assert np.all(got.view(np.uint32) == np.full(shape, v, np.float32).view(np.uint32))
    x = (10 * np.arange(R)[:, None] + np.arange(K)[None, :]).astype(np.float32)
    assert orc.mean_to_shape(x, (K,)).f32.tolist() == [j + 5.0 * (R - 1) for j in range(K)]
    assert orc.mean_to_shape(x, (R, 1)).f32.ravel().tolist() == [
        10.0 * i + (K - 1) / 2 for i in range(R)]
    # the whole mean of x: 5 (R - 1) + (K - 1) / 2
    assert float(orc.mean_to_shape(x, ()).f32) == 5.0 * (R - 1) + (K - 1) / 2


def test_mean_library_cases_and_edges(orc):
    """Against numpy's binary64 mean; a size-1 (or unreduced) dim is a copy;
    an empty reduced dim gives NaN (0 / 0); the divisor is the count of the
    reduced dims only."""
    rng = np.random.default_rng(31)
    x = rng.standard_normal((5, 3, 8)).astype(np.float32)
    x64 = x.astype(np.float64)
    for shape, axes in (((), (0, 1, 2)), ((8,), (0, 1)), ((3, 1), (0, 2)),
                        ((5, 1, 1), (1, 2)), ((1, 3, 8), (0,))):
        want = x64.mean(axis=axes).reshape(shape)
        got = orc.mean_to_shape(x, shape)
        assert np.allclose(got.f64, want, rtol=1e-14, atol=1e-16), shape
        assert np.allclose(got.abs, np.abs(x64).mean(axis=axes).reshape(shape), rtol=1e-14)
        # rounded once from the binary64 mean
        assert np.array_equal(got.f32, got.f64.astype(np.float32))
    assert np.array_equal(orc.mean_to_shape(x, x.shape).f32, x)
    y = x[:, :1, :]
    assert np.array_equal(orc.mean_to_shape(y, (5, 1, 8)).f32, y)
    e = orc.mean_to_shape(np.zeros((0, 4), np.float32), (4,)).f32
    assert e.shape == (4,) and np.all(np.isnan(e))
    assert orc.mean_to_shape(np.zeros((0, 4), np.float32), (0, 1)).f32.shape == (0, 1)
    with pytest.raises(orc.OracleError):
        orc.mean_to_shape(x, (4,))


def test_mean_backward(orc):
    """d/dx_i of sum_j g_j mean(x)_j is g_j / count for the output j that
    x_i is averaged into (finite differences of the linear form); with a
    power-of-two count the division is exact and the gradient's mass equals
    the upstream gradient's."""
    rng = np.random.default_rng(32)
    x = rng.standard_normal((3, 5, 4)).astype(np.float32)
    for shape in ((5, 1), (), (1, 5, 4), (4,)):
        g = rng.standard_normal(shape).astype(np.float32)
        gx = orc.mean_bwd(g, x.shape)
        assert gx.shape == x.shape

        def L(x64):
            m = x64.mean(axis=tuple(k for k in range(3) if _reduced(k, x.shape, shape)),
                         keepdims=True).reshape(shape)
            return math.fsum((g.astype(np.float64) * m).ravel())

        x64 = x.astype(np.float64)
        for j in [(0, 0, 0), (2, 4, 3), (1, 2, 1)]:
            h = 1e-3
            xp, xm = x64.copy(), x64.copy()
            xp[j] += h
            xm[j] -= h
            fd = (L(xp) - L(xm)) / (2 * h)
            assert abs(fd - float(gx[j])) <= 1e-6 * max(1e-3, abs(fd)), (shape, j)
    g = rng.standard_normal((3, 1, 4)).astype(np.float32)
    gx = orc.mean_bwd(g, (3, 8, 4))  # count 8: exact division
    assert np.array_equal(gx * np.float32(8), np.broadcast_to(g, (3, 8, 4)))
    assert math.fsum(gx.astype(np.float64).ravel()) == math.fsum(g.astype(np.float64).ravel())
    with pytest.raises(orc.OracleError):
        orc.mean_bwd(g, (3, 8, 5))


def _reduced(k, shape_in, shape_out):
    ko = k - (len(shape_in) - len(shape_out))
    return ko < 0 or (shape_out[ko] == 1 and shape_in[k] != 1)


def test_grad_norm_pins(orc):
    """Closed form for constants (0.5 repeated 64 times has norm 4 exactly),
    additivity of squared norms over the list, numpy's binary64 norm of the
    concatenation, and empty tensors / lists contributing nothing."""
    assert orc.grad_norm([np.full(64, 0.5, np.float32)]) == 4.0
    assert orc.grad_norm([np.full(9, -3.0, np.float32), np.full(16, 0.0, np.float32)]) == 9.0
    assert orc.grad_norm([]) == 0.0
    assert orc.grad_norm([np.zeros(0, np.float32)]) == 0.0
    rng = np.random.default_rng(33)
    gs = [rng.standard_normal(n).astype(np.float32) * np.float32(s)
          for n, s in ((1000, 0.01), (3, 5.0), (0, 1.0), (4097, 0.1))]
    whole = np.linalg.norm(np.concatenate([g.astype(np.float64) for g in gs]))
    assert orc.grad_norm(gs) == pytest.approx(whole, rel=1e-14)
    parts = math.fsum(orc.grad_norm([g]) ** 2 for g in gs)
    assert orc.grad_norm(gs) ** 2 == pytest.approx(parts, rel=1e-14)
    # scaling by a power of two scales the norm exactly
    assert orc.grad_norm([g * np.float32(4) for g in gs]) == 4 * orc.grad_norm(gs)


def test_clip_grad_norm_pins(orc):
    """Below or at the threshold nothing changes (the pages scale only when
    the norm exceeds c); above it every element is multiplied by the same
    factor, the direction is kept, the new norm is c * n / (n + 1e-6), and
    the 1e-6 sits beside the norm (visible when the norm is small)."""
    rng = np.random.default_rng(34)
    gs = [rng.standard_normal(n).astype(np.float32) * np.float32(0.01) for n in (50, 7)]
    n = orc.grad_norm(gs)
    out, norm, clipped, f = orc.clip_grad_norm(gs, 2 * n)
    assert not clipped and norm == n and f == 1.0
    assert all(np.array_equal(a, b) for a, b in zip(out, gs))
    # norm exactly equal to the threshold: [3, 4] has norm 5
    out, norm, clipped, _ = orc.clip_grad_norm([np.array([3.0, 4.0], np.float32)], 5.0)
    assert norm == 5.0 and not clipped and out[0].tolist() == [3.0, 4.0]
    # small norm: c = 1e-3, ||g|| = 5e-3 -> factor 1e-3 / (5e-3 + 1e-6)
    g = np.array([3e-3, 4e-3], np.float32)
    out, norm, clipped, f = orc.clip_grad_norm([g], 1e-3)
    n64 = math.sqrt(float(g[0]) ** 2 + float(g[1]) ** 2)
    assert clipped and norm == pytest.approx(n64, rel=1e-15)
    want = 1e-3 * n64 / (n64 + 1e-6)
    got = math.sqrt(float(out[0][0]) ** 2 + float(out[0][1]) ** 2)
    assert got == pytest.approx(want, rel=3e-7)
    assert abs(got - 1e-3) > 1e-7  # without the 1e-6 the new norm would be c
    # one factor for every element of every tensor, direction kept
    out, norm, clipped, f = orc.clip_grad_norm(gs, 0.5 * n)
    assert clipped and 0.49 < f < 0.5
    for a, b in zip(out, gs):
        r = a.astype(np.float64) / b.astype(np.float64)
        assert np.all(np.abs(r - float(f)) <= float(f) * 2.0 ** -23)
    assert orc.grad_norm(out) == pytest.approx(0.5 * n * n / (n + 1e-6), rel=1e-6)


# ------------------------------------------------------- row statistics
# Mean, variance and softmax are the reductions the GPU chapter lists beside
# the gradient norm; LayerNorm takes the first two of each row, the
# attention's softmax the row max and the sum of exponentials.


def test_row_moments_pins(orc):
    """Constant rows: mean exact, variance 0; an arithmetic sequence a + d j
    (j < n): mean a + d (n - 1)/2, variance d^2 (n^2 - 1)/12; numpy's
    binary64 mean and var (ddof 0); the variance is shift invariant; a row
    pitch beyond the row is skipped."""
    c = np.full((3, 384), np.float32(0.7), np.float32)
    m, v = orc.row_moments(c)
    assert np.all(m.f32 == np.float32(0.7)) and np.all(v.f64 == 0.0)
    n, a, d = 384, np.float32(-3.0), np.float32(0.5)
    x = (a + d * np.arange(n, dtype=np.float32))[None, :]
    m, v = orc.row_moments(x)
    assert m.f64[0] == float(a) + float(d) * (n - 1) / 2
    assert v.f64[0] == pytest.approx(float(d) ** 2 * (n * n - 1) / 12, rel=1e-14)
    rng = np.random.default_rng(81)
    y = rng.standard_normal((17, 300)).astype(np.float32) * np.float32(3) + np.float32(1)
    m, v = orc.row_moments(y)
    y64 = y.astype(np.float64)
    assert np.allclose(m.f64, y64.mean(axis=1), rtol=1e-14, atol=1e-15)
    assert np.allclose(v.f64, y64.var(axis=1), rtol=1e-13)
    assert np.array_equal(m.f32, m.f64.astype(np.float32))
    assert np.allclose(m.abs, np.abs(y64).mean(axis=1), rtol=1e-14)
    # on a 2^-10 grid, adding 64 is exact in binary32 (|y| < 64)
    yq = (np.round(y * 1024) / 1024).astype(np.float32)
    _, vq = orc.row_moments(yq)
    _, v2 = orc.row_moments(yq + np.float32(64))
    assert np.allclose(v2.f64, vq.f64, rtol=1e-12)
    # pitch: rows of 300 inside a buffer with rows of 320
    buf = np.zeros((17, 320), np.float32)
    buf[:, :300] = y
    mp, vp = orc.row_moments(buf.reshape(-1)[:16 * 320 + 300], cols=300, ld=320)
    assert np.array_equal(mp.f32, m.f32) and np.array_equal(vp.f32, v.f32)
    e, ev = orc.row_moments(np.zeros((2, 0), np.float32))
    assert np.all(np.isnan(e.f32)) and np.all(np.isnan(ev.f32))


def test_row_softmax_stats_pins(orc):
    """The max is exact (numpy's); a constant row sums to its length; x_j =
    -j t is a geometric series (1 - e^(-n t)) / (1 - e^(-t)); log(sum) + max
    equals scipy's binary64 logsumexp; NaN rows give NaN, a row of -inf gives
    NaN (exp of -inf minus -inf), an empty row gives max -inf and sum 0."""
    from scipy.special import logsumexp
    mx, s = orc.row_softmax_stats(np.full((2, 256), np.float32(-1e9), np.float32))
    assert np.all(mx == np.float32(-1e9)) and np.all(s.f64 == 256.0)
    t = 0.25
    x = (-t * np.arange(100)).astype(np.float32)[None, :]  # exact in binary32
    mx, s = orc.row_softmax_stats(x)
    assert mx[0] == 0.0
    assert s.f64[0] == pytest.approx((1 - math.exp(-100 * t)) / (1 - math.exp(-t)), rel=1e-14)
    rng = np.random.default_rng(82)
    y = rng.standard_normal((9, 256)).astype(np.float32) * np.float32(4)
    y[3, 100:] = np.float32(-1e9)  # a causal-mask style row
    mx, s = orc.row_softmax_stats(y)
    assert np.array_equal(mx, y.max(axis=1))
    lse = logsumexp(y.astype(np.float64), axis=1)
    assert np.allclose(np.log(s.f64) + mx.astype(np.float64), lse, rtol=0, atol=1e-13)
    z = y.copy()
    z[1, 7] = np.nan
    z[2, :] = -np.inf
    mz, sz = orc.row_softmax_stats(z)
    assert np.isnan(mz[1]) and np.isnan(sz.f32[1])
    assert mz[2] == -np.inf and np.isnan(sz.f32[2])
    me, se = orc.row_softmax_stats(np.zeros((2, 0), np.float32))
    assert np.all(me == -np.inf) and np.all(se.f32 == 0)
