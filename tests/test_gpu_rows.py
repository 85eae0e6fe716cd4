"""GPU parity of the per-row statistics (GPU chapter, "reduction": mean,
variance and softmax are reductions; a LayerNorm takes the first two of each
row, the attention's softmax the row max and sum of exponentials) against
the CPU oracle.

Mean: within 2e-6 * sum|x| / cols (+ the binary32 subnormal step).
Variance and sum of exponentials: within 2e-6 of their own value (every term
is non-negative).  Row max: bit-exact.  NaN exactly where the oracle has NaN.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from broadcast_autograd_amd import zk  # noqa: E402
from gpu_util import assert_bitexact, assert_bwd, dev, host  # noqa: E402


@pytest.fixture(autouse=True)
def _name(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    sys.stdout.flush()
    yield
    torch.cuda.synchronize()


def _check(got, ref, what):
    from oracle import Grad
    nan = np.isnan(ref.f32)
    assert np.array_equal(np.isnan(got), nan), what
    k = ~nan
    assert_bwd(got[k], Grad(ref.f32[k], ref.f64[k], ref.abs[k]), what)


def _view(x, pad=0, off=0):
    """Device view of host rows x with a row pitch of cols + pad, starting
    `off` elements into its buffer; returns (tensor, flat host buffer, ld)."""
    rows, cols = x.shape
    ld = cols + pad
    buf = np.zeros(off + max(rows * ld, 1), np.float32)
    for r in range(rows):
        buf[off + r * ld: off + r * ld + cols] = x[r]
    t = torch.from_numpy(buf).to("cuda")
    v = torch.as_strided(t, (rows, cols), (ld, 1), off)
    return v, buf[off:], ld


COLS = [1, 3, 64, 255, 256, 257, 384, 1000, 2048, 4096, 4097, 10000]


@pytest.mark.parametrize("cols", COLS)
@pytest.mark.parametrize("layout", ["dense", "pitched", "unaligned"])
def test_row_stats(orc, cols, layout):
    rows = 37
    rng = np.random.default_rng(cols)
    x = (rng.standard_normal((rows, cols)) * 3 + 1).astype(np.float32)
    if cols >= 8:
        x[5, cols // 2:] = np.float32(-1e9)  # a masked tail
    pad, off = {"dense": (0, 0), "pitched": (12, 0), "unaligned": (1, 1)}[layout]
    t, flat, ld = _view(x, pad, off)
    m, v = zk.row_moments(t)
    rm, rv = orc.row_moments(flat, cols=cols, ld=ld) if rows * ld > 0 else orc.row_moments(x)
    _check(host(m), rm, f"mean cols={cols} {layout}")
    _check(host(v), rv, f"var cols={cols} {layout}")
    mx, s = zk.row_softmax_stats(t)
    rmx, rs = orc.row_softmax_stats(flat, cols=cols, ld=ld)
    assert_bitexact(host(mx), rmx, f"max cols={cols} {layout}")
    _check(host(s), rs, f"sumexp cols={cols} {layout}")
    again = host(zk.row_softmax_stats(t)[1])
    assert np.array_equal(again.view(np.uint32), host(s).view(np.uint32))


@pytest.mark.parametrize("cols", [300, 256, 512, 5000])
def test_row_stats_special_values(orc, cols):
    """NaN, +-inf and huge values in every row kernel: 256 and 512 columns
    take the rows that fill every lane, 300 the guarded ones, 5000 the
    streamed one."""
    x = np.random.default_rng(3).standard_normal((10, cols)).astype(np.float32)
    x[0, 17] = np.nan
    x[1, :] = -np.inf
    x[2, 3] = np.inf
    x[3, :] = np.float32(-1e9)
    x[4, 0] = np.float32(3e38)
    x[5, 7], x[5, 200] = np.inf, np.nan
    x[6, :] = np.nan
    x[7, ::2] = -np.inf
    x[8, :] = -np.inf
    x[8, 100] = np.nan
    t = dev(x)
    mx, s = zk.row_softmax_stats(t)
    rmx, rs = orc.row_softmax_stats(x)
    assert_bitexact(host(mx), rmx, "max")
    got = host(s)
    assert np.array_equal(np.isnan(got), np.isnan(rs.f32))
    k = ~np.isnan(rs.f32)
    assert np.allclose(got[k], rs.f64[k], rtol=2e-6, atol=0)
    m, v = zk.row_moments(t)
    rm, rv = orc.row_moments(x)
    assert np.array_equal(np.isnan(host(m)), np.isnan(rm.f32))


def test_row_stats_edges(orc):
    e = torch.zeros((3, 0), device="cuda")
    m, v = zk.row_moments(e)
    assert np.all(np.isnan(host(m))) and np.all(np.isnan(host(v)))
    mx, s = zk.row_softmax_stats(e)
    assert np.all(host(mx) == -np.inf) and np.all(host(s) == 0)
    z = torch.zeros((0, 5), device="cuda")
    assert zk.row_moments(z)[0].shape == (0,)
    # one row of 1 element
    one = dev(np.array([[2.5]], np.float32))
    m, v = zk.row_moments(one)
    assert float(host(m)[0]) == 2.5 and float(host(v)[0]) == 0.0
    mx, s = zk.row_softmax_stats(one)
    assert float(host(mx)[0]) == 2.5 and float(host(s)[0]) == 1.0


def test_row_stats_gpt_shapes(orc):
    """The GPT configuration's LayerNorm rows ([64*256, 384]) and causal
    attention rows ([64*6*256, 256], masked above the diagonal), sampled
    rows checked against the oracle, all rows for finiteness."""
    from broadcast_autograd_amd import workloads as W
    h = W.gpt_row_stats()
    x, s = h["x"], h["scores"]
    m, v = zk.row_moments(dev(x))
    mx, se = zk.row_softmax_stats(dev(s))
    rows = np.random.default_rng(5).choice(x.shape[0], 64, replace=False)
    rm, rv = orc.row_moments(x[rows])
    _check(host(m)[rows], rm, "gpt mean")
    _check(host(v)[rows], rv, "gpt var")
    rows = np.random.default_rng(6).choice(s.shape[0], 64, replace=False)
    rmx, rs = orc.row_softmax_stats(s[rows])
    assert_bitexact(host(mx)[rows], rmx, "gpt max")
    _check(host(se)[rows], rs, "gpt sumexp")
    assert np.all(np.isfinite(host(se))) and np.all(host(se) >= 1.0)
