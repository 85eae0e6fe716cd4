"""GPU parity of the other reductions: the mean back to a shape and its
gradient (GPU chapter, "reduction"; GPT chapter, "training loop": the
per-token loss averaged over dim 0), and the global L2 norm of a list of
gradients with the ClipGradNorm scaling (GPT chapter, "training loop").

Mean: within 2e-6 * sum|x| / count of the oracle (+ the binary32 subnormal
step), NaN exactly where the oracle has NaN.  Mean gradient: bit-exact (one
binary32 division on both sides).  Norm: within 2e-6 of the oracle's norm
relative, and in practice equal after rounding to binary32 (both round a
binary64 sum of exact squares; only the summation order differs).  Clip: each
scaled element within 2e-6 relative of the oracle's; the tests' seeds also
give bit-exact results, since both sides round the same binary64 factor.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from broadcast_autograd_amd import zk  # noqa: E402
from gpu_util import (BWD_TOL, F32_SUBNORMAL_STEP, assert_bitexact, assert_bwd, dev,  # noqa: E402
                      host, strided_pair)


@pytest.fixture(autouse=True)
def _name(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    sys.stdout.flush()
    yield
    torch.cuda.synchronize()


def _check_mean(got, ref, what):
    nan = np.isnan(ref.f32)
    assert np.array_equal(np.isnan(got), nan), what
    if nan.all():
        return
    from oracle import Grad
    keep = ~nan
    assert_bwd(got[keep], Grad(ref.f32[keep], ref.f64[keep], ref.abs[keep]), what)


MEAN_CASES = [
    # (sizes, strides or None, target)
    ((4096, 1024), None, (1024,)),             # column means: red_col
    ((1024, 4096), None, (1024, 1)),           # row means: red_row
    ((16384,), None, ()),                      # per-token loss -> scalar
    ((64, 128, 256), None, (128, 1)),          # outer and inner dims reduced
    ((512, 384), (1, 512), (384,)),            # transposed view: red_tile
    ((3, 5, 7, 2, 9), None, (5, 1, 2, 1)),     # generic rank 5
    ((37, 13), None, (37, 13)),                # nothing reduced: x / 1
    ((6, 1, 4), None, (1, 1, 4)),              # a size-1 dim is not counted
    ((257, 3), (3, 1), (1, 3)),                # ragged rows
]


@pytest.mark.parametrize("case", MEAN_CASES)
def test_mean_to_shape(orc, case):
    sizes, strides, target = case
    rng = np.random.default_rng(sum(sizes) + len(target))
    if strides is None:
        x = rng.standard_normal(sizes).astype(np.float32)
        t = dev(x)
        v = x
    else:
        span = sum((n - 1) * s for n, s in zip(sizes, strides)) + 1
        st = rng.standard_normal(span).astype(np.float32)
        v, t, _ = strided_pair(st, sizes, strides)
    got = host(zk.mean_to_shape(t, target))
    _check_mean(got, orc.mean_to_shape(v, target), f"mean {case}")
    again = host(zk.mean_to_shape(t, target))
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))


def test_mean_edges(orc):
    # an empty reduced dim: 0 / 0 = NaN, like the oracle
    e = torch.zeros((0, 5), device="cuda")
    got = host(zk.mean_to_shape(e, (5,)))
    assert got.shape == (5,) and np.all(np.isnan(got))
    # an empty target: nothing to write
    assert zk.mean_to_shape(torch.zeros((0, 5), device="cuda"), (0, 1)).shape == (0, 1)
    # a constant mean is that constant, bit for bit
    c = torch.full((300, 7), 0.3, device="cuda")
    got = host(zk.mean_to_shape(c, (7,)))
    assert np.array_equal(got, np.full(7, np.float32(0.3)))


MEAN_BWD_CASES = [
    ((), (16384,)),                 # the per-token loss mean
    ((1024,), (4096, 1024)),        # column means
    ((1024, 1), (1024, 4096)),      # row means
    ((128, 1), (64, 128, 256)),
    ((5, 1, 2, 1), (3, 5, 7, 2, 9)),
    ((37, 13), (37, 13)),           # count 1
    ((1, 3), (257, 3)),             # count 257: an inexact division
]


@pytest.mark.parametrize("case", MEAN_BWD_CASES)
def test_mean_bwd(orc, case):
    sout, sin = case
    g = np.random.default_rng(len(sin) + len(sout)).standard_normal(sout).astype(np.float32)
    got = host(zk.mean_bwd(dev(g), sin))
    assert_bitexact(got, orc.mean_bwd(g, sin), f"mean_bwd {case}")


def test_mean_bwd_count_rounds_to_binary32(orc):
    """A count above 2^24 is rounded to binary32 before the division."""
    n = (1 << 24) + 1
    g = np.array(3.0, np.float32)
    got = host(zk.mean_bwd(dev(g), (n,)))
    want = np.float32(3.0) / np.float32(n)
    assert np.all(got == want)
    assert_bitexact(got[:8], orc.mean_bwd(g, (n,))[:8])


# ------------------------------------------------------------- L2 norm

def _tensors(sizes, seed, sigma=0.01, offsets=None):
    """Device tensors of the given sizes (slices of one buffer at element
    offsets when given, to vary alignment) and their host copies."""
    rng = np.random.default_rng(seed)
    hs = [(rng.standard_normal(n).astype(np.float32) * np.float32(sigma)) for n in sizes]
    if offsets is None:
        return [dev(h) for h in hs], hs
    total = sum(sizes) + sum(offsets) + 16
    buf = torch.zeros(total, device="cuda")
    ts, pos = [], 0
    for h, o in zip(hs, offsets):
        pos += o
        t = buf[pos:pos + h.size]
        t.copy_(torch.from_numpy(h))
        ts.append(t)
        pos += h.size
    return ts, hs


def _check_norm(got, want64, what):
    got = float(got)
    assert abs(got - want64) <= BWD_TOL * want64 + F32_SUBNORMAL_STEP, (what, got, want64)
    assert np.float32(got) == np.float32(want64), (what, got, want64)


NORM_SIZES = [
    [1], [3], [8191], [8192], [8193], [100003], [(1 << 20) + 5],
    [384, 384, 147456, 0, 1152, 589824, 1536, 5],
]


@pytest.mark.parametrize("sizes", NORM_SIZES)
def test_grad_norm(orc, sizes):
    ts, hs = _tensors(sizes, len(sizes) + sum(sizes))
    got = zk.grad_norm(ts)
    _check_norm(host(got), orc.grad_norm(hs), f"norm {sizes}")
    again = zk.grad_norm(ts)
    assert host(got).view(np.uint32) == host(again).view(np.uint32)


def test_grad_norm_unaligned_and_many(orc):
    """Bases off 16-byte alignment, and more tensors than one launch's table
    (empty ones among them)."""
    rng = np.random.default_rng(7)
    sizes = [int(s) for s in rng.integers(0, 20000, 150)]
    sizes[3] = sizes[70] = 0
    offsets = [int(o) for o in rng.integers(0, 4, 150)]
    ts, hs = _tensors(sizes, 8, offsets=offsets)
    _check_norm(host(zk.grad_norm(ts)), orc.grad_norm(hs), "150 tensors")


def test_grad_norm_empty_lists():
    assert float(host(zk.grad_norm([]))) == 0.0
    assert float(host(zk.grad_norm([torch.zeros(0, device="cuda")]))) == 0.0


def _check_clip(ts, hs, want, what):
    outs, n64, clipped, f = want
    for t, o in zip(ts, outs):
        got = host(t)
        lim = BWD_TOL * np.abs(o.astype(np.float64)) + F32_SUBNORMAL_STEP
        assert np.all(np.abs(got.astype(np.float64) - o) <= lim), what
        assert_bitexact(got, o, what)


@pytest.mark.parametrize("ratio", [0.25, 0.999, 1.5])
def test_clip_grad_norm(orc, ratio):
    """max_norm = ratio * norm: clipped below 1, untouched above."""
    sizes = [384, 147456, 1152, 0, 589824, 1536, 7]
    ts, hs = _tensors(sizes, 11, offsets=[0, 1, 2, 3, 0, 0, 1])
    n64 = orc.grad_norm(hs)
    c = float(np.float32(ratio * n64))
    want = orc.clip_grad_norm(hs, c)
    before = [t.clone() for t in ts]
    norm = zk.clip_grad_norm(ts, c)
    _check_norm(host(norm), n64, "clip norm")
    assert want[2] == (ratio < 1)
    _check_clip(ts, hs, want, f"clip ratio {ratio}")
    if ratio >= 1:
        for t, b in zip(ts, before):
            assert torch.equal(t.view(torch.int32), b.view(torch.int32))


def test_clip_at_the_threshold_and_small_norm(orc):
    """The norm equal to max_norm is not clipped; with a small norm the 1e-6
    beside it shows."""
    t = dev(np.array([3.0, 4.0], np.float32))
    assert float(host(zk.clip_grad_norm([t], 5.0))) == 5.0
    assert host(t).tolist() == [3.0, 4.0]
    h = np.array([3e-3, 4e-3], np.float32)
    t = dev(h)
    zk.clip_grad_norm([t], 1e-3)
    _check_clip([t], [h], orc.clip_grad_norm([h], float(np.float32(1e-3))), "small norm")


def test_clip_special_values(orc):
    """An infinite gradient gives an infinite norm and the factor 0 (inf * 0 =
    NaN); a NaN gradient gives a NaN norm, which is not above the threshold,
    so nothing is scaled.  Same as the oracle."""
    for bad in (np.inf, np.nan):
        h = np.array([1.0, bad, -2.0, 0.5] * 3, np.float32)
        t = dev(h)
        norm = float(host(zk.clip_grad_norm([t], 1.0)))
        outs, n64, clipped, f = orc.clip_grad_norm([h], 1.0)
        assert (np.isnan(norm) and np.isnan(n64)) or norm == n64
        assert_bitexact(host(t), outs[0], f"clip with {bad}")


def test_clip_gpt_parameter_list(orc):
    """The GPT training configuration's parameter gradients (hidden 384, 6
    blocks, sequence 256), N(0, 0.01): the norm is about 35, so the clip
    scales every element."""
    from broadcast_autograd_amd import workloads as W
    shapes = W.gpt_param_shapes()
    sizes = [int(np.prod(s)) for s in shapes]
    ts, hs = _tensors(sizes, 12)
    want = orc.clip_grad_norm(hs, 1.0)
    assert want[2]
    norm = zk.clip_grad_norm(ts, 1.0)
    _check_norm(host(norm), want[1], "gpt norm")
    _check_clip(ts, hs, want, "gpt clip")


def test_clip_threshold_edges(orc):
    """max_norm = 0 scales by 0 (any nonzero norm exceeds it) and leaves all
    zeros untouched; max_norm = inf never scales; rank-0 and empty tensors in
    the list."""
    h = np.random.default_rng(21).standard_normal(1000).astype(np.float32)
    for c in (0.0, float("inf")):
        t = dev(h)
        s = dev(np.array(2.5, np.float32))
        e = torch.zeros(0, device="cuda")
        norm = float(host(zk.clip_grad_norm([t, s.reshape(1), e], c)))
        outs, n64, clipped, f = orc.clip_grad_norm([h, np.array([2.5], np.float32)], c)
        assert np.float32(norm) == np.float32(n64)
        assert_bitexact(host(t), outs[0], f"clip c={c}")
        assert_bitexact(host(s).reshape(1), outs[1], f"clip scalar c={c}")
        assert clipped == (c == 0.0)
    z = torch.zeros(100, device="cuda")
    assert float(host(zk.clip_grad_norm([z], 0.0))) == 0.0
    assert np.all(host(z) == 0)


def test_mean_rank0_and_size1(orc):
    """Means over nothing (rank 0, all size-1 dims) are copies; the gradient
    through them is the upstream gradient itself."""
    x = np.array(3.25, np.float32)
    assert float(host(zk.mean_to_shape(dev(x), ()))) == 3.25
    y = np.random.default_rng(22).standard_normal((1, 1, 5)).astype(np.float32)
    assert_bitexact(host(zk.mean_to_shape(dev(y), (1, 5))), y.reshape(1, 5))
    g = np.random.default_rng(23).standard_normal((1, 5)).astype(np.float32)
    assert_bitexact(host(zk.mean_bwd(dev(g), (1, 1, 5))), g.reshape(1, 1, 5))
    assert_bitexact(host(zk.mean_bwd(dev(x), ())), x)
