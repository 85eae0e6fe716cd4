"""GPU parity past 2^31 elements: the 64-bit index paths of the forward,
backward and reduction kernels, on tensors of 2^31 + 4096 elements (8.6 GB
each).  The large operands are constant fills made by torch (plain
plumbing, not this library), so the oracle reads them as stride-0 views of
one value; the small operands are seeded random.  Forward: bit-exact at
sampled positions on both sides of 2^31.  Reductions: their exact sums (every
term is the same binary32 product, exact in binary64)."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from broadcast_autograd_amd import zk  # noqa: E402
from gpu_util import assert_bitexact, dev, host  # noqa: E402

C = 1024
R = ((1 << 31) + 4096) // C      # R * C = 2^31 + 4096
N = R * C


@pytest.fixture(autouse=True)
def _name(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    sys.stdout.flush()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _positions(seed):
    rng = np.random.default_rng(seed)
    edge = [0, 1, C - 1, C, (1 << 31) - 1, 1 << 31, (1 << 31) + 1, N - C, N - 1]
    return np.concatenate([np.array(edge, np.int64), rng.integers(0, N, 4000)])


def _take(t, pos):
    return host(t.reshape(-1)[torch.from_numpy(pos).to("cuda")])


def test_forward_past_2_31(orc):
    b_np = np.random.default_rng(1).standard_normal(C).astype(np.float32)
    a = torch.full((R, C), 1.5, device="cuda")
    info = zk.plan_describe("fwd", "mul", zk.desc_of(a), zk.make_desc((C,)))
    assert info["index64"] and info["kernel"] == "fwd_row", info
    out = zk.binary_fwd("mul", a, dev(b_np))
    va = orc.View(np.array([1.5], np.float32), (R, C), (0, 0))
    pos = _positions(2)
    assert_bitexact(_take(out, pos), orc.fwd_at("mul", va, b_np, pos), "fwd_row 64-bit")
    del out, a
    # a broadcast row plus a column: no operand is dense -> the gather kernel
    s_np = np.random.default_rng(3).standard_normal(C).astype(np.float32)
    col_np = np.random.default_rng(4).standard_normal((R, 1)).astype(np.float32)
    srow = torch.as_strided(dev(s_np), (R, C), (0, 1))
    info = zk.plan_describe("fwd", "add", zk.desc_of(srow), zk.make_desc((R, 1)))
    assert info["index64"] and info["kernel"] == "fwd_generic", info
    out = zk.binary_fwd("add", srow, dev(col_np))
    vs = orc.View(s_np, (R, C), (0, 1))
    assert_bitexact(_take(out, pos), orc.fwd_at("add", vs, col_np, pos), "fwd_generic 64-bit")


def test_shared_row_vector_past_2_31(orc):
    """A dense [rows, 65536] operand against a shared row vector, 2^31 +
    131072 elements: the 64-bit index path of the kernel that applies each
    piece of the vector to two rows."""
    cols = 1 << 16
    rows = ((1 << 31) + 2 * cols) // cols  # even
    v_np = np.random.default_rng(6).standard_normal(cols).astype(np.float32)
    a = torch.full((rows, cols), -2.5, device="cuda")
    info = zk.plan_describe("fwd", "sub", zk.desc_of(a), zk.make_desc((cols,)))
    assert info["index64"] and info["kernel"] == "fwd_row", info
    out = zk.binary_fwd("sub", dev(v_np), a)  # the row vector first
    va = orc.View(np.array([-2.5], np.float32), (rows, cols), (0, 0))
    n = rows * cols
    rng = np.random.default_rng(7)
    pos = np.concatenate([np.array([0, cols - 1, cols, (1 << 31) - 1, 1 << 31, n - 1], np.int64),
                          rng.integers(0, n, 4000)])
    assert_bitexact(_take(out, pos), orc.fwd_at("sub", v_np, va, pos), "bcrows 64-bit")


def test_fused_shared_row_vector_past_2_31(orc):
    """(a * b) + c with a [rows, 65536] constant, b a shared row vector and c a
    scalar per row, 2^31 + 131072 elements: the 64-bit index path of the
    fused kernel that applies each piece of the vector to two rows."""
    cols = 1 << 16
    rows = ((1 << 31) + 2 * cols) // cols  # even
    v_np = np.random.default_rng(8).standard_normal(cols).astype(np.float32)
    c_np = np.random.default_rng(9).standard_normal((rows, 1)).astype(np.float32)
    a = torch.full((rows, cols), 0.75, device="cuda")
    out = zk.binary2_fwd("mul", "add", a, dev(v_np), dev(c_np))
    va = orc.View(np.array([0.75], np.float32), (rows, cols), (0, 0))
    n = rows * cols
    rng = np.random.default_rng(10)
    pos = np.concatenate([np.array([0, cols - 1, cols, (1 << 31) - 1, 1 << 31, n - 1], np.int64),
                          rng.integers(0, n, 4000)])
    assert_bitexact(_take(out, pos), orc.fwd2_at("mul", "add", va, v_np, c_np, pos),
                    "fused bcrows 64-bit")


def test_backward_and_reductions_past_2_31(orc):
    b_np = np.random.default_rng(5).standard_normal(C).astype(np.float32)
    a = torch.full((R, C), 1.5, device="cuda")
    g = torch.full((R, C), 0.5, device="cuda")
    ga, gb = zk.binary_bwd("mul", g, a, dev(b_np))
    # grad_b[j] = sum over R rows of 0.5 * 1.5, exact
    assert np.all(host(gb) == np.float32(0.75 * R))
    pos = _positions(6)
    want = (np.float32(0.5) * b_np)[pos % C]
    assert_bitexact(_take(ga, pos), want, "grad_a 64-bit")
    del ga, a
    # reductions of the full tensor: to a row, to a scalar, and the mean
    assert np.all(host(zk.reduce_to_shape(g, (C,))) == np.float32(0.5 * R))
    assert float(host(zk.reduce_to_shape(g.view(-1), ()))) == 0.5 * N
    assert float(host(zk.mean_to_shape(g.view(-1), ()))) == 0.5


def test_column_sums_beyond_the_grid_limit():
    """[2, 2^30 + 1024] summed to its columns: 2^22 + 4 column groups of 256,
    more than one launch may hold, so red_col walks its blocks with a grid
    stride.  Column j holds (j mod 4096, 1), so a skipped or misplaced block
    shows; the sums and the multiply backward's are exact in binary32."""
    K = (1 << 30) + 1024
    info = zk.plan_describe("reduce", "add", zk.make_desc((2, K)), zk.make_desc((K,)))
    assert info["kernel"] == "red_col" and info["partials"] == 1, info
    col = (torch.arange(K, device="cuda", dtype=torch.int32) % 4096).to(torch.float32)
    x = torch.stack([col, torch.ones_like(col)])
    out = torch.full((K,), float("nan"), device="cuda")
    zk.reduce_to_shape(x, (K,), out=out)
    assert torch.equal(out, col + 1.0)
    del out
    g = torch.full((2, K), 0.5, device="cuda")
    b = torch.full((K,), 2.0, device="cuda")
    ga, gb = zk.binary_bwd("mul", g, x, b)
    assert torch.equal(gb, 0.5 * col + 0.5)     # sum_r g * x[r, j]
    assert bool((ga == 1.0).all())               # g * b
