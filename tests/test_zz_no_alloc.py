"""zk_binary_bwd_noalloc: the backward with the library's own device scratch
array in place of a caller workspace, for callers that cannot allocate.

Called through the C ABI (ctypes) with caller-allocated outputs, and checked
bit for bit against zk_binary_bwd with a workspace (the same plan and
kernels, so the same bits): two calls in a row per reduction class, the
second on a smaller input, so that the second call reuses the array the
first left full of its partials.  A shape whose partials need more than
ZK_SCRATCH_BYTES is refused before any launch; the outputs stay untouched.
"""
import ctypes
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from broadcast_autograd_amd import zk  # noqa: E402
from gpu_util import assert_bwd, dev, host  # noqa: E402

SCRATCH_BYTES = 16 << 20  # ZK_SCRATCH_BYTES in include/zk.h


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _noalloc(op, epi, g, a, b, ga, gb, acc_a=None, acc_b=None, stream=None):
    da, db = zk.desc_of(a), zk.desc_of(b)
    s = torch.cuda.current_stream() if stream is None else stream
    return zk.lib().zk_binary_bwd_noalloc(
        zk.OPS[op], zk.EPIS[epi], zk._ptr(g), zk._ptr(a), ctypes.byref(da), zk._ptr(b),
        ctypes.byref(db), zk._ptr(ga), zk._ptr(acc_a), zk._ptr(gb), zk._ptr(acc_b),
        ctypes.c_void_p(s.cuda_stream))


# (op, epi, big shape, small shape, smaller big shape, smaller small shape):
# column sums (16 and 4 waves a block), the interleaved long-column sum whose
# 512 partials a column fill the scratch exactly, GeLU column sums, row
# sums, the transposed tile, a one-pass gather and a gather with partials
CASES = [
    ("mul", "none", (4096, 4096), (4096,), (1000, 2048), (2048,)),
    ("mul", "none", (32768, 4096), (4096,), (8192, 4096), (4096,)),
    ("add", "gelu", (4096, 1024), (1024,), (300, 512), (512,)),
    ("mul", "none", (8, 16, 65536), (1, 16, 1), (2, 16, 8192), (1, 16, 1)),
    ("div", "none", (2, 3, 4, 5, 6, 7, 8, 9), (1, 3, 1, 5, 1, 7, 1, 9),
     (2, 3, 2, 5, 2, 7, 2, 9), (1, 3, 1, 5, 1, 7, 1, 9)),
    ("sub", "none", (6000, 8), (6000, 1), (600, 8), (600, 1)),
]


def _operands(rng, sa, sb, transposed=False):
    a = rng.standard_normal(sa).astype(np.float32)
    b = rng.uniform(0.5, 2.0, sb).astype(np.float32)
    g = rng.standard_normal(sa).astype(np.float32)
    return a, b, g


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}-{len(c[2])}d")
def test_noalloc_matches_workspace_call(orc, case):
    op, epi, sa, sb, sa2, sb2 = case
    rng = np.random.default_rng(sum(sa) + len(op))
    for shape_a, shape_b in ((sa, sb), (sa2, sb2)):
        say(f"  {op}/{epi} {shape_a} x {shape_b}")
        a_np, b_np, g_np = _operands(rng, shape_a, shape_b)
        a, b, g = dev(a_np), dev(b_np), dev(g_np)
        assert zk.bwd_workspace_bytes(op, a, b, epi=epi) <= SCRATCH_BYTES
        ga, gb = zk.binary_bwd(op, g, a, b, epi=epi)
        ga2 = torch.full_like(a, float("nan"))
        gb2 = torch.full_like(b, float("nan"))
        assert _noalloc(op, epi, g, a, b, ga2, gb2) == 0
        torch.cuda.synchronize()
        for x, y, name in ((ga, ga2, "grad_a"), (gb, gb2, "grad_b")):
            assert np.array_equal(host(x).view(np.uint32), host(y).view(np.uint32)), name
        e = orc.EPI_GELU if epi == "gelu" else orc.EPI_NONE
        ra, rb = orc.bwd(op, g_np, a_np, b_np, epi=e)
        assert_bwd(host(ga2), ra, "grad_a")
        assert_bwd(host(gb2), rb, "grad_b")


def test_noalloc_transposed_and_acc(orc):
    """The transposed tile reduction, with the reduced gradient accumulated in
    place and the full one's acc being the upstream gradient; again smaller."""
    rng = np.random.default_rng(5)
    for n, m in ((2048, 1024), (256, 512)):
        say(f"  transposed {n} x {m}")
        s = rng.uniform(-1, 1, n * m).astype(np.float32)
        st = dev(s)
        a = torch.as_strided(st, (n, m), (1, n))
        b_np = rng.uniform(-1, 1, m).astype(np.float32)
        g_np = rng.standard_normal((n, m)).astype(np.float32)
        prev = rng.standard_normal(m).astype(np.float32)
        b, g = dev(b_np), dev(g_np)
        ga = torch.empty(n, m, device="cuda")
        gb = dev(prev)
        ga2 = torch.empty(n, m, device="cuda")
        gb2 = dev(prev)
        zk.binary_bwd("mul", g, a, b, grad_a=ga, grad_b=gb, acc_a=g, acc_b=gb)
        assert _noalloc("mul", "none", g, a, b, ga2, gb2, acc_a=g, acc_b=gb2) == 0
        torch.cuda.synchronize()
        assert torch.equal(ga, ga2) and torch.equal(gb, gb2)
        va = orc.View(s, (n, m), (1, n))
        ra, rb = orc.bwd("mul", g_np, va, b_np, acc_a=g_np, acc_b=prev)
        assert_bwd(host(ga2), ra, "grad_a")
        assert_bwd(host(gb2), rb, "grad_b")


def test_noalloc_side_stream():
    """On a side stream of the current device, after the default stream's
    uploads."""
    rng = np.random.default_rng(9)
    a, b, g = (dev(x) for x in _operands(rng, (2048, 2048), (2048,)))
    ga, gb = zk.binary_bwd("mul", g, a, b)
    ga2, gb2 = torch.empty_like(a), torch.empty_like(b)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    assert _noalloc("mul", "none", g, a, b, ga2, gb2, stream=side) == 0
    torch.cuda.synchronize()
    assert torch.equal(ga, ga2) and torch.equal(gb, gb2)


def test_noalloc_refuses_more_than_the_scratch():
    """A transposed operand of 131072 x 4096 leaves 1024 partials a column,
    32 MiB: refused with ZK_ERR_WORKSPACE before anything is launched (the
    outputs keep their fill)."""
    st = torch.empty(4096 * 131072, device="cuda")
    a = torch.as_strided(st, (131072, 4096), (1, 131072))
    b = torch.empty(4096, device="cuda")
    g = torch.empty(131072, 4096, device="cuda")
    assert zk.bwd_workspace_bytes("mul", a, b) > SCRATCH_BYTES
    ga = torch.full((131072, 4096), 7.0, device="cuda")
    gb = torch.full((4096,), 7.0, device="cuda")
    assert _noalloc("mul", "none", g, a, b, ga, gb) == zk.ERR["ZK_ERR_WORKSPACE"]
    torch.cuda.synchronize()
    assert bool((gb == 7.0).all()) and bool((ga[:4] == 7.0).all())
