"""GPU parity of the scalar-operand calls, the stand-alone activations and
the ReLU epilogue against the CPU oracle (a host scalar is the rank-0 case of
the broadcast rule).  Forward bit-exact; backward within 2e-6 * sum|terms|."""
import sys
import zlib

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from broadcast_autograd_amd import zk  # noqa: E402
from gpu_util import assert_bitexact, assert_bwd, assert_gelu_exact, dev, host, strided_pair  # noqa: E402

OPS = ["add", "sub", "mul", "div"]


@pytest.fixture(autouse=True)
def _name(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    sys.stdout.flush()
    yield
    torch.cuda.synchronize()


def _epi(orc, epi):
    return {"none": orc.EPI_NONE, "gelu": orc.EPI_GELU, "relu": orc.EPI_RELU}[epi]


def _check_fwd(orc, got, want, hv, epi):
    if epi == "gelu":
        assert_gelu_exact(got, want, hv)
    else:
        assert_bitexact(got, want, "fwd")


LAYOUTS = [
    ("dense", (64, 256), None, 0),        # row kernel, scalar by value
    ("ragged", (7, 13), None, 0),         # inner dim not a multiple of 4
    ("transposed", (96, 64), (1, 96), 0),  # generic path
    ("offset", (32, 128), (128, 1), 1),   # misaligned base
    ("scalar", (), None, 0),
]


@pytest.mark.parametrize("layout", LAYOUTS, ids=[x[0] for x in LAYOUTS])
@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("epi", ["none", "gelu", "relu"])
@pytest.mark.parametrize("first", [False, True])
def test_scalar_operand(orc, layout, op, epi, first):
    _, sizes, strides, off = layout
    rng = np.random.default_rng(zlib.crc32(repr((layout[0], op, epi, first)).encode()))
    n = int(np.prod(sizes)) if sizes else 1
    if strides is None:
        strides = tuple(int(np.prod(sizes[k + 1:])) for k in range(len(sizes)))
    span = off + sum((m - 1) * s for m, s in zip(sizes, strides)) + 1
    st = rng.uniform(0.5, 2.0, span).astype(np.float32)
    st *= np.where(rng.random(span) < 0.5, -1, 1).astype(np.float32)
    v, t, _ = strided_pair(st, sizes, strides, off)
    s = np.float32(rng.uniform(0.5, 2.0))
    s0 = np.array(s, np.float32)
    args = (s0, v) if first else (v, s0)
    e = _epi(orc, epi)
    want = orc.fwd(op, *args, epi=e)
    got = host(zk.scalar_fwd(op, t, float(s), scalar_first=first, epi=epi))
    _check_fwd(orc, got, want, orc.fwd(op, *args), epi)
    g = rng.standard_normal(want.shape).astype(np.float32)
    acc = rng.standard_normal(want.shape).astype(np.float32)
    gt = host(zk.scalar_bwd(op, dev(g), t, float(s), scalar_first=first, acc_t=dev(acc),
                            epi=epi))
    ref = orc.bwd(op, g, *args, acc_a=None if first else acc, acc_b=acc if first else None,
                  want=(not first, first), epi=e)
    assert_bwd(gt.reshape(want.shape) if want.shape else gt, ref[1] if first else ref[0],
               f"grad_t {op} {epi}")
    assert n == g.size


@pytest.mark.parametrize("f", ["gelu", "relu"])
def test_unary_special_values(orc, f):
    x = np.linspace(-14, 14, 1 << 16, dtype=np.float32)
    x[:12] = [0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45, 1e-38, -1e-38, -0.7518, 6.4, -6.4]
    z = np.zeros((), np.float32)
    e = _epi(orc, f)
    want = orc.fwd("sub", x, z, epi=e)
    got = host(zk.unary_fwd(f, dev(x)))
    _check_fwd(orc, got, want, x, f)
    g = np.random.default_rng(2).standard_normal(x.shape).astype(np.float32)
    gx = host(zk.unary_bwd(f, dev(g), dev(x)))
    ref, _ = orc.bwd("sub", g, x, z, want=(True, False), epi=e)
    assert_bwd(gx, ref, f"unary {f}")


@pytest.mark.parametrize("shapes", [((512, 1024), (1024,)), ((300, 1000), (1000,)),
                                    ((8, 64, 256), (64, 1)), ((2, 3, 4, 5), (3, 1, 5))])
@pytest.mark.parametrize("op", OPS)
def test_relu_epilogue_with_broadcast(orc, shapes, op):
    """bias + ReLU: forward bit-exact; backward of both operands (the
    broadcast one reduced) within tolerance, on the column, row and generic
    reduction paths."""
    sa, sb = shapes
    rng = np.random.default_rng(zlib.crc32(repr((shapes, op)).encode()))
    a = rng.standard_normal(sa).astype(np.float32)
    b = rng.uniform(0.5, 2.0, sb).astype(np.float32)
    want = orc.fwd(op, a, b, epi=orc.EPI_RELU)
    assert_bitexact(host(zk.binary_fwd(op, dev(a), dev(b), epi="relu")), want, "relu fwd")
    g = rng.standard_normal(want.shape).astype(np.float32)
    ga, gb = zk.binary_bwd(op, dev(g), dev(a), dev(b), epi="relu")
    ra, rb = orc.bwd(op, g, a, b, epi=orc.EPI_RELU)
    assert_bwd(host(ga), ra, "grad_a")
    assert_bwd(host(gb), rb, "grad_b")


def test_unary_errors():
    x = dev(np.ones(4, np.float32))
    with pytest.raises(zk.ZkError) as e:
        zk.unary_fwd("none", x)
    assert e.value.name == "ZK_ERR_UNSUPPORTED"
