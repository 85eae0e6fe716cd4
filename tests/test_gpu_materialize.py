"""GPU parity of zk_materialize (stride-aware copy of a view into dense
storage, broadcast to a target shape; Operator chapter, "view backward")
against the CPU oracle: bit-exact, on every kernel path."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from broadcast_autograd_amd import zk  # noqa: E402
from gpu_util import assert_bitexact, dev, host, strided_pair  # noqa: E402


@pytest.fixture(autouse=True)
def _name(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    sys.stdout.flush()
    yield
    torch.cuda.synchronize()


CASES = [
    # (sizes, strides, offset, target or None)
    ((256, 512), (1, 256), 0, None),        # transposed -> tile path (aligned)
    ((130, 260), (1, 130), 0, None),        # transposed, columns not 16-byte aligned
    ((61, 128), (1, 64), 0, None),          # transposed, ragged last row group
    ((128, 96), (1, 128), 1, None),         # transposed, misaligned base
    ((64, 3, 256), (1024, 256, 1), 0, None),  # padded rows -> row path, contiguous inner
    ((32, 128), (256, 2), 0, None),         # inner stride 2 -> gather
    ((1024,), (1,), 0, (16, 1024)),         # broadcast a row (OpBroadcastTo)
    ((8, 1), (1, 1), 0, (8, 512)),          # broadcast a column -> inner stride 0
    ((3, 5, 7), (35, 7, 1), 0, (2, 3, 5, 7)),  # inner 7: generic
    ((2, 3, 4, 5, 6), (1, 2, 6, 24, 120), 0, None),  # rank 5 fully permuted: generic
    ((), (), 0, (4, 4)),                    # scalar broadcast
]


@pytest.mark.parametrize("case", CASES)
def test_materialize_paths(orc, case):
    sizes, strides, off, target = case
    span = off + sum((n - 1) * s for n, s in zip(sizes, strides)) + 1
    st = np.random.default_rng(len(sizes) + span).standard_normal(span).astype(np.float32)
    v, t, _ = strided_pair(st, sizes, strides, off)
    shape = tuple(sizes) if target is None else target
    got = host(zk.materialize(t, shape))
    assert_bitexact(got, orc.materialize(v, shape), f"materialize {case}")


def test_materialize_special_values(orc):
    x = np.array([[0.0, -0.0, np.inf], [-np.inf, np.nan, 1e-45]], np.float32)
    t = dev(x).t()
    got = host(zk.materialize(t))
    assert np.array_equal(got.view(np.uint32), np.ascontiguousarray(x.T).view(np.uint32))


def test_materialize_empty_and_errors():
    t = dev(np.zeros((0, 3), np.float32))
    assert tuple(zk.materialize(t).shape) == (0, 3)
    with pytest.raises(zk.ZkError) as e:
        zk.materialize(dev(np.ones((2, 3), np.float32)), (4, 3))
    assert e.value.name == "ZK_ERR_SHAPE"


def test_materialize_large_transpose(orc):
    """The 4096 x 4096 transposed view of the strided workload, sampled."""
    rng = np.random.default_rng(4001)
    n = 4096
    st = rng.uniform(-1, 1, n * n).astype(np.float32)
    s = dev(st)
    t = torch.as_strided(s, (n, n), (1, n))
    got = host(zk.materialize(t))
    pos = np.unique(rng.integers(0, n * n, 20000))
    i, j = pos // n, pos % n
    want = st[i + j * n]
    assert_bitexact(got.reshape(-1)[pos], want, "sampled transpose")
