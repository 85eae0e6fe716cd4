"""GeLU forward on every binary32 argument in [-10, 10], against the oracle.

GeLU is named by the MLP passages of the "Zero" book (Operator chapter,
"fusion"; GPT chapter, the feed-forward block) without a formula; both sides
compute GeLU(h) = h Phi(h) rounded once to binary32 (the oracle from the C
library's binary64 erfc, the kernels from their own piecewise polynomials
with a binary64 libm fallback near rounding ties).  Here every one of the
2,185,232,386 binary32 values in [-10, 10] (both zeros included) goes through
the MLP layout the benchmark times, act[rows, 1024] + bias[1024] with a zero
bias, and each result must equal the oracle's bit for bit, apart from the
documented near-tie exception (results one unit apart where the exact value
lies within 1e-12 relative of the midpoint between them).
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from broadcast_autograd_amd import zk  # noqa: E402
from gpu_util import assert_gelu_exact, dev, host  # noqa: E402

COLS = 1024
CHUNK = 1 << 26  # elements per launch: 65536 rows of 1024
TEN = 0x41200000  # bit pattern of 10.0f


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _sweep(orc, sign_bit):
    bias_np = np.zeros(COLS, np.float32)
    bias = dev(bias_np)
    total = ties = 0
    for lo in range(0, TEN + 1, CHUNK):
        hi = min(lo + CHUNK, TEN + 1)
        bits = np.arange(lo, hi, dtype=np.uint32) | np.uint32(sign_bit)
        n = bits.size
        pad = (-n) % COLS
        if pad:
            bits = np.concatenate([bits, np.zeros(pad, np.uint32)])
        h = bits.view(np.float32).reshape(-1, COLS)
        got = host(zk.binary_fwd("add", dev(h), bias, epi="gelu"))
        want = orc.fwd("add", h, bias_np, epi=orc.EPI_GELU)
        ties += assert_gelu_exact(got.reshape(-1)[:n], want.reshape(-1)[:n],
                                  h.reshape(-1)[:n])
        total += n
        say(f"  bits {lo:#010x}..{hi - 1:#010x} (sign {sign_bit >> 31}): {n} values, "
            f"near-tie exceptions so far {ties}")
    assert total == TEN + 1
    return ties


def test_gelu_every_nonnegative_binary32_to_ten(orc):
    _sweep(orc, 0)


def test_gelu_every_nonpositive_binary32_to_minus_ten(orc):
    _sweep(orc, 0x80000000)
