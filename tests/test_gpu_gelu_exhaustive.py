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

The backward GeLU'(h) = Phi(h) + h phi(h) is swept over every 16th binary32
bit pattern in [-14, 14] (every exponent, 2^19 significands of each; past the
kernels' binary32 range |h| <= 9; the oracle's binary64 derivative costs
about 100 ns an element, too slow for all 2.2e9): with an upstream gradient
of ones, the full-shape gradient is GeLU'(h) itself and the bias gradient
sums it over 65536 rows; both must stay within 2e-6 of the sum of the
magnitudes of their terms {g Phi(h), g h phi(h)}.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from broadcast_autograd_amd import zk  # noqa: E402
from gpu_util import assert_bwd, assert_gelu_exact, dev, host  # noqa: E402

COLS = 1024
CHUNK = 1 << 26  # elements per launch: 65536 rows of 1024
TEN = 0x41200000  # bit pattern of 10.0f
FOURTEEN = 0x41600000  # bit pattern of 14.0f
BWD_STEP = 16  # backward: every 16th bit pattern


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


def _chunks(top, sign_bit, step):
    """(first bit pattern, count, h[rows, COLS]) over patterns 0, step, ...
    up to top with the sign bit set as given; the last chunk is padded with
    zeros."""
    for lo in range(0, top + 1, CHUNK * step):
        hi = min(lo + CHUNK * step, top + 1)
        bits = np.arange(lo, hi, step, dtype=np.uint32) | np.uint32(sign_bit)
        n = bits.size
        pad = (-n) % COLS
        if pad:
            bits = np.concatenate([bits, np.zeros(pad, np.uint32)])
        yield lo, n, bits.view(np.float32).reshape(-1, COLS)


def _sweep_bwd(orc, sign_bit):
    bias_np = np.zeros(COLS, np.float32)
    bias = dev(bias_np)
    worst_a = worst_b = 0.0
    total = 0
    for lo, n, h in _chunks(FOURTEEN, sign_bit, BWD_STEP):
        g_np = np.ones_like(h)
        ga, gb = zk.binary_bwd("add", dev(g_np), dev(h), bias, epi="gelu")
        ra, rb = orc.bwd("add", g_np, h, bias_np, epi=orc.EPI_GELU)
        worst_a = max(worst_a, assert_bwd(host(ga), ra, "grad_act"))
        worst_b = max(worst_b, assert_bwd(host(gb), rb, "grad_bias"))
        total += n
        say(f"  bits {lo:#010x}.. (sign {sign_bit >> 31}): {n} values, largest error "
            f"so far {worst_a:.3f} (full) / {worst_b:.3f} (bias) of the allowance")
    assert total == FOURTEEN // BWD_STEP + 1
    say(f"  largest error {worst_a:.3f} (full) / {worst_b:.3f} (bias) of the allowance")
    return worst_a, worst_b


def test_gelu_grad_nonnegative_binary32_to_fourteen(orc):
    _sweep_bwd(orc, 0)


def test_gelu_grad_nonpositive_binary32_to_minus_fourteen(orc):
    _sweep_bwd(orc, 0x80000000)
