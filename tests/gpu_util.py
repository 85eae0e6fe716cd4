"""Helpers for the GPU parity tests: seeded views on both sides and the
comparison rules.

Forward: bit-exact (any NaN matches any NaN), the GeLU epilogue included: both
sides round the exact h * Phi(h) correctly (the oracle through binary128 where
binary64 cannot decide, the kernels through double-double).
Backward: |gpu - oracle| <= 2e-6 * sum|terms| + 2^-149 per element, and
exactly +-0 where that sum is 0.  The 2^-149 term is the spacing of binary32
subnormals: a binary32 result below 2^-126 cannot carry the relative accuracy
2e-6, so there the bound also admits the neighbouring subnormal of the
correctly rounded value.
"""
import numpy as np

BWD_TOL = 2e-6
F32_SUBNORMAL_STEP = 2.0 ** -149


def torch_mod():
    import torch
    return torch


def dev(x):
    torch = torch_mod()
    # np.array keeps 0-d arrays 0-d (ascontiguousarray would make them 1-d)
    return torch.from_numpy(np.array(x, dtype=np.float32, order="C")).to("cuda")


def strided_pair(storage, sizes, strides, offset=0):
    """(oracle View, device tensor) reading the same storage the same way."""
    import oracle
    torch = torch_mod()
    st = dev(storage.reshape(-1))
    t = torch.as_strided(st, tuple(sizes), tuple(strides), offset)
    return oracle.View(storage.reshape(-1), sizes, strides, offset), t, st


def host(t):
    return t.detach().cpu().numpy()


def assert_bitexact(got, want, what=""):
    got = np.asarray(got, dtype=np.float32)
    want = np.asarray(want, dtype=np.float32)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    gb, wb = got.view(np.uint32), want.view(np.uint32)
    nan = np.isnan(got) & np.isnan(want)
    bad = (gb != wb) & ~nan
    if bad.any():
        i = np.flatnonzero(bad.reshape(-1))[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} differ; first at "
                             f"{i}: got {got.reshape(-1)[i]} want {want.reshape(-1)[i]}")


def assert_gelu_exact(got, want, hval=None, what="gelu"):
    """GeLU forward: bit for bit (``hval``, the binary32 arguments, only
    names the first differing ones).  Returns 0, the number of differences
    allowed."""
    got = np.asarray(got, dtype=np.float32).reshape(-1)
    want = np.asarray(want, dtype=np.float32).reshape(-1)
    diff = np.flatnonzero((got.view(np.uint32) != want.view(np.uint32)) &
                          ~(np.isnan(got) & np.isnan(want)))
    if diff.size:
        i = diff[:5]
        h = None if hval is None else np.asarray(hval, np.float32).reshape(-1)[i]
        raise AssertionError(f"{what}: {diff.size} of {got.size} differ; first at {i}: "
                             f"h {h} got {got[i]} want {want[i]}")
    return 0


def assert_bwd(got, ref, what=""):
    """ref is an oracle.Grad."""
    got = np.asarray(got, dtype=np.float32)
    assert got.shape == ref.f32.shape, (what, got.shape, ref.f32.shape)
    g64 = got.astype(np.float64)
    err = np.abs(g64 - ref.f32.astype(np.float64))
    lim = BWD_TOL * ref.abs + F32_SUBNORMAL_STEP
    bad = err > lim
    zero = ref.abs == 0
    bad |= zero & (got != 0)
    if bad.any():
        i = np.flatnonzero(bad.reshape(-1))[:5]
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at {i}: "
            f"got {got.reshape(-1)[i]} want {ref.f32.reshape(-1)[i]} "
            f"abs {ref.abs.reshape(-1)[i]}")
    # largest error as a fraction of 2e-6*sum|terms| over the results in the
    # binary32 normal range (the tolerance margin)
    normal = np.abs(ref.f32) >= np.float32(2.0 ** -126)
    with np.errstate(invalid="ignore", divide="ignore"):
        r = err[normal] / (BWD_TOL * ref.abs[normal])
    r = r[np.isfinite(r)]
    return float(r.max()) if r.size else 0.0
