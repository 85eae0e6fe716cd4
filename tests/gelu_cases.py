"""GeLU reference values and hard arguments shared by the oracle pins and the
host check of the library's double-double GeLU.

GeLU is read as the exact h * Phi(h) rounded once to binary32 (the Zero book
names the activation in its GPU chapter, element-wise section, and its GPT
chapter's FFN, without a formula).  The reference is mpmath at 400 bits.
"""
import os

import numpy as np

F32 = np.float32
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def mp_gelu_f32(h):
    """h * Phi(h) from mpmath at 400 bits, correctly rounded to binary32
    (nearest; no exact tie occurs for a binary32 h != 0, since h * Phi(h) is
    then irrational)."""
    import mpmath
    with mpmath.workprec(400):
        hx = mpmath.mpf(float(h))
        y = hx * mpmath.ncdf(hx)
        c = np.float32(float(y))
        cands = [np.nextafter(c, F32(-np.inf)), c, np.nextafter(c, F32(np.inf))]
        dist = [abs(mpmath.mpf(float(v)) - y) for v in cands]
        k = min(range(3), key=lambda i: dist[i])
        assert sorted(dist)[0] != sorted(dist)[1], ("exact tie", h)
        return cands[k]


def near_tie_arguments():
    """The binary32 h in [-10, 10] whose binary64 GeLU lies within 1e-14 of a
    binary32 midpoint (golden/gelu_near_ties.txt, an exhaustive scan)."""
    with open(os.path.join(GOLDEN, "gelu_near_ties.txt")) as f:
        pats = [int(ln, 16) for ln in f if ln.strip() and not ln.startswith("#")]
    return np.array(pats, dtype=np.uint32).view(np.float32)


def constructed_arguments():
    """Arguments built to sit on or next to binary32 midpoints: odd multiples
    of 2^-149 (h/2 is exactly a midpoint and h * Phi(h) = h/2 + h^2 phi(0) +
    ... lies just above it), normal h whose half is a subnormal midpoint, the
    run near h = 7.45e-8 where GeLU(h) / (h/2) - 1 = 0.8 h crosses half a
    binary32 unit, the crossing near h = 5.2 where h - GeLU(h) = h Phi(-h)
    passes half a unit of h, h near -1 and near +-5 (where evaluation forms
    switch), and the subnormal results near h = -14."""
    import mpmath
    tiny = 2.0 ** -149
    hs = [s * k * tiny for k in (1, 3, 5, 7, 2 ** 23 - 1, 2 ** 23 + 1, 12345) for s in (1, -1)]
    hs += [s * k * tiny for k in (2, 4, 1024) for s in (1, -1)]           # h/2 exact
    m = F32(2.0 ** -126)
    hs += [s * float(np.nextafter(m, F32(1))) for s in (1, -1)]            # (1 + 2^-23) 2^-126
    hs += [s * float(F32(1.5) * m + F32(2.0 ** -149)) for s in (1, -1)]
    base = int(F32(7.45e-8).view(np.uint32))
    hs += list(np.arange(base - 48, base + 48, 3, dtype=np.uint32).view(np.float32))
    lo, hi = 5.0, 5.5                                   # h Phi(-h) = 2^-22
    with mpmath.workprec(80):
        for _ in range(60):
            mid = 0.5 * (lo + hi)
            if mid * mpmath.ncdf(-mid) > mpmath.mpf(2) ** -22:
                lo = mid
            else:
                hi = mid
    c = int(F32(lo).view(np.uint32))
    hs += list(np.arange(c - 32, c + 32, dtype=np.uint32).view(np.float32))
    for v in (1.0, 5.0):
        u = int(F32(v).view(np.uint32))
        around = np.arange(u - 4, u + 4, dtype=np.uint32).view(np.float32)
        hs += [float(x) for x in around] + [-float(x) for x in around]
    hs += list(np.linspace(-14.6, -13.0, 41, dtype=np.float32))
    return np.array(hs, dtype=np.float32)
