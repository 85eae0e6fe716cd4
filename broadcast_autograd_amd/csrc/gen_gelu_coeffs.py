"""Writes zk_gelu_coeffs.h: polynomial coefficients of the device GeLU.

    python broadcast_autograd_amd/csrc/gen_gelu_coeffs.py

Forward (binary64, rounded once to binary32).  GeLU(h) = h*Phi(h) with
Phi(h) = erfc(|h|/sqrt2)/2 for h < 0 and 1 - erfc(|h|/sqrt2)/2 otherwise, so
the device needs E(a) = erfc(a/sqrt2) for a = |h| to a small relative error.
E is tabulated as piecewise polynomials in d = a - c (c the interval's
midpoint) of degree TAB_DEG on intervals of a in [0, TAB_AMAX]: the
intervals are uniform in w = a^2 + TAB_K*a (TAB_S per unit of w), so their
width shrinks like 1/a
where E falls off like exp(-a^2/2) (each piece then spans a bounded change
of log E) and is uniform near a = 0 where E is smooth; the interval of a is
floor(w) (w rounded any way: a piece is accurate slightly past its ends).
Each piece is a least-squares fit on a dense grid weighted for relative error
(near-minimax), computed in binary64 from scipy's erfcx times exp (erfc with
full relative accuracy), converted from the Chebyshev to the monomial basis
in d.  Beyond TAB_AMAX (|h| > 6.36) GeLU(h) rounds to h for h > 0, and the
kernel evaluates negative h there with its double-double path.

Backward (binary32, tolerance 2e-6): erfcx(u)*(u + K) as a polynomial in s,
an affine image onto [-1, 1] of t = (u - K)/(u + K), u = |h|/sqrt2 in
[0, UMAX]; the same reciprocal 1/(u + K) gives t and undoes the factor (the
rational substitution of Chebyshev expansions of the scaled complementary
error function, e.g. Schonfelder, Math. Comp. 32 (1978); Shepherd &
Laframboise, Math. Comp. 36 (1981)); exp comes from the hardware exp2 after
a Cody-Waite reduction.  Also a weighted least-squares fit on Chebyshev
nodes.

The script reports each fit's error measured on a dense grid.
"""
import os

import numpy as np
from numpy.polynomial import chebyshev as C
from numpy.polynomial import polynomial as P
from scipy.special import erfcx

K = 3.75
UMAX = 10.6          # beyond, |GeLU(h)| < 2^-150: the result is -0
TAB_DEG = 8
TAB_S = 1                       # pieces per unit of w
TAB_AMAX = 4.5 * np.sqrt(2.0)   # |h| <= 6.364: Phi(-h) > 2^-33
TAB_K = 3.0 * np.sqrt(2.0)      # w = a^2 + TAB_K*a, intervals w in [j, j+1)


def fit_erfcx(deg, n=6000):
    tmin, tmax = -1.0, (UMAX - K) / (UMAX + K)
    th = np.cos(np.pi * (np.arange(n) + 0.5) / n)
    s = th
    t = 0.5 * (tmax - tmin) * s + 0.5 * (tmax + tmin)
    u = K * (1 + t) / (1 - t)
    y = erfcx(u) * (u + K)
    w = 1.0 / y
    c = C.chebfit(s, y, deg, w=w)
    mono = C.cheb2poly(c)
    a = 2.0 / (tmax - tmin)
    b = -(tmax + tmin) / (tmax - tmin)
    return mono, a, b


def fit_table():
    """Pieces of E(a) = erfc(a/sqrt2): rows (c, a_0 .. a_DEG) and the
    dense-grid maximum relative error."""
    wmax = TAB_AMAX ** 2 + TAB_K * TAB_AMAX
    n = int(np.ceil(wmax * TAB_S - 1e-9))
    wb = np.arange(n + 1, dtype=np.float64) / TAB_S
    ab = (-TAB_K + np.sqrt(TAB_K * TAB_K + 4.0 * wb)) / 2.0   # a^2 + K a = w
    rows, worst = [], 0.0
    for i in range(n):
        lo, hi = ab[i], ab[i + 1]
        c, hw = 0.5 * (lo + hi), 0.5 * (hi - lo)
        a = np.linspace(lo, hi, 6001)
        u = a / np.sqrt(2.0)
        e = erfcx(u) * np.exp(-u * u)
        x = (a - c) / hw
        v = C.chebvander(x, TAB_DEG) / e[:, None]
        b, *_ = np.linalg.lstsq(v, np.ones_like(e), rcond=None)
        mono = C.cheb2poly(b)
        coef = np.array([m / hw ** k for k, m in enumerate(mono)])
        p = np.zeros_like(a)
        for ck in coef[::-1]:
            p = p * (a - c) + ck
        worst = max(worst, float(np.max(np.abs(p / e - 1))))
        rows.append([c] + list(coef))
    return np.array(rows), worst


def report_f32(me, a, b):
    """Error of the binary32 evaluation (coefficients and arithmetic)."""
    m32 = me.astype(np.float32)
    uu = np.concatenate([np.linspace(0, UMAX, 200001),
                         np.geomspace(1e-7, UMAX, 20001)]).astype(np.float32)
    rc = np.float32(1) / (uu + np.float32(K))
    s = ((uu - np.float32(K)) * rc) * np.float32(a) + np.float32(b)
    p = np.full_like(s, m32[-1])
    for ck in m32[-2::-1]:
        p = p * s + ck
    e = np.max(np.abs((p * rc).astype(np.float64) / erfcx(uu.astype(np.float64)) - 1))
    print(f"F32: erfcx rel err {e:.2e} (degree {len(me) - 1}, binary32 arithmetic)")
    return e


def arr32(name, v):
    body = ",\n    ".join(repr(float(np.float32(x))) + "f" for x in v)
    return f"static constexpr float {name}[{len(v)}] = {{\n    {body}}};\n"


def main():
    rows, terr = fit_table()
    print(f"forward table: {len(rows)} pieces of degree {TAB_DEG}, erfc rel err {terr:.2e}")
    me, a, b = fit_erfcx(9)
    e32 = report_f32(me, a, b)
    # Rows are padded with zeros to a stride of an odd number of 16-byte
    # units: lanes reading random rows with 128-bit LDS reads then start in
    # all 16 of the LDS's 16-byte bank groups (a stride of 64 bytes would
    # use 4 of them, and its reads would conflict four times as often).
    stride = TAB_DEG + 2 + (TAB_DEG % 2)
    if (stride // 2) % 2 == 0:
        stride += 2
    rows = [list(r) + [0.0] * (stride - len(r)) for r in rows]
    tab = ",\n    ".join(", ".join(float(v).hex() for v in r) for r in rows)
    hdr = ("// zk_gelu_coeffs.h -- generated by gen_gelu_coeffs.py; do not edit.\n"
           "// Forward: erfc(a/sqrt2), a = |h| with a^2 <= kGeluTabAmax2, as piecewise\n"
           "// polynomials sum_k c_k (a - mid)^k; the piece of a is\n"
           "// floor((a^2 + kGeluTabK*a) * kGeluTabS).\n"
           "// Backward: erfcx(u)*(u+K) ~ sum c_k s^k, s = A*t + B, t = (u-K)/(u+K).\n"
           "#pragma once\n\nnamespace zk {\n\n"
           f"// forward table: erfc rel. error {terr:.2e} (dense-grid maximum at fit time)\n"
           f"static constexpr int kGeluTabN = {len(rows)};\n"
           f"static constexpr int kGeluTabW = {TAB_DEG + 2};  // mid, c_0 .. c_{TAB_DEG}\n"
           f"static constexpr int kGeluTabStride = {stride};  // doubles per row (zero padded)\n"
           f"static constexpr double kGeluTabK = {float(TAB_K).hex()};\n"
           f"static constexpr double kGeluTabS = {float(TAB_S).hex()};  // pieces per unit of w\n"
           f"static constexpr double kGeluTabAmax2 = {float(TAB_AMAX * TAB_AMAX).hex()};\n"
           f"static constexpr double kGeluTab[{len(rows) * stride}] = {{\n    {tab}}};\n\n"
           f"static constexpr double kErfcxK = {float(K).hex()};\n"
           f"static constexpr double kErfcxUmax = {float(UMAX).hex()};\n\n"
           f"// F32: erfcx rel. error {e32:.2e} evaluated in binary32\n"
           + arr32("kErfcxF32", me) + arr32("kErfcxABF32", [a, b])
           + "\n}  // namespace zk\n")
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zk_gelu_coeffs.h")
    with open(path, "w") as f:
        f.write(hdr)
    print("wrote", path)


if __name__ == "__main__":
    main()
