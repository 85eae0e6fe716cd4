"""Writes zk_gelu_dd_coeffs.h: the double-double table of the device GeLU's
rounding path (the arguments the binary64 table of zk_gelu_coeffs.h cannot
round with certainty).

    python broadcast_autograd_amd/csrc/gen_gelu_dd_coeffs.py

E(a) = erfc(a/sqrt2) on the same pieces as the binary64 forward table
(uniform in w = a^2 + K a, K = 3 sqrt2, one piece per unit of w, a = |h| up
to 4.5 sqrt2), each as a polynomial sum_k C_k d^k in d = a - c (c the
piece's midpoint, the same binary64 number as in the binary64 table) of
degree DEG, with every C_k a double-double (hi = RN64(C_k), lo =
RN64(C_k - hi)).  The polynomial interpolates E at Chebyshev nodes of the
piece widened by a hair (the device computes the piece index from a rounded
w, so an argument a rounding away from a piece's end may use its
neighbour), all in mpmath at 300 bits; the script then evaluates the rounded
polynomial exactly at dense points of every piece and reports the largest
relative error against E.  It also picks kGeluDDSplit, the lowest degree from
which the device may sum the terms in binary64 (the rest in double-double)
with a rounding error below 2^-60 of E.
"""
import os

import mpmath
import numpy as np

DEG = 16
# the device sums the terms of degree SPLIT and above in binary64: SPLIT is the
# smallest split whose rounding bound stays below 2^-SPLIT_BITS of E
SPLIT_BITS = 60
TAB_S = 1
TAB_AMAX = 4.5 * np.sqrt(2.0)
TAB_K = 3.0 * np.sqrt(2.0)
PREC = 300


def pieces():
    """Binary64 piece ends and midpoints, computed as the binary64 table's
    generator does."""
    wmax = TAB_AMAX ** 2 + TAB_K * TAB_AMAX
    n = int(np.ceil(wmax * TAB_S - 1e-9))
    wb = np.arange(n + 1, dtype=np.float64) / TAB_S
    ab = (-TAB_K + np.sqrt(TAB_K * TAB_K + 4.0 * wb)) / 2.0
    return [(float(ab[i]), float(ab[i + 1]), float(0.5 * (ab[i] + ab[i + 1]))) for i in range(n)]


def E(a):
    return mpmath.erfc(a / mpmath.sqrt(2))


def fit_piece(lo, hi, c):
    """Double-double monomial coefficients in d = a - c, and the measured
    relative error of the rounded polynomial."""
    mp = mpmath.mpf
    width = mp(hi) - mp(lo)
    pad = width * mp("1e-9") + mp("1e-12")
    # nodes symmetric about c so that the Chebyshev variable is d / hw
    hw = max(mp(hi) - mp(c), mp(c) - mp(lo)) + pad
    n = DEG + 1
    nodes = [mpmath.cos(mpmath.pi * (j + mp(0.5)) / n) for j in range(n)]
    vals = [E(mp(c) + hw * t) for t in nodes]
    # Chebyshev coefficients by the discrete cosine sums
    cheb = []
    for k in range(n):
        s = mp(0)
        for j in range(n):
            s += vals[j] * mpmath.cos(mpmath.pi * k * (j + mp(0.5)) / n)
        cheb.append(s * 2 / n)
    cheb[0] /= 2
    # monomial coefficients in t = d / hw (Chebyshev polynomials expanded)
    mono = [mp(0)] * n
    tk_prev, tk = [mp(1)], [mp(0), mp(1)]
    polys = [tk_prev, tk]
    for k in range(2, n):
        nxt = [mp(0)] * (k + 1)
        for i, v in enumerate(polys[k - 1]):
            nxt[i + 1] += 2 * v
        for i, v in enumerate(polys[k - 2]):
            nxt[i] -= v
        polys.append(nxt)
    for k in range(n):
        for i, v in enumerate(polys[k]):
            mono[i] += cheb[k] * v
    coef = [m / hw ** i for i, m in enumerate(mono)]
    dd = []
    for ck in coef:
        h = float(ck)
        dd.append((h, float(ck - mp(h))))
    # exact evaluation of the rounded polynomial against E
    worst = mp(0)
    for a in mpmath.linspace(mp(lo), mp(hi), 97):
        d = a - mp(c)
        p = mp(0)
        for h, lw in reversed(dd):
            p = p * d + (mp(h) + mp(lw))
        worst = max(worst, abs(p / E(a) - 1))
    return dd, worst


def tail_bound(rows, S):
    """Largest rounding error, relative to E, of the binary64 Horner sum of
    the terms of degree S and above: gamma_2n * sum_{k>=S} |C_k| |d|^k / E
    (n = DEG - S fma steps, u = 2^-53), over 33 points of each piece."""
    u = mpmath.mpf(2) ** -53
    n = DEG - S
    gam = 2 * n * u / (1 - 2 * n * u)
    worst = mpmath.mpf(0)
    for (lo, hi, c), r in zip(pieces(), rows):
        C = [abs(mpmath.mpf(r[1 + 2 * k])) for k in range(DEG + 1)]
        for a in mpmath.linspace(mpmath.mpf(lo), mpmath.mpf(hi), 33):
            d = abs(a - mpmath.mpf(c))
            t = sum(C[k] * d ** k for k in range(S, DEG + 1))
            worst = max(worst, gam * t / E(a))
    return worst


def main():
    mpmath.mp.prec = PREC
    rows, worst = [], mpmath.mpf(0)
    for lo, hi, c in pieces():
        dd, w = fit_piece(lo, hi, c)
        worst = max(worst, w)
        rows.append([c] + [x for pair in dd for x in pair])
    print(f"double-double table: {len(rows)} pieces of degree {DEG}, "
          f"largest relative error {float(worst):.2e} (2^{float(mpmath.log(worst, 2)):.1f})")
    split, bound = None, None
    for S in range(1, DEG + 1):
        bound = tail_bound(rows, S)
        if bound <= mpmath.mpf(2) ** -SPLIT_BITS:
            split = S
            break
    print(f"binary64 terms from degree {split}: rounding bound 2^{float(mpmath.log(bound, 2)):.1f} of E")
    width = 1 + 2 * (DEG + 1)
    tab = ",\n    ".join(", ".join(float(v).hex() for v in r) for r in rows)
    hdr = ("// zk_gelu_dd_coeffs.h -- generated by gen_gelu_dd_coeffs.py; do not edit.\n"
           "// erfc(a/sqrt2) on the pieces of zk_gelu_coeffs.h (piece of a: floor((a^2 +\n"
           "// kGeluTabK*a) * kGeluTabS)) as sum_k C_k (a - mid)^k with double-double C_k;\n"
           "// a row holds mid, then (hi, lo) of C_0 .. C_kGeluDDDeg.\n"
           "#pragma once\n\nnamespace zk {\n\n"
           f"// largest relative error {float(worst):.2e} (exact evaluation at fit time)\n"
           f"static constexpr int kGeluDDDeg = {DEG};\n"
           f"static constexpr int kGeluDDWidth = {width};  // doubles per row\n"
           f"static constexpr int kGeluDDN = {len(rows)};\n"
           f"// terms of degree kGeluDDSplit and above are summed in binary64: their\n"
           f"// rounding error is at most 2^{float(mpmath.log(bound, 2)):.1f} of E (gamma_2n times the sum of\n"
           f"// |C_k| |d|^k, n binary64 steps, over 33 points of every piece)\n"
           f"static constexpr int kGeluDDSplit = {split};\n"
           f"static constexpr double kGeluDDTab[{len(rows) * width}] = {{\n    {tab}}};\n\n"
           "}  // namespace zk\n")
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zk_gelu_dd_coeffs.h")
    with open(path, "w") as f:
        f.write(hdr)
    print("wrote", path)


if __name__ == "__main__":
    main()
