"""Exact-rational models of IEEE fp32/fp64 rounding, for pins that must not
trust the floating point they check.

fl32(x) / fl64(x) round a Fraction to the nearest fp32 / fp64 value, ties to
even (normal range only, which every pin stays in).  inv_rms_exact gives the
RMSNorm factor 1 / sqrt(sum x^2 / K + eps) of an fp32 row to ~100 bits, and
fp32_margin how far a value sits from the nearest point where fp32 rounding
changes its result (a midpoint between two fp32 neighbours).
"""
import math
from fractions import Fraction


def _round_to_bits(x: Fraction, mant_bits: int) -> Fraction:
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    x = abs(x)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    if Fraction(2) ** (e + 1) <= x:
        e += 1
    ulp = Fraction(2) ** (e - mant_bits)
    m = x / ulp
    fl = math.floor(m)
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def fl32(x) -> Fraction:
    """Nearest fp32 value (24-bit significand), ties to even."""
    return _round_to_bits(Fraction(x), 23)


def fl64(x) -> Fraction:
    """Nearest fp64 value (53-bit significand), ties to even."""
    return _round_to_bits(Fraction(x), 52)


def rint_half_even(x: Fraction) -> int:
    fl = math.floor(x)
    rem = x - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def inv_rms_exact(x, eps: float, bits: int = 100) -> Fraction:
    """1 / sqrt(sum_k x_k^2 / K + eps) for the fp32 values x, eps taken as
    the fp64 value of its fp32 argument, to `bits` fractional bits (the
    integer square root is exact; the result is within 2^-bits of the true
    value relative to 1)."""
    xs = [Fraction(float(v)) for v in x]
    v = sum(t * t for t in xs) / len(xs) + Fraction(float(eps))
    # inv = sqrt(1 / v): isqrt of floor(4^bits / v), scaled back
    scaled = (Fraction(4) ** bits) / v
    r = math.isqrt(scaled.numerator // scaled.denominator)
    return Fraction(r, 2 ** bits)


def fp32_margin(v: Fraction) -> float:
    """Relative distance from v (> 0) to the nearest fp32 midpoint, the
    points where rounding to fp32 switches between neighbours."""
    r = fl32(v)
    e = r.numerator.bit_length() - r.denominator.bit_length()
    if Fraction(2) ** e > r:
        e -= 1
    ulp = Fraction(2) ** (e - 23)
    lo, hi = r - ulp / 2, r + ulp / 2
    # just above a power of two the lower midpoint is a quarter ulp away
    if r == Fraction(2) ** e:
        lo = r - ulp / 4
    return float(min(abs(v - lo), abs(hi - v)) / v)


def rms_fp64_error_bound(K: int) -> float:
    """Relative bound on the error of any fp64 evaluation of the RMSNorm
    factor of a K-row with nonnegative squares: a sum of K terms in any
    order (K - 1 roundings), the divide, the add of eps, the square root and
    the reciprocal, each a relative error of at most 2^-53."""
    return (K + 8) * 2.0 ** -53


def rms_undecided_rows(X, eps: float):
    """Rows of the fp32 matrix X whose RMSNorm factor, rounded to fp32, may
    depend on the order of the fp64 sum of squares: rows whose (nearly
    exact) factor lies closer to an fp32 rounding switch point than any fp64
    evaluation order can err.  Every other row rounds to one fp32 value
    whatever order a correct fp64 implementation sums in, so its factor --
    and everything cast from it -- must agree bit for bit.  Returns
    [(row, margin, bound)]."""
    import numpy as np
    X = np.asarray(X, np.float32)
    M, K = X.shape
    bound = rms_fp64_error_bound(K) + 2.0 ** -51  # + this reference's own error
    out = []
    sq = X.astype(np.float64) ** 2  # exact: fp32 squares fit fp64
    for m in range(M):
        s = Fraction(math.fsum(sq[m]))  # correctly rounded sum of exact squares
        v = s / K + Fraction(float(eps))
        if v == 0:
            continue  # 1/sqrt(0) is +inf in any order: nothing to round
        scaled = (Fraction(4) ** 100) / v
        inv = Fraction(math.isqrt(scaled.numerator // scaled.denominator), 2 ** 100)
        margin = fp32_margin(inv)
        if margin <= bound:
            out.append((m, margin, bound))
    return out


def check_rms_cast_rows(Q_gpu, X, g, eps, Q_ref, what=""):
    """Compare the int8 codes a GPU RMSNorm cast produced (Q_gpu, M x K) with
    the oracle's (Q_ref) row by row: bit for bit on every row whose factor is
    decided (rms_undecided_rows); an undecided row is reported and must equal
    the oracle's cast of (x * inv') * g for inv' the oracle's factor or one of
    its fp32 neighbours.  X is the norm's fp32 input (the residual sum for
    the add variant).  Returns the undecided rows."""
    import sys
    import numpy as np
    import oracle as O
    und = rms_undecided_rows(X, eps)
    skip = {m for m, _, _ in und}
    rows = [m for m in range(X.shape[0]) if m not in skip]
    np.testing.assert_array_equal(Q_gpu[rows], Q_ref[rows], err_msg=what)
    for m, margin, bound in und:
        print(f"[undecided rmsnorm factor] {what} row {m}: margin {margin:.3g} <= bound {bound:.3g}",
              file=sys.stderr, flush=True)
        _, _, _, _, inv = O.rmsnorm_quant_act(X[m:m + 1], g, eps)
        inv0 = np.float32(inv[0])
        ok = False
        for cand in (inv0, np.nextafter(inv0, np.float32(np.inf)), np.nextafter(inv0, np.float32(0))):
            xh = (X[m] * cand).astype(np.float32)
            if g is not None:
                xh = (xh * g).astype(np.float32)
            Qc, _, _ = O.quant_act(xh[None, :])
            ok = ok or bool(np.array_equal(Q_gpu[m], Qc[0]))
        assert ok, f"{what}: undecided row {m} matches no neighbouring factor"
    return und


def decided_or_skip(Xin, eps, where):
    """A chain compares every later stage bit for bit, which holds only when
    each RMSNorm factor on the way is decided (rms_undecided_rows); a chain
    that meets an undecided factor is reported and skipped."""
    import pytest
    und = rms_undecided_rows(Xin, eps)
    if und:
        m, margin, bound = und[0]
        pytest.skip(f"undecided RMSNorm factor at {where}, row {m}: margin {margin:.3g} <= {bound:.3g}")
