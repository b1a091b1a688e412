"""Pins of the oracle's correctly rounded tier against facts fixed outside it.

The tier (Carbon README, "Roadmap", v0.2: exact, order-independent summation with a
superaccumulator) is read as: every output is the exact real value of its dot product
(+ bias), rounded once to the dtype, ties to even. So the pins are:
  * exact rational sums (Python Fraction) of the products on small random shapes with
    wide exponent ranges, rounded by an independent rational round-to-nearest-even;
  * hand-made witnesses: a value just above a rounding midpoint that a detour through
    float64 would round down, a cancellation that the tiled float64 chain loses, ties,
    subnormal and overflowing results, exact zeros and non-finite inputs;
  * exact invariances: any permutation of the reduction gives the same bits; negating
    one operand negates the result; integer inputs give the exact tier's result.
Each check takes an Oracle handle and raises AssertionError on a mismatch.
"""
from fractions import Fraction

import numpy as np

import synthetic as syn
from tests.pins import stor, vals, wide_f32

DTS = ("f32", "bf16", "f16")
FORMAT = {"f32": (24, -126, 127), "bf16": (8, -126, 127), "f16": (11, -14, 15)}   # p, emin, emax
INF = {"f32": 0x7F800000, "bf16": 0x7F80, "f16": 0x7C00}
SIGN = {"f32": 0x80000000, "bf16": 0x8000, "f16": 0x8000}


def _encode(value, dt):
    """Storage code of a float64 value that dt holds exactly (non-negative)."""
    if dt == "f32":
        return int(np.array([value], dtype=np.float32).view(np.uint32)[0])
    if dt == "f16":
        return int(np.array([value], dtype=np.float16).view(np.uint16)[0])
    return int(np.array([value], dtype=np.float32).view(np.uint32)[0]) >> 16


def round_fraction(fr, dt):
    """Round-to-nearest-even of an exact rational to dt, by rational arithmetic; returns the code."""
    p, emin, emax = FORMAT[dt]
    if fr == 0:
        return 0
    neg = fr < 0
    a = -fr if neg else fr
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e, emin) - (p - 1)                        # exponent of the last kept bit
    scaled = a / Fraction(2) ** q
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    value = Fraction(n) * Fraction(2) ** q
    max_finite = (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    code = INF[dt] if value > max_finite else _encode(float(value), dt)
    return code | (SIGN[dt] if neg else 0)


def _codes(y, dt):
    return y.view(np.uint32).astype(np.int64) if dt == "f32" else y.view(np.uint16).astype(np.int64)


def _operands(op, A, B, m, k, n):
    """(lhs(row), rhs(col)) sequences along the reduction for op, as float64 arrays."""
    if op == "fwd":
        return (lambda i: A[i, :]), (lambda j: B[:, j])
    if op == "dx":
        return (lambda i: A[i, :]), (lambda j: B[j, :])
    return (lambda i: A[:, i]), (lambda j: B[:, j])


def brute_force(O):
    """Every output equals the rational RNE of the exact Fraction sum."""
    for dt in DTS:
        for si, (op, m, k, n) in enumerate((("fwd", 3, 70, 5), ("dx", 4, 6, 40), ("dw", 45, 3, 4), ("fwd", 2, 1, 3))):
            if dt == "f32":
                A = wide_f32(1300 + si, 0, (m, k) if op != "dx" else (m, n), emin=-60, emax=60)
                B = wide_f32(1300 + si, 1, (k, n) if op != "dw" else (m, n), emin=-60, emax=60)
            else:
                lim = (-20, 20) if dt == "bf16" else (-6, 6)
                A = syn.to_storage(vals(wide_f32(1300 + si, 0, (m, k) if op != "dx" else (m, n), *lim), "f32"), dt)
                B = syn.to_storage(vals(wide_f32(1300 + si, 1, (k, n) if op != "dw" else (m, n), *lim), "f32"), dt)
            bias = syn.normal(1300 + si, 2, (n,), sigma=3.0, dt=dt) if op == "fwd" else None
            y = O.gemm_cr(op, dt, A, B, m, k, n, bias=bias)
            Av, Bv = vals(A, dt), vals(B, dt)
            lhs, rhs = _operands(op, Av, Bv, m, k, n)
            rows_out, cols = (k if op == "dw" else m), (k if op == "dx" else n)
            codes = _codes(y, dt)
            for i in range(rows_out):
                for j in range(cols):
                    ex = sum((Fraction(a) * Fraction(b) for a, b in zip(lhs(i), rhs(j))), Fraction(0))
                    if bias is not None:
                        ex += Fraction(vals(bias, dt)[j])
                    assert codes[i, j] == round_fraction(ex, dt), (dt, op, si, i, j)


def _dot_case(O, dt, terms, bias=None):
    """One output: x = terms' a values, w = their b values (a column), optional bias; returns the code."""
    a = np.array([t[0] for t in terms])
    b = np.array([t[1] for t in terms])
    X = stor(a.reshape(1, -1), dt)
    W = stor(b.reshape(-1, 1), dt)
    bb = stor(np.array([bias]), dt) if bias is not None else None
    return int(_codes(O.gemm_cr("fwd", dt, X, W, 1, len(terms), 1, bias=bb), dt)[0, 0])


def witnesses(O):
    """Hand-made cases: just above a midpoint (a float64 detour rounds it to even instead),
    cancellation lost by a float64 chain, ties, subnormals, overflow, zeros, non-finite."""
    # 1 + 2^-8 + 2^-60: exact sum is above the bf16 midpoint between 1 and 1 + 2^-7
    assert _dot_case(O, "bf16", [(1.0, 1.0), (2.0 ** -8, 1.0), (2.0 ** -30, 2.0 ** -30)]) == 0x3F81
    assert _dot_case(O, "bf16", [(1.0, 1.0), (2.0 ** -8, 1.0)]) == 0x3F80          # tie to even
    assert _dot_case(O, "bf16", [(1.0, 1.0), (3 * 2.0 ** -8, 1.0)]) == 0x3F82      # tie to even, upward
    assert _dot_case(O, "bf16", [(1.0, 1.0), (2.0 ** -8, 1.0), (-(2.0 ** -30), 2.0 ** -30)]) == 0x3F80
    # f32: 1 + 2^-24 + 2^-80 rounds up
    assert _dot_case(O, "f32", [(1.0, 1.0), (2.0 ** -24, 1.0), (2.0 ** -40, 2.0 ** -40)]) == 0x3F800001
    # cancellation inside one tile: the float64 chain gives 0, the exact value is 1
    for dt in ("f32", "bf16"):
        terms = [(2.0 ** 100, 1.0), (1.0, 1.0), (-(2.0 ** 100), 1.0)]
        assert _dot_case(O, dt, terms) == _encode(1.0, dt), dt
        assert _dot_case(O, dt, terms[::-1]) == _encode(1.0, dt), dt
        assert _dot_case(O, dt, [(2.0 ** 100, 1.0), (-(2.0 ** 100), 1.0)], bias=2.0 ** -100) == _encode(2.0 ** -100, dt)
    # exact zero is +0; a negative result below half the smallest subnormal is -0
    assert _dot_case(O, "f16", [(1.0, 1.0), (-1.0, 1.0)]) == 0
    assert _dot_case(O, "f16", [(-(2.0 ** -14), 2.0 ** -12)]) == 0x8000
    assert _dot_case(O, "f16", [(2.0 ** -14, 2.0 ** -11)]) == 0x0000                 # exactly half: tie to 0
    assert _dot_case(O, "f16", [(2.0 ** -14, 3 * 2.0 ** -12)]) == 0x0001             # 0.75 ulp: up
    assert _dot_case(O, "f16", [(2.0 ** -14, 2.0 ** -10), (2.0 ** -14, 2.0 ** -11)]) == 0x0002   # 1.5 -> 2
    # just above half the smallest subnormal: rounding to 11 significant bits first would make it a tie
    assert _dot_case(O, "f16", [(2.0 ** -14, 2.0 ** -11), (2.0 ** -14, 2.0 ** -22)]) == 0x0001
    assert _dot_case(O, "f32", [(2.0 ** -100, 2.0 ** -48), (2.0 ** -100, 2.0 ** -50)]) == 0x00000002   # 2.5 -> 2
    # overflow to infinity; the largest finite value stays
    assert _dot_case(O, "f16", [(256.0, 256.0)]) == 0x7C00
    assert _dot_case(O, "f16", [(65504.0, 1.0), (8.0, 1.0)]) == 0x7BFF            # below the midpoint
    assert _dot_case(O, "f16", [(65504.0, 1.0), (16.0, 1.0)]) == 0x7C00           # at the midpoint: to inf
    assert _dot_case(O, "bf16", [(2.0 ** 127, 2.0), (-(2.0 ** 127), 2.0), (2.0 ** 127, 1.0)]) == 0x7F00
    # non-finite inputs
    assert _dot_case(O, "f32", [(np.inf, 1.0), (1.0, 1.0)]) == 0x7F800000
    assert _dot_case(O, "f32", [(np.inf, 1.0), (-np.inf, 1.0)]) & 0x7FC00000 == 0x7FC00000
    assert _dot_case(O, "f32", [(np.inf, 0.0)]) & 0x7FC00000 == 0x7FC00000


def invariances(O):
    """Reduction order does not matter; negating an operand negates the result; integer
    inputs give exactly the exact tier's bits."""
    rng = np.random.default_rng(1350)
    for dt in DTS:
        m, k, n = 5, 200, 7
        A = syn.normal(1350, 0, (m, k), dt=dt)
        B = syn.normal(1350, 1, (k, n), sigma=0.02, dt=dt)
        bias = syn.normal(1350, 2, (n,), dt=dt)
        y = O.gemm_cr("fwd", dt, A, B, m, k, n, bias=bias)
        for _ in range(3):
            perm = rng.permutation(k)
            yp = O.gemm_cr("fwd", dt, np.ascontiguousarray(A[:, perm]), np.ascontiguousarray(B[perm, :]), m, k, n,
                           bias=bias)
            assert np.array_equal(_codes(yp, dt), _codes(y, dt)), dt
        An = syn.to_storage(-vals(A, dt), dt)
        yn = O.gemm_cr("fwd", dt, An, B, m, k, n)
        y0 = O.gemm_cr("fwd", dt, A, B, m, k, n)
        assert np.array_equal(vals(yn, dt), -vals(y0, dt)), dt
        Ai = syn.integers(1351, 0, (m, k), -8, 8, dt)
        Bi = syn.integers(1351, 1, (k, n), -8, 8, dt)
        bi = syn.integers(1351, 2, (n,), -8, 8, dt)
        assert np.array_equal(_codes(O.gemm_cr("fwd", dt, Ai, Bi, m, k, n, bias=bi), dt),
                              _codes(O.fwd(dt, Ai, Bi, bi)[0], dt)), dt


def near_exact_tier(O):
    """On ordinary data the exact tier is within its error bound of the exact value, so the two
    tiers' outputs are at most one unit apart (and mostly equal)."""
    for dt in DTS:
        for op, m, k, n in (("fwd", 20, 300, 30), ("dx", 16, 40, 300), ("dw", 300, 20, 24)):
            A = syn.normal(1360, 0, (m, k) if op != "dx" else (m, n), dt=dt)
            B = syn.normal(1360, 1, (k, n) if op != "dw" else (m, n), sigma=0.5, dt=dt)
            yc = _codes(O.gemm_cr(op, dt, A, B, m, k, n), dt)
            ye = _codes(O.gemm(op, dt, A, B, m, k, n)[0], dt)
            top = SIGN[dt]
            mono = lambda c: np.where(c & top, -(c & (top - 1)), c)
            d = np.abs(mono(yc) - mono(ye))
            assert d.max() <= 1 and (d > 0).mean() < 0.01, (dt, op, int(d.max()), float((d > 0).mean()))


def exact_sum_rounding(O):
    """The rounding step alone, on random exact sums of float64 values against rational RNE."""
    rng = np.random.default_rng(1370)
    for dt in DTS:
        for _ in range(300):
            cnt = int(rng.integers(1, 6))
            v = rng.standard_normal(cnt) * np.exp2(rng.integers(-30, 30, cnt).astype(float))
            if dt == "f16":
                v = v * 2.0 ** -20
            ex = sum((Fraction(float(t)) for t in v), Fraction(0))
            got = int(np.array([O.exact_sum(dt, v)]).view(np.uint32 if dt == "f32" else np.uint16)[0])
            assert got == round_fraction(ex, dt), (dt, v)


ALL = [brute_force, witnesses, invariances, near_exact_tier, exact_sum_rounding]
