"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each check takes an oracle handle (oracle.Oracle) so the same checks can be run
against deliberately broken builds of the oracle (tests/test_oracle_mutants.py)
to show that each one has teeth. A check raises AssertionError on failure.

What pins what (definitions: Carbon README, alia-carbon 0.2.0, "How It Works";
sgemm-bi 0.1.2 PyPI page, "Use" and "Determinism contracts"):
  integer_exact       index/operand handling of fwd, dx, dw, bias; any order is exact on small integers
  rational_bound      the float64 arithmetic against exact rational sums and the method's error bound
  order_witnesses     ascending chain inside a tile, tiles anchored at 0, compensation only across tiles
  neumaier_textbook   Neumaier's compensation (not Kahan's, not naive) across tiles
  kbn_vs_partials     the compensated combine of the tile partials rounds their exact sum almost correctly
  downcast_*          single round-to-nearest-even from float64, ties to even, overflow, subnormals
  invariants          row/column permutation, negation and power-of-two scaling
  transpose           dx and dw equal fwd on materialised transposes
  closed_form_k1      K = 1 reduces to one float64 add and one rounding
  numpy_fp64          agreement with a library float64 matmul within the error bound
"""
import json
import os
from fractions import Fraction

import numpy as np

import synthetic as syn

DTS = ("f32", "bf16", "f16")


# ---------------------------------------------------------------- helpers ----

def stor(v, dt):
    """Exactly representable float64 values -> storage (raises if not exact)."""
    s = syn.to_storage(np.asarray(v, dtype=np.float64), dt)
    back = syn.from_storage(s, dt)
    assert np.array_equal(back, np.asarray(v, dtype=np.float64)), "value not exact in " + dt
    return s


def vals(a, dt):
    return syn.from_storage(a, dt)


def _nearest_by_fraction(v, cands, dt_bits_even):
    """Pick the candidate (code, value) nearest to v by exact rational distance, ties to even code."""
    fv = Fraction(v)
    best = None
    for code, cv in cands:
        d = abs(Fraction(cv) - fv)
        key = (d, 0 if dt_bits_even(code) else 1)
        if best is None or key < best[0]:
            best = (key, code)
    return best[1]


def brute_round_bf16(v):
    """Nearest bf16 code of a finite float64 v by exact distances over a small neighbourhood."""
    sign = 0x8000 if np.signbit(v) else 0
    a = abs(float(v))
    with np.errstate(over="ignore"):
        f = np.float32(a)  # any nearby f32; the bf16 neighbours of a lie within a few codes of its top half
    base = int(np.array(f, dtype=np.float32).view(np.uint32)) >> 16
    cands = []
    for code in range(max(0, base - 2), min(0x7f80, base + 3) + 1):
        cv = float(np.array([code << 16], dtype=np.uint32).view(np.float32)[0]) if code < 0x7f80 else 2.0 ** 128
        cands.append((code, cv))
    code = _nearest_by_fraction(a, cands, lambda c: c % 2 == 0)
    return code | sign


def brute_round_f32(v):
    a = float(v)
    f = np.float32(a)
    cands = []
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        if np.isfinite(c):
            cands.append((int(np.array(c, dtype=np.float32).view(np.uint32)), float(c)))
    code = _nearest_by_fraction(a, cands, lambda c: c % 2 == 0)
    return np.array([code], dtype=np.uint32).view(np.float32)[0]


def lib_round(v, dt):
    """Library rounding of float64 values that are exact in float32 (or any double for f16)."""
    v = np.asarray(v, dtype=np.float64)
    if dt == "f32":
        return v.astype(np.float32)
    if dt == "f16":
        return v.astype(np.float16).view(np.uint16)  # numpy rounds float64 -> half once
    f = v.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), v), "bf16 library rounding needs f32-exact inputs"
    return syn.to_storage(f.astype(np.float64), "bf16")


def operands(op, m, k, n):
    """Shapes of (A, B) for an op, with (m, k, n) always the forward problem."""
    return {"fwd": ((m, k), (k, n)), "dx": ((m, n), (k, n)), "dw": ((m, k), (m, n))}[op]


def run(O, op, dt, A, B, m, k, n, bias=None, **kw):
    return O.gemm(op, dt, A, B, m, k, n, bias=bias, **kw)


def exact_products_sum(op, Af, Bf):
    """Exact float64 matrix of the op on small-integer operands (int64 arithmetic)."""
    Ai = Af.astype(np.int64)
    Bi = Bf.astype(np.int64)
    if op == "fwd":
        return Ai @ Bi
    if op == "dx":
        return Ai @ Bi.T
    return Ai.T @ Bi


# ---------------------------------------------------------------- pins ----

def integer_exact(O, shapes=((5, 97, 7), (33, 70, 65), (3, 1, 9), (1, 33, 1), (64, 64, 64), (2, 200, 3))):
    for op in ("fwd", "dx", "dw"):
        for dt in DTS:
            for si, (m, k, n) in enumerate(shapes):
                sa, sb = operands(op, m, k, n)
                A = syn.integers(100 + si, 0, sa, -8, 8, dt)
                B = syn.integers(100 + si, 1, sb, -8, 8, dt)
                bias = syn.integers(100 + si, 2, (n,), -8, 8, dt) if op == "fwd" else None
                y, r, _ = run(O, op, dt, A, B, m, k, n, bias=bias, want_r=True)
                ex = exact_products_sum(op, vals(A, dt), vals(B, dt))
                if bias is not None:
                    ex = ex + vals(bias, dt).astype(np.int64)
                assert np.array_equal(r, ex.astype(np.float64)), (op, dt, m, k, n)
                assert np.array_equal(y, lib_round(ex.astype(np.float64), dt)), (op, dt, m, k, n)


def wide_f32(seed, tid, shape, emin=-30, emax=30):
    """float32 values with spread exponents (exact products and sums stay far from over/underflow)."""
    mant = syn.from_storage(syn.normal(seed, tid, shape), "f32")
    ex = syn.from_storage(syn.integers(seed, tid + 50, shape, emin, emax), "f32")
    return (mant * 2.0 ** ex).astype(np.float32)


def rational_bound(O):
    u = 2.0 ** -53
    for si, (m, k, n) in enumerate(((3, 96, 4), (2, 33, 5), (4, 64, 3), (1, 95, 2))):
        X = wide_f32(200 + si, 0, (m, k))
        W = wide_f32(200 + si, 1, (k, n))
        b = wide_f32(200 + si, 2, (n,))
        y, r, S = run(O, "fwd", "f32", X, W, m, k, n, bias=b, want_r=True, want_S=True)
        Xf, Wf, bf = X.astype(np.float64), W.astype(np.float64), b.astype(np.float64)
        for i in range(m):
            for j in range(n):
                ex = sum((Fraction(Xf[i, q]) * Fraction(Wf[q, j]) for q in range(k)), Fraction(0)) + Fraction(bf[j])
                Sx = sum((abs(Fraction(Xf[i, q]) * Fraction(Wf[q, j])) for q in range(k)), Fraction(0)) + abs(Fraction(bf[j]))
                err = abs(Fraction(r[i, j]) - ex)
                # chain error <= 31u S, compensated combine <= 2u|sum| + O(u^2), bias add <= u|r|
                assert err <= Fraction(64 * u) * Sx + Fraction(4 * u) * abs(ex), (si, i, j, float(err), float(Sx))
                assert abs(Fraction(S[i, j]) - Sx) <= Fraction(2.0 ** -40) * Sx


def _witness_operands(op, dt, L, placements):
    """One output whose reduction sequence holds the given (index, x, w) terms, zeros elsewhere.

    The output is element (0, 0) of the op's result; the reduction has length L.
    Returns (A, B, m, k, n)."""
    if op == "fwd":
        m, k, n = 1, L, 1
        a = np.zeros((1, L)); b = np.zeros((L, 1))
        for idx, xv, wv in placements:
            a[0, idx] = xv; b[idx, 0] = wv
    elif op == "dx":
        m, k, n = 1, 1, L
        a = np.zeros((1, L)); b = np.zeros((1, L))
        for idx, xv, wv in placements:
            a[0, idx] = xv; b[0, idx] = wv
    else:
        m, k, n = L, 1, 1
        a = np.zeros((L, 1)); b = np.zeros((L, 1))
        for idx, xv, wv in placements:
            a[idx, 0] = xv; b[idx, 0] = wv
    return stor(a, dt), stor(b, dt), m, k, n


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "witnesses.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _golden_terms(case):
    return [(int(i), float.fromhex(x), float.fromhex(w)) for i, x, w in case["terms"]]


def order_witnesses(O):
    """Hand-derived cases of tests/golden/witnesses.json, each laid along the reduction of fwd, dx and dw."""
    for case in golden()["cases"]:
        if case["name"] == "neumaier_not_kahan":
            continue
        want = float.fromhex(case["r"])
        for op in ("fwd", "dx", "dw"):
            for dt in DTS:
                A, B, m, k, n = _witness_operands(op, dt, case["L"], _golden_terms(case))
                y, r, _ = run(O, op, dt, A, B, m, k, n, want_r=True)
                assert r[0, 0] == want and not np.signbit(r[0, 0]), (case["name"], op, dt, r[0, 0], want)


def neumaier_textbook(O):
    """Tile partials [u, B, u, -B], B/u = 2^54: Neumaier gives 2u where plain and Kahan summation give 0."""
    case = [c for c in golden()["cases"] if c["name"] == "neumaier_not_kahan"][0]
    want = float.fromhex(case["r"])
    for op in ("fwd", "dx", "dw"):
        for dt in DTS:
            A, Bm, m, k, n = _witness_operands(op, dt, case["L"], _golden_terms(case))
            y, r, _ = run(O, op, dt, A, Bm, m, k, n, want_r=True)
            assert r[0, 0] == want, (op, dt, r[0, 0])


def kbn_vs_partials(O):
    """The combine of T tile partials is within u|sum| + tiny of their exact sum.

    The partials come from the oracle itself run on K-slices of one tile each
    (a single tile is exactly the fma chain); cancellation across tiles is heavy,
    so a plain or misplaced float64 sum would miss the bound by far."""
    u = 2.0 ** -53
    m, n, T = 4, 5, 6
    K = 32 * T - 7
    X = wide_f32(300, 0, (m, K), -5, 5)
    W = wide_f32(300, 1, (K, n), -5, 5)
    # alternate tile magnitudes so consecutive partials cancel
    for t in range(T):
        X[:, 32 * t:32 * t + 32] *= np.float32(2.0 ** (40 if t % 2 else 0))
        if t % 4 == 3:
            X[:, 32 * t:32 * t + 32] *= np.float32(-1.0)
    _, r, _ = O.fwd("f32", X, W, want_r=True)
    parts = []
    for t in range(T):
        sl = slice(32 * t, min(32 * t + 32, K))
        _, p, _ = O.fwd("f32", np.ascontiguousarray(X[:, sl]), np.ascontiguousarray(W[sl, :]), want_r=True)
        parts.append(p)
    for i in range(m):
        for j in range(n):
            ex = sum((Fraction(p[i, j]) for p in parts), Fraction(0))
            ab = sum((abs(Fraction(p[i, j])) for p in parts), Fraction(0))
            assert abs(Fraction(r[i, j]) - ex) <= Fraction(u) * abs(ex) + Fraction(4 * T * T * u * u) * ab, (i, j)
    # T = 2: the combine returns exactly RNE64(p0 + p1)
    X2 = np.ascontiguousarray(X[:, :64]); W2 = np.ascontiguousarray(W[:64, :])
    _, r2, _ = O.fwd("f32", X2, W2, want_r=True)
    assert np.array_equal(r2, parts[0] + parts[1])


def downcast_witnesses(O):
    for case in golden()["downcast"]:
        dt = case["dt"]
        A, B, m, k, n = _witness_operands("fwd", dt, case["L"], _golden_terms(case))
        y, r, _ = O.fwd(dt, A, B, want_r=True)
        assert r[0, 0] == float.fromhex(case["r"]) and int(y[0, 0]) == int(case["code"], 16), case["name"]
    # special values of the rounding itself
    bf = O.round_to("bf16", np.array([0.0, -0.0, np.inf, -np.inf, 2.0 ** 128, 3.3895313892515355e38,
                                      3.3961775292304974e38, 2.0 ** -133, 2.0 ** -134, 2.0 ** -134 * 1.5]))
    assert [int(v) for v in bf] == [0x0000, 0x8000, 0x7F80, 0xFF80, 0x7F80, 0x7F7F, 0x7F80, 0x0001, 0x0000, 0x0001]
    assert np.isnan(syn.from_storage(O.round_to("bf16", np.array([np.nan])), "bf16")[0])
    hf = O.round_to("f16", np.array([65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -25, -0.0]))
    assert [int(v) for v in hf] == [0x7BFF, 0x7BFF, 0x7C00, 0x0001, 0x0000, 0x0001, 0x8000]


def _random_doubles(seed, count, emin, emax):
    mant = syn.from_storage(syn.normal(seed, 0, (count,)), "f32") * (1 + syn.uniform(seed, 1, 0, count) * 2.0 ** -20)
    ex = syn.from_storage(syn.integers(seed, 2, (count,), emin, emax), "f32")
    return mant * 2.0 ** ex


def downcast_random_f16(O, count=20000):
    v = _random_doubles(11, count, -30, 17)
    # exact midpoints between neighbouring f16 values (ties), in normal and subnormal range
    codes = syn.integers(12, 0, (2000,), 0, 0x7BFE, "f32").astype(np.int64).astype(np.uint16)
    lo = codes.view(np.float16).astype(np.float64)
    hi = (codes + 1).view(np.float16).astype(np.float64)
    v = np.concatenate([v, (lo + hi) / 2, -(lo + hi) / 2])
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(O.round_to("f16", v), want)


def downcast_random_bf16(O, count=3000):
    v = _random_doubles(13, count, -140, 130)
    codes = syn.integers(14, 0, (500,), 0, 0x7F7E, "f32").astype(np.int64)
    lo = (codes << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    hi = ((codes + 1) << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    v = np.concatenate([v, (lo + hi) / 2, -(lo + hi) / 2])
    got = O.round_to("bf16", v)
    want = np.array([brute_round_bf16(x) for x in v], dtype=np.uint16)
    assert np.array_equal(got, want)


def downcast_random_f32(O, count=3000):
    v = _random_doubles(15, count, -160, 120)
    got = O.round_to("f32", v)
    want = np.array([brute_round_f32(x) for x in v], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def invariants(O):
    m, k, n = 37, 100, 45
    for dt in ("f32", "bf16"):
        X = syn.normal(400, 0, (m, k), dt=dt)
        W = syn.normal(400, 1, (k, n), sigma=0.5, dt=dt)
        b = syn.normal(400, 2, (n,), sigma=0.1, dt=dt)
        y, r, _ = O.fwd(dt, X, W, b, want_r=True)
        assert not np.any(np.signbit(r) & (r == 0))
        pr = np.array([(7 * i + 3) % m for i in range(m)])
        pc = np.array([(11 * j + 5) % n for j in range(n)])
        y2, _, _ = O.fwd(dt, np.ascontiguousarray(X[pr]), W, b)
        assert np.array_equal(y2, y[pr])
        y3, _, _ = O.fwd(dt, X, np.ascontiguousarray(W[:, pc]), np.ascontiguousarray(b[pc]))
        assert np.array_equal(y3, y[:, pc])
        Xn = stor(-vals(X, dt), dt); bn = stor(-vals(b, dt), dt)
        _, rn, _ = O.fwd(dt, Xn, W, bn, want_r=True)
        assert np.array_equal(rn, -r)
        Xs = stor(vals(X, dt) * 2.0 ** 7, dt); bs = stor(vals(b, dt) * 2.0 ** 7, dt)
        ys, rs, _ = O.fwd(dt, Xs, W, bs, want_r=True)
        assert np.array_equal(rs, r * 2.0 ** 7)
        assert np.array_equal(vals(ys, dt), vals(y, dt) * 2.0 ** 7)
        Xz = X.copy(); Xz[5] = 0
        yz, rz, _ = O.fwd(dt, Xz, W, b, want_r=True)
        assert np.array_equal(rz[5], vals(b, dt)) and np.array_equal(yz[5], b)
        # dx is batch-row independent too
        dY = syn.normal(400, 3, (m, n), dt=dt)
        gx, _, _ = O.dx(dt, dY, W)
        gx2, _, _ = O.dx(dt, np.ascontiguousarray(dY[pr]), W)
        assert np.array_equal(gx2, gx[pr])


def transpose(O):
    m, k, n = 19, 70, 41
    for dt in DTS:
        X = syn.normal(500, 0, (m, k), dt=dt)
        W = syn.normal(500, 1, (k, n), dt=dt)
        dY = syn.normal(500, 3, (m, n), dt=dt)
        gx, _, _ = O.dx(dt, dY, W)
        gx_ref, _, _ = O.fwd(dt, dY, np.ascontiguousarray(W.T))
        assert np.array_equal(gx, gx_ref)
        gw, _, _ = O.dw(dt, X, dY)
        gw_ref, _, _ = O.fwd(dt, np.ascontiguousarray(X.T), dY)
        assert np.array_equal(gw, gw_ref)


def closed_form_k1(O):
    m, n = 16, 24
    for dt in DTS:
        X = syn.normal(600, 0, (m, 1), dt=dt)
        W = syn.normal(600, 1, (1, n), dt=dt)
        b = syn.normal(600, 2, (n,), dt=dt)
        y, r, _ = O.fwd(dt, X, W, b, want_r=True)
        ref = vals(X, dt) * vals(W, dt) + vals(b, dt)   # product exact, one float64 add
        assert np.array_equal(r, ref)
        if dt == "bf16":
            want = np.array([[brute_round_bf16(v) for v in row] for row in ref], dtype=np.uint16)
        else:
            want = lib_round(ref, dt)
        assert np.array_equal(y.view(np.uint16 if dt != "f32" else np.uint32),
                              want.view(np.uint16 if dt != "f32" else np.uint32))


def numpy_fp64(O):
    m, k, n = 48, 300, 40
    for dt in DTS:
        X = syn.normal(700, 0, (m, k), dt=dt)
        W = syn.normal(700, 1, (k, n), sigma=0.3, dt=dt)
        b = syn.normal(700, 2, (n,), sigma=0.1, dt=dt)
        dY = syn.normal(700, 3, (m, n), dt=dt)
        Xf, Wf, bf, Gf = (vals(a, dt) for a in (X, W, b, dY))
        _, r, S = O.fwd(dt, X, W, b, want_r=True, want_S=True)
        assert np.all(np.abs(r - (Xf @ Wf + bf)) <= 2.0 ** -40 * S)
        assert np.allclose(S, np.abs(Xf) @ np.abs(Wf) + np.abs(bf), rtol=1e-12)
        _, r, S = O.dx(dt, dY, W, want_r=True, want_S=True)
        assert np.all(np.abs(r - Gf @ Wf.T) <= 2.0 ** -40 * S)
        _, r, S = O.dw(dt, X, dY, want_r=True, want_S=True)
        assert np.all(np.abs(r - Xf.T @ Gf) <= 2.0 ** -40 * S)


ALL = [integer_exact, rational_bound, order_witnesses, neumaier_textbook, kbn_vs_partials,
       downcast_witnesses, downcast_random_f16, downcast_random_bf16, downcast_random_f32,
       invariants, transpose, closed_form_k1, numpy_fp64]
