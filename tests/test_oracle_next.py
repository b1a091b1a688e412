"""Pins of the oracle's bias gradient and of dW rounded to f32, against facts
fixed outside the oracle: exact integer column sums, exact rational sums within
the method's error bound, the hand-derived order witnesses laid along a column,
and a brute-force f32 rounding.

db[n] = sum_i dy[i, n] is the dW of a column of ones (the reduction over i in
tiles of 32 rows, Neumaier across tiles; sgemm-bi 0.1.2 PyPI page, note after
"Determinism contracts": the bias gradient is a column sum of dY). dW for f32
master weights (Carbon README, "Roadmap", v0.3 mixed precision) is the same
float64 value rounded once to f32 instead of the input dtype.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic as syn
from tests.pins import brute_round_f32, golden, lib_round, stor, vals, wide_f32

DTS = ("f32", "bf16", "f16")


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("out_dt", [None, "f32"])
def test_db_integer_exact(dt, out_dt):
    for si, (m, n) in enumerate(((1, 1), (31, 5), (32, 7), (33, 9), (200, 3), (1000, 17))):
        dy = syn.integers(600 + si, 3, (m, n), -8, 8, dt)
        y, r, _ = oracle.db(dt, dy, out_dt=out_dt, want_r=True)
        ex = vals(dy, dt).astype(np.int64).sum(axis=0).astype(np.float64)
        assert np.array_equal(r, ex), (dt, m, n)
        assert np.array_equal(y, lib_round(ex, out_dt or dt)), (dt, m, n)


def test_db_rational_bound():
    u = 2.0 ** -53
    for si, m in enumerate((1, 31, 33, 96, 130)):
        dy = wide_f32(650 + si, 3, (m, 4))
        _, r, S = oracle.db("f32", dy, want_r=True, want_S=True)
        d = dy.astype(np.float64)
        for j in range(4):
            ex = sum((Fraction(d[i, j]) for i in range(m)), Fraction(0))
            Sx = sum((abs(Fraction(d[i, j])) for i in range(m)), Fraction(0))
            assert abs(Fraction(r[j]) - ex) <= Fraction(64 * u) * Sx + Fraction(4 * u) * abs(ex), (m, j)
            assert abs(Fraction(S[j]) - Sx) <= Fraction(2.0 ** -40) * Sx


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_db_order_witnesses(dt):
    """Each golden case's product values laid down one column of dY (rows = reduction index)."""
    for case in golden()["cases"]:
        L = case["L"]
        col = np.zeros(L)
        for idx, xs, ws in case["terms"]:
            col[idx] = float.fromhex(xs) * float.fromhex(ws)   # exact: powers of two
        dy = np.stack([col, np.zeros(L), -col], axis=1)
        _, r, _ = oracle.db(dt, stor(dy, dt), want_r=True)
        want = float.fromhex(case["r"])
        assert r[0] == want and r[2] == -want and r[1] == 0.0, (case["name"], r)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_dw_f32_out_single_rounding(dt):
    m, k, n = 70, 5, 6
    X = syn.normal(700, 0, (m, k), dt=dt)
    G = syn.normal(700, 3, (m, n), dt=dt)
    y32, r, _ = oracle.dw_out(dt, "f32", X, G, want_r=True)
    y16, _, _ = oracle.dw(dt, X, G)
    assert y32.dtype == np.float32 and y32.shape == (k, n)
    for q in range(k):
        for j in range(n):
            assert y32[q, j] == brute_round_f32(r[q, j]), (q, j)
    # the input-dtype output of dw_out is dw's own
    assert np.array_equal(oracle.dw_out(dt, dt, X, G)[0], y16)


def test_dw_f32_out_integer_exact():
    m, k, n = 65, 3, 4
    X = syn.integers(710, 0, (m, k), -8, 8, "bf16")
    G = syn.integers(710, 3, (m, n), -8, 8, "bf16")
    y32, _, _ = oracle.dw_out("bf16", "f32", X, G)
    ex = vals(X, "bf16").astype(np.int64).T @ vals(G, "bf16").astype(np.int64)
    assert np.array_equal(y32, ex.astype(np.float32))
