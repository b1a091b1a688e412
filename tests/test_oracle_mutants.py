"""Mistakes planted in copies of the oracle (on the CPU) must each fail some pin.

Each mutant is oracle.cpp with one plausible slip, compiled into a temporary
directory; the pins of tests/pins.py are run against it and at least one must
fail. This shows that the pins constrain the oracle rather than restate it.
Also: the oracle's results do not depend on the compiler or optimisation level.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import synthetic as syn
from oracle.build import SRC, build
from tests import pins

MUTANTS = {
    "tile_width_16": ("constexpr int64_t KT = 32;", "constexpr int64_t KT = 16;"),
    "plain_sum_across_tiles": ("c = c + ((s - tt) + p);", "c = c;"),
    "neumaier_branch_swapped": ("if (std::fabs(s) >= std::fabs(p)) {", "if (std::fabs(s) < std::fabs(p)) {"),
    "chain_descending": ("for (int64_t k = t0; k < t1; ++k) {", "for (int64_t k = t1 - 1; k >= t0; --k) {"),
    "ties_down": ("else code = (lo % 2 == 0) ? lo : hi;", "else code = lo;"),
    "bias_dropped": ("v = v + bj;", "v = v + 0.0 * bj;"),
    "compensation_dropped_at_end": ("return s + c;\n}", "return s;\n}"),
    # ways a four-deep matrix instruction could order its products: each
    # group of four indices (from the tile start) summed pairwise, or as a
    # chain from 0 and only then added to the running partial, or exactly
    # (in long double) with the running partial and rounded once
    "pairwise_in_groups_of_four": (
        "p = std::fma(a[k], b[k], p);",
        "if ((k - t0) % 4 == 0) { double v[4] = {0.0, 0.0, 0.0, 0.0}; "
        "for (int64_t q = k; q < std::min(k + 4, t1); ++q) v[q - k] = a[q] * b[q]; "
        "p = p + ((v[0] + v[1]) + (v[2] + v[3])); }"),
    "group_chain_then_added": (
        "p = std::fma(a[k], b[k], p);",
        "if ((k - t0) % 4 == 0) { double g = 0.0; "
        "for (int64_t q = k; q < std::min(k + 4, t1); ++q) g = std::fma(a[q], b[q], g); p = p + g; }"),
    "group_fused_with_partial": (
        "p = std::fma(a[k], b[k], p);",
        "if ((k - t0) % 4 == 0) { long double g = p; "
        "for (int64_t q = k; q < std::min(k + 4, t1); ++q) g += (long double)a[q] * (long double)b[q]; "
        "p = (double)g; }"),
}


def _compile_variant(tmp_path, name, src_text, compiler="g++", opt=None):
    src = tmp_path / f"{name}.cpp"
    src.write_text(src_text)
    out = str(tmp_path / f"lib{name}.so")
    flags = [f for f in oracle.build.FLAGS if not (opt and f.startswith("-O"))] + ([opt] if opt else [])
    subprocess.run([compiler, *flags, str(src), "-o", out], check=True)
    return oracle.Oracle(out)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not found exactly once"
    O = _compile_variant(tmp_path, name, text.replace(old, new))
    failed = []
    for check in pins.ALL:
        try:
            check(O)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"planted mistake {name} passed every pin"


@pytest.mark.parametrize("compiler,opt", [("g++", "-O0"), ("clang++", "-O0"), ("clang++", "-O2"), ("g++", "-O3")])
def test_compiler_independence(tmp_path, compiler, opt):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not installed")
    O = _compile_variant(tmp_path, f"v_{compiler}_{opt}".replace("+", "p"), open(SRC).read(), compiler, opt)
    ref = oracle.default()
    m, k, n = 23, 150, 31
    for dt in pins.DTS:
        X = syn.normal(800, 0, (m, k), dt=dt)
        W = syn.normal(800, 1, (k, n), dt=dt)
        b = syn.normal(800, 2, (n,), sigma=0.1, dt=dt)
        dY = syn.normal(800, 3, (m, n), dt=dt)
        for a, r in ((O.fwd(dt, X, W, b, want_r=True), ref.fwd(dt, X, W, b, want_r=True)),
                     (O.dx(dt, dY, W, want_r=True), ref.dx(dt, dY, W, want_r=True)),
                     (O.dw(dt, X, dY, want_r=True), ref.dw(dt, X, dY, want_r=True))):
            assert np.array_equal(a[0], r[0])
            assert np.array_equal(a[1].view(np.uint64), r[1].view(np.uint64))
