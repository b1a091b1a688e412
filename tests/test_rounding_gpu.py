"""The tiers' output roundings on the device against the oracle's rounding
(sgemm-bi 0.1.2 PyPI page, "Determinism contracts": the round-to-nearest-even
downcast; Carbon README, "How It Works": one rounding at the end).

Fast tier: every one of the 2^32 f32 bit patterns goes through round_from_f32,
the function every fast-tier epilogue calls, to bf16 and to f16, and is
compared bit for bit with the oracle's single rounding of the same value
(oracle_round on it as float64, which holds it exactly); a NaN must stay a NaN
(its payload is not part of the contract). Exact tier: round_from_f64 (round to
odd at f32, then the hardware's round to nearest even) on float64 values chosen
where a double rounding would go wrong -- each midpoint between neighbouring
outputs, and values a hair above or below it that round to the midpoint at f32
-- together with the neighbours of every output value, the overflow and
subnormal edges, specials and random values, to bf16, f16 and f32. The same
values go through round_group, the LayerNorm forward's rounding of eight values
per lane (for bf16 a plain rounding at f32 unless the wave meets a bf16
midpoint): every value above that rounds to a midpoint at f32 takes its slow
path, and its neighbours in the same wave are checked with it."""
import concurrent.futures as cf
import os

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

CHUNK = 1 << 24
WORKERS = min(16, os.cpu_count() or 1)


def _is_nan16(bits, dt):
    bits = bits.astype(np.uint16)
    if dt == "bf16":
        return ((bits & 0x7f80) == 0x7f80) & ((bits & 0x007f) != 0)
    return ((bits & 0x7c00) == 0x7c00) & ((bits & 0x03ff) != 0)


def _compare_f32_chunk(first, got, dt):
    """Oracle rounding of the f32 values with bits first .. first + len(got) - 1."""
    bits = (np.arange(len(got), dtype=np.uint64) + np.uint64(first)).astype(np.uint32)
    v = bits.view(np.float32)
    with np.errstate(invalid="ignore"):
        want = oracle.round_to(dt, v.astype(np.float64)).view(np.uint16)
    got = got.view(np.uint16)
    nan_in = np.isnan(v)
    bad = (got != want) & ~nan_in
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        return f"{dt}: f32 bits {int(bits[i]):#010x}: device {int(got[i]):#06x}, oracle {int(want[i]):#06x}"
    if not _is_nan16(got[nan_in], dt).all():
        return f"{dt}: a NaN input did not give a NaN"
    return None


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_fast_tier_rounding_of_every_f32(dt):
    import deterministic_invariant_gemm_det_amd as dg
    import torch
    print(f"all 2^32 f32 patterns -> {dt}", flush=True)
    failures = []
    with cf.ThreadPoolExecutor(max_workers=WORKERS) as ex:
        futures = []
        for first in range(0, 1 << 32, CHUNK):
            got = dg.det_gemm_debug_round_f32(first, CHUNK, dt)
            torch.cuda.synchronize()
            futures.append(ex.submit(_compare_f32_chunk, first, got.cpu().numpy(), dt))
            if len(futures) >= 2 * WORKERS:
                failures += [f.result() for f in futures[:WORKERS]]
                futures = futures[WORKERS:]
        failures += [f.result() for f in futures]
    failures = [f for f in failures if f]
    assert not failures, failures[:5]


def test_fast_tier_f32_output_is_the_value():
    import deterministic_invariant_gemm_det_amd as dg
    first = 0x7f000000
    got = dg.det_gemm_debug_round_f32(first, CHUNK, "f32").cpu().numpy().view(np.uint32)
    want = (np.arange(CHUNK, dtype=np.uint64) + np.uint64(first)).astype(np.uint32)
    assert np.array_equal(got, want)


def _values_of(dt):
    """Every finite value of the output type in increasing order (f32: a sample)."""
    if dt == "bf16":
        bits = np.arange(1 << 16, dtype=np.uint32)
        with np.errstate(invalid="ignore"):
            v = (bits << 16).view(np.float32).astype(np.float64)
    elif dt == "f16":
        v = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    else:
        rng = np.random.default_rng(11)
        bits = np.unique(np.concatenate([rng.integers(0, 1 << 32, 1 << 22, dtype=np.uint64).astype(np.uint32),
                                         np.arange(0, 4096, dtype=np.uint32),           # smallest subnormals
                                         np.arange(0x7f7ff000, 0x7f800000, dtype=np.uint32)]))  # up to the largest
        with np.errstate(invalid="ignore"):
            v = bits.view(np.float32).astype(np.float64)
    v = np.unique(v[np.isfinite(v)])
    return v


def _hard_cases(dt):
    v = _values_of(dt)
    lo, hi = v[:-1], v[1:]
    gap = hi - lo
    mid = lo + gap / 2                      # exact in float64
    up, down = np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)
    eps = gap * 2.0 ** -30                  # rounds to the midpoint at f32 precision
    top = v[-1]
    over = [top + (top - v[-2]) / 2 * f for f in (0.5, 1.0 - 2.0 ** -40, 1.0, 1.0 + 2.0 ** -40, 2.0)]
    rng = np.random.default_rng(12)
    rand = (rng.standard_normal(1 << 20) * np.exp2(rng.integers(-150, 140, 1 << 20))).astype(np.float64)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e300, -1e300, 1e-300, -1e-300, 2.0 ** -1074])
    cases = np.concatenate([mid, up, down, mid + eps, mid - eps, lo, np.nextafter(lo, np.inf),
                            np.nextafter(lo, -np.inf), lo + gap * 2.0 ** -40, hi - gap * 2.0 ** -40,
                            np.array(over), rand, specials])
    return np.concatenate([cases, -cases])


@pytest.mark.parametrize("grouped", [False, True])
@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_exact_tier_rounding_of_hard_float64_values(dt, grouped):
    import deterministic_invariant_gemm_det_amd as dg
    import torch
    x = _hard_cases(dt)
    print(f"{dt} grouped={grouped}: {x.size} float64 values", flush=True)
    hook = dg.det_gemm_debug_round_f64_grouped if grouped else dg.det_gemm_debug_round_f64
    got = hook(torch.from_numpy(x).to("cuda:0"), dt).cpu().numpy()
    with np.errstate(invalid="ignore"):
        want = oracle.round_to(dt, x)
    if dt == "f32":
        got, want = got.view(np.uint32), want.view(np.uint32)
        nan_out = np.isnan(got.view(np.float32))
    else:
        got, want = got.view(np.uint16), want.view(np.uint16)
        nan_out = _is_nan16(got, dt)
    nan_in = np.isnan(x)
    assert np.array_equal(nan_out, nan_in), "NaN in and NaN out differ"
    bad = (got != want) & ~nan_in
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        pytest.fail(f"{dt}: {x[i]!r} ({x[i].hex()}): device {int(got[i]):#x}, oracle {int(want[i]):#x} "
                    f"({int(bad.sum())} of {x.size} differ)")
