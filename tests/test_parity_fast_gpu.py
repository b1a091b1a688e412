"""Fast tier on the GPU: within the stated tolerance of the oracle, exact on
integer inputs, identical across reruns and across the two tile families."""
import numpy as np
import pytest

import oracle
import synthetic as syn
from tests.gpu_util import assert_bits_equal, assert_within_tolerance, gpu_op, operand_shapes

pytestmark = pytest.mark.gpu

DTS = ("f32", "bf16", "f16")
SHAPES = [(1, 1, 1), (3, 33, 65), (127, 70, 129), (64, 64, 64), (200, 300, 100), (17, 1000, 5),
          (65, 31, 63), (2, 97, 250), (130, 200, 1100), (257, 129, 1030),
          # reduction lengths that are multiples of 64 for every op (large-tile kernel), ragged edges
          (320, 128, 192), (512, 256, 136), (192, 640, 1000), (64, 64, 1088), (576, 192, 64)]


@pytest.fixture(autouse=True)
def _auto_family():
    import deterministic_invariant_gemm_det_amd as dg
    dg.det_gemm_debug_force_family(-1)
    yield
    dg.det_gemm_debug_force_family(-1)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("op", ["fwd", "dx", "dw"])
def test_tolerance_and_families(op, dt):
    import deterministic_invariant_gemm_det_amd as dg
    for si, (m, k, n) in enumerate(SHAPES):
        print(f"fast {op} {dt} {(m, k, n)}", flush=True)
        sa, sb = operand_shapes(op, m, k, n)
        A = syn.normal(1100 + si, 0, sa, dt=dt)
        B = syn.normal(1100 + si, 1, sb, sigma=0.5, dt=dt)
        bias = syn.normal(1100 + si, 2, (n,), sigma=0.1, dt=dt) if op == "fwd" else None
        _, r, S = oracle.gemm(op, dt, A, B, m, k, n, bias=bias, want_r=True, want_S=True)
        y = gpu_op(op, dt, A, B, bias, tier="fast")
        assert_within_tolerance(y, r, S, dt, f"fast {op} {dt} {(m, k, n)}")
        assert_bits_equal(gpu_op(op, dt, A, B, bias, tier="fast"), y, "rerun")
        for fam in (0, 1, 10, 12, 14, 15):
            dg.det_gemm_debug_force_family(fam)
            assert_bits_equal(gpu_op(op, dt, A, B, bias, tier="fast"), y, f"family {fam}")
        dg.det_gemm_debug_force_family(-1)


@pytest.mark.parametrize("dt", DTS)
def test_integer_inputs_exact(dt):
    for op in ("fwd", "dx", "dw"):
        for si, (m, k, n) in enumerate(SHAPES):
            sa, sb = operand_shapes(op, m, k, n)
            A = syn.integers(1200 + si, 0, sa, -8, 8, dt)
            B = syn.integers(1200 + si, 1, sb, -8, 8, dt)
            want, _, _ = oracle.gemm(op, dt, A, B, m, k, n)
            assert_bits_equal(gpu_op(op, dt, A, B, tier="fast"), want, f"int fast {op} {dt} {(m, k, n)}")


# dW shapes whose reduction (m) is long enough to be split into chunks: the
# split count comes from the shape alone, so both families (and the eight-wave
# kernel where the shape allows it) must give the same bits. m = 1100 and
# 2101 are not multiples of 64 (register-staged kernel only, ragged last chunk).
SPLIT_SHAPES = [(1088, 100, 136), (2048, 192, 320), (4160, 64, 64), (1100, 72, 200), (2101, 136, 64)]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_dw_split(dt):
    import deterministic_invariant_gemm_det_amd as dg
    for si, (m, k, n) in enumerate(SPLIT_SHAPES):
        print(f"fast dw split {dt} {(m, k, n)}", flush=True)
        A = syn.normal(1300 + si, 0, (m, k), dt=dt)
        B = syn.normal(1300 + si, 1, (m, n), sigma=0.5, dt=dt)
        _, r, S = oracle.gemm("dw", dt, A, B, m, k, n, want_r=True, want_S=True)
        y = gpu_op("dw", dt, A, B, tier="fast")
        assert_within_tolerance(y, r, S, dt, f"fast dw {dt} {(m, k, n)}")
        assert_bits_equal(gpu_op("dw", dt, A, B, tier="fast"), y, "rerun")
        for fam in (0, 1, 10, 11, 12, 13, 14, 15):
            dg.det_gemm_debug_force_family(fam)
            assert_bits_equal(gpu_op("dw", dt, A, B, tier="fast"), y, f"family {fam}")
        dg.det_gemm_debug_force_family(-1)


# The forward for at most 32 rows (one 32-column block per workgroup, the weight streamed
# through LDS): bit-identical to the tiled kernels; k a multiple of 8 (other k take the tiled
# kernels); ragged n, k past the last 128-index chunk, with and without the bias.
SKINNY = [(1, 768, 3072), (3, 768, 3072), (17, 3072, 768), (32, 72, 1000), (31, 8, 5), (2, 200, 40), (9, 1032, 136),
          (1, 11008, 64)]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_skinny_forward_matches_tiled(dt):
    import deterministic_invariant_gemm_det_amd as dg
    for si, (m, k, n) in enumerate(SKINNY):
        print(f"skinny fwd {dt} {(m, k, n)}", flush=True)
        X = syn.normal(1500 + si, 0, (m, k), dt=dt)
        W = syn.normal(1500 + si, 1, (k, n), sigma=0.1, dt=dt)
        b = syn.normal(1500 + si, 2, (n,), sigma=0.1, dt=dt)
        _, r, S = oracle.fwd(dt, X, W, b, want_r=True, want_S=True)
        for bias in (b, None):
            dg.det_gemm_debug_force_family(16)
            y16 = gpu_op("fwd", dt, X, W, bias, tier="fast")
            dg.det_gemm_debug_force_family(0)
            y0 = gpu_op("fwd", dt, X, W, bias, tier="fast")
            dg.det_gemm_debug_force_family(-1)
            assert_bits_equal(y16, y0, f"skinny vs tiled {dt} {(m, k, n)} bias={bias is not None}")
            assert_bits_equal(gpu_op("fwd", dt, X, W, bias, tier="fast"), y0, "automatic")
        assert_within_tolerance(gpu_op("fwd", dt, X, W, b, tier="fast"), r, S, dt, f"skinny {dt} {(m, k, n)}")
