"""Exact tier on the GPU, bit for bit against the CPU oracle."""
import numpy as np
import pytest

import oracle
import synthetic as syn
from tests import pins
from tests.gpu_util import assert_bits_equal, gpu_op, operand_shapes

pytestmark = pytest.mark.gpu

DTS = ("f32", "bf16", "f16")
SHAPES = [(1, 1, 1), (3, 33, 65), (127, 70, 129), (64, 64, 64), (200, 300, 100), (17, 1000, 5), (65, 31, 63), (2, 97, 250),
          (96, 100, 144), (49, 48, 47)]


def test_config1_fp32_fwd_dx_dw():
    """M=256 K=512 N=512 f32, X, W ~ N(0,1), bias ~ N(0,0.1), dY ~ N(0,1), seed 42: full outputs."""
    m, k, n = 256, 512, 512
    X = syn.normal(42, syn.TID_X, (m, k))
    W = syn.normal(42, syn.TID_W, (k, n))
    b = syn.normal(42, syn.TID_B, (n,), sigma=0.1)
    G = syn.normal(42, syn.TID_DY, (m, n))
    print("config1 fwd", flush=True)
    assert_bits_equal(gpu_op("fwd", "f32", X, W, b), oracle.fwd("f32", X, W, b)[0], "fwd")
    assert_bits_equal(gpu_op("fwd", "f32", X, W), oracle.fwd("f32", X, W)[0], "fwd nobias")
    print("config1 dx", flush=True)
    assert_bits_equal(gpu_op("dx", "f32", G, W), oracle.dx("f32", G, W)[0], "dx")
    print("config1 dw", flush=True)
    assert_bits_equal(gpu_op("dw", "f32", X, G), oracle.dw("f32", X, G)[0], "dw")


@pytest.fixture(autouse=True)
def _auto_variant():
    import deterministic_invariant_gemm_det_amd as dg
    dg.det_gemm_debug_force_exact_kernel(-1)
    yield
    dg.det_gemm_debug_force_exact_kernel(-1)


@pytest.mark.parametrize("variant", [0, 1, 2, 3, 4, 5, 6, 7],
                         ids=["m16s", "mfma16", "valu", "mfma4db", "m16s48", "skinny", "mfma4", "mfma4r48"])
@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("op", ["fwd", "dx", "dw"])
def test_ragged_shapes(op, dt, variant):
    import deterministic_invariant_gemm_det_amd as dg
    dg.det_gemm_debug_force_exact_kernel(variant)
    for si, (m, k, n) in enumerate(SHAPES):
        print(f"exact {op} {dt} {(m, k, n)} variant {variant}", flush=True)
        sa, sb = operand_shapes(op, m, k, n)
        A = syn.normal(900 + si, 0, sa, dt=dt)
        B = syn.normal(900 + si, 1, sb, sigma=0.5, dt=dt)
        bias = syn.normal(900 + si, 2, (n,), sigma=0.1, dt=dt) if op == "fwd" else None
        want, _, _ = oracle.gemm(op, dt, A, B, m, k, n, bias=bias)
        assert_bits_equal(gpu_op(op, dt, A, B, bias), want, f"{op} {dt} {(m, k, n)}")


@pytest.mark.parametrize("dt", DTS)
def test_integer_inputs_exact(dt):
    for op in ("fwd", "dx", "dw"):
        for si, (m, k, n) in enumerate(SHAPES):
            sa, sb = operand_shapes(op, m, k, n)
            A = syn.integers(950 + si, 0, sa, -8, 8, dt)
            B = syn.integers(950 + si, 1, sb, -8, 8, dt)
            want, _, _ = oracle.gemm(op, dt, A, B, m, k, n)
            assert_bits_equal(gpu_op(op, dt, A, B), want, f"int {op} {dt} {(m, k, n)}")


VARIANTS = [0, 1, 2, 3, 4, 5, 6, 7]
VARIANT_IDS = ["m16s", "mfma16", "valu", "mfma4db", "m16s48", "skinny", "mfma4", "mfma4r48"]


@pytest.mark.parametrize("variant", VARIANTS, ids=VARIANT_IDS)
def test_golden_witnesses(variant):
    """Every hand-derived witness as a single output, through each exact kernel."""
    import deterministic_invariant_gemm_det_amd as dg
    dg.det_gemm_debug_force_exact_kernel(variant)
    for case in pins.golden()["cases"] + pins.golden()["downcast"]:
        dts = [case["dt"]] if "dt" in case else DTS
        for op in ("fwd", "dx", "dw"):
            for dt in dts:
                A, B, m, k, n = pins._witness_operands(op, dt, case["L"], pins._golden_terms(case))
                want, r, _ = oracle.gemm(op, dt, A, B, m, k, n, want_r=True)
                assert r[0, 0] == float.fromhex(case["r"])
                assert_bits_equal(gpu_op(op, dt, A, B), want, f"{case['name']} {op} {dt} variant {variant}")


# Output positions of the embedded witnesses: first, middle and last rows and
# columns of 64-, 48- and 16-wide blocks and of the lanes' 4 x 4 sub-blocks.
EMB_ROWS = [0, 5, 14, 31, 33, 47, 48, 63, 64, 70, 81, 95]
EMB_COLS = [0, 3, 16, 31, 32, 47, 50, 63, 64, 66, 75, 79]


def _embedded(op, dt, seed):
    """All witness cases of the golden file inside one 96 x 80 output over a reduction of 128, the
    rest of the operands random: witness q sits at output (EMB_ROWS[q], EMB_COLS[q]), its row of
    the first operand zero except its terms, its column of the second holding the term values."""
    cases = pins.golden()["cases"]
    assert len(cases) <= len(EMB_ROWS)
    L, R, C = 128, 96, 80
    m, k, n = {"fwd": (R, L, C), "dx": (R, C, L), "dw": (L, R, C)}[op]
    sa, sb = operand_shapes(op, m, k, n)
    A = syn.from_storage(syn.normal(seed, 0, sa, dt=dt), dt).copy()
    B = syn.from_storage(syn.normal(seed, 1, sb, sigma=0.5, dt=dt), dt).copy()
    for case, i, j in zip(cases, EMB_ROWS, EMB_COLS):
        assert case["L"] <= L
        if op == "dw":
            A[:, i] = 0.0
        else:
            A[i, :] = 0.0
        for idx, xv, wv in pins._golden_terms(case):
            if op == "fwd":
                A[i, idx], B[idx, j] = xv, wv
            elif op == "dx":
                A[i, idx], B[j, idx] = xv, wv
            else:
                A[idx, i], B[idx, j] = xv, wv
    return cases, pins.stor(A, dt), pins.stor(B, dt), m, k, n


@pytest.mark.parametrize("variant", VARIANTS, ids=VARIANT_IDS)
@pytest.mark.parametrize("op", ["fwd", "dx", "dw"])
def test_witnesses_inside_blocks(op, variant):
    """The order witnesses (a sequential fma chain inside each four-index matrix-instruction group,
    the running partial entering each group first, ties to even, tiles anchored at 0, Neumaier
    across tiles) at many positions of full blocks of every exact kernel, random data around them:
    the oracle's float64 value at each witness is the hand-derived one, and the whole output is
    the oracle's bit for bit."""
    import deterministic_invariant_gemm_det_amd as dg
    dg.det_gemm_debug_force_exact_kernel(variant)
    for dt in DTS:
        print(f"embedded witnesses {op} {dt} variant {variant}", flush=True)
        cases, A, B, m, k, n = _embedded(op, dt, 1200 + DTS.index(dt))
        want, r, _ = oracle.gemm(op, dt, A, B, m, k, n, want_r=True)
        for case, i, j in zip(cases, EMB_ROWS, EMB_COLS):
            assert r[i, j] == float.fromhex(case["r"]) and not np.signbit(r[i, j]), (case["name"], op, dt)
        assert_bits_equal(gpu_op(op, dt, A, B), want, f"embedded {op} {dt} variant {variant}")
        if op == "dw" and dt != "f32" and variant in (0, 4):
            # the f32-output dW (the default kernel in its two row-block forms)
            want32 = oracle.round_to("f32", r)
            got32 = _dw_f32(dt, A, B)
            assert_bits_equal(got32, want32, f"embedded dw->f32 {dt} variant {variant}")


def _dw_f32(dt, A, B):
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    from tests.gpu_util import to_dev
    out = dg.dw(to_dev(A, dt), to_dev(B, dt), "exact", out_dtype=torch.float32)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("dt,scale_x,scale_w", [
    ("f32", 2.0 ** -70, 2.0 ** -70),    # f32 subnormal outputs
    ("bf16", 2.0 ** -70, 2.0 ** -65),   # bf16 subnormal outputs
    ("f16", 2.0 ** -8, 2.0 ** -10),     # f16 subnormal outputs
    ("bf16", 2.0 ** 100, 2.0 ** 27),    # bf16 overflow to inf
    ("f16", 2.0 ** 6, 2.0 ** 8),        # f16 overflow to inf
    ("f32", 2.0 ** 100, 2.0 ** 27),     # f32 overflow to inf
])
def test_rounding_edges(dt, scale_x, scale_w):
    m, k, n = 40, 37, 50
    X = syn.to_storage(syn.from_storage(syn.normal(990, 0, (m, k), dt=dt), dt) * scale_x, dt)
    W = syn.to_storage(syn.from_storage(syn.normal(990, 1, (k, n), dt=dt), dt) * scale_w, dt)
    want, _, _ = oracle.fwd(dt, X, W)
    assert_bits_equal(gpu_op("fwd", dt, X, W), want, f"edges {dt}")
