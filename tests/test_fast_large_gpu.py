"""Fast tier at the GPT-2-124M MLP sizes (8192 tokens, 768 <-> 3072, bf16), in
the launch configuration the benchmark times: sampled output rows within the
stated tolerance of the oracle, identical bits on reruns and across every tile
family and tile shape (the large shapes are the only ones that exercise the
eight-wave kernel's full-size tiles over many stages)."""
import numpy as np
import pytest

import oracle
import synthetic as syn
from tests.gpu_util import assert_bits_equal, assert_within_tolerance, to_dev, to_host

pytestmark = pytest.mark.gpu

M = 8192
LAYERS = [("c_fc", 768, 3072), ("c_proj", 3072, 768)]
FAMILIES = (0, 1, 10, 11, 12, 13, 14, 15)
ROWS = np.array([0, 1, 31, 32, 255, 256, 1000, 4095, 4096, 8190, 8191])


@pytest.fixture(autouse=True)
def _auto_family():
    import deterministic_invariant_gemm_det_amd as dg
    dg.det_gemm_debug_force_family(-1)
    yield
    dg.det_gemm_debug_force_family(-1)


@pytest.mark.parametrize("layer", LAYERS, ids=[l[0] for l in LAYERS])
@pytest.mark.parametrize("op", ["fwd", "dx", "dw"])
def test_gpt2_shapes(op, layer):
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    dt = "bf16"
    _, k, n = layer
    X = syn.normal(42, syn.TID_X, (M, k), dt=dt)
    W = syn.normal(42, syn.TID_W, (k, n), sigma=0.02, dt=dt)
    b = syn.normal(42, syn.TID_B, (n,), sigma=0.1, dt=dt)
    G = syn.normal(42, syn.TID_DY, (M, n), dt=dt)
    x, w, bb, g = to_dev(X, dt), to_dev(W, dt), to_dev(b, dt), to_dev(G, dt)
    run = {"fwd": lambda: dg.fwd(x, w, bb, "fast"), "dx": lambda: dg.dx(g, w, "fast"),
           "dw": lambda: dg.dw(x, g, "fast")}[op]
    print(f"fast large {op} {layer}", flush=True)
    y = to_host(run(), dt)
    # sampled rows against the oracle (dW's rows are the k index, at most k)
    rows = ROWS[ROWS < (k if op == "dw" else M)]
    A, B, bias = {"fwd": (X, W, b), "dx": (G, W, None), "dw": (X, G, None)}[op]
    _, r, S = oracle.gemm(op, dt, A, B, M, k, n, bias=bias, rows=rows, want_r=True, want_S=True)
    assert_within_tolerance(y[rows], r, S, dt, f"fast {op} {layer[0]} sampled rows")
    for rep in range(3):
        assert_bits_equal(to_host(run(), dt), y, f"rerun {rep}")
    for fam in FAMILIES:
        print(f"  family {fam}", flush=True)
        dg.det_gemm_debug_force_family(fam)
        outs = [run() for _ in range(2)]
        for i, o in enumerate(outs):
            assert_bits_equal(to_host(o, dt), y, f"family {fam} call {i}")
    dg.det_gemm_debug_force_family(-1)
    torch.cuda.synchronize()
