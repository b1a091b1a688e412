"""Batch invariance: rows of a smaller-M result equal the matching rows of the
M = 8192 result bit for bit (K = 768, N = 3072), for fwd and dx, both tiers.
The smaller inputs are the first M rows copied into separate buffers."""
import numpy as np
import pytest

import oracle
import synthetic as syn
from tests.gpu_util import assert_bits_equal, to_dev, to_host

pytestmark = pytest.mark.gpu

MS = (1, 3, 17, 64, 127, 512, 2048, 8192)
K, N = 768, 3072


@pytest.mark.parametrize("tier", ["exact", "fast"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_m_sweep(dt, tier):
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    X = syn.normal(42, syn.TID_X, (8192, K), dt=dt)
    W = syn.normal(42, syn.TID_W, (K, N), sigma=0.02, dt=dt)
    b = syn.normal(42, syn.TID_B, (N,), sigma=0.1, dt=dt)
    G = syn.normal(42, syn.TID_DY, (8192, N), dt=dt)
    w = to_dev(W, dt)
    bb = to_dev(b, dt)
    full_y = to_host(dg.fwd(to_dev(X, dt), w, None, tier), dt)
    full_yb = to_host(dg.fwd(to_dev(X, dt), w, bb, tier), dt)
    full_dx = to_host(dg.dx(to_dev(G, dt), w, tier), dt)
    for M in MS:
        print(f"sweep {dt} {tier} M={M}", flush=True)
        x = to_dev(np.ascontiguousarray(X[:M]), dt)
        g = to_dev(np.ascontiguousarray(G[:M]), dt)
        assert_bits_equal(to_host(dg.fwd(x, w, None, tier), dt), full_y[:M], f"fwd M={M}")
        assert_bits_equal(to_host(dg.fwd(x, w, bb, tier), dt), full_yb[:M], f"fwd+bias M={M}")
        assert_bits_equal(to_host(dg.dx(g, w, tier), dt), full_dx[:M], f"dx M={M}")
    torch.cuda.synchronize()
    if tier == "exact":
        rows = np.array([0, 1, 2, 16, 63, 126, 511, 2047, 4095, 8191])
        assert_bits_equal(full_y[rows], oracle.fwd(dt, X, W, rows=rows)[0], "fwd vs oracle")
        assert_bits_equal(full_yb[rows], oracle.fwd(dt, X, W, b, rows=rows)[0], "fwd+bias vs oracle")
        assert_bits_equal(full_dx[rows], oracle.dx(dt, G, W, rows=rows)[0], "dx vs oracle")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_m_sweep_long_reduction_fast(dt):
    """K = 3072, N = 768 (GPT-2 c_proj): from m = 4096 on, the fast forward
    first copies the weight transposed (for K = 768, N = 3072 the same switch
    sits inside the main sweep's 4095/4096); rows must not change across that
    switch (nor anywhere else in the sweep), with and without the bias."""
    import deterministic_invariant_gemm_det_amd as dg
    k, n = 3072, 768
    X = syn.normal(43, syn.TID_X, (8192, k), dt=dt)
    W = syn.normal(43, syn.TID_W, (k, n), sigma=0.02, dt=dt)
    b = syn.normal(43, syn.TID_B, (n,), sigma=0.1, dt=dt)
    w, bb = to_dev(W, dt), to_dev(b, dt)
    full = to_host(dg.fwd(to_dev(X, dt), w, bb, "fast"), dt)
    full_nb = to_host(dg.fwd(to_dev(X, dt), w, None, "fast"), dt)
    for M in (1, 17, 2048, 4095, 4096, 6000):
        print(f"long-reduction sweep {dt} M={M}", flush=True)
        x = to_dev(np.ascontiguousarray(X[:M]), dt)
        assert_bits_equal(to_host(dg.fwd(x, w, bb, "fast"), dt), full[:M], f"fwd+bias M={M}")
        assert_bits_equal(to_host(dg.fwd(x, w, None, "fast"), dt), full_nb[:M], f"fwd M={M}")


# Row counts on both sides of every point where the fast tier's choice of kernel changes
# with m for K = 768, N = 3072 (each choice gives the same bits; the rows must not change):
#   fwd: 128 x 64 tiles when m is a multiple of 128 and 256 x 192 tiles would number fewer
#        than 256 (m <= 3840), else 256 x 192 tiles -- m = 127/128/129, 3840/3841/3968;
#        from m = 4096 on, the weight copied transposed first -- m = 4095/4096;
#   dX (768 columns): 64 x 192 tiles when m is a multiple of 64 and 128 x 192 tiles would
#        number fewer than 256 (m <= 8064), else 128 x 192 -- m = 63/64/65, 8064/8065/8128;
#   plus the few-rows limit of the exact tier (m = 32/33).
SWITCH_MS = (32, 33, 63, 64, 65, 127, 128, 129, 3840, 3841, 3968, 4095, 4096, 8064, 8065, 8128)


@pytest.mark.parametrize("tier", ["fast", "exact"])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_m_sweep_switch_points(dt, tier):
    import deterministic_invariant_gemm_det_amd as dg
    X = syn.normal(44, syn.TID_X, (8192, K), dt=dt)
    W = syn.normal(44, syn.TID_W, (K, N), sigma=0.02, dt=dt)
    b = syn.normal(44, syn.TID_B, (N,), sigma=0.1, dt=dt)
    G = syn.normal(44, syn.TID_DY, (8192, N), dt=dt)
    w, bb = to_dev(W, dt), to_dev(b, dt)
    full_yb = to_host(dg.fwd(to_dev(X, dt), w, bb, tier), dt)
    full_dx = to_host(dg.dx(to_dev(G, dt), w, tier), dt)
    Ms = SWITCH_MS if tier == "fast" else (32, 33, 63, 64, 65)
    for M in Ms:
        print(f"switch sweep {dt} {tier} M={M}", flush=True)
        x = to_dev(np.ascontiguousarray(X[:M]), dt)
        g = to_dev(np.ascontiguousarray(G[:M]), dt)
        assert_bits_equal(to_host(dg.fwd(x, w, bb, tier), dt), full_yb[:M], f"fwd+bias M={M}")
        assert_bits_equal(to_host(dg.dx(g, w, tier), dt), full_dx[:M], f"dx M={M}")
