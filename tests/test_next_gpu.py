"""Bias gradient (det_gemm_db) and dW with an f32 output (det_gemm_dw_out) on the
GPU against the oracle: db bit for bit in both tiers; dW to f32 bit for bit in
the exact tier and within the fast tier's tolerance (identical across reruns
and tile families, split reductions included)."""
import numpy as np
import pytest

import oracle
import synthetic as syn
from tests.gpu_util import assert_bits_equal, assert_within_tolerance, to_dev, to_host

pytestmark = pytest.mark.gpu

DB_SHAPES = [(1, 1), (31, 5), (32, 33), (33, 70), (200, 130), (1000, 3), (8300, 65), (4096, 3072)]


@pytest.fixture(autouse=True)
def _auto_family():
    import deterministic_invariant_gemm_det_amd as dg
    dg.det_gemm_debug_force_family(-1)
    dg.det_gemm_debug_force_db_chunk(0)
    yield
    dg.det_gemm_debug_force_family(-1)
    dg.det_gemm_debug_force_db_chunk(0)


def _db_gpu(G, dt, out_dt, tier):
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    from tests.gpu_util import torch_dtype
    g = to_dev(G, dt)
    out = dg.db(g, tier, out_dtype=torch_dtype(out_dt))
    torch.cuda.synchronize()
    return to_host(out, out_dt)


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_db_bit_exact(dt):
    for si, (m, n) in enumerate(DB_SHAPES):
        print(f"db {dt} {(m, n)}", flush=True)
        G = syn.normal(1400 + si, syn.TID_DY, (m, n), dt=dt)
        for out_dt in sorted({dt, "f32"}):
            want, _, _ = oracle.db(dt, G, out_dt=out_dt)
            for tier in ("exact", "fast"):
                assert_bits_equal(_db_gpu(G, dt, out_dt, tier), want, f"db {dt}->{out_dt} {tier} {(m, n)}")


@pytest.mark.parametrize("chunk", [1, 3, 128])
def test_db_chunked(chunk):
    """Tiles handled in several chunks (the pass state carried between them) give the same bits."""
    import deterministic_invariant_gemm_det_amd as dg
    m, n = 8300, 260   # 260 tiles, the last one short
    G = syn.normal(1440, syn.TID_DY, (m, n), dt="bf16")
    want, _, _ = oracle.db("bf16", G, out_dt="f32")
    dg.det_gemm_debug_force_db_chunk(chunk)
    assert_bits_equal(_db_gpu(G, "bf16", "f32", "exact"), want, f"db chunk {chunk}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_db_unaligned_base(dt):
    """dY starting one element past an aligned address takes the per-element load path."""
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    from tests.gpu_util import torch_dtype
    m, n = 100, 64
    G = syn.normal(1445, syn.TID_DY, (m, n), dt=dt)
    want, _, _ = oracle.db(dt, G)
    flat = to_dev(np.concatenate([G.reshape(-1)[:1], G.reshape(-1)]), dt)
    g = flat[1:].view(m, n)
    assert g.data_ptr() % 16 != 0
    out = dg.db(g, "exact")
    torch.cuda.synchronize()
    assert_bits_equal(to_host(out, dt), want, f"db unaligned {dt}")
    assert out.dtype == torch_dtype(dt)


def test_db_integer_columns():
    m, n = 5000, 40
    G = syn.integers(1450, 3, (m, n), -8, 8, "bf16")
    want = syn.from_storage(G, "bf16").astype(np.int64).sum(axis=0).astype(np.float32)
    assert_bits_equal(_db_gpu(G, "bf16", "f32", "exact"), want, "integer column sums")


DW_SHAPES = [(64, 64, 64), (100, 33, 65), (257, 129, 200), (1088, 100, 136), (2048, 192, 320), (1100, 72, 200)]


def _dw_out_gpu(X, G, dt, tier):
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    out = dg.dw(to_dev(X, dt), to_dev(G, dt), tier, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return to_host(out, "f32")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_dw_f32_out(dt):
    import deterministic_invariant_gemm_det_amd as dg
    for si, (m, k, n) in enumerate(DW_SHAPES):
        print(f"dw->f32 {dt} {(m, k, n)}", flush=True)
        X = syn.normal(1500 + si, 0, (m, k), dt=dt)
        G = syn.normal(1500 + si, 3, (m, n), sigma=0.5, dt=dt)
        want, r, S = oracle.dw_out(dt, "f32", X, G, want_r=True, want_S=True)
        assert_bits_equal(_dw_out_gpu(X, G, dt, "exact"), want, f"exact dw->f32 {dt} {(m, k, n)}")
        y = _dw_out_gpu(X, G, dt, "fast")
        assert_within_tolerance(y, r, S, "f32", f"fast dw->f32 {dt} {(m, k, n)}")
        assert_bits_equal(_dw_out_gpu(X, G, dt, "fast"), y, "rerun")
        for fam in (0, 1, 10, 11):
            dg.det_gemm_debug_force_family(fam)
            assert_bits_equal(_dw_out_gpu(X, G, dt, "fast"), y, f"family {fam}")
        dg.det_gemm_debug_force_family(-1)


def test_dw_f32_out_gpt2_c_fc():
    """The GPT-2 c_fc weight gradient (8192 tokens, 768 x 3072) as f32: sampled rows of
    the exact tier against the oracle, the fast tier within tolerance."""
    dt, m, k, n = "bf16", 8192, 768, 3072
    X = syn.normal(42, syn.TID_X, (m, k), dt=dt)
    G = syn.normal(42, syn.TID_DY, (m, n), dt=dt)
    rows = np.array([0, 1, 47, 48, 383, 767])
    want, r, S = oracle.dw_out(dt, "f32", X, G, rows=rows, want_r=True, want_S=True)
    assert_bits_equal(_dw_out_gpu(X, G, dt, "exact")[rows], want, "exact c_fc dW -> f32")
    assert_within_tolerance(_dw_out_gpu(X, G, dt, "fast")[rows], r, S, "f32", "fast c_fc dW -> f32")


def test_measured_peaks_are_plausible():
    """The peak-rate microkernels run and report rates between a fifth of the datasheet peak
    and a little above it (the datasheet figures assume the top clock)."""
    from deterministic_invariant_gemm_det_amd import peak
    for kind, iters, datasheet in ((0, 4000, 78.6), (1, 4000, 78.6), (2, 2000, 2516.6)):
        print(f"peak kind {kind}", flush=True)
        tf = peak.measure(kind, iters, reps=3)
        assert 0.2 * datasheet < tf < 1.1 * datasheet, (kind, tf)
