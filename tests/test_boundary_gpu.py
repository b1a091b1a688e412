"""The C-ABI boundary on a device: the refusal of an unsupported architecture, the
binding's checks of caller-supplied outputs, calls from two threads on one stream,
and workspace growth inside one stream's sequence of calls."""
import threading

import numpy as np
import pytest

import oracle
import synthetic as syn
from tests.gpu_util import assert_bits_equal, to_dev, to_host

pytestmark = pytest.mark.gpu


def test_unsupported_arch_is_refused_with_a_clear_message():
    """With the architecture check pointed at another name (sgemm-bi 0.1.2 PyPI page,
    introduction: unsupported platforms are refused with a clear message), every entry point
    returns DET_EDEVICE, names the architecture, and writes nothing; restoring the device's own
    name restores service."""
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    L = dg.lib()
    x = to_dev(syn.normal(5, 0, (64, 96), dt="bf16"), "bf16")
    w = to_dev(syn.normal(5, 1, (96, 80), dt="bf16"), "bf16")
    y = torch.full((64, 80), 7.0, dtype=torch.bfloat16, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    try:
        dg.det_gemm_debug_force_arch("gfx942")
        for tier in (0, 1, 2):
            st = L.det_gemm_fwd(y.data_ptr(), x.data_ptr(), w.data_ptr(), None, 64, 96, 80, 1, tier, stream)
            assert st == -4, st
            msg = dg.det_gemm_last_error()
            assert "gfx942" in msg and "gfx950" in msg, msg
        # every buffer sized for its call, so that nothing could go out of bounds even if a call ran
        gx = torch.full((64, 96), 7.0, dtype=torch.bfloat16, device="cuda:0")
        gw = torch.full((96, 80), 7.0, dtype=torch.bfloat16, device="cuda:0")
        gb = torch.full((80,), 7.0, dtype=torch.bfloat16, device="cuda:0")
        assert L.det_gemm_dx(gx.data_ptr(), y.data_ptr(), w.data_ptr(), 64, 96, 80, 1, 0, stream) == -4
        assert L.det_gemm_dw(gw.data_ptr(), x.data_ptr(), y.data_ptr(), 64, 96, 80, 1, 1, stream) == -4
        assert L.det_gemm_db(gb.data_ptr(), 1, y.data_ptr(), 64, 80, 1, 0, stream) == -4
        with pytest.raises(dg.DetGemmError, match="gfx942"):
            dg.fwd(x, w, None, "exact")
        torch.cuda.synchronize()
        for t in (y, gx, gw, gb):
            assert bool((t == 7.0).all()), "a refused call wrote its output"
    finally:
        dg.det_gemm_debug_force_arch(None)
    got = dg.fwd(x, w, None, "exact")
    torch.cuda.synchronize()
    want, _, _ = oracle.fwd("bf16", to_host(x, "bf16"), to_host(w, "bf16"))
    assert_bits_equal(to_host(got, "bf16"), want, "after restoring the architecture")


def test_out_checks_on_device_tensors():
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    x = to_dev(syn.normal(6, 0, (32, 48), dt="f16"), "f16")
    w = to_dev(syn.normal(6, 1, (48, 40), dt="f16"), "f16")
    g = to_dev(syn.normal(6, 2, (32, 40), dt="f16"), "f16")
    dev = x.device
    with pytest.raises(ValueError):
        dg.fwd(x, w, out=torch.empty((32, 39), dtype=torch.float16, device=dev))
    with pytest.raises(ValueError):
        dg.fwd(x, w, out=torch.empty((32, 40), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        dg.dx(g, w, out=torch.empty((48, 32), dtype=torch.float16, device=dev).t())
    with pytest.raises(ValueError):
        dg.dx(g, w, out=torch.empty((32, 48), dtype=torch.float16))   # host tensor
    y = torch.empty((32, 40), dtype=torch.float16, device=dev)
    assert dg.fwd(x, w, out=y) is y
    gx = torch.empty((32, 48), dtype=torch.float16, device=dev)
    assert dg.dx(g, w, out=gx) is gx


def test_two_threads_on_one_stream():
    """Calls from two host threads on the same stream, each needing the stream's workspace
    (split fast dW, few-rows exact forward, bias gradient): each call's launches stay together
    in the stream, so every result equals the one computed alone."""
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    xa = to_dev(syn.normal(80, 0, (4096, 768), dt="bf16"), "bf16")
    ga = to_dev(syn.normal(80, 3, (4096, 1024), dt="bf16"), "bf16")
    xs = to_dev(syn.normal(81, 0, (9, 768), dt="bf16"), "bf16")
    wa = to_dev(syn.normal(81, 1, (768, 1024), sigma=0.02, dt="bf16"), "bf16")
    seqs = {
        "a": [lambda: dg.dw(xa, ga, "fast"), lambda: dg.db(ga, "exact")],
        "b": [lambda: dg.fwd(xs, wa, None, "exact"), lambda: dg.dw(xa, ga, "exact")],
    }
    ref = {k: [f().view(torch.int16).cpu().numpy() for f in v] for k, v in seqs.items()}
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    out, errors = {}, []
    barrier = threading.Barrier(2)

    def run(tag):
        try:
            barrier.wait(timeout=60)
            with torch.cuda.stream(s):
                res = [[f() for f in seqs[tag]] for _ in range(6)]
            s.synchronize()
            out[tag] = [[t.view(torch.int16).cpu().numpy() for t in r] for r in res]
        except Exception as e:   # reported by the main thread
            errors.append(f"{tag}: {e!r}")

    print("two threads, one stream", flush=True)
    threads = [threading.Thread(target=run, args=(t,)) for t in ("a", "b")]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    for tag in ("a", "b"):
        for r, res in enumerate(out[tag]):
            for i, (got, want) in enumerate(zip(res, ref[tag])):
                assert np.array_equal(got, want), f"thread {tag} round {r} call {i}"


def test_workspace_growth_in_stream_order():
    """A stream's workspace grows (a larger buffer taken, the old one kept) while earlier calls
    that use the old one are still queued: every result equals the oracle's."""
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    outs = []
    for i, (m, k, n) in enumerate([(5, 64, 96), (17, 512, 700), (31, 4096, 1000), (3, 9000, 2000)]):
        X = syn.normal(90 + i, 0, (m, k), dt="bf16")
        W = syn.normal(90 + i, 1, (k, n), sigma=0.1, dt="bf16")
        outs.append((X, W, dg.fwd(to_dev(X, "bf16"), to_dev(W, "bf16"), None, "exact")))   # few-rows path
    torch.cuda.synchronize()
    for X, W, y in outs:
        want, _, _ = oracle.fwd("bf16", X, W)
        assert_bits_equal(to_host(y, "bf16"), want, f"few rows {X.shape} x {W.shape}")
