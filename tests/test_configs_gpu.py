"""The larger workloads at full size, in the launch configuration the library uses:

* the GPT-2-124M linears at 8192 tokens, bf16: QKV (768 -> 2304), attention
  projection (768 -> 768), MLP (768 -> 3072, 3072 -> 768); fwd, dX and dW in both
  tiers. Every output element against the oracle (bit for bit in the exact tier,
  within the stated tolerance in the fast tier), bias included on the forward; the
  plain single-threaded oracle runs on blocks of output rows in parallel host
  threads (each row's arithmetic is independent of the others, so the bits are
  those of one thread);
* f32 4096^3 and the bf16 4096 x 4096 x 11008 / 4096 x 11008 x 4096 products, fwd,
  dX and dW in both tiers: 100 back-to-back reruns give identical bits (checked on
  the device, the first output's SHA-256 printed), and sampled rows match the oracle
  as above.
"""
import concurrent.futures as cf
import functools
import hashlib
import os

import numpy as np
import pytest

import oracle
import synthetic as syn
from tests.gpu_util import assert_bits_equal, assert_within_tolerance, to_dev, to_host

pytestmark = pytest.mark.gpu

GPT2 = [(768, 2304), (768, 768), (768, 3072), (3072, 768)]


def _run(dg, op, x, w, g, b, tier):
    if op == "fwd":
        return dg.fwd(x, w, b, tier)
    if op == "dx":
        return dg.dx(g, w, tier)
    return dg.dw(x, g, tier)


def _check_rows(op, dt, tier, X, W, G, b, m, k, n, y, rows, what):
    A, B, bias = {"fwd": (X, W, b), "dx": (G, W, None), "dw": (X, G, None)}[op]
    out_rows = k if op == "dw" else m
    rows = rows[rows < out_rows]
    want, r, S = oracle.gemm(op, dt, A, B, m, k, n, bias=bias, rows=rows, want_r=True, want_S=True)
    if tier == "exact":
        assert_bits_equal(y[rows], want, what)
    else:
        assert_within_tolerance(y[rows], r, S, dt, what)


def _host_threads():
    """Oracle threads: the host cores this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _oracle_full(op, dt, A, B, m, k, n, bias):
    """The oracle's y, r and S of every output element, blocks of rows on parallel threads."""
    out_rows = k if op == "dw" else m
    blocks = np.array_split(np.arange(out_rows, dtype=np.int64), 4 * _host_threads())
    with cf.ThreadPoolExecutor(_host_threads()) as ex:
        parts = list(ex.map(lambda rows: oracle.gemm(op, dt, A, B, m, k, n, bias=bias, rows=rows, want_r=True,
                                                     want_S=True), [b for b in blocks if b.size]))
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(3))


@pytest.mark.parametrize("kn", GPT2, ids=[f"{k}x{n}" for k, n in GPT2])
def test_gpt2_linears(kn):
    """Every output element of fwd, dX and dW in both tiers: exact tier bit for bit, fast tier
    within the tolerance; two runs give identical bits."""
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    dt, m = "bf16", 8192
    k, n = kn
    X = syn.normal(42, syn.TID_X, (m, k), dt=dt)
    W = syn.normal(42, syn.TID_W, (k, n), sigma=0.02, dt=dt)
    b = syn.normal(42, syn.TID_B, (n,), sigma=0.1, dt=dt)
    G = syn.normal(42, syn.TID_DY, (m, n), dt=dt)
    x, w, bb, g = to_dev(X, dt), to_dev(W, dt), to_dev(b, dt), to_dev(G, dt)
    for op in ("fwd", "dx", "dw"):
        A, B, bias = {"fwd": (X, W, b), "dx": (G, W, None), "dw": (X, G, None)}[op]
        print(f"gpt2 {k}x{n} {op}: oracle on {_host_threads()} threads", flush=True)
        want, r, S = _oracle_full(op, dt, A, B, m, k, n, bias)
        for tier in ("exact", "fast"):
            print(f"gpt2 {k}x{n} {tier} {op}", flush=True)
            y0 = _run(dg, op, x, w, g, bb, tier)
            y1 = _run(dg, op, x, w, g, bb, tier)
            torch.cuda.synchronize()
            assert torch.equal(y0.view(torch.int16), y1.view(torch.int16)), "rerun"
            got = to_host(y0, dt)
            if tier == "exact":
                assert_bits_equal(got, want, f"gpt2 {k}x{n} exact {op}")
            else:
                assert_within_tolerance(got, r, S, dt, f"gpt2 {k}x{n} fast {op}")


LARGE = [("f32", 4096, 4096, 4096), ("bf16", 4096, 4096, 11008), ("bf16", 4096, 11008, 4096)]


@functools.lru_cache(maxsize=None)
def _large_inputs(cfg):
    dt, m, k, n = cfg
    print(f"generating {cfg}", flush=True)
    return (syn.normal(42, syn.TID_X, (m, k), dt=dt), syn.normal(42, syn.TID_W, (k, n), sigma=0.02, dt=dt),
            syn.normal(42, syn.TID_DY, (m, n), dt=dt))


@pytest.mark.parametrize("cfg", LARGE, ids=[f"{c[0]}-{c[1]}x{c[2]}x{c[3]}" for c in LARGE])
@pytest.mark.parametrize("tier", ["exact", "fast"])
def test_large_reruns(cfg, tier):
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    dt, m, k, n = cfg
    X, W, G = _large_inputs(cfg)
    x, w, g = to_dev(X, dt), to_dev(W, dt), to_dev(G, dt)
    rows = np.array([0, 1, 2047, 4095])
    view = torch.int32 if dt == "f32" else torch.int16
    for op in ("fwd", "dx", "dw"):
        print(f"large {dt} {m}x{k}x{n} {tier} {op}", flush=True)
        y0 = _run(dg, op, x, w, g, None, tier)
        for rep in range(99):
            assert torch.equal(_run(dg, op, x, w, g, None, tier).view(view), y0.view(view)), f"{op}: rerun {rep} differs"
        host = to_host(y0, dt)
        print(f"  sha256 {hashlib.sha256(host.tobytes()).hexdigest()[:16]}", flush=True)
        _check_rows(op, dt, tier, X, W, G, None, m, k, n, host, rows, f"large {dt} {m}x{k}x{n} {tier} {op}")
