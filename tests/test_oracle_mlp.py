"""The oracle's toy-MLP training run against a plain float64-matmul run of the same model.

The compensated GEMM differs from a library float64 matmul only by rounding far
below float32 resolution, so a few training steps of both must stay within a
few float32 ulps; a wrong transpose, activation mask, gradient scale or update
would not.
"""
import numpy as np

import synthetic as syn
from oracle import mlp

F32 = np.float32


def _numpy_step(params, X, T, lr=syn.MLP_LR):
    acts, pre = [X], []
    a = X
    for l, (W, b) in enumerate(params):
        h = (a.astype(np.float64) @ W.astype(np.float64) + b.astype(np.float64)).astype(F32)
        pre.append(h)
        a = np.where(h > 0, h, F32(0)) if l < len(params) - 1 else h
        acts.append(a)
    g = ((acts[-1] - T) * F32(2.0 ** -12)).astype(F32)
    grads = [None] * len(params)
    for l in range(len(params) - 1, -1, -1):
        W, _ = params[l]
        gW = (acts[l].astype(np.float64).T @ g.astype(np.float64)).astype(F32)
        gb = g.astype(np.float64).sum(axis=0).astype(F32)
        grads[l] = (gW, gb)
        if l > 0:
            gx = (g.astype(np.float64) @ W.astype(np.float64).T).astype(F32)
            g = np.where(pre[l - 1] > 0, gx, F32(0)).astype(F32)
    return [((W - F32(lr) * gW).astype(F32), (b - F32(lr) * gb).astype(F32)) for (W, b), (gW, gb) in zip(params, grads)]


def test_mlp_tracks_float64_reference():
    seed = 42
    p_or = syn.mlp_init(seed)
    p_np = syn.mlp_init(seed)
    for s in range(3):
        X, T = syn.mlp_batch(seed, s)
        p_or, loss = mlp.step(p_or, X, T)
        p_np = _numpy_step(p_np, X, T)
        assert np.isfinite(loss)
    for (Wo, bo), (Wn, bn) in zip(p_or, p_np):
        assert np.allclose(Wo, Wn, rtol=1e-5, atol=1e-6)
        assert np.allclose(bo, bn, rtol=1e-5, atol=1e-6)
    assert sum(W.size + b.size for W, b in p_or) == 542016


def test_mlp_digest_is_reproducible():
    p1, l1 = mlp.train(7, steps=2)
    p2, l2 = mlp.train(7, steps=2)
    d1, per1 = mlp.digest(p1)
    d2, per2 = mlp.digest(p2)
    assert d1 == d2 and per1 == per2 and len(per1) == 8 and l1 == l2
