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


def _rne32(x):
    """Round an exact rational to the nearest float32, ties to the even encoding (brute force
    over the neighbours of float32(float(x)); independent of numpy's own conversion path)."""
    from fractions import Fraction
    c = np.float32(float(x))
    best = None
    for v in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        key = (abs(Fraction(float(v)) - x), int(np.array(v).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, v)
    return best[1]


def test_relu_mask_is_strict_at_zero():
    """A hidden unit whose pre-activation is exactly 0 passes no gradient (the derivative of the
    ReLU is taken as 0 at 0): with x = [3, 0], W1 = [[0, 1], [0, 0]], b1 = 0 the first unit's
    pre-activation is +0, so after one step its weights and bias are still exactly 0, while
    reading the mask as h >= 0 would move them by -fl32(0.01 * 3 * 2^-11)."""
    params = [(np.array([[0, 1], [0, 0]], dtype=F32), np.zeros(2, dtype=F32)),
              (np.array([[1], [1]], dtype=F32), np.zeros(1, dtype=F32))]
    X = np.array([[3, 0]], dtype=F32)
    T = np.array([[1]], dtype=F32)
    new, _ = mlp.step(params, X, T)
    (W1, b1), (W2, b2) = new
    # y = 3, g2 = fl32(3 - 1) * 2^-12 = 2^-11, g1 = [0, 2^-11]; dW1[0] = 3 * g1, db1 = g1
    assert W1[0, 0] == 0 and not np.signbit(W1[0, 0]) and b1[0] == 0
    from fractions import Fraction
    step = _rne32(Fraction(float(np.float32(0.01))) * Fraction(3 * 2 ** -11))
    assert step != 0   # what a >= mask would have subtracted from W1[0, 0]
    assert W1[0, 1] == _rne32(Fraction(1) - Fraction(float(step)))
    assert b1[1] == -_rne32(Fraction(float(np.float32(0.01))) * Fraction(2 ** -11))


def test_sgd_update_rounds_twice():
    """The update is w = fl32(w - fl32(lr * g)), two roundings: on a one-unit linear model
    (x = 1, W = 2^-30, b = 0, target t) chosen so that lr * g nearly cancels W, the two-rounding
    value differs from the fused fl32(w - lr * g) -- the oracle must give the former."""
    from fractions import Fraction
    Fr = lambda v: Fraction(float(v))   # noqa: E731
    W0 = np.float32(2.0 ** -30)
    t = np.float32(float(W0) - float(W0) / 0.01 * 2 ** 12 * 1.0001)
    lr = np.float32(0.01)
    params = [(np.array([[W0]], dtype=F32), np.zeros(1, dtype=F32))]
    new, _ = mlp.step(params, np.array([[1]], dtype=F32), np.array([[t]], dtype=F32))
    (W1, b1), = new
    # y = RNE32(1 * W0 + 0) = W0; g = fl32(y - t) * 2^-12 (exact scaling); dW = RNE32(1 * g) = g
    g = Fraction(float(_rne32(Fr(W0) - Fr(t)))) * Fraction(2 ** -12)
    q = _rne32(Fr(lr) * g)
    two = _rne32(Fr(W0) - Fr(q))
    fused = _rne32(Fr(W0) - Fr(lr) * g)
    assert two != fused
    assert W1[0, 0] == two, (float(W1[0, 0]), float(two), float(fused))
    assert b1[0] == _rne32(-Fr(q))
