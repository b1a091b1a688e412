"""Toy-MLP training run on the CPU oracle (test infrastructure only).

End-to-end reproducibility check in the spirit of the Carbon README
(alia-carbon 0.2.0), "The Proof": train a small model from a seed and hash
every weight tensor with SHA-256. The model, data and optimiser are not given
there; this module fixes them as follows:
  forward  h_l = fwd(a_{l-1}, W_l, b_l) with the compensated tiled GEMM;
           a_l = h_l if h_l > 0 else +0.0 for l = 1..3; the last layer is linear;
  loss     mean squared error over the 128 x 64 outputs; its gradient is
           g_4 = fl32(y - T) * 2^-12 (2 / 8192 is a power of two, so exact);
  backward dW_l = dw(a_{l-1}, g_l); db_l = dw(ones[128,1], g_l);
           g_{l-1} = dx(g_l, W_l) where h_{l-1} > 0, else +0.0;
  update   w = fl32(w - fl32(0.01f * g)), all gradients taken before any update.
"""
import hashlib

import numpy as np

import synthetic as syn
from . import dw, dx, fwd

F32 = np.float32


def relu(h):
    return np.where(h > 0, h, F32(0.0)).astype(F32)


def step(params, X, T, lr=syn.MLP_LR):
    acts = [X]
    pre = []
    a = X
    for l, (W, b) in enumerate(params):
        h, _, _ = fwd("f32", a, W, b)
        pre.append(h)
        a = relu(h) if l < len(params) - 1 else h
        acts.append(a)
    y = acts[-1]
    g = ((y - T).astype(F32) * F32(2.0 ** -12)).astype(F32)
    ones = np.ones((X.shape[0], 1), dtype=F32)
    grads = [None] * len(params)
    for l in range(len(params) - 1, -1, -1):
        W, b = params[l]
        gW, _, _ = dw("f32", np.ascontiguousarray(acts[l]), g)
        gb, _, _ = dw("f32", ones, g)
        grads[l] = (gW, gb.reshape(-1))
        if l > 0:
            gx, _, _ = dx("f32", g, W)
            g = np.where(pre[l - 1] > 0, gx, F32(0.0)).astype(F32)
    lr32 = F32(lr)
    new = []
    for (W, b), (gW, gb) in zip(params, grads):
        W2 = (W - (lr32 * gW).astype(F32)).astype(F32)
        b2 = (b - (lr32 * gb).astype(F32)).astype(F32)
        new.append((np.ascontiguousarray(W2), np.ascontiguousarray(b2)))
    loss = float(np.mean((y.astype(np.float64) - T.astype(np.float64)) ** 2))
    return new, loss


def digest(params):
    """SHA-256 over W1, b1, ..., W4, b4 (raw little-endian bytes), plus one per tensor."""
    h = hashlib.sha256()
    per = []
    for W, b in params:
        for t in (W, b):
            raw = np.ascontiguousarray(t, dtype="<f4").tobytes()
            h.update(raw)
            per.append(hashlib.sha256(raw).hexdigest())
    return h.hexdigest(), per


def train(seed, steps=50):
    params = syn.mlp_init(seed)
    losses = []
    for s in range(steps):
        X, T = syn.mlp_batch(seed, s)
        params, loss = step(params, X, T)
        losses.append(loss)
    return params, losses
