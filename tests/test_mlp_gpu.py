"""Toy-MLP training (256-512-512-256-64, batch 128, f32, 50 SGD steps) through
the exact tier: the SHA-256 of the final weights equals the oracle's, for the
five seeds of the Carbon README's proof table, and training twice gives the
same hash (the sgemm-bi example's pattern)."""
import concurrent.futures as cf
import hashlib
import multiprocessing as mp

import numpy as np
import pytest

import synthetic as syn

pytestmark = pytest.mark.gpu

STEPS = 50


def _oracle_digest(seed):
    from oracle import mlp
    params, losses = mlp.train(seed, STEPS)
    return mlp.digest(params)[0], losses[-1]


def gpu_train(seed, steps=STEPS):
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    dev = torch.device("cuda:0")
    params = []
    for W, b in syn.mlp_init(seed):
        params.append((torch.from_numpy(W).to(dev).requires_grad_(True),
                       torch.from_numpy(b).to(dev).requires_grad_(True)))
    lr = torch.tensor(syn.MLP_LR, dtype=torch.float32, device=dev)
    zero = torch.zeros((), dtype=torch.float32, device=dev)
    for s in range(steps):
        X, T = syn.mlp_batch(seed, s)
        a = torch.from_numpy(X).to(dev)
        t = torch.from_numpy(T).to(dev)
        for l, (W, b) in enumerate(params):
            h = dg.deterministic_linear(a, W, b, tier="exact")
            a = torch.where(h > 0, h, zero) if l < len(params) - 1 else h
        g = ((a - t) * (2.0 ** -12)).detach()
        a.backward(g)
        with torch.no_grad():
            for W, b in params:
                for p in (W, b):
                    step = p.grad * lr
                    p.copy_(p - step)
                    p.grad = None
    torch.cuda.synchronize()
    h = hashlib.sha256()
    for W, b in params:
        for p in (W, b):
            h.update(np.ascontiguousarray(p.detach().cpu().numpy(), dtype="<f4").tobytes())
    return h.hexdigest()


def test_mlp_sha256_matches_oracle_all_seeds():
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=len(syn.MLP_SEEDS), mp_context=ctx) as ex:
        futs = {seed: ex.submit(_oracle_digest, seed) for seed in syn.MLP_SEEDS}
        gpu = {}
        for seed in syn.MLP_SEEDS:
            print("gpu mlp seed", seed, flush=True)
            gpu[seed] = gpu_train(seed)
        for seed in syn.MLP_SEEDS:
            want, loss = futs[seed].result()
            print(f"seed {seed}: gpu {gpu[seed][:16]} oracle {want[:16]} final loss {loss:.6f}", flush=True)
            assert gpu[seed] == want, seed


def test_mlp_train_twice_same_hash():
    assert gpu_train(42, steps=10) == gpu_train(42, steps=10)
