"""Toy-MLP training (256-512-512-256-64, batch 128, f32, 50 SGD steps) through
the exact tier: the SHA-256 of the final weights equals the oracle's, for the
five seeds of the Carbon README's proof table; training twice gives the same
hash (the sgemm-bi example's pattern), and so does resuming at step 25 from
weights saved to the host."""
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


def gpu_train(seed, steps=STEPS, start=0, params=None):
    """Steps start .. steps - 1 of the run on the GPU, from the seed's initial weights or from
    `params` (host arrays [(W, b), ...], as a checkpoint holds them); returns the SHA-256 of the
    final weights and the weights themselves as host arrays."""
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    dev = torch.device("cuda:0")
    dev_params = []
    for W, b in (params if params is not None else syn.mlp_init(seed)):
        dev_params.append((torch.from_numpy(np.ascontiguousarray(W)).to(dev).requires_grad_(True),
                           torch.from_numpy(np.ascontiguousarray(b)).to(dev).requires_grad_(True)))
    lr = torch.tensor(syn.MLP_LR, dtype=torch.float32, device=dev)
    zero = torch.zeros((), dtype=torch.float32, device=dev)
    for s in range(start, steps):
        X, T = syn.mlp_batch(seed, s)   # the data stream's position is the step index
        a = torch.from_numpy(X).to(dev)
        t = torch.from_numpy(T).to(dev)
        for l, (W, b) in enumerate(dev_params):
            h = dg.deterministic_linear(a, W, b, tier="exact")
            a = torch.where(h > 0, h, zero) if l < len(dev_params) - 1 else h
        g = ((a - t) * (2.0 ** -12)).detach()
        a.backward(g)
        with torch.no_grad():
            for W, b in dev_params:
                for p in (W, b):
                    step = p.grad * lr
                    p.copy_(p - step)
                    p.grad = None
    torch.cuda.synchronize()
    host = [(W.detach().cpu().numpy().copy(), b.detach().cpu().numpy().copy()) for W, b in dev_params]
    h = hashlib.sha256()
    for W, b in host:
        for p in (W, b):
            h.update(np.ascontiguousarray(p, dtype="<f4").tobytes())
    return h.hexdigest(), host


@pytest.fixture(scope="module")
def oracle_digests():
    """The oracle's 50-step SHA-256 and final loss for every seed, computed in parallel processes."""
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=len(syn.MLP_SEEDS), mp_context=ctx) as ex:
        futs = {seed: ex.submit(_oracle_digest, seed) for seed in syn.MLP_SEEDS}
        return {seed: f.result() for seed, f in futs.items()}


def test_mlp_sha256_matches_oracle_all_seeds(oracle_digests):
    for seed in syn.MLP_SEEDS:
        print("gpu mlp seed", seed, flush=True)
        got, _ = gpu_train(seed)
        want, loss = oracle_digests[seed]
        print(f"seed {seed}: gpu {got[:16]} oracle {want[:16]} final loss {loss:.6f}", flush=True)
        assert got == want, seed


def test_mlp_resume_at_step_25(oracle_digests):
    """Train 25 steps, keep the weights on the host as a checkpoint, start again from it with
    fresh device tensors at step 25 (the data stream is indexed by step): the 50-step SHA-256 is
    the uninterrupted run's, which is the oracle's (Carbon README, "The Proof": the same hash of
    every weight tensor)."""
    for seed in syn.MLP_SEEDS:
        print("gpu mlp resume seed", seed, flush=True)
        _, ckpt = gpu_train(seed, steps=25)
        got, _ = gpu_train(seed, steps=STEPS, start=25, params=ckpt)
        assert got == oracle_digests[seed][0], seed


def test_mlp_train_twice_same_hash():
    assert gpu_train(42, steps=10)[0] == gpu_train(42, steps=10)[0]
