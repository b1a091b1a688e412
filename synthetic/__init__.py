"""Seeded synthetic inputs shared by the tests, the oracle harness and the benchmark.

This module holds no GEMM arithmetic: it only turns a (seed, tensor id) pair
into a tensor of f32/bf16/f16 values, so that the CPU oracle and the GPU
library are fed the very same bytes.

Generator (fixed here so that every run draws the same values):
  * one SplitMix64 stream per tensor (Steele, Lea and Flood, "Fast splittable
    pseudorandom number generators", OOPSLA 2014), started from
    state0 = seed XOR (0x9E3779B97F4A7C15 * (tensor_id + 1)) mod 2^64;
  * uniform u = (draw >> 11) * 2^-53 in [0, 1);
  * standard normal by Box-Muller from two consecutive uniforms:
    z = sqrt(-2 ln(1 - u1)) * cos(2 pi u2), in float64, then times sigma;
  * conversion to storage: float64 -> float32 (RNE, numpy), then float32 ->
    bf16 (RNE, torch) or float32 -> f16 (RNE, numpy).
Storage arrays are float32 for "f32" and uint16 bit patterns for "bf16"/"f16".
"""
import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)
CHUNK = 1 << 22

STORAGE = {"f32": np.float32, "bf16": np.uint16, "f16": np.uint16}


def _state0(seed, tid):
    s = (int(seed) & 0xFFFFFFFFFFFFFFFF) ^ ((0x9E3779B97F4A7C15 * (int(tid) + 1)) & 0xFFFFFFFFFFFFFFFF)
    return np.uint64(s)


def splitmix64(seed, tid, start, count):
    """Draws start .. start+count-1 of the tensor's SplitMix64 stream (uint64)."""
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = _state0(seed, tid) + idx * GAMMA
        z = (z ^ (z >> np.uint64(30))) * M1
        z = (z ^ (z >> np.uint64(27))) * M2
    return z ^ (z >> np.uint64(31))


def uniform(seed, tid, start, count):
    return (splitmix64(seed, tid, start, count) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal_f64(seed, tid, count, sigma=1.0):
    out = np.empty(count, dtype=np.float64)

    def fill(c0):   # chunks are independent: their values do not depend on the threads
        c = min(CHUNK, count - c0)
        u = uniform(seed, tid, 2 * c0, 2 * c)
        u1, u2 = u[0::2], u[1::2]
        out[c0:c0 + c] = np.sqrt(-2.0 * np.log(1.0 - u1)) * np.cos(2.0 * np.pi * u2) * sigma

    starts = range(0, count, CHUNK)
    if count <= CHUNK:
        for c0 in starts:
            fill(c0)
    else:
        import os
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=max(1, min(8, os.cpu_count() or 1))) as ex:
            list(ex.map(fill, starts))
    return out


def to_storage(v, dt):
    """float64 values -> storage of dt (via float32, RNE at each step)."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    if dt == "f32":
        return f
    if dt == "f16":
        return f.astype(np.float16).view(np.uint16)
    if dt == "bf16":
        import torch
        return torch.from_numpy(np.ascontiguousarray(f)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dt)


def from_storage(a, dt):
    """Storage of dt -> float64 values (exact)."""
    if dt == "f32":
        return a.astype(np.float64)
    if dt == "f16":
        return a.view(np.float16).astype(np.float64)
    if dt == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(dt)


def normal(seed, tid, shape, sigma=1.0, dt="f32"):
    count = int(np.prod(shape))
    return np.ascontiguousarray(to_storage(normal_f64(seed, tid, count, sigma), dt).reshape(shape))


def integers(seed, tid, shape, lo, hi, dt="f32"):
    """Uniform integers in [lo, hi] (inclusive), stored exactly in dt."""
    count = int(np.prod(shape))
    span = np.uint64(hi - lo + 1)
    v = (splitmix64(seed, tid, 0, count) % span).astype(np.int64) + lo
    return np.ascontiguousarray(to_storage(v.astype(np.float64), dt).reshape(shape))


# Tensor ids used across the suite (one stream per logical tensor).
TID_X, TID_W, TID_B, TID_DY = 0, 1, 2, 3


# ---- toy multilayer perceptron used by the end-to-end reproducibility check ----
# Widths 256 -> 512 -> 512 -> 256 -> 64, batch 128, float32, weights stored
# [in, out] and He-initialised (normal, sigma = sqrt(2 / fan_in)), biases zero.
MLP_WIDTHS = (256, 512, 512, 256, 64)
MLP_BATCH = 128
MLP_LR = 0.01
MLP_SEEDS = (42, 123, 7, 999, 2024)


def mlp_init(seed):
    """[(W_l float32 [in,out], b_l float32 [out]) for l = 1..4]."""
    params = []
    for l in range(len(MLP_WIDTHS) - 1):
        fan_in, fan_out = MLP_WIDTHS[l], MLP_WIDTHS[l + 1]
        W = normal(seed, 10 + l, (fan_in, fan_out), sigma=float(np.sqrt(2.0 / fan_in)))
        b = np.zeros(fan_out, dtype=np.float32)
        params.append((W, b))
    return params


def mlp_batch(seed, step):
    """(X_s [128,256], T_s [128,64]) float32 for training step `step`."""
    X = normal(seed, 1000 + 2 * step, (MLP_BATCH, MLP_WIDTHS[0]))
    T = normal(seed, 1001 + 2 * step, (MLP_BATCH, MLP_WIDTHS[-1]))
    return X, T
