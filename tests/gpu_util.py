"""Helpers for the GPU tests: storage arrays <-> device tensors, bit compares, tolerance."""
import numpy as np

import synthetic as syn

P = {"f32": 24, "bf16": 8, "f16": 11}
EMIN = {"f32": -126, "bf16": -126, "f16": -14}


def torch_dtype(dt):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dt]


def to_dev(a, dt, device="cuda:0"):
    import torch
    if dt == "f32":
        t = torch.from_numpy(np.ascontiguousarray(a))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch_dtype(dt))
    return t.to(device)


def to_host(t, dt):
    import torch
    t = t.detach().contiguous().cpu()
    if dt == "f32":
        return t.numpy().copy()
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


def assert_bits_equal(got, want, what=""):
    g, w = bits(got), bits(want)
    if g.shape != w.shape:
        raise AssertionError(f"{what}: shape {g.shape} vs {w.shape}")
    bad = np.argwhere(g != w)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {g.size} elements differ; first at {i}: "
                             f"got {hex(int(g[i]))} want {hex(int(w[i]))}")


def ulp(v, dt):
    v = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    e = np.maximum(np.where(v > 0, e, EMIN[dt]), EMIN[dt])
    return np.exp2(e - (P[dt] - 1))


def assert_within_tolerance(got, r, S, dt, what=""):
    """|y - r| <= 2^-20 * S + ulp_D(max(|r|, |y|)) per element."""
    y = syn.from_storage(got, dt)
    err = np.abs(y - r)
    bound = 2.0 ** -20 * S + ulp(np.maximum(np.abs(r), np.abs(y)), dt)
    bad = np.argwhere(~(err <= bound))
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {y.size} outside tolerance; first at {i}: "
                             f"y={y[i]!r} r={r[i]!r} S={S[i]!r} bound={bound[i]!r}")


def operand_shapes(op, m, k, n):
    return {"fwd": ((m, k), (k, n)), "dx": ((m, n), (k, n)), "dw": ((m, k), (m, n))}[op]


def gpu_op(op, dt, A, B, bias=None, tier="exact"):
    """Run one op through the C-ABI (via the binding) on host storage arrays; returns host storage."""
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    a, b = to_dev(A, dt), to_dev(B, dt)
    bb = to_dev(bias, dt) if bias is not None else None
    if op == "fwd":
        out = dg.fwd(a, b, bb, tier)
    elif op == "dx":
        out = dg.dx(a, b, tier)
    else:
        out = dg.dw(a, b, tier)
    torch.cuda.synchronize()
    return to_host(out, dt)
