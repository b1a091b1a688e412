"""det_gemm_dw_noalloc (the weight gradient for callers that cannot allocate) against
det_gemm_dw_out through the C-ABI: the same bits on two calls in a row, the second with a
smaller input, in every tier and path that needs a workspace; a call whose workspace exceeds
the fixed scratch is refused with DET_EINVAL and writes nothing."""
import numpy as np
import pytest

import synthetic as syn
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu

# (dt, dw_dt, tier, [(m, k, n) larger, then smaller]) -- every case uses the scratch:
#   fast bf16/f16 dW split into chunks, with the smaller operand copied transposed;
#   exact few-rows dW (k <= 32: every tile partial in the scratch);
#   the correctly rounded tier (statistics and slices).
CASES = [
    ("bf16", "bf16", "fast", [(8192, 768, 3072), (2048, 256, 512)]),
    ("bf16", "f32", "fast", [(8192, 3072, 768), (4096, 768, 768)]),
    ("f16", "f16", "fast", [(8192, 768, 2304), (1088, 100, 136)]),
    ("bf16", "bf16", "exact", [(4096, 17, 1000), (640, 5, 300)]),
    ("f32", "f32", "exact", [(2000, 32, 700), (96, 3, 50)]),
    ("bf16", "bf16", "cr", [(1024, 96, 200), (300, 40, 64)]),
]
TORCH = {"f32": "float32", "bf16": "bfloat16", "f16": "float16"}


def _pair(dg, torch, dt, odt, tier, m, k, n, seed):
    x = to_dev(syn.normal(seed, 0, (m, k), dt=dt), dt)
    g = to_dev(syn.normal(seed, 3, (m, n), dt=dt), dt)
    tdt = getattr(torch, TORCH[odt])
    ref = torch.empty((k, n), dtype=tdt, device=x.device)
    got = torch.full((k, n), 3.0, dtype=tdt, device=x.device)
    st = torch.cuda.current_stream().cuda_stream
    dg.det_gemm_dw_out(ref, odt, x, g, m, k, n, dt, tier, st)
    dg.det_gemm_dw_noalloc(got, odt, x, g, m, k, n, dt, tier, st)
    return ref, got


@pytest.mark.parametrize("case", CASES, ids=[f"{c[2]}-{c[0]}-{c[1]}" for c in CASES])
def test_noalloc_matches_dw_out(case):
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    dt, odt, tier, shapes = case
    outs = []
    for i, (m, k, n) in enumerate(shapes):   # two calls in a row, the second smaller
        print(f"noalloc {tier} {dt}->{odt} {(m, k, n)}", flush=True)
        outs.append(_pair(dg, torch, dt, odt, tier, m, k, n, 2000 + 10 * i + CASES.index(case)))
    torch.cuda.synchronize()
    ints = {2: torch.int16, 4: torch.int32}
    for (m, k, n), (ref, got) in zip(shapes, outs):
        v = ints[ref.element_size()]
        assert torch.equal(ref.view(v), got.view(v)), f"{tier} {dt}->{odt} {(m, k, n)}"


def test_noalloc_refuses_a_workspace_beyond_the_scratch():
    """The correctly rounded dW of 8192 x 768 x 3072 needs about 250 MB of slices: refused with
    DET_EINVAL and a message giving both sizes; the output is untouched; a later call works."""
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    m, k, n = 8192, 768, 3072
    x = to_dev(syn.normal(7, 0, (m, k), dt="bf16"), "bf16")
    g = to_dev(syn.normal(7, 3, (m, n), dt="bf16"), "bf16")
    out = torch.full((k, n), 3.0, dtype=torch.bfloat16, device=x.device)
    st = torch.cuda.current_stream().cuda_stream
    status = dg.lib().det_gemm_dw_noalloc(out.data_ptr(), 1, x.data_ptr(), g.data_ptr(), m, k, n, 1, 2, st)
    assert status == -1, status
    msg = dg.det_gemm_last_error()
    assert "scratch" in msg and str(64 << 20) in msg, msg
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()), "a refused call wrote its output"
    ref, got = _pair(dg, torch, "bf16", "bf16", "fast", m, k, n, 8)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))
