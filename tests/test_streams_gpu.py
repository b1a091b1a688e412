"""Streams and threads: every call is enqueued on the caller's current stream,
workspace users (the fast tier's split dW, the exact tier's few-rows path, the
bias gradient) keep one workspace per stream, and calls from two host threads
on two streams at once give the same bits as the same calls one after another
on the default stream."""
import threading

import pytest

import synthetic as syn
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu


def _workloads():
    """Two call sequences with workspaces of different sizes (and dtypes)."""
    import deterministic_invariant_gemm_det_amd as dg
    a = {
        "x": to_dev(syn.normal(77, syn.TID_X, (8192, 768), dt="bf16"), "bf16"),
        "g": to_dev(syn.normal(77, syn.TID_DY, (8192, 3072), dt="bf16"), "bf16"),
        "w": to_dev(syn.normal(77, syn.TID_W, (768, 3072), sigma=0.02, dt="bf16"), "bf16"),
    }
    b = {
        "x": to_dev(syn.normal(78, syn.TID_X, (2048, 512), dt="f16"), "f16"),
        "g": to_dev(syn.normal(78, syn.TID_DY, (2048, 1024), dt="f16"), "f16"),
        "w": to_dev(syn.normal(78, syn.TID_W, (512, 1024), sigma=0.02, dt="f16"), "f16"),
        "xs": to_dev(syn.normal(79, syn.TID_X, (17, 512), dt="f16"), "f16"),
    }
    seq_a = [
        ("fast dw", lambda: dg.dw(a["x"], a["g"], "fast")),          # split dW: partials + transposed copy
        ("fast dx", lambda: dg.dx(a["g"], a["w"], "fast")),
        ("db", lambda: dg.db(a["g"], "exact")),                       # tile partials in the workspace
    ]
    seq_b = [
        ("exact dw", lambda: dg.dw(b["x"], b["g"], "exact")),
        ("exact fwd few rows", lambda: dg.fwd(b["xs"], b["w"], None, "exact")),   # per-tile partials
        ("fast dw", lambda: dg.dw(b["x"], b["g"], "fast")),
    ]
    return seq_a, seq_b


def _hosts(outs):
    """The outputs' bits on the host (integer views of the same bytes)."""
    import torch
    ints = {2: torch.int16, 4: torch.int32, 8: torch.int64}
    return [o.detach().cpu().view(ints[o.element_size()]).numpy().copy() for o in outs]


def test_user_stream_and_two_threads_match_default_stream():
    import torch
    seq_a, seq_b = _workloads()
    torch.cuda.synchronize()
    ref_a = _hosts([f() for _, f in seq_a])
    ref_b = _hosts([f() for _, f in seq_b])
    torch.cuda.synchronize()

    # one user stream, the calls ordered on it alone
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        outs = [f() for _, f in seq_a]
    s.synchronize()
    for (name, _), got, want in zip(seq_a, _hosts(outs), ref_a):
        assert (got == want).all(), f"user stream: {name}"

    # two host threads, each on its own stream, several rounds at once
    results, errors = {}, []

    def run(tag, seq, rounds=4):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                outs = [[f() for _, f in seq] for _ in range(rounds)]
            st.synchronize()
            results[tag] = [_hosts(o) for o in outs]
        except Exception as e:   # reported by the main thread
            errors.append(f"{tag}: {e!r}")

    print("two threads, two streams", flush=True)
    threads = [threading.Thread(target=run, args=("a", seq_a)), threading.Thread(target=run, args=("b", seq_b))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    for tag, seq, ref in (("a", seq_a, ref_a), ("b", seq_b, ref_b)):
        for r, outs in enumerate(results[tag]):
            for (name, _), got, want in zip(seq, outs, ref):
                assert (got == want).all(), f"thread {tag} round {r}: {name}"
