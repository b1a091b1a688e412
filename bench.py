"""Benchmark of the deterministic GEMM hot path on one MI355X.

One step = one training pass of the GPT-2-124M MLP linears at 8192 tokens
(c_fc 768->3072 and c_proj 3072->768, bf16 storage): forward, dX and dW of
both layers, through the exact tier (float64 tiles + Neumaier) and then the
fast tier (bf16 matrix cores, f32 accumulate): 12 GEMM launches, all inputs
resident in HBM before the timed region.

Prints one JSON line. `value` is useful TFLOP/s of the whole step
(2*M*N*K per GEMM over the step time); per-tier and per-op rates, the
roofline of the dominant kernel (measured with HIP events on the stream the
kernels run on) and the CPU oracle's rate on a bounded sample are included.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "deterministic GEMM TFLOP/s (fp64-KBN & bf16-MFMA tiers) + % of peak, 1 GPU"
PEAK_FP64 = 78.6      # TFLOP/s, MI355X FP64 vector and FP64 matrix
PEAK_BF16 = 2516.6    # TFLOP/s, MI355X dense bf16 MFMA
TOKENS = 8192
LAYERS = (("c_fc", 768, 3072), ("c_proj", 3072, 768))
OPS = ("fwd", "dx", "dw")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU-oracle sample")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    return p.parse_args()


def make_inputs(dev):
    import torch
    import numpy as np
    import synthetic as syn

    def to_dev(a, dt, device):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

    data = {}
    for li, (name, k, n) in enumerate(LAYERS):
        X = syn.normal(42 + li, syn.TID_X, (TOKENS, k), dt="bf16")
        W = syn.normal(42 + li, syn.TID_W, (k, n), sigma=0.02, dt="bf16")
        G = syn.normal(42 + li, syn.TID_DY, (TOKENS, n), dt="bf16")
        data[name] = dict(X=X, W=W, G=G, x=to_dev(X, "bf16", dev), w=to_dev(W, "bf16", dev),
                          g=to_dev(G, "bf16", dev), k=k, n=n,
                          y=torch.empty((TOKENS, n), dtype=torch.bfloat16, device=dev),
                          gx=torch.empty((TOKENS, k), dtype=torch.bfloat16, device=dev),
                          gw=torch.empty((k, n), dtype=torch.bfloat16, device=dev))
    return data


def launches(data):
    """The step as a list of (tier, layer, op, callable)."""
    import deterministic_invariant_gemm_det_amd as dg
    out = []
    for tier in ("exact", "fast"):
        for name, _, _ in LAYERS:
            d = data[name]
            out.append((tier, name, "fwd", lambda d=d, t=tier: dg.fwd(d["x"], d["w"], None, t, out=d["y"])))
            out.append((tier, name, "dx", lambda d=d, t=tier: dg.dx(d["g"], d["w"], t, out=d["gx"])))
            out.append((tier, name, "dw", lambda d=d, t=tier: dg.dw(d["x"], d["g"], t, out=d["gw"])))
    return out


def cpu_baseline(data, budget_s):
    """The oracle, as it stands, on a bounded sample of the step's exact-tier GEMMs (one core)."""
    import numpy as np
    import oracle
    flops = 0.0
    t0 = time.perf_counter()
    per_op = budget_s / 6.0
    pieces = []
    for name, k, n in LAYERS:
        d = data[name]
        for op in OPS:
            rows_done = 0
            t_op = time.perf_counter()
            chunk = 8 if op != "dw" else 2
            while time.perf_counter() - t_op < per_op:
                rows = np.arange(rows_done, rows_done + chunk)
                if op == "fwd":
                    oracle.fwd("bf16", d["X"], d["W"], rows=rows)
                    flops += 2.0 * chunk * k * n
                elif op == "dx":
                    oracle.dx("bf16", d["G"], d["W"], rows=rows)
                    flops += 2.0 * chunk * n * k
                else:
                    oracle.dw("bf16", d["X"], d["G"], rows=rows)
                    flops += 2.0 * chunk * TOKENS * n
                rows_done += chunk
            pieces.append(f"{name}.{op}:{rows_done} rows")
    secs = time.perf_counter() - t0
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": "exact-tier output rows of the step's six GEMMs (" + ", ".join(pieces) +
                      f"), {secs:.1f} s single-threaded, useful 2*M*N*K flops per row"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: only one GPU is used here (asked for {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    dev = torch.device("cuda:0")
    data = make_inputs(dev)
    steps = launches(data)
    stream = torch.cuda.current_stream(dev)

    for _ in range(args.warmup):
        for _, _, _, f in steps:
            f()
    torch.cuda.synchronize()

    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in steps]
          for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(args.steps):
        for i, (_, _, _, f) in enumerate(steps):
            ev[s][i][0].record(stream)
            f()
            ev[s][i][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps

    per = {}
    for i, (tier, name, op, _) in enumerate(steps):
        ms = sum(ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)) / args.steps
        k, n = data[name]["k"], data[name]["n"]
        fl = 2.0 * TOKENS * k * n
        per[f"{tier}.{name}.{op}"] = {"us": round(ms * 1e3, 2), "tflops": round(fl / (ms * 1e-3) / 1e12, 2)}

    def tier_stats(tier, peak):
        keys = [k for k in per if k.startswith(tier + ".")]
        fl = sum(2.0 * TOKENS * data[k.split(".")[1]]["k"] * data[k.split(".")[1]]["n"] for k in keys)
        us = sum(per[k]["us"] for k in keys)
        tf = fl / (us * 1e-6) / 1e12
        return {"tflops": round(tf, 2), "pct_of_peak": round(100 * tf / peak, 2), "peak_tflops": peak, "us": round(us, 1)}

    total_flops = 2 * sum(2.0 * TOKENS * k * n * len(OPS) for _, k, n in LAYERS)
    value = total_flops / (ms_step * 1e-3) / 1e12

    # dominant kernel: the exact-tier launch with the largest share of the step
    exact_keys = [k for k in per if k.startswith("exact.")]
    dom = max(exact_keys, key=lambda k: per[k]["us"])
    dom_tf = per[dom]["tflops"]
    roofline = {"bound": "mfma", "achieved": dom_tf, "peak": PEAK_FP64, "unit": "TFLOP/s",
                "frac": round(dom_tf / PEAK_FP64, 4), "traffic": None, "kernel": dom,
                "note": "exact tier on FP64 matrix cores; peak is the FP64 (vector = matrix) rate"}

    result = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f64+bf16", "data": "synthetic",
        "config": {"workload": "GPT-2-124M MLP linears (c_fc 768->3072, c_proj 3072->768), 8192 tokens, "
                               "bf16 storage, fwd+dX+dW, exact tier then fast tier (12 GEMMs per step)",
                   "tokens": TOKENS, "layers": [list(l) for l in LAYERS]},
        "tiers": {"exact": tier_stats("exact", PEAK_FP64), "fast": tier_stats("fast", PEAK_BF16)},
        "per_gemm": per,
        "roofline": roofline,
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(data, args.cpu_seconds)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
