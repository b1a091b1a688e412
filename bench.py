"""Benchmark of the deterministic GEMM hot path on one MI355X.

One step = one training pass of the GPT-2-124M MLP linears at 8192 tokens
(c_fc 768->3072 and c_proj 3072->768, bf16 storage): forward, dX and dW of
both layers, through the exact tier (float64 tiles + Neumaier) and then the
fast tier (bf16 matrix cores, f32 accumulate): 12 GEMM launches, all inputs
resident in HBM before the timed region.

Prints one JSON line. `value` is useful TFLOP/s of the whole step
(2*M*N*K per GEMM over the step time); per-tier and per-op rates, the
roofline of the dominant kernel (measured with HIP events on the stream the
kernels run on; its HBM traffic comes from the committed counter summary
under profiles/ while the kernel source is unchanged), skinny-M forward
bandwidth and the CPU oracle's rate on a bounded sample are included.

Per launch the mean time gives the reported rate (median and minimum beside
it); the SHA-256 of every output is recorded, and each tier is also stated as
a fraction of the peak the library's own microkernels measure on the same GPU. For context only, the vendor
BLAS behind torch.matmul is timed on the same tensors (it carries no
determinism contract and is not the product path).

Profiling aids (not part of the measured step): --only tier.op runs just
those launches, --copy-mib N times a plain device copy of N MiB, the known
size against which memory counters are scaled.
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
PEAK_INT8 = 5033.2    # TOP/s, MI355X dense int8 MFMA
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
    p.add_argument("--cpu-full", action="store_true",
                   help="time the oracle on configs 1-4 in full (several minutes) instead of the bounded sample")
    p.add_argument("--no-skinny", action="store_true", help="skip the skinny-M bandwidth measurements")
    p.add_argument("--skinny-only", action="store_true",
                   help="profiling aid: only the skinny-M measurements (one JSON line)")
    p.add_argument("--skinny-light", action="store_true", help="a tenth of the skinny-M calls (for runs under a profiler)")
    p.add_argument("--no-vendor", action="store_true", help="skip the vendor-BLAS context timings")
    p.add_argument("--no-peak", action="store_true", help="skip the measured-peak microkernels")
    p.add_argument("--shapes", action="store_true",
                   help="instead of the step: fwd/dX/dW in both tiers on the other workloads' shapes (one JSON line)")
    p.add_argument("--no-next", action="store_true",
                   help="skip the bias-gradient, f32-dW and LayerNorm measurements")
    p.add_argument("--only", default=None,
                   help="profiling aid: run only the launches of one tier and op (e.g. exact.dw, cr.fwd) and print their times")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="profiling aid: time a plain device copy of this many MiB instead (counter calibration)")
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


def launches(data, only=None):
    """The step as a list of (tier, layer, op, callable); `only` = "tier.op" keeps those launches
    (tier "cr", the correctly rounded tier, is not part of the step: profiling only)."""
    import deterministic_invariant_gemm_det_amd as dg
    out = []
    for tier in ("exact", "fast") + (("cr",) if only and only.startswith("cr.") else ()):
        for name, _, _ in LAYERS:
            d = data[name]
            out.append((tier, name, "fwd", lambda d=d, t=tier: dg.fwd(d["x"], d["w"], None, t, out=d["y"])))
            out.append((tier, name, "dx", lambda d=d, t=tier: dg.dx(d["g"], d["w"], t, out=d["gx"])))
            out.append((tier, name, "dw", lambda d=d, t=tier: dg.dw(d["x"], d["g"], t, out=d["gw"])))
    if only:
        out = [l for l in out if f"{l[0]}.{l[2]}" == only]
        if not out:
            raise SystemExit(f"bench.py: --only {only!r} matches no launch (use tier.op, e.g. exact.dw)")
    return out


def time_launches(steps, n_steps, warmup, stream):
    """Warm up, then time n_steps passes over `steps` with an event pair around
    every launch and one around the whole region, all on `stream`."""
    import torch
    for _ in range(warmup):
        for _, _, _, f in steps:
            f()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in steps]
          for _ in range(n_steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(n_steps):
        for i, (_, _, _, f) in enumerate(steps):
            ev[s][i][0].record(stream)
            f()
            ev[s][i][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    per_launch_ms = [[ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(n_steps)] for i in range(len(steps))]
    return t_start.elapsed_time(t_end), per_launch_ms


# Kernel sources whose HBM traffic the stored counter summary describes; the
# stored figure is reported only while these files are unchanged.
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "exact_dw_bf16_gpt2mlp_8192tok_traffic.md")
TRAFFIC_SOURCES = ("deterministic_invariant_gemm_det_amd/csrc/exact.hip",
                   "deterministic_invariant_gemm_det_amd/csrc/common.hpp")


def sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration),
    or None when the summary is missing or the kernel source changed since."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            text = f.read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        line = line.strip().lstrip("-* ").replace("`", "")
        if ":" in line:
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    if fields.get("kernel_sources_sha256") != sources_sha256():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(dev, mib, n_steps, warmup):
    """A plain device-to-device copy of known size, for scaling memory counters."""
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    steps = [("copy", "copy", "copy", lambda: dst.copy_(src))]
    total_ms, per = time_launches(steps, n_steps, warmup, stream)
    ms = sum(per[0]) / len(per[0])
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "us_per_copy": round(ms * 1e3, 2),
                      "GB_per_s": round(2 * n / (ms * 1e-3) / 1e9, 1)}))


def skinny(data, dev, light=False):
    """Skinny-M forward, both tiers: M = 1, 3, 17 (the first rows of the c_fc
    input, k=768, n=3072) and M = 1 on c_proj (k=3072, n=768). Achieved GB/s of
    algorithmic bytes (x, w and y once each):
      warm:  a HIP graph of 50 back-to-back calls replayed (the weight stays in
             the last-level cache between calls; no host call overhead);
      eager: 200 back-to-back calls through the Python binding (host-paced
             when the kernel is shorter than the call);
      cold:  one call after a 512 MiB buffer is written, so the weight comes
             from HBM (median of 20).
    light: a tenth of the calls (for runs under a profiler)."""
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    out = {}
    cases = [("c_fc", m) for m in (1, 3, 17)] + [("c_proj", 1)]
    for layer, m in cases:
        d = data[layer]
        k, n = d["k"], d["n"]
        x = d["x"][:m].clone()
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        algo_bytes = 2 * (m * k + k * n + m * n)
        for tier in ("exact", "fast"):
            f = lambda: dg.fwd(x, d["w"], None, tier, out=y)
            n_eager, n_graph, n_replay, n_cold = (20, 10, 2, 5) if light else (200, 50, 4, 20)
            side = torch.cuda.Stream(dev)
            side.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.stream(side):
                for _ in range(5):
                    f()
                side.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(side)
                for _ in range(n_eager):
                    f()
                e1.record(side)
                side.synchronize()
                eager_us = e0.elapsed_time(e1) * 1e3 / n_eager
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    for _ in range(n_graph):
                        f()
                g.replay()
                side.synchronize()
                e0.record(side)
                for _ in range(n_replay):
                    g.replay()
                e1.record(side)
                side.synchronize()
                warm_us = e0.elapsed_time(e1) * 1e3 / (n_graph * n_replay)
                cold = []
                for _ in range(n_cold):
                    flush.fill_(7)
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(side)
                    f()
                    b.record(side)
                    side.synchronize()
                    cold.append(a.elapsed_time(b) * 1e3)
            del g
            cold_us = sorted(cold)[len(cold) // 2]
            gbps = lambda us: round(algo_bytes / (us * 1e-6) / 1e9, 1)
            key = f"{tier}.M{m}" if layer == "c_fc" else f"{tier}.{layer}.M{m}"
            out[key] = {"us_warm": round(warm_us, 2), "GBps_warm": gbps(warm_us),
                        "us_eager": round(eager_us, 2), "GBps_eager": gbps(eager_us),
                        "us_cold": round(cold_us, 2), "GBps_cold": gbps(cold_us),
                        "algo_bytes": algo_bytes, "k": k, "n": n}
    return out


PEAK_HBM = 8000.0   # GB/s, MI355X HBM3E


def _time_calls(f, stream, reps=50, warmup=5):
    """Average microseconds per call of f, HIP events on `stream` around `reps` back-to-back calls."""
    import torch
    for _ in range(warmup):
        f()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        f()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def next_rows(data, dev):
    """The ops beside the GEMMs, on the step's own tensors: the bias gradient of both layers
    (f32 out), dW of c_fc written as f32 in both tiers, and the GPT-2 LayerNorm (8192 x 768,
    bf16, float64 statistics) forward and backward. HBM-bound ops report GB/s of algorithmic
    bytes against the HBM peak."""
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    stream = torch.cuda.current_stream(dev)
    out = {}

    def hbm(us, nbytes):
        gbps = nbytes / (us * 1e-6) / 1e9
        return {"us": round(us, 2), "algo_bytes": nbytes,
                "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM, "unit": "GB/s",
                             "frac": round(gbps / PEAK_HBM, 4)}}

    for name, k, n in LAYERS:
        g = data[name]["g"]
        db = torch.empty(n, dtype=torch.float32, device=dev)
        us = _time_calls(lambda: dg.db(g, "exact", out=db, out_dtype=torch.float32), stream)
        out[f"db.{name}"] = hbm(us, TOKENS * n * 2 + n * 4)
    d = data["c_fc"]
    gw32 = torch.empty((d["k"], d["n"]), dtype=torch.float32, device=dev)
    fl = 2.0 * TOKENS * d["k"] * d["n"]
    for tier, peak in (("exact", PEAK_FP64), ("fast", PEAK_BF16)):
        us = _time_calls(lambda: dg.dw(d["x"], d["g"], tier, out=gw32, out_dtype=torch.float32), stream, reps=10)
        tf = fl / (us * 1e-6) / 1e12
        out[f"dw_f32.c_fc.{tier}"] = {"us": round(us, 2), "tflops": round(tf, 2),
                                      "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": peak,
                                                   "unit": "TFLOP/s", "frac": round(tf / peak, 4)}}
    # The correctly rounded tier on c_fc: tflops = useful 2MNK rate; the roofline is the int8
    # matrix work its 7-bit slice path issues (every 64 x 64 tile of these operands takes it).
    xb = d["x"].view(torch.int16).cpu().numpy().view("uint16")              # [m][k]
    wb = d["w"].view(torch.int16).cpu().numpy().view("uint16")              # [k][n]
    gb = d["g"].view(torch.int16).cpu().numpy().view("uint16")              # [m][n]
    int8_ops = {"fwd": cr_int8_ops(xb, wb.T.copy(), d["k"]),                 # X rows, W columns
                "dx": cr_int8_ops(gb, wb, d["n"]),                           # dY rows, W rows
                "dw": cr_int8_ops(xb.T.copy(), gb.T.copy(), TOKENS)}         # X columns, dY columns
    for op, f in (("fwd", lambda: dg.fwd(d["x"], d["w"], None, "cr", out=d["y"])),
                  ("dx", lambda: dg.dx(d["g"], d["w"], "cr", out=d["gx"])),
                  ("dw", lambda: dg.dw(d["x"], d["g"], "cr", out=d["gw"]))):
        us = _time_calls(f, stream, reps=10, warmup=2)
        tf = fl / (us * 1e-6) / 1e12
        tops = int8_ops[op] / (us * 1e-6) / 1e12
        out[f"cr.c_fc.{op}"] = {"us": round(us, 2), "tflops": round(tf, 2), "int8_ops": int8_ops[op],
                                "roofline": {"bound": "mfma", "achieved": round(tops, 2), "peak": PEAK_INT8,
                                             "unit": "TOP/s", "frac": round(tops / PEAK_INT8, 4)}}
    h = 768
    x = data["c_fc"]["x"]                      # 8192 x 768 bf16
    gy = data["c_proj"]["g"]                   # 8192 x 768 bf16, the LayerNorm's incoming gradient
    gamma = torch.ones(h, dtype=torch.bfloat16, device=dev).add_(x[0] * 0.01)
    beta = (x[1] * 0.1).contiguous()
    y = torch.empty_like(x)
    _, mean, rstd = dg.layer_norm(x, gamma, beta, 1e-5, out=y)
    us = _time_calls(lambda: dg.layer_norm(x, gamma, beta, 1e-5, out=y), stream)
    out["layernorm_fwd.8192x768"] = hbm(us, 2 * TOKENS * h * 2 + 2 * h * 2 + 16 * TOKENS)
    us = _time_calls(lambda: dg.layer_norm_backward(gy, x, mean, rstd, gamma, param_dtype=torch.float32), stream)
    out["layernorm_bwd.8192x768"] = hbm(us, 3 * TOKENS * h * 2 + 16 * TOKENS + h * 2 + 2 * h * 4)
    return out


def cr_int8_ops(a_rows, b_cols, red):
    """Integer operations the correctly rounded tier's int8 path issues for bf16 operands given as
    uint16 bit arrays a_rows[rows][red] and b_cols[cols][red] (each reduction line contiguous):
    2 * 64 * 64 * kp per slice pair of every 64 x 64 tile that path takes (kp = red rounded up to
    128; a line needs (top - low) // 7 + 1 slices of 7 bits, a tile the most of its lines, at
    most five each side)."""
    import numpy as np

    def slices(bits):
        b = bits.astype(np.int32)
        e, f = (b >> 7) & 0xff, b & 0x7f
        sig = np.where(e > 0, f | 0x80, f)
        lsb = np.where(e > 0, e - 134, -133)
        nz = sig > 0
        hi = np.where(nz, lsb + np.floor(np.log2(np.maximum(sig, 1))).astype(np.int32), -(1 << 20))
        ctz = np.log2(sig & -sig, where=nz, out=np.zeros(sig.shape)).astype(np.int32)
        lo = np.where(nz, lsb + ctz, 1 << 20)
        top, low = hi.max(axis=1), lo.min(axis=1)
        n = np.where(top > -(1 << 20), (top - low) // 7 + 1, 0)
        pad = (-len(n)) % 64
        return np.pad(n, (0, pad)).reshape(-1, 64).max(axis=1)

    la, lb = slices(a_rows), slices(b_cols)
    ok_a, ok_b = la <= 5, lb <= 5
    kp = (red + 127) // 128 * 128
    pairs = float((la * ok_a).sum()) * float((lb * ok_b).sum())
    return 2.0 * 64 * 64 * kp * pairs


def output_hashes(data, steps):
    """SHA-256 (first 16 hex digits) of every GEMM output of one more pass of the step, so runs
    on different machines and days can be compared bit for bit."""
    import hashlib
    import torch
    out = {}
    for tier, name, op, f in steps:
        f()
        t = data[name][{"fwd": "y", "dx": "gx", "dw": "gw"}[op]]
        torch.cuda.synchronize()
        out[f"{tier}.{name}.{op}"] = hashlib.sha256(t.view(torch.int16).cpu().numpy().tobytes()).hexdigest()[:16]
    return out


def host_cpu():
    """The host's CPU model name and logical CPU count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count()


SWEEP = (("gpt2_qkv", "bf16", 8192, 768, 2304), ("gpt2_attn_proj", "bf16", 8192, 768, 768),
         ("gpt2_c_fc", "bf16", 8192, 768, 3072), ("gpt2_c_proj", "bf16", 8192, 3072, 768),
         ("f32_4096", "f32", 4096, 4096, 4096), ("bf16_up", "bf16", 4096, 4096, 11008),
         ("bf16_down", "bf16", 4096, 11008, 4096))
PEAKS = {("exact", "bf16"): PEAK_FP64, ("exact", "f32"): PEAK_FP64, ("fast", "bf16"): PEAK_BF16,
         ("fast", "f32"): 157.3}


def shape_sweep(dev):
    """fwd, dX and dW in both tiers on the other workloads' shapes (M x K x N): mean microseconds
    per launch (HIP events around back-to-back calls on the current stream), TFLOP/s and the
    fraction of the tier's peak for the dtype (FP64 for the exact tier; bf16 or FP32 matrix
    peak for the fast tier)."""
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    stream = torch.cuda.current_stream(dev)
    out = {}
    for name, dt, m, k, n in SWEEP:
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        g0 = torch.Generator(device=dev)
        g0.manual_seed(42)
        x = torch.randn(m, k, device=dev, generator=g0).to(tdt)
        w = (torch.randn(k, n, device=dev, generator=g0) * 0.02).to(tdt)
        g = torch.randn(m, n, device=dev, generator=g0).to(tdt)
        y, gx, gw = (torch.empty(m, n, device=dev, dtype=tdt), torch.empty(m, k, device=dev, dtype=tdt),
                     torch.empty(k, n, device=dev, dtype=tdt))
        fl = 2.0 * m * k * n
        for tier in ("exact", "fast"):
            for op, f in (("fwd", lambda: dg.fwd(x, w, None, tier, out=y)), ("dx", lambda: dg.dx(g, w, tier, out=gx)),
                          ("dw", lambda: dg.dw(x, g, tier, out=gw))):
                reps = 3 if tier == "exact" else 20
                us = _time_calls(f, stream, reps=reps, warmup=1)
                tf = fl / (us * 1e-6) / 1e12
                out[f"{name}.{tier}.{op}"] = {"mkn": [m, k, n], "dtype": dt, "us": round(us, 1), "tflops": round(tf, 1),
                                              "frac_of_peak": round(tf / PEAKS[(tier, dt)], 4)}
                print(f"{name} {tier} {op}: {us:.1f} us {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)
        del x, w, g, y, gx, gw
    return out


def vendor_context(data, dev, fast_per):
    """Context only, not the product path: the vendor BLAS behind torch.matmul (hipBLASLt)
    on the step's own bf16 tensors in their natural layouts (X @ W, dY @ W^T, X^T @ dY, the
    transposes as views), with no determinism or batch-invariance contract. Each fast-tier
    launch's time is reported beside it."""
    import torch
    stream = torch.cuda.current_stream(dev)
    out = {}
    for name, k, n in LAYERS:
        d = data[name]
        x, w, g = d["x"], d["w"], d["g"]
        fl = 2.0 * TOKENS * k * n
        for op, f in (("fwd", lambda: torch.matmul(x, w)), ("dx", lambda: torch.matmul(g, w.t())),
                      ("dw", lambda: torch.matmul(x.t(), g))):
            us = _time_calls(f, stream)
            ours = fast_per[f"fast.{name}.{op}"]["us"]
            out[f"{name}.{op}"] = {"us": round(us, 2), "tflops": round(fl / (us * 1e-6) / 1e12, 1),
                                   "fast_tier_us": ours, "fast_over_vendor_time": round(ours / us, 3)}
    tot_v = sum(v["us"] for v in out.values())
    tot_f = sum(v["fast_tier_us"] for v in out.values())
    out["total"] = {"us": round(tot_v, 1), "fast_tier_us": round(tot_f, 1), "fast_over_vendor_time": round(tot_f / tot_v, 3)}
    return out


CONFIG4 = (("qkv", 768, 2304), ("attn_proj", 768, 768), ("c_fc", 768, 3072), ("c_proj", 3072, 768))


def cpu_baseline(budget_s, full=False):
    """The oracle, as it stands, single-threaded on this host, on the workloads' own inputs.

    Bounded (default, about budget_s seconds): config 1 (f32 256 x 512 x 512 fwd, dX, dW) and
    one training step of config 3 (the f32 MLP) in full, config 2's forward at M = 1, 3, 17 in
    full (f32 and bf16), and output rows of config 4's twelve bf16 GEMMs (the four GPT-2 linears
    at 8192 tokens, fwd/dX/dW) for equal shares of the rest of the budget. full=True times
    configs 1 to 4 in full instead: all 50 MLP steps, every M prefix of config 2, every output
    of config 4 (several minutes; progress on stderr). `value` is config 4's useful rate
    (2*M*N*K flops per second over the rows done)."""
    import numpy as np
    import oracle
    import synthetic as syn
    from oracle import mlp

    per = {}

    def record(key, flops, secs, note=None):
        per[key] = {"gflop": round(flops / 1e9, 4), "s": round(secs, 3), "gflops": round(flops / secs / 1e9, 3)}
        if note:
            per[key]["rows"] = note
        if full:
            print(f"cpu_baseline {key}: {secs:.1f} s", file=sys.stderr, flush=True)

    def timed(f):
        t0 = time.perf_counter()
        f()
        return time.perf_counter() - t0

    t_all = time.perf_counter()
    # config 1: f32, M=256, K=512, N=512, seed 42
    m, k, n = 256, 512, 512
    X = syn.normal(42, syn.TID_X, (m, k))
    W = syn.normal(42, syn.TID_W, (k, n))
    b = syn.normal(42, syn.TID_B, (n,), sigma=0.1)
    G = syn.normal(42, syn.TID_DY, (m, n))
    record("cfg1.fwd", 2.0 * m * k * n, timed(lambda: oracle.fwd("f32", X, W, b)))
    record("cfg1.dx", 2.0 * m * k * n, timed(lambda: oracle.dx("f32", G, W)))
    record("cfg1.dw", 2.0 * m * k * n, timed(lambda: oracle.dw("f32", X, G)))

    # config 3: the f32 MLP (seed 42), one step or all 50
    widths, batch = syn.MLP_WIDTHS, syn.MLP_BATCH
    layers = list(zip(widths[:-1], widths[1:]))
    step_flops = sum(2.0 * batch * i * o * 2 + 2.0 * batch * o for i, o in layers)   # fwd, dW, db
    step_flops += sum(2.0 * batch * i * o for i, o in layers[1:])                      # dX below layer 1
    steps = 50 if full else 1

    def train():
        params = syn.mlp_init(42)
        for s_ in range(steps):
            Xs, Ts = syn.mlp_batch(42, s_)
            params, _ = mlp.step(params, Xs, Ts)
    record("cfg3.mlp_steps", step_flops * steps, timed(train), note=f"{steps} of 50 steps")

    # config 2: forward of the M prefixes of an 8192-row X, K=768, N=3072, f32 and bf16
    for dt in ("f32", "bf16"):
        X8 = syn.normal(42, syn.TID_X, (8192, 768), dt=dt)
        W2 = syn.normal(42, syn.TID_W, (768, 3072), sigma=0.02, dt=dt)
        for M in (1, 3, 17, 64, 127, 512, 2048, 8192):
            if full or M <= 17:
                record(f"cfg2.{dt}.M{M}", 2.0 * M * 768 * 3072, timed(lambda: oracle.fwd(dt, X8[:M], W2)))

    # config 4: GPT-2 linears at 8192 tokens, bf16, seed 42
    spent = time.perf_counter() - t_all
    share = max(0.2, (budget_s - spent) / 12.0)
    flops4, secs4 = 0.0, 0.0
    for name, k, n in CONFIG4:
        m = TOKENS
        X = syn.normal(42, syn.TID_X, (m, k), dt="bf16")
        W = syn.normal(42, syn.TID_W, (k, n), sigma=0.02, dt="bf16")
        G = syn.normal(42, syn.TID_DY, (m, n), dt="bf16")
        for op in OPS:
            A, B = {"fwd": (X, W), "dx": (G, W), "dw": (X, G)}[op]
            out_rows = k if op == "dw" else m
            row_flops = 2.0 * m * k * n / out_rows
            if full:
                secs = timed(lambda: oracle.gemm(op, "bf16", A, B, m, k, n))
                done = out_rows
            else:
                # one call, as in the full run (the oracle upcasts the other operand once per
                # call), with as many rows as fill the share at about 1.5 GFLOP/s
                done = int(max(1, min(out_rows, share * 1.5e9 / row_flops)))
                rows = np.arange(done, dtype=np.int64)
                secs = timed(lambda: oracle.gemm(op, "bf16", A, B, m, k, n, rows=rows))
            record(f"cfg4.{name}.{op}", row_flops * done, secs, note=f"{done} of {out_rows}")
            flops4 += row_flops * done
            secs4 += secs
    total = time.perf_counter() - t_all
    model, ncpu = host_cpu()
    what = ("configs 1-4 in full" if full else
            "config 1 and one config-3 step in full, config 2 at M=1,3,17 in full, output rows of config 4's "
            "twelve GEMMs")
    return {"value": flops4 / secs4 / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "host_cpu": model, "host_logical_cpus": ncpu,
            "sample": f"{what}; single-threaded, {total:.1f} s; value = config 4's useful 2*M*N*K flops per second",
            "per_workload": per}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: only one GPU is used here (asked for {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    dev = torch.device("cuda:0")
    if args.copy_mib:
        copy_calibration(dev, args.copy_mib, args.steps, args.warmup)
        return
    if args.shapes:
        print(json.dumps({"shape_sweep": shape_sweep(dev)}))
        return
    data = make_inputs(dev)
    if args.skinny_only:
        print(json.dumps({"skinny_fwd_bf16": skinny(data, dev, light=args.skinny_light)}))
        return
    steps = launches(data, args.only)
    stream = torch.cuda.current_stream(dev)
    total_ms, per_launch_ms = time_launches(steps, args.steps, args.warmup, stream)
    ms_step = total_ms / args.steps

    # per launch: mean over the timed steps (the figure rocprofv3's average duration
    # is compared with), median and minimum beside it
    per = {}
    for i, (tier, name, op, _) in enumerate(steps):
        times = sorted(per_launch_ms[i])
        h = len(times) // 2
        med = times[h] if len(times) % 2 else 0.5 * (times[h - 1] + times[h])
        mean = sum(times) / len(times)
        k, n = data[name]["k"], data[name]["n"]
        fl = 2.0 * TOKENS * k * n
        per[f"{tier}.{name}.{op}"] = {"us": round(mean * 1e3, 2), "tflops": round(fl / (mean * 1e-3) / 1e12, 2),
                                      "us_median": round(med * 1e3, 2), "us_min": round(times[0] * 1e3, 2),
                                      "tflops_median": round(fl / (med * 1e-3) / 1e12, 2)}
    if args.only:
        print(json.dumps({"only": args.only, "steps": args.steps, "warmup": args.warmup, "per_gemm": per}))
        return

    def tier_stats(tier, peak):
        keys = [k for k in per if k.startswith(tier + ".")]
        fl = sum(2.0 * TOKENS * data[k.split(".")[1]]["k"] * data[k.split(".")[1]]["n"] for k in keys)
        us = sum(per[k]["us"] for k in keys)
        us_med = sum(per[k]["us_median"] for k in keys)
        tf, tf_med = fl / (us * 1e-6) / 1e12, fl / (us_med * 1e-6) / 1e12
        return {"tflops": round(tf, 2), "pct_of_peak": round(100 * tf / peak, 2), "peak_tflops": peak, "us": round(us, 1),
                "tflops_median": round(tf_med, 2), "pct_of_peak_median": round(100 * tf_med / peak, 2)}

    total_flops = 2 * sum(2.0 * TOKENS * k * n * len(OPS) for _, k, n in LAYERS)
    value = total_flops / (ms_step * 1e-3) / 1e12

    # Dominant kernel: the exact-tier dW kernel (its two launches, c_fc and
    # c_proj, are one kernel with the same flops and the largest share of the
    # step). achieved = algorithmic flops per launch / its average launch time.
    dom = [k for k in per if k.startswith("exact.") and k.endswith(".dw")]
    dom_us = sum(per[k]["us"] for k in dom) / len(dom)
    dom_flops = 2.0 * TOKENS * LAYERS[0][1] * LAYERS[0][2]
    dom_tf = dom_flops / (dom_us * 1e-6) / 1e12
    roofline = {"bound": "mfma", "achieved": round(dom_tf, 2), "peak": PEAK_FP64, "unit": "TFLOP/s",
                "frac": round(dom_tf / PEAK_FP64, 4), "traffic": stored_traffic(),
                "kernel": "exact_m16s_kernel<BF16, 48-row blocks, dW> (exact.c_fc.dw, exact.c_proj.dw)",
                "avg_launch_us": round(dom_us, 2), "flops_per_launch": dom_flops,
                "note": "exact tier on FP64 matrix cores (V_MFMA_F64_16X16X4); peak is MI355X FP64 (vector = matrix)"}
    fast = tier_stats("fast", PEAK_BF16)
    roofline_fast = {"bound": "mfma", "achieved": fast["tflops"], "peak": PEAK_BF16, "unit": "TFLOP/s",
                     "frac": round(fast["tflops"] / PEAK_BF16, 4), "traffic": None,
                     "kernel": "fast tier, all six launches (eight-wave bf16 MFMA 32x32x16 kernel, f32 accumulate; dW split into shape-fixed chunks plus an ordered combine)"}

    result = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f64+bf16", "data": "synthetic",
        "config": {"workload": "GPT-2-124M MLP linears (c_fc 768->3072, c_proj 3072->768), 8192 tokens, "
                               "bf16 storage, fwd+dX+dW, exact tier then fast tier (12 GEMMs per step)",
                   "tokens": TOKENS, "layers": [list(l) for l in LAYERS]},
        "tiers": {"exact": tier_stats("exact", PEAK_FP64), "fast": fast},
        "per_gemm": per,
        "roofline": roofline,
        "roofline_fast": roofline_fast,
    }
    result["output_sha256"] = output_hashes(data, steps)
    if not args.no_peak:
        from deterministic_invariant_gemm_det_amd import peak as dpeak
        peaks = {"fp64_mfma_4x4x4": round(dpeak.measure(0, 4000), 2), "fp64_fma_valu": round(dpeak.measure(1, 4000), 2),
                 "bf16_mfma_32x32x16": round(dpeak.measure(2, 2000), 2), "unit": "TFLOP/s",
                 "note": "peak-rate microkernels (libdetpeak.so) at the GPU's running clock (no memory traffic)"}
        result["measured_peak"] = peaks
        result["tiers"]["exact"]["pct_of_measured_peak"] = round(100 * result["tiers"]["exact"]["tflops"] / peaks["fp64_mfma_4x4x4"], 2)
        result["tiers"]["fast"]["pct_of_measured_peak"] = round(100 * result["tiers"]["fast"]["tflops"] / peaks["bf16_mfma_32x32x16"], 2)
    if not args.no_skinny:
        result["skinny_fwd_bf16"] = skinny(data, dev, light=args.skinny_light)
    if not args.no_next:
        result["next_rows"] = next_rows(data, dev)
    if not args.no_vendor:
        result["vendor_blas_context"] = vendor_context(data, dev, per)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds, full=args.cpu_full)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
