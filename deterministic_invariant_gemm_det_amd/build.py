"""Build libdetgemm.so (the C-ABI HIP library) and libdetpeak.so (the
benchmark's peak-rate microkernels, a separate library) for gfx950 with hipcc.

Every source under csrc/ is compiled ahead of time for gfx950 only. Floating
point contraction is off (the exact tier's float64 operations are written out
one by one and must stay that way), and packed-f32 instructions are disabled.
"""
import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libdetgemm.so")
PEAK_LIB = os.path.join(HERE, "libdetpeak.so")
SOURCES = ["abi.cpp", "exact.hip", "fast.hip", "fast16.hip", "fast16w.hip", "colsum.hip", "layernorm.hip", "cr.hip",
           "noalloc.hip", "skinny.hip", "debug_round.hip"]
PEAK_SOURCES = ["peak.hip"]
# Per-source extra flags. The exact tier keeps matrix-core results in ordinary
# VGPRs: the Neumaier update reads every partial on the vector ALU, and the
# accumulator-register form would add a copy per partial.
EXTRA = {"exact.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src, build_dir):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(out=LIB, jobs=4, peak_out=PEAK_LIB):
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir), SOURCES + PEAK_SOURCES))
    _link(objs[:len(SOURCES)], out)
    _link(objs[len(SOURCES):], peak_out)
    return out


if __name__ == "__main__":
    print(build())
