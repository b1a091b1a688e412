"""Build the CPU oracle's shared object (test infrastructure only).

The oracle is plain single-threaded C++17. It is compiled with contraction off
and without fast-math so that every float64 operation in it is the one written
in the source.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.cpp")
LIB = os.path.join(HERE, "liboracle.so")

FLAGS = ["-std=c++17", "-O2", "-mfma", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(out=LIB, compiler="g++", opt=None):
    """Compile oracle.cpp into `out` with `compiler` (g++ or clang++)."""
    flags = list(FLAGS)
    if opt is not None:
        flags = [f for f in flags if not f.startswith("-O")] + [opt]
    tmp = out + ".tmp"
    cmd = [compiler, *flags, SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
