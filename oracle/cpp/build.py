"""Build the C++ oracle (mx_oracle.cpp) into oracle/libmxoracle.so with g++ (C++17, OpenMP).

    python -m oracle.cpp.build

Test infrastructure: only tests/, the smoke check and the CPU baseline load the library.
No fast-math flags: the oracle's float64 and FP32 steps keep IEEE semantics.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(os.path.dirname(HERE), "libmxoracle.so")


def build(verbose=False, out=LIB):
    tmp = out + ".tmp"
    cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-fPIC", "-shared", "-Wall",
           os.path.join(HERE, "mx_oracle.cpp"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("g++ failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
