"""Build libmxattn.so in-tree with hipcc for gfx950.

    python -m block_scaled_mxfp8_amd.build [--verbose] [--variant max-ilp]

All HIP sources under csrc/ are compiled into one shared library next to this file. Packed
FP32 instructions are disabled for the device code (-packed-fp32-ops); the host pass of
hipcc warns that it does not know that target feature, which is harmless. MFMA accumulators
are kept in the VGPR form (-amdgpu-mfma-vgpr-form): left to its heuristic, the backend put the
backward's dK/dV accumulators in AGPRs and copied them to VGPRs and back around every MFMA
(~450 v_accvgpr moves per 64-query step).
"""
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmxattn.so")

# Builds of the same sources under another instruction scheduler, loaded only by tests: the
# kernels' counted memory waits must not depend on the order a scheduler picks (LLVM's max-ilp
# scheduler once hoisted the dQ-from-store kernel's dS loads above its K-tile LDS-DMA).
VARIANTS = {"max-ilp": ("libmxattn_maxilp.so", ("-mllvm", "-amdgpu-sched-strategy=max-ilp"))}


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmxattn)")


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose=False, out=LIB, extra=(), info=True):
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form=1",
           "-Wno-unused-command-line-argument",
           "-I", os.path.join(ROOT, "include"), *extra, *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(line for line in (res.stdout + res.stderr).splitlines() if noise not in line and "(ignoring feature)" not in line)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msgs)
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, out)
    if info:
        write_build_info(os.path.join(HERE, "build_info.json"))
    return out


def build_variant(name, verbose=False):
    """Build one of VARIANTS next to the library (its own file; build_info.json is untouched)."""
    fname, extra = VARIANTS[name]
    return build(verbose, os.path.join(HERE, fname), extra, info=False)


def write_build_info(path):
    """Identity of this build (read by the benchmark): git revision of the tree, hipcc version,
    hash of the sources compiled."""
    import hashlib
    import json
    h = hashlib.sha256()
    for src in sorted(glob.glob(os.path.join(HERE, "csrc", "*"))):
        with open(src, "rb") as f:
            h.update(os.path.relpath(src, ROOT).encode() + b"\0" + f.read())
    def run(cmd):
        try:
            return subprocess.run(cmd, capture_output=True, text=True, cwd=ROOT, timeout=30).stdout.strip()
        except Exception:  # noqa: BLE001 - informational
            return None
    git = run(["git", "rev-parse", "--short=12", "HEAD"])
    if git and run(["git", "status", "--porcelain", "--", "block_scaled_mxfp8_amd", "include"]):
        git += "+uncommitted"
    hip = run([hipcc(), "--version"])
    info = {"git": git, "hipcc": hip.splitlines()[0] if hip else None, "source_sha256": h.hexdigest()}
    with open(path, "w") as f:
        json.dump(info, f)


if __name__ == "__main__":
    if "--variant" in sys.argv:
        print(build_variant(sys.argv[sys.argv.index("--variant") + 1], verbose="--verbose" in sys.argv))
    else:
        print(build(verbose="--verbose" in sys.argv))
