"""Build ``libdp.so`` (the HIP kernels and the C ABI) for gfx950 with hipcc.

Each ``csrc/*.hip`` file is compiled to an object in parallel, then linked
into ``linear_rnn_sequence_amd/libdp.so`` (in-tree, so it travels with the
source tree).  All device code is built with packed-FP32 instructions
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdp.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the scans convert every accumulator tile
    # to an fp16 operand, which the accumulator-register form would copy first
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass reports the device-only feature flag as unknown: harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP source for gfx950 and link libdp.so (always rebuilds)."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
