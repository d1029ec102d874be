"""Build libkvq.so (HIP kernels for gfx950 + the C ABI host library) in place."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libkvq.so")
OBJDIR = os.path.join(HERE, "_build")

ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]
# The quantizer must round exactly like IEEE binary32: no contraction, and
# hipcc's default correctly rounded division is relied on.
SOURCES = {
    "kvq_append.hip": ["-ffp-contract=off"],
    # MFMA accumulators in ArchVGPRs: the softmax rescale multiplies them with
    # VALU, which otherwise costs AGPR<->VGPR copies every chunk
    "kvq_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
    "kvq_merge.hip": [],
    # KL terms are products and sums rounded one by one, as in the oracle
    "kvq_drift.hip": ["-ffp-contract=off"],
    "kvq_api.cpp": ["-ffp-contract=off"],
}


def _compile(src: str, extra: list[str], verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(x for x in r.stderr.splitlines() if noise not in x and x.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err and verbose:
        print(err, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda kv: _compile(kv[0], kv[1], verbose), SOURCES.items()))
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
