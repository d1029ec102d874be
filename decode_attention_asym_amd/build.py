"""Build libkvq.so (HIP kernels for gfx950 + the C ABI host library) in place."""
from __future__ import annotations

import os
import re
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
    # VALU, which otherwise costs AGPR<->VGPR copies every chunk; the resource
    # remarks feed check_no_scratch
    "kvq_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true", "-Rpass-analysis=kernel-resource-usage"],
    "kvq_merge.hip": [],
    "kvq_noalloc.hip": [],
    # KL terms are products and sums rounded one by one, as in the oracle
    "kvq_drift.hip": ["-ffp-contract=off"],
    "kvq_api.cpp": ["-ffp-contract=off"],
}


def resource_usage(remarks: str) -> dict:
    """{kernel symbol: {field: value}} from hipcc's kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+(.+?): (\S+) \[-Rpass-analysis=kernel-resource-usage\]", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return out


def check_no_scratch(usage: dict) -> None:
    """The decode kernels wait for their LDS copies with static vmcnt counts
    that assume every vector-memory instruction in the chunk loop is one of
    those copies; a register spill (scratch loads and stores) would break the
    count and give wrong results without a fault.  Refuse such a build."""
    bad = []
    kernels = [k for k in usage if any(n in k for n in ("decode_kernel", "decode_mixed_kernel", "decode_fused_kernel"))]
    if not kernels:
        raise RuntimeError("no decode kernel resource remarks found (is -Rpass-analysis on?)")
    for k in kernels:
        u = usage[k]
        if u.get("ScratchSize [bytes/lane]") != "0" or u.get("VGPRs Spill") != "0" or u.get("SGPRs Spill") != "0":
            bad.append(f"{k}: scratch {u.get('ScratchSize [bytes/lane]')} B/lane, VGPR spill {u.get('VGPRs Spill')}, "
                       f"SGPR spill {u.get('SGPRs Spill')}")
    if bad:
        raise RuntimeError("decode kernels must not use scratch (their vmcnt waits count only the LDS copies):\n"
                           + "\n".join(bad))


def _compile(src: str, extra: list[str], verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    lines = [x for x in r.stderr.splitlines() if noise not in x and x.strip()]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(lines))
    if any("kernel-resource-usage" in x for x in lines):
        check_no_scratch(resource_usage(r.stderr))
        lines = [x for x in lines if "kernel-resource-usage" not in x]
    err = "\n".join(lines)
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
