"""Builds libfa8.so (the C-ABI library with the gfx950 kernels) in-tree with hipcc."""
from __future__ import annotations

import json
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa8.so")
SOURCES = ["fa8_host.cpp", "fa8_kernels.hip", "fa8_quant.hip"]

# Packed-fp32 VALU forms are turned off for every HIP translation unit.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


# Per-lane scratch a kernel may use: a register or two spilled outside the tile loop is
# harmless, anything more means a template instance spills in its hot loop (or a helper became a
# real call with a stack frame) and the build fails.
MAX_SCRATCH_BYTES = 16
RESOURCES = os.path.join(PKG, "_build", "resource_usage.json")


def _resources(remarks: str) -> dict:
    """Kernel -> {VGPRs, AGPRs, ScratchSize, Occupancy, ...} from clang's kernel-resource-usage
    remarks."""
    out, cur = {}, None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+|True|False) \[", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return out


def _compile(src: str, obj: str, verbose: bool) -> dict:
    cmd = [hipcc()] + HIP_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return _resources(r.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source and link libfa8.so next to this file. Returns the library path."""
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        usage = {}
        for u in ex.map(lambda a: _compile(a[0], a[1], verbose), zip(SOURCES, objs)):
            usage.update(u)
    with open(RESOURCES, "w") as f:
        json.dump(usage, f, indent=1, sort_keys=True)
    bad = {k: v for k, v in usage.items()
           if int(v.get("ScratchSize", 0)) > MAX_SCRATCH_BYTES or v.get("Dynamic Stack") == "True"}
    if bad:
        raise RuntimeError("kernels using scratch memory (register spills or stack frames): " +
                           ", ".join(f"{k} ({v.get('ScratchSize')} B/lane)" for k, v in bad.items()))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
