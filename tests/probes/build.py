"""Builds the test probes (tests/probes/*.hip) in-tree with hipcc for gfx950. Test
infrastructure: nothing in the library loads these."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
PROBES = {"mfma_dot.hip": "libmfma_dot.so", "mfma_acc.hip": "libmfma_acc.so"}


def build() -> None:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    hipcc = os.path.join(rocm, "bin", "hipcc")
    for src, lib in PROBES.items():
        out = os.path.join(HERE, lib)
        tmp = out + ".tmp"
        subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        os.path.join(HERE, src), "-o", tmp], check=True, capture_output=True)
        os.replace(tmp, out)


if __name__ == "__main__":
    build()
