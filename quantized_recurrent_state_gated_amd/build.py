"""Build libsq.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m quantized_recurrent_state_gated_amd.build [-v]

Packed-FP32 instructions are disabled for all device code.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libsq.so")
SOURCES = ["sq_kernels.hip", "sq_api.hip"]
ARCH = os.environ.get("SQ_OFFLOAD_ARCH", "gfx950")


def hipcc_cmd(out: str) -> list:
    return (["/opt/rocm/bin/hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             "-shared", "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-o", out] + [os.path.join(CSRC, s) for s in SOURCES])


def build(verbose: bool = False) -> str:
    cmd = hipcc_cmd(OUT + ".tmp")
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
