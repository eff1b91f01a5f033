"""Build tests/abi_smoke (a plain C caller of libsq) with gcc, linking the HIP
runtime's C API and the in-tree libsq.so.  Called by __graft_entry__.build();
the GPU test runs the binary it leaves next to this file."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "abi_smoke.c")
OUT = os.path.join(HERE, "abi_smoke.bin")
LIBDIR = os.path.join(ROOT, "quantized_recurrent_state_gated_amd")


def cmd(out: str = OUT) -> list:
    return ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
            "-I/opt/rocm/include", SRC, "-o", out, "-L/opt/rocm/lib", "-lamdhip64",
            f"-L{LIBDIR}", "-lsq", f"-Wl,-rpath,{LIBDIR}", "-Wl,-rpath,/opt/rocm/lib", "-lm"]


def build(verbose: bool = False) -> str:
    if not os.path.exists(os.path.join(LIBDIR, "libsq.so")):
        raise RuntimeError("libsq.so is not built")
    c = cmd()
    if verbose:
        print(" ".join(c), flush=True)
    subprocess.run(c, check=True)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
