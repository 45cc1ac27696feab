"""Build the HIP library libmamba_scan.so in-tree, for gfx950 only."""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libmamba_scan.so")
SOURCES = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "scan_kernels.hip")]
ARCH = "gfx950"


def hipcc():
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def compile_library(output=LIBRARY, extra=()):
    """Compile every source into one shared library and return its path.

    Packed fp32 VALU forms are switched off (-packed-fp32-ops) so the
    compiler emits only scalar fp32 vector instructions.
    """
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-function",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           f"-I{INCLUDE}", f"-I{CSRC}", *extra, *SOURCES, "-o", output + ".tmp"]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "is not a recognized feature for this target"
    out = "\n".join(l for l in res.stdout.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    os.replace(output + ".tmp", output)
    return output


if __name__ == "__main__":
    print(compile_library())
