"""Build the HIP library libmamba_scan.so in-tree, for gfx950 only.

Each translation unit is compiled to an object on its own, in parallel,
and the objects are linked into one shared library. The chunked-scan
kernels are compiled eight times from scan_variant.hip, once per
(I/O dtype, delta softplus, half of the dstate range).
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libmamba_scan.so")
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

# (object name, source, extra defines)
UNITS = [("api", "api.cpp", ()), ("noalloc", "noalloc.hip", ()), ("launch", "launch.hip", ()),
         ("conv1d", "conv1d.hip", ()),
         ("scan_bwd", "scan_bwd.hip", ()), ("ssd", "ssd.hip", ())] + [
    (f"scan_io{io}_sp{sp}_n{part}", "scan_variant.hip",
     (f"-DMAMBA_VARIANT_IO={io}", f"-DMAMBA_VARIANT_SP={sp}", f"-DMAMBA_VARIANT_PART={part}"))
    for io in (0, 1) for sp in (0, 1) for part in (0, 1)]


def hipcc():
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _flags(extra):
    # Packed fp32 VALU forms are switched off (-packed-fp32-ops) so the
    # compiler emits only scalar fp32 vector instructions.
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{INCLUDE}", f"-I{CSRC}", *extra]


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "is not a recognized feature for this target"
    out = "\n".join(l for l in res.stdout.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    return out


def compile_library(output=LIBRARY, extra=(), jobs=None):
    """Compile every unit (in parallel) and link them into `output`; returns
    its path. `extra` flags go to every compile."""
    build_dir = os.path.join(os.path.dirname(os.path.abspath(output)), "_build")
    os.makedirs(build_dir, exist_ok=True)
    tag = os.path.basename(output).replace(".", "_")
    objs = []
    cmds = []
    for name, src, defs in UNITS:
        obj = os.path.join(build_dir, f"{tag}_{name}.o")
        objs.append(obj)
        cmds.append([hipcc(), *_flags(list(extra) + list(defs)), "-c", os.path.join(CSRC, src),
                     "-o", obj])
    jobs = jobs or min(len(cmds), max(1, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        list(pool.map(_run, cmds))
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", output + ".tmp"])
    os.replace(output + ".tmp", output)
    return output


if __name__ == "__main__":
    print(compile_library())
