"""Build libapex4.so (HIP for gfx950) in-tree with hipcc.

    python -m w4a4_group_quantized_amd.build

Flags: correctly rounded fp32 division (the quantizer's codes depend on it),
no packed-fp32 instructions, -O3.  The library links only the HIP runtime.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libapex4.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str, bdir: str, defines: tuple, verbose: bool) -> str:
    obj = os.path.join(bdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *HIP_FLAGS, *[f"-D{d}" for d in defines], "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; anything else is shown
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if verbose:
        print(" ".join(cmd), flush=True)
        if msg.strip():
            print(msg)
    return obj


def build(verbose: bool = False, out: str | None = None, defines: tuple = ()) -> str:
    """Compile every source (in parallel) and link libapex4.so (or `out`, with extra -D defines)."""
    from concurrent.futures import ThreadPoolExecutor
    lib = out or LIB
    bdir = os.path.join(os.path.dirname(lib), "_build")
    os.makedirs(bdir, exist_ok=True)
    jobs = max(1, min(8, os.cpu_count() or 1))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, bdir, defines, verbose), sources()))
    tmp = lib + ".tmp"
    subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
