"""Build the HIP library liblsq.so for gfx950 (in-tree, hipcc)."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblsq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# No fp contraction (every fused multiply-add in the kernels is an explicit
# fmaf, as the arithmetic contract requires), IEEE division, and packed fp32
# instructions disabled.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument", f"-I{os.path.join(ROOT, 'include')}"]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _headers() -> list[str]:
    return glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(ROOT, "include", "*.h"))


def _compile(src: str, incremental: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if incremental and os.path.exists(obj):
        t = os.path.getmtime(obj)
        if all(os.path.getmtime(d) < t for d in [src, __file__, *_headers()]):
            return obj
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = False, incremental: bool = False) -> str:
    """Compile every HIP/C++ source and link liblsq.so next to this file
    (incremental: skip objects newer than their source and every header)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda x: _compile(x, incremental), srcs))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def device_asm(src: str, out: str) -> None:
    """AMD assembly of one translation unit (for reading the generated ISA)."""
    cmd = [HIPCC, *FLAGS, "--cuda-device-only", "-S", src, "-o", out]
    subprocess.run(cmd, check=True)


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv)
    sys.exit(0)
