"""Build libsxattn.so in-tree for gfx950 with hipcc.

    python -m block_sparse_cross_anchor_amd.build        # compile + link

Every HIP source is compiled to an object in parallel, then linked into
``block_sparse_cross_anchor_amd/libsxattn.so`` next to this file.  Packed fp32
instructions are disabled for all device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libsxattn.so")
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

SOURCES = ["api.hip", "cost.hip", "combine.hip", "gather.hip", "order.hip", "plan.hip", "attn_f32.hip",
           "attn_fwd.hip", "attn_bwd.hip",
           "lpt.cpp"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, bdir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".cpp"):
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC, "-c", path,
               "-o", obj]
    else:
        cmd = [_hipcc(), *HIPCC_FLAGS, *extra, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    msgs = [ln for ln in (r.stderr or "").splitlines()
            if ln.strip() and "packed-fp32-ops" not in ln and "is not a recognized feature" not in ln]
    if any("warning" in m for m in msgs):
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(verbose: bool = True, out: str = OUT, defines=()) -> str:
    """Compile every source and link `out`.  `defines` (e.g. ["SXA_KV_WAVES=4"]) are
    passed to hipcc as -D flags, for building tuning variants out of tree."""
    bdir = BUILD_DIR if out == OUT else out + "_objs"
    os.makedirs(bdir, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    extra = [f"-D{d}" for d in defines]
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, bdir, extra), SOURCES))
    tmp = out + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


DRIVER_SRC = os.path.join(ROOT, "tests", "c_abi", "sxattn_c_driver.cpp")
DRIVER_OUT = os.path.join(ROOT, "tests", "c_abi", "sxattn_c_driver")


def build_c_driver(verbose: bool = True) -> str:
    """Compile the host program that drives the library through its C ABI alone
    (used by the GPU tests); it finds libsxattn.so next to this file at run time."""
    if not os.path.exists(DRIVER_SRC):
        return ""
    tmp = DRIVER_OUT + ".tmp"
    cmd = [_hipcc(), "-O2", "-std=c++17", "-Wall", "-I", INCLUDE, DRIVER_SRC, "-o", tmp,
           "-L", HERE, "-lsxattn", "-Wl,-rpath,$ORIGIN/../../block_sparse_cross_anchor_amd"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"driver build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, DRIVER_OUT)
    if verbose:
        print(f"built {DRIVER_OUT}")
    return DRIVER_OUT


if __name__ == "__main__":
    build()
    build_c_driver()
