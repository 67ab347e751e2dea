"""Build the HIP library ``libpa.so`` in-tree for gfx950.

Every ``csrc/*.hip`` file is compiled with hipcc into ``_build/`` (in
parallel) and linked into ``paged_kv_cache_44_amd/libpa.so``. Packed fp32
VALU instructions are disabled for the device code.

    python -m paged_kv_cache_44_amd.build
"""

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libpa.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src).replace(".hip", ".o"))
    cmd = [hipcc(), "-c", src, "-o", obj] + common_flags()
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libpa.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = min(len(sources), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "-shared", "-o", tmp] + objs + [f"--offload-arch={ARCH}", "-fPIC"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(sources)} sources")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
