"""Build libpkv.so for gfx950 with hipcc, in the package directory.

    python -m paged_kv_cache_334_amd.build        # or __graft_entry__.build()

Every .hip file under csrc/ is compiled with hipcc and every .cpp file (host
code only) with g++ to an object in _build/ (in parallel), then linked into
paged_kv_cache_334_amd/libpkv.so.  Always rebuilds.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpkv.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CXX = shutil.which("g++") or "c++"
HOST_FLAGS = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-I", os.path.join(ROOT, "include")]
FLAGS = [
    "-O3",
    f"--offload-arch={ARCH}",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Wno-unused-result",
    # packed float32 instructions are left to no part of this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: the decode kernels rescale and
    # read them between instructions, which the AGPR form turns into copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    base, ext = os.path.splitext(os.path.basename(src))
    obj = os.path.join(BUILD, base + ext.replace(".", "_") + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj] if ext == ".hip" else [CXX, *HOST_FLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature; drop that line only
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(line for line in res.stderr.splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    jobs = min(len(sources), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(sources)} sources")
    return LIB


if __name__ == "__main__":
    build()
