"""Build libpa.so (the HIP kernels, the host block manager and the C ABI) in-tree for gfx950.

Every HIP source (csrc/*.hip) is compiled by hipcc with packed-fp32 instructions disabled (the
compiler would otherwise form v_pk_* fp32 ops from ordinary float code); host-only C++
(csrc/*.cpp) is compiled by the host compiler. Everything is linked into one shared library
next to this file, where the Python binding loads it.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpa.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, obj: str, extra) -> None:
    cmd = [hipcc(), *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    # the host pass does not know the packed-fp32 feature and says so: harmless, filtered
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")


HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]


def _compile_host(src: str, obj: str) -> None:
    cmd = [os.environ.get("CXX", "g++"), *HOST_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host compiler failed for {src}:\n{r.stderr}")
    if r.stderr.strip():
        sys.stderr.write(r.stderr)


def build(out: str = LIB, extra=(), jobs: int = 8) -> str:
    """Compile csrc/*.hip and csrc/*.cpp and link them into `out`. Returns the library path."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    host_srcs = sorted(glob.glob(os.path.join(CSRC, "*.cpp")))
    with tempfile.TemporaryDirectory(prefix="pa_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs + host_srcs]

        def one(i):
            if i < len(srcs):
                _compile(srcs[i], objs[i], extra)
            else:
                _compile_host(host_srcs[i - len(srcs)], objs[i])

        with ThreadPoolExecutor(max(1, min(jobs, len(objs)))) as ex:
            list(ex.map(one, range(len(objs))))
        tmp_lib = out + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(tmp_lib, out)
    return out


if __name__ == "__main__":
    print(build())
