"""Build libpkv.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m paged_kv_cache_315_amd.build              # libpkv.so
    python -m paged_kv_cache_315_amd.build --timeline   # libpkv_timeline.so (profiling build)

Every HIP source is compiled with packed-fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops): the compiler otherwise forms
v_pk_{add,mul,fma}_f32 from ordinary float code. Host-only sources (csrc/*.cpp: the block
manager) are plain C++ built with g++ and linked into the same library.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libpkv.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def host_sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def build(out_path: str = LIB_PATH, extra_flags: tuple[str, ...] = (), verbose: bool = False) -> str:
    """Compile every csrc/*.hip to an object, link them into one shared library."""
    objs = []
    with tempfile.TemporaryDirectory(prefix="pkv_build_") as tmp:
        procs = []
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                           text=True), src))
            objs.append(obj)
        for src in host_sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = ["g++", *CXX_FLAGS, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                           text=True), src))
            objs.append(obj)
        failed = []
        for p, src in procs:
            out, _ = p.communicate()
            # hipcc's host pass does not know the packed-fp32 feature; drop that one warning
            lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
            if lines and (verbose or p.returncode):
                print("\n".join(lines), file=sys.stderr)
            if p.returncode:
                failed.append(src)
        if failed:
            raise RuntimeError(f"hipcc failed for {failed}")
        tmp_out = out_path + ".tmp"
        subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_out],
                       check=True)
        os.replace(tmp_out, out_path)
    return out_path


TIMELINE_LIB_PATH = os.path.join(PKG, "libpkv_timeline.so")


if __name__ == "__main__":
    if "--timeline" in sys.argv:
        # profiling build: the balanced decode kernel stamps its phases per workgroup
        # (bench.py --timeline loads it through PKV_LIBRARY)
        print(build(TIMELINE_LIB_PATH, extra_flags=("-DPKV_TIMELINE",), verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
