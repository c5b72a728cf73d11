"""Build libcsa2.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m compressed_kv_cache_csa2_amd.build

Every call recompiles. Objects go to compressed_kv_cache_csa2_amd/_build/, the library
to compressed_kv_cache_csa2_amd/libcsa2.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcsa2.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    return obj, out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    if verbose:
        for obj, out in results:
            if out.strip():
                print(out)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host-check build: the C ABI's host code (csa2_api.hip compiled as C++ by g++, no device
# code) with every kernel launcher stubbed out (hostcheck/launch_stubs.cpp), under
# AddressSanitizer and UndefinedBehaviorSanitizer. The CPU tests load it in place of
# libcsa2.so (CSA2_LIBRARY) with the sanitizer runtimes preloaded.
HOSTCHECK_SRC = os.path.join(PKG, "hostcheck", "launch_stubs.cpp")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_hostcheck(out_path: str) -> str:
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-x", "c++", os.path.join(CSRC, "csa2_api.hip"), "-x", "c++", HOSTCHECK_SRC,
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", out_path]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host-check build failed:\n{r.stdout}{r.stderr}")
    return out_path


def sanitizer_runtimes() -> list:
    """Paths of g++'s ASan and UBSan runtimes (to preload into a Python process)."""
    out = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True,
                           text=True).stdout.strip()
        out.append(p)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
