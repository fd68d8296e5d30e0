"""Build libdf11.so in-tree: host codec with g++, gfx950 kernels with hipcc.

The shared library links the HIP runtime by its SONAME (libamdhip64.so.7) with
torch's library directory first on the run path, so that a process that has
imported torch resolves it to the runtime torch already loaded and torch's
streams and allocations are valid inside the library.
"""

from __future__ import annotations

import importlib.util
import os
import shutil
import subprocess
from typing import List

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
BUILD_DIR = os.path.join(REPO_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libdf11.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
OFFLOAD_ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={OFFLOAD_ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    # Packed FP32 instructions are kept out of every HIP build.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Atomics are issued as written (the optimizer would wrap one-lane LDS
    # adds in a loop over the active lanes).
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall",
]


def _torch_lib_dir() -> str:
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.origin:
        return ""
    return os.path.join(os.path.dirname(spec.origin), "lib")


def _run(cmd: List[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")


def build(verbose: bool = False) -> str:
    """Compile every source of the library and return the path of libdf11.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    host_objs = []
    for src in ("df11_host.cpp", "df11_rans_host.cpp"):
        obj = os.path.join(BUILD_DIR, src.replace(".cpp", ".o"))
        _run(["g++", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", f"-I{INCLUDE}", f"-I{CSRC}",
              "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        host_objs.append(obj)
    dev_objs = []
    for src in ("df11_decode.hip", "df11_rans_decode.hip"):
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        _run([hipcc, *HIP_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        dev_objs.append(obj)
    rpaths = [p for p in (_torch_lib_dir(), os.path.join(ROCM, "lib")) if p]
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={OFFLOAD_ARCH}", "-shared", "-fPIC", "-o", tmp, *host_objs, *dev_objs,
          *[f"-Wl,-rpath,{p}" for p in rpaths]], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


# Host code of the sanitizer build: AddressSanitizer and UndefinedBehaviorSanitizer,
# every report fatal.  Each flag goes to the host compilation only.
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime that a process loading the
    sanitizer build must preload."""
    import glob
    found = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not found:
        raise RuntimeError("the clang AddressSanitizer runtime is not installed")
    return found[-1]


def build_sanitized(out_path: str, verbose: bool = False) -> str:
    """Build the whole library with the host code (the codec, the argument
    checks and launch arithmetic of the device entry points) under
    AddressSanitizer and UndefinedBehaviorSanitizer, for CPU tests; the
    gfx950 code objects are built as usual.  A process that loads it needs
    asan_runtime() preloaded."""
    work = os.path.join(BUILD_DIR, "sanitized")
    os.makedirs(work, exist_ok=True)
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    objs = []
    for src in ("df11_host.cpp", "df11_rans_host.cpp", "df11_decode.hip", "df11_rans_decode.hip"):
        obj = os.path.join(work, src.split(".")[0] + ".o")
        lang = [] if src.endswith(".hip") else ["-x", "hip"]
        _run([hipcc, *HIP_FLAGS, *SAN_HOST, "-O1", f"-I{INCLUDE}", f"-I{CSRC}", *lang, "-c",
              os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    rpaths = [p for p in (_torch_lib_dir(), os.path.join(ROCM, "lib")) if p]
    _run([hipcc, f"--offload-arch={OFFLOAD_ARCH}", "-shared", "-fPIC", "-shared-libasan", *SAN_HOST, "-o", out_path,
          *objs, *[f"-Wl,-rpath,{p}" for p in rpaths]], verbose)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
