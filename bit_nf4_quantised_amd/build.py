"""Build libqlora_nf4.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: python bit_nf4_quantised_amd/build.py   (or __graft_entry__.build()). It does not import the
package, whose import needs the library this script produces.
Each translation unit is compiled to an object under bit_nf4_quantised_amd/_build/, then linked
into bit_nf4_quantised_amd/libqlora_nf4.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqlora_nf4.so")
SOURCES = ["quant.hip", "gemm.hip", "lora.hip", "skinny.hip", "merge.hip", "optim.hip", "variants.hip", "abi.hip"]
ARCH = os.environ.get("NF4_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          # no packed-fp32 instructions in device code
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [hipcc()] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the C ABI layer (argument
# validation and kernel sequencing). Each -fsanitize= applies to the host compilation only; the
# device code is unchanged. The library leaves the sanitizer runtime unresolved: a process that
# loads it preloads libclang_rt.asan (which carries the UBSan handlers too).
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_LIB = os.path.join(BUILD, "libqlora_nf4_san.so")


def asan_runtime() -> str:
    """Path of clang's shared AddressSanitizer runtime next to hipcc."""
    root = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "lib", "clang")
    for base in (root, "/opt/rocm/lib/llvm/lib/clang"):
        if os.path.isdir(base):
            for ver in sorted(os.listdir(base), reverse=True):
                cand = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
                if os.path.exists(cand):
                    return os.path.realpath(cand)
    raise RuntimeError("clang's AddressSanitizer runtime (libclang_rt.asan-x86_64.so) not found")


def build_sanitized(verbose: bool = True) -> str:
    """Build _build/libqlora_nf4_san.so: abi.hip with host sanitizers, the kernels as usual."""
    os.makedirs(BUILD, exist_ok=True)
    others = [s for s in SOURCES if s != "abi.hip"]
    with ThreadPoolExecutor(max_workers=min(len(others), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, others))
    san_obj = os.path.join(BUILD, "abi_san.o")
    cmd = [hipcc()] + COMMON + ["-g"] + SANITIZE + ["-c", os.path.join(CSRC, "abi.hip"), "-o", san_obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stderr}")
    tmp = SAN_LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, san_obj] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
