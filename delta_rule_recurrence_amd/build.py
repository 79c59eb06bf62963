"""Build libfalcon.so (the HIP kernels and the C ABI) in-tree for gfx950.

Usage: ``python -m delta_rule_recurrence_amd.build`` (or ``build()``).  Each
``csrc/*.hip`` file is compiled by hipcc to an object under ``_build/`` and
the objects are linked into ``delta_rule_recurrence_amd/libfalcon.so``.

``python -m delta_rule_recurrence_amd.build --sanitize`` (or
``build_sanitized()``) builds ``libfalcon_san.so`` under ``_build_san/`` for
host-side checking on a machine without a GPU: the host code with
AddressSanitizer and UndefinedBehaviorSanitizer and with the launchers'
bounds model compiled in (FALCON_BOUNDS_CHECK), the device code unoptimised
(it is never run from this build).  A process that loads it must preload the
ASan runtime (``asan_runtime()``).
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfalcon.so")
BUILD_SAN = os.path.join(PKG, "_build_san")
LIB_SAN = os.path.join(PKG, "libfalcon_san.so")

ARCH = "gfx950"
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # Packed fp32 arithmetic stays off (the compiler otherwise forms
    # v_pk_*_f32 from ordinary float code).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


# Host code sanitised and bounds-checked, device code unoptimised (never run).
SAN_FLAGS = [
    "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all",
    "-Xarch_device", "-O0", "-Xarch_device", "-g0",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", "-DFALCON_BOUNDS_CHECK",
    "-I", INCLUDE, "-I", CSRC,
]


def asan_runtime() -> str:
    """The shared ASan runtime of the ROCm compiler (to preload)."""
    llvm = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm")
    for root in (os.path.join(llvm, "lib", "clang"), "/opt/rocm/llvm/lib/clang"):
        if os.path.isdir(root):
            for ver in sorted(os.listdir(root), reverse=True):
                cand = os.path.join(root, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
                if os.path.exists(cand):
                    return os.path.realpath(cand)
    raise RuntimeError("the ASan runtime of the ROCm compiler was not found")


def _compile(src: str, obj: str, flags=None) -> None:
    cmd = [hipcc(), *(HIPCC_FLAGS if flags is None else flags), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{res.stdout}\n{res.stderr}")


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [os.path.join(BUILD, s[:-4] + ".o") for s in sources]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        futs = [ex.submit(_compile, os.path.join(CSRC, s), o) for s, o in zip(sources, objs)]
        for f in futs:
            f.result()
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(sources)} sources")
    return LIB


def build_sanitized(verbose: bool = True) -> str:
    os.makedirs(BUILD_SAN, exist_ok=True)
    sources = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [os.path.join(BUILD_SAN, s[:-4] + ".o") for s in sources]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        futs = [ex.submit(_compile, os.path.join(CSRC, s), o, SAN_FLAGS) for s, o in zip(sources, objs)]
        for f in futs:
            f.result()
    tmp = LIB_SAN + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_SAN)
    if verbose:
        print(f"built {LIB_SAN} from {len(sources)} sources (host sanitizers, bounds checks)")
    return LIB_SAN


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized()
    else:
        build()
    sys.exit(0)
