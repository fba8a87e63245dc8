"""Builds libmoe.so (all HIP sources of the package) for gfx950 with hipcc, in-tree.

``build(sanitize=True)`` builds libmoe_san.so instead: the same sources with the host code
(argument validation, size arithmetic, launch set-up) under AddressSanitizer and
UndefinedBehaviorSanitizer; the device code is compiled as usual. It is loaded only on the CPU,
with the sanitizer runtime preloaded (``sanitizer_runtime()``), to check the host layer."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")
BUILD_SAN = os.path.join(PKG, "_build_san")
LIB_SAN = os.path.join(PKG, "libmoe_san.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    # keep hipcc from emitting packed fp32 VALU ops (v_pk_add/mul/fma_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# host-side sanitizers only: each flag goes to the host compilation alone
SAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]
SAN_LINK = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-shared-libsan"]


def sanitizer_runtime() -> str:
    """Path of the clang ASan runtime (with UBSan) that a process loading libmoe_san.so preloads."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True).stdout.strip()
    return out


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(BUILD_SAN if sanitize else BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *(SAN_FLAGS if sanitize else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(jobs: int | None = None, sanitize: bool = False) -> str:
    """Compile every source and link libmoe.so (libmoe_san.so with ``sanitize``) next to this
    file. Always rebuilds."""
    os.makedirs(BUILD_SAN if sanitize else BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), srcs))
    lib = LIB_SAN if sanitize else LIB
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *(SAN_LINK if sanitize else []),
           "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    import sys
    print(build(sanitize="--sanitize" in sys.argv[1:]))
