"""Build libtokengate.so in-tree with hipcc for gfx950 (runs without a GPU).

Each csrc/*.hip file compiles to an object in _build/ (in parallel), then the
objects link into learned_token_pruning_post_amd/libtokengate.so.

``--sanitize`` builds the same library with AddressSanitizer and
UndefinedBehaviorSanitizer on its host code only (device code as usual) into
_build/san/libtokengate.so, for running the argument-validation tests on the
CPU: load it with TG_LIBRARY=<that path> and the clang ASan runtime
(asan_runtime()) in LD_PRELOAD. It is never the product library.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtokengate.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    "-Wno-unused-command-line-argument",
]


# host-side sanitizers only: every -fsanitize flag is scoped to the host pass
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-O1", "-Xarch_host", "-g"]
SANITIZE_LINK = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-shared-libasan"]
SAN_LIB = os.path.join(BUILD, "san", "libtokengate.so")


def asan_runtime() -> str:
    """The clang ASan runtime the sanitized build links against (to LD_PRELOAD)."""
    llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(HIPCC))), "llvm")
    hits = sorted(glob.glob(os.path.join(llvm, "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("no clang ASan runtime under %s" % llvm)
    return hits[-1]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, sanitize: bool = False) -> str:
    out = os.path.dirname(SAN_LIB) if sanitize else BUILD
    obj = os.path.join(out, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC] + FLAGS + (SANITIZE if sanitize else []) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr[-8000:]))
    return obj


def build(verbose: bool = True, sanitize: bool = False) -> str:
    """Compile and link; returns the library's path (SAN_LIB with ``sanitize``)."""
    if not os.path.exists(HIPCC):
        raise RuntimeError("hipcc not found at %s" % HIPCC)
    lib = SAN_LIB if sanitize else LIB
    os.makedirs(os.path.dirname(SAN_LIB) if sanitize else BUILD, exist_ok=True)
    srcs = sources()
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", "8")), os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + (SANITIZE_LINK if sanitize else []) + \
        ["-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr[-8000:]))
    shutil.move(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv[1:])
    sys.exit(0)
