"""Build libmoba.so (HIP, gfx950) in-tree with hipcc.

``python -m block_sparse_long_gating_amd.build`` compiles every source under
``csrc/`` to ``_build/*.o`` in parallel and links ``libmoba.so`` next to this
file. It always recompiles. With ``--host-sanitized`` it builds a debug copy,
``_build/hostsan/libmoba.so``, whose host code runs under AddressSanitizer and
UndefinedBehaviorSanitizer (load it with ``MOBA_LIBRARY`` set to its path and
the runtime from ``asan_runtime()`` preloaded).
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoba.so")

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler away from packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libmoba")
    return path


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "is not a recognized feature for this target"
    out = "\n".join(l for l in r.stdout.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host-sanitized debug build: the host code that checks arguments and plans
# the workspace (the .cpp sources and the host side of noalloc.hip) is rebuilt
# with AddressSanitizer and UndefinedBehaviorSanitizer on the host pass only;
# the device code is unchanged (the other objects are those of build()).
SAN_DIR = os.path.join(BUILD, "hostsan")
SAN_LIB = os.path.join(SAN_DIR, "libmoba.so")
SAN_SOURCES = ("moba_api.cpp", "noalloc.hip")
SAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (it must be
    preloaded into a process that loads the sanitized library)."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE,
                       stderr=subprocess.DEVNULL, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        rdir = subprocess.run([hipcc(), "-print-runtime-dir"], stdout=subprocess.PIPE, stderr=subprocess.DEVNULL,
                              text=True).stdout.strip()
        path = os.path.join(rdir, "libclang_rt.asan-x86_64.so")
    if not os.path.exists(path):
        raise RuntimeError("the shared AddressSanitizer runtime of the ROCm compiler was not found")
    return path


def build_host_sanitized() -> str:
    """Builds _build/hostsan/libmoba.so; returns its path."""
    srcs = sources()
    objs = {s: os.path.join(BUILD, os.path.basename(s) + ".o") for s in srcs}
    if not all(os.path.exists(o) for o in objs.values()):
        build(verbose=False)
    os.makedirs(SAN_DIR, exist_ok=True)
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1"] + SAN_FLAGS

    def compile_san(src):
        obj = os.path.join(SAN_DIR, os.path.basename(src) + ".o")
        r = subprocess.run([hipcc(), *flags, "-c", src, "-o", obj], stdout=subprocess.PIPE,
                           stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (host sanitizers) failed on {src}:\n{r.stdout}")
        return obj

    san = [s for s in srcs if os.path.basename(s) in SAN_SOURCES]
    with concurrent.futures.ThreadPoolExecutor(len(san)) as ex:
        san_objs = dict(zip(san, ex.map(compile_san, san)))
    link = [san_objs.get(s, objs[s]) for s in srcs]
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", SAN_LIB, *link]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (host sanitizers) failed:\n{r.stdout}")
    return SAN_LIB


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv[1:]:
        print(build_host_sanitized())
    else:
        build()
