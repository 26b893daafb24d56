"""Build libmoe.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run as ``python -m grouped_gemm_softmax_amd.build``; ``__graft_entry__.build()``
calls :func:`build`. Objects go to ``grouped_gemm_softmax_amd/_build`` and the
library to ``grouped_gemm_softmax_amd/libmoe.so`` (in-tree).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 math.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(os.path.dirname(PKG), "include")]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    lines = [l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l
             and "is not a recognized feature for this target" not in l]
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + "\n".join(lines))
    return "\n".join(lines)


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(OUT_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        futs = [ex.submit(_run, [HIPCC, *HIP_FLAGS, "-c", s, "-o", o])
                for s, o in zip(srcs, objs)]
        for f in futs:
            out = f.result()
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


# Host code of the C ABI (argument validation, workspace carving, the
# diagnostics) under AddressSanitizer and UndefinedBehaviorSanitizer; the
# device code is unchanged. Each sanitizer flag applies to the host pass only.
SANITIZED_SOURCES = ("api.hip", "diagnostics.hip")
HOST_SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                       "-Xarch_host", "-fno-sanitize-recover=undefined",
                       "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The compiler's AddressSanitizer runtime, to preload into a process
    that loads a sanitized build."""
    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib",
                                         "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so next to " + HIPCC)
    return hits[-1]


def build_host_sanitized(out_dir: str) -> str:
    """libmoe with its host-side C ABI layer sanitized, in `out_dir`; the
    kernels' objects are those of the in-tree build (made first if missing)."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(OUT_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    if not all(os.path.exists(o) for o in objs):
        build()
    os.makedirs(out_dir, exist_ok=True)
    flags = [f for f in HIP_FLAGS if f != "-O3"] + ["-O1", "-g"] + HOST_SANITIZE_FLAGS
    link = []
    for s, o in zip(srcs, objs):
        if os.path.basename(s) in SANITIZED_SOURCES:
            o = os.path.join(out_dir, os.path.basename(s)[:-4] + ".san.o")
            _run([HIPCC, *flags, "-c", s, "-o", o])
        link.append(o)
    lib = os.path.join(out_dir, "libmoe_sanitized.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SANITIZE_FLAGS[:4],
          "-shared-libsan", "-o", lib, *link])
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
