"""Build the Parallax HIP library (libparallax_hip.so) in-tree for gfx950.

Each source is compiled to an object in parallel (hipcc -c), then linked.
Usage: python -m parameterized_local_linear_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["api.hip", "decode.hip", "prefill.hip", "backward.hip"]
LIB = os.path.join(HERE, "libparallax_hip.so")
OBJDIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed fp32 instructions: keep plain v_fma/v_mul/v_add
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(line for line in res.stderr.splitlines() if "packed-fp32-ops" not in line)
    return res.returncode, errs


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    objs = [os.path.join(OBJDIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        results = list(ex.map(_run, cmds))
    for (rc, errs), src in zip(results, SOURCES):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {src} ({rc}):\n{errs}")
        if errs.strip() and verbose:
            print(errs, file=sys.stderr)
    tmp = LIB + ".tmp"
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    rc, errs = _run(link)
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{errs}")
    os.replace(tmp, LIB)
    return LIB


CLANG_RT = "/opt/rocm/llvm/lib/clang"


def asan_runtime() -> str:
    """The ROCm clang's shared AddressSanitizer runtime (to preload)."""
    for ver in sorted(os.listdir(CLANG_RT), reverse=True):
        p = os.path.join(CLANG_RT, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    raise RuntimeError("no libclang_rt.asan-x86_64.so under " + CLANG_RT)


def build_host_sanitized() -> str:
    """The library with its host code (the C ABI's argument checks, the decode
    split planner, the launch wrappers of api.hip) built with AddressSanitizer
    and UBSan, for the host test tier: _build/libparallax_hip_san.so. Device
    code is built as usual; the kernels' objects are those of build(). A process
    that loads it must preload asan_runtime()."""
    objs = [os.path.join(OBJDIR, os.path.splitext(s)[0] + ".o") for s in SOURCES[1:]]
    if not all(os.path.exists(o) for o in objs):
        build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    api_o = os.path.join(OBJDIR, "api_san.o")
    rc, errs = _run([HIPCC, *FLAGS, "-g", *san, "-c", os.path.join(CSRC, SOURCES[0]), "-o", api_o])
    if rc != 0:
        raise RuntimeError(f"hipcc failed on {SOURCES[0]} ({rc}):\n{errs}")
    out = os.path.join(OBJDIR, "libparallax_hip_san.so")
    rc, errs = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *san, "-shared-libsan",
                     api_o, *objs, "-o", out])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{errs}")
    return out


if __name__ == "__main__":
    print(build(verbose=True))
