"""Builds libgdn (HIP kernels + C-ABI host code) in-tree for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libgdn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM_INCLUDE = "/opt/rocm/include"
ROCM_LIB = "/opt/rocm/lib"
# A plain-C program that drives the C-ABI without Python (built next to the library).
C_EXAMPLE_SRC = os.path.join(ROOT, "examples", "c_abi_decode.c")
C_EXAMPLE = os.path.join(LIBDIR, "c_abi_decode")
# Memory-stream probes the benchmark times next to the update (not part of libgdn).
PROBE_SRC = os.path.join(CSRC, "stream_probe.hip")
PROBE_LIB = os.path.join(LIBDIR, "libgdn_stream_probe.so")

DEVICE_SOURCES = ["gdn_kernels.hip", "gdn_rows.hip", "gdn_chunk.hip", "gdn_chunk_ws.hip", "gdn_scratch.hip"]
HOST_SOURCES = ["gdn_api.cpp"]

# Packed fp32 VALU forms are disabled: hipcc -O3 otherwise forms them from
# scalar float code.  No implicit FMA contraction: the kernels spell out every
# fused multiply-add, so all instances round the same way.
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]
DEVICE = ["-x", "hip", "--offload-arch=gfx950", "-ffp-contract=off", "-Xclang", "-target-feature",
          "-Xclang", "-packed-fp32-ops"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer (device code is
# compiled as usual).  The library is then loaded into a process that preloads
# clang's ASan runtime (asan_runtime()); the CPU tests run the host-only ABI
# tests that way.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """clang's shared ASan runtime, to preload into a process that loads a
    sanitized build."""
    import glob
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise FileNotFoundError("clang's libclang_rt.asan-x86_64.so was not found under /opt/rocm/llvm")
    return found[-1]


def build(verbose: bool = False, extra_device_flags=(), out: str = LIB, sanitize: bool = False) -> str:
    """Compiles libgdn to `out`.  sanitize=True instruments the host code
    (argument checks, planning, launches) with ASan and UBSan; such a build
    is for tests only and skips the C example."""
    libdir = os.path.dirname(os.path.abspath(out))
    os.makedirs(libdir, exist_ok=True)
    extra = HOST_SANITIZE if sanitize else []
    tag = ".san" if sanitize else ""
    cmds, objs = [], []
    for src in DEVICE_SOURCES:
        obj = os.path.join(libdir, src + tag + ".o")
        cmds.append([HIPCC, *COMMON, *DEVICE, *extra_device_flags, *extra, "-c",
                     os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(libdir, src + tag + ".o")
        cmds.append([HIPCC, *COMMON, "-I", ROCM_INCLUDE, "-D__HIP_PLATFORM_AMD__", "-x", "c++", *extra,
                     "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    # one compiler process per source, at most MAX_JOBS (default 4) at a time
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "4"))))
    with ThreadPoolExecutor(jobs) as pool:
        for f in [pool.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = out + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    for o in objs:
        os.remove(o)
    if not sanitize:
        build_c_example(verbose)
        build_stream_probe(verbose)
    return out


def build_stream_probe(verbose: bool = False) -> str:
    tmp = PROBE_LIB + ".tmp"
    _run([HIPCC, *COMMON, *DEVICE, "-shared", PROBE_SRC, "-o", tmp], verbose)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def c_example_command(out: str = C_EXAMPLE, syntax_only: bool = False):
    """gcc command line of the C example (C11, the HIP runtime's C API)."""
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", INCLUDE, "-I", ROCM_INCLUDE, C_EXAMPLE_SRC]
    if syntax_only:
        return cmd + ["-fsyntax-only"]
    return cmd + ["-L", LIBDIR, "-lgdn", "-L", ROCM_LIB, "-lamdhip64", "-lm",
                  "-Wl,-rpath,$ORIGIN", "-Wl,-rpath," + ROCM_LIB, "-o", out]


def build_c_example(verbose: bool = False) -> str:
    tmp = C_EXAMPLE + ".tmp"
    _run(c_example_command(tmp), verbose)
    os.replace(tmp, C_EXAMPLE)
    return C_EXAMPLE


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
