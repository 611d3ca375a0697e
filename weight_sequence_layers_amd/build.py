"""Build libttt.so in-tree with hipcc for gfx950.

    python -m weight_sequence_layers_amd.build        # or build() from Python
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libttt.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["ttt_kernels.hip", "ttt_backward.hip", "ttt_small.hip", "ttt_noalloc.hip",
           "ttt_ns_small.hip", "ttt_block.hip", "libttt.cpp", "ttt_block.cpp"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
    "-I" + os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed:\n" + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link libttt.so next to this file. Always recompiles."""
    build_dir = os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)
    objs = [os.path.join(build_dir, src.replace(".", "_") + ".o") for src in SOURCES]
    # one compiler process per source, a few at a time (each takes about a GB of memory)
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", "0")) or os.cpu_count() or 1, 8))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        outs = list(ex.map(lambda so: _run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, so[0]),
                                             "-o", so[1]]), zip(SOURCES, objs)))
    if verbose:
        for out in outs:
            if out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


HOST_SOURCES = [f for f in SOURCES if f.endswith(".cpp")]
# sanitizers compiled into the host code only; the device code is built as always.
# "ubsan": undefined-behaviour checks as traps (no runtime library); "asan": address checks,
# whose runtime (asan_runtime()) must be preloaded into the process that loads the library
HOST_SANITIZE = {
    "ubsan": ["-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fsanitize-trap=undefined",
              "-Xarch_host", "-fno-sanitize=vptr"],
    "asan": ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"],
}


def asan_runtime() -> str:
    """Path of the compiler's shared address-sanitizer runtime."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang")
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       stdout=subprocess.PIPE, text=True)
    return r.stdout.strip()


def build_host_sanitized(out_path: str, kind: str = "ubsan") -> str:
    """A copy of the library at out_path whose host sources (argument checks, state and
    workspace handling, launch order) carry the sanitizer `kind`, linked with the kernel
    objects of the last build(). For CPU tests of the host logic."""
    build_dir = os.path.join(PKG, "_build")
    objs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".", "_") + ".o")
        if src in HOST_SOURCES:
            obj = out_path + "." + src.replace(".", "_") + ".o"
            _run([HIPCC, *FLAGS, "-O1", "-g", *HOST_SANITIZE[kind], "-c",
                  os.path.join(CSRC, src), "-o", obj])
        elif not os.path.exists(obj):
            raise FileNotFoundError(f"{obj} missing: run build() first")
        objs.append(obj)
    link = ["-shared-libsan", "-Xarch_host", "-fsanitize=address"] if kind == "asan" else []
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *link, *objs, "-o", out_path])
    return out_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
