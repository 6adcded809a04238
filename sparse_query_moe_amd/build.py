"""Build libgqe.so (the gfx950 kernels and the C ABI) in-tree with hipcc.

    python -m sparse_query_moe_amd.build          # compiles every time
    python -m sparse_query_moe_amd.build --debug  # libgqe_debug.so (-DGQE_DEBUG)
    python -m sparse_query_moe_amd.build --asan   # host AddressSanitizer build

Each .hip source is compiled to an object in parallel, then linked into
sparse_query_moe_amd/libgqe.so next to this file.  The debug library adds
the index checks of every routing and dispatch-list access (include/gqe.h,
"Debug build").  The ASan library instruments the host code only (the ABI's
argument validation and launch sequence; device code is built as usual) and
is loaded with the compiler's ASan runtime preloaded (asan_runtime()).
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgqe.so")
DEBUG_LIB = os.path.join(HERE, "libgqe_debug.so")
ASAN_LIB = os.path.join(HERE, "libgqe_asan.so")
# extra flags, object folder and library of each variant
VARIANTS = {
    "release": ([], BUILD, LIB),
    "debug": (["-DGQE_DEBUG"], os.path.join(HERE, "_build_debug"), DEBUG_LIB),
    # host code only: each -fsanitize applies to the host pass
    "asan": (["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"],
             os.path.join(HERE, "_build_asan"), ASAN_LIB),
}
SOURCES = ["router.hip", "dispatch.hip", "gemm.hip", "attention.hip", "decode.hip", "backward.hip", "peaks.hip", "api.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 math is kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str, extra, folder) -> str:
    obj = os.path.join(folder, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    return obj


def _link(variant: str, objs) -> str:
    lib = VARIANTS[variant][2]
    tmp = lib + ".tmp"
    link_extra = ["-fsanitize=address"] if variant == "asan" else []
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False, variant: str = "release") -> str:
    """Compile all sources and link one library variant (release, debug or
    asan); returns the library path."""
    return build_variants((variant,), verbose)[0]


def build_variants(variants=tuple(VARIANTS), verbose: bool = False):
    """Compile the sources of every listed variant in one pool of hipcc jobs
    (at most 8 at a time), then link each library; returns their paths."""
    jobs = []
    for v in variants:
        extra, folder, _ = VARIANTS[v]
        os.makedirs(folder, exist_ok=True)
        jobs += [(v, src, extra, folder) for src in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: (j[0], _compile(j[1], j[2], j[3])), jobs))
    libs = []
    for v in variants:
        libs.append(_link(v, [o for vv, o in objs if vv == v]))
        if verbose:
            print(f"built {libs[-1]}")
    return libs


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime (to preload with the ASan
    library)."""
    res = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the compiler's ASan runtime was not found")
    return path


if __name__ == "__main__":
    which = "debug" if "--debug" in sys.argv else "asan" if "--asan" in sys.argv else "release"
    build(verbose=True, variant=which)
    sys.exit(0)
