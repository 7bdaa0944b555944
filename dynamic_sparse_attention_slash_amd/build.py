"""Build libdsa.so (all HIP sources under csrc/) for gfx950 with hipcc.

Usage: python -m dynamic_sparse_attention_slash_amd.build  (or build() here).
The library lands next to this file, in-tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libdsa.so")
BUILD_DIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 (v_pk_*_f32) code generation
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# per-source extra flags: the attention kernels take maxima of scores that are
# finite or -inf, never NaN, and rely on NaN-free fmaxf for single v_max3_f32
EXTRA = {"sparse_attention.hip": ["-fno-honor-nans"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# host-side AddressSanitizer + UndefinedBehaviorSanitizer (device code is built
# as usual): for checking the library's host code, argument validation above all
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def _compile(src: str, build_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True, out: str = OUT, sanitize: bool = False) -> str:
    """Compile every source and link ``out``. ``sanitize`` adds the host-side
    sanitizers; such a library needs the sanitizer runtime loaded first (link
    it into an executable built with the same -fsanitize flags)."""
    build_dir = BUILD_DIR if out == OUT else out + ".build"
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    extra = SANITIZE if sanitize else []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, extra), srcs))
    tmp = out + ".tmp"
    link_extra = [*SANITIZE, "-Xarch_host", "-shared-libsan"] if sanitize else []
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    shutil.rmtree(build_dir, ignore_errors=True)
    if verbose:
        print(f"built {out}", file=sys.stderr)
    return out


if __name__ == "__main__":
    build()
