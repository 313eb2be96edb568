"""Build libqlinear.so in-tree: hipcc for gfx950, one object per source,
linked into ``weight_quantized_linear_amd/libqlinear.so``.

Run ``python weight_quantized_linear_amd/build.py`` (or ``__graft_entry__.build()``);
this file imports nothing from the package, whose import needs the built
library.  Every call recompiles every source.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libqlinear.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# The benchmark's ceiling kernels (stream read, matrix-core loop): a library
# of their own, not part of libqlinear's ABI.
CEILING_SRC = os.path.join(PKG, "ceiling", "ceiling.hip")
CEILING_PATH = os.path.join(PKG, "libqlinear_ceiling.so")

ARCH = "gfx950"
# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in any kernel.  No fast-math:
# the int8 quantiser relies on the correctly rounded float32 division.
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# QLINEAR_TILE_ORDER=flat builds the tiled GEMMs with the plain row-major
# tile order instead of the XCD-aware one, to measure what the latter buys.
if os.environ.get("QLINEAR_TILE_ORDER") == "flat":
    COMMON_FLAGS.append("-DQLINEAR_FLAT_TILE_ORDER")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; libqlinear needs ROCm's hipcc to build")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *COMMON_FLAGS, *lang, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)
    return obj


def _link(objs, path: str, verbose: bool) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source, link libqlinear.so and the benchmark's
    libqlinear_ceiling.so; returns the path of libqlinear.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources() + [CEILING_SRC]
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:-1], LIB_PATH, verbose)
    _link(objs[-1:], CEILING_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
