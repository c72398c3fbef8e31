"""Build libdualar.so (gfx950) in-tree with hipcc.

    python -m dual_autoregressive_tts_amd.build [--checked | --all]

Variants:
  release  libdualar.so: the library the binding loads.
  checked  libdualar_checked.so: the same kernels compiled with
           DUALAR_DEVICE_CHECKS, which checks cache positions and
           partial-sum slots in the kernels and reports a failed check as
           DUALAR_ERR_DEVICE_INDEX at dualar_sync.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libdualar.so")
LIB_CHECKED = os.path.join(HERE, "libdualar_checked.so")
SOURCES = ["api.hip", "gemv.hip", "gemm.hip", "gemm_tile.hip", "attention.hip", "attn_o.hip", "prefill.hip", "depth.hip", "sample.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM_LIB = "/opt/rocm/lib"

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# host-side marker ranges (prefill / frame / slow / head / fast) for rocprofv3 --marker-trace
LINK_LIBS = ["-L" + ROCM_LIB, "-lrocprofiler-sdk-roctx"]


def _run(cmd, what):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{what} failed:\n{' '.join(cmd)}\n{r.stderr}")


def _compile(src: str, objdir: str, flags) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    _run([HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj], f"hipcc {src}")
    return obj


def _objects(objdir: str, flags) -> list:
    os.makedirs(objdir, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        return list(ex.map(lambda s: _compile(s, objdir, flags), SOURCES))


def build(verbose: bool = False, checked: bool = False) -> str:
    """Compile and link libdualar.so (or, with checked, libdualar_checked.so)."""
    objdir = os.path.join(OBJ, "checked") if checked else OBJ
    flags = FLAGS + (["-DDUALAR_DEVICE_CHECKS"] if checked else [])
    objs = _objects(objdir, flags)
    lib = LIB_CHECKED if checked else LIB
    tmp = lib + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, *LINK_LIBS, "-o", tmp], "link")
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


def build_all(verbose: bool = False) -> None:
    build(verbose)
    build(verbose, checked=True)


if __name__ == "__main__":
    if "--all" in sys.argv:
        build_all(verbose=True)
    else:
        build(verbose=True, checked="--checked" in sys.argv)
    sys.exit(0)
