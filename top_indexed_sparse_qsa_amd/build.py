"""Builds libqsa.so in-tree with hipcc for gfx950.

Each source compiles to an object in parallel, then one shared library is
linked next to this file.  Run ``python -m top_indexed_sparse_qsa_amd.build``;
``--sanitize`` builds ``libqsa_san.so`` instead, with the host code under
AddressSanitizer and UndefinedBehaviorSanitizer (for the boundary tests).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqsa.so")
SOURCES = ["api.cpp", "indexer.hip", "sparse_attention.hip", "decode_attention.hip", "noalloc.hip", "front_end.hip"]
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off; hipcc forms them itself otherwise
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# The kernels take finite inputs: without NaN semantics a max (softmax,
# relu) needs no quieting of MFMA results.
EXTRA = {"sparse_attention.hip": ["-fno-honor-nans"], "decode_attention.hip": ["-fno-honor-nans"], "indexer.hip": ["-fno-honor-nans"],
         "front_end.hip": ["-fno-honor-nans"]}


def _hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; libqsa needs ROCm to build")
    return p


# Host-side sanitizers (the device code is left as it is): the host layer's
# argument checks, workspace arithmetic and launch planning run under
# AddressSanitizer and UndefinedBehaviorSanitizer.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_LIB = os.path.join(HERE, "libqsa_san.so")
# measurement-only kernels (the part's own ceilings), a library of their own
CEIL_SRC = "ceilings.hip"
CEIL_LIB = os.path.join(HERE, "libqsa_ceilings.so")


def asan_runtime() -> str:
    """Path of the shared ASan runtime the sanitized library needs preloaded."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else ""


def _compile(src: str, obj: str, extra=()) -> None:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_hipcc(), *COMMON, *EXTRA.get(src, []), *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SAN_LIB if sanitize else LIB
    extra = SANITIZE if sanitize else []
    with tempfile.TemporaryDirectory(prefix="qsa_build_") as tmp:
        objs = [os.path.join(tmp, s + ".o") for s in SOURCES]
        with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            list(ex.map(lambda so: _compile(*so, extra=extra), zip(SOURCES, objs)))
        out_tmp = out + ".tmp"
        link_extra = ["-shared-libasan", "-fsanitize=address,undefined"] if sanitize else []
        cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, *objs, "-o", out_tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        os.replace(out_tmp, out)
    if not sanitize:
        r = subprocess.run([_hipcc(), *COMMON, "-x", "hip", "-shared", os.path.join(CSRC, CEIL_SRC), "-o",
                            CEIL_LIB + ".tmp"], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {CEIL_SRC}:\n{r.stdout}\n{r.stderr}")
        os.replace(CEIL_LIB + ".tmp", CEIL_LIB)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv[1:])
    sys.exit(0)
