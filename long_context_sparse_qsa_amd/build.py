"""Build libqsa.so (HIP, gfx950) in-tree with hipcc.

Every source under csrc/ is compiled to an object in parallel, then linked
into ``long_context_sparse_qsa_amd/libqsa.so``; the measurement kernels
under probe/ become ``libqsa_probe.so`` (loaded by the benchmark only).
Flags:
  --offload-arch=gfx950      CDNA4 only
  -O3, no fast-math          pooling must keep IEEE adds in a fixed order
  -packed-fp32-ops disabled  packed float32 VALU ops stay out of the code
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
PROBE = os.path.join(PKG, "probe")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqsa.so")
PROBE_LIB = os.path.join(PKG, "libqsa_probe.so")

ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mcode-object-version=5",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the QSA library needs ROCm's hipcc to build")


def sources(d: str = CSRC) -> list:
    return sorted(os.path.join(d, f) for f in os.listdir(d) if f.endswith(".hip"))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(os.path.dirname(src)) + "_" + os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIP_FLAGS, f"-I{INCLUDE}", f"-I{os.path.dirname(src)}", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is expected
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def _link(objs: list, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(lib)} failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libqsa.so and libqsa_probe.so;
    returns the path of libqsa.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs, psrcs = sources(CSRC), sources(PROBE)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(psrcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs + psrcs))
    _link(objs[:len(srcs)], LIB, verbose)
    _link(objs[len(srcs):], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
