"""Build libaa.so in-tree with hipcc for gfx950.

    python -m associative_algebra_block_amd.build

compiles the HIP kernels, the host plan code and the C entry points into
associative_algebra_block_amd/libaa.so.  hipcc cross-compiles the device code,
so no GPU is needed.  Only symbols named aa_* are exported.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libaa.so")

SOURCES = ["aa_plan.cpp", "aa_api.cpp", "aa_kernels.hip", "aa_backward.hip", "aa_small.hip", "aa_tile32.hip"]
ARCH = "gfx950"

# Device-code flags.  Packed fp32 arithmetic is switched off for every HIP
# translation unit (-packed-fp32-ops); the host pass prints a harmless notice
# that it does not know the feature.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain is required to build libaa.so")


def build(verbose: bool = False) -> str:
    """Compile every source and link libaa.so.  Returns the library path."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="aa_build_") as tmp:
        objs, cmds = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmds.append([cc, *HIP_FLAGS, *lang, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)
        # the translation units are independent: compile them side by side
        with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        vscript = os.path.join(tmp, "aa.map")
        with open(vscript, "w") as f:
            f.write("{ global: aa_*; local: *; };\n")
        out_tmp = LIB + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp, *objs,
               f"-Wl,--version-script={vscript}", "-Wl,-rpath,/opt/rocm/lib"]
        _run(cmd, verbose)
        os.replace(out_tmp, LIB)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
