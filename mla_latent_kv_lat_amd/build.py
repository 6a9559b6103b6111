"""Build libmla.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python mla_latent_kv_lat_amd/build.py

(run it as a script: importing the package loads the library being built).

Each source compiles to an object in parallel, then one shared library is
linked next to this file.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmla.so")
SOURCES = ["mla_api.hip", "generic_kernels.hip", "combine.hip", "mfma_kernels.hip", "decode_split.hip",
           "combine_proj.hip", "kv_append.hip", "prefill.hip", "out_fused.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


# sources the split-K decode kernel is built from (its measurements are tied to these)
DECODE_SOURCES = ("decode_split.hip", "decode_common.hpp", "mfma_common.hpp", "common.hpp",
                  "kernels.hpp")
PREFILL_SOURCES = ("prefill.hip", "decode_common.hpp", "mfma_common.hpp", "common.hpp",
                   "kernels.hpp")
OUT_FUSED_SOURCES = ("out_fused.hip", "mfma_common.hpp", "common.hpp", "kernels.hpp")


def source_digest(files=None) -> str:
    """Hash of library sources and the header (ties measurements to code):
    the library's build inputs (SOURCES and the headers under csrc/), or
    only `files` (names under csrc/).  Other files lying in csrc/ do not
    enter the library and do not change the hash."""
    import hashlib
    h = hashlib.sha256()
    names = sorted(files) if files else sorted(
        set(SOURCES) | {f for f in os.listdir(CSRC) if f.endswith(".hpp")})
    for f in names:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    with open(os.path.join(HERE, "..", "include", "mla.h"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
