"""Build libfastgen.so for gfx950 with hipcc (in-tree, next to this file).

Usage: python -m adaptive_kv_cache_fg_amd.build  (or call build()).
Each .hip source is compiled to an object in parallel, then linked into a
shared library.  Packed fp32 VALU instructions are disabled for every device
compile.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
from pathlib import Path

HERE = Path(__file__).resolve().parent
CSRC = HERE / "csrc"
INCLUDE = HERE.parent / "include"
BUILD = HERE / "_build"
LIB = HERE / "libfastgen.so"

ARCH = os.environ.get("FG_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: no accumulator-register copies before the softmax VALU work
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-source additions.  The profiling sweeps never see NaN (masked scores are
# -inf, never NaN), so max reductions need no NaN quieting of their operands.
EXTRA = {"profile_kernels": ["-fno-honor-nans"]}


def _compile(src: Path) -> Path:
    obj = BUILD / (src.stem + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(src.stem, []), "-c", str(src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src.name}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> Path:
    BUILD.mkdir(exist_ok=True)
    sources = sorted(CSRC.glob("*.hip"))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *map(str, objs), "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(sources)} sources for {ARCH}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
