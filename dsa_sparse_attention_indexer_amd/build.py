"""Build libdsa.so (gfx950 only) in-tree with hipcc.

    python -m dsa_sparse_attention_indexer_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
INCLUDE = PKG.parent / "include"
LIB = PKG / "libdsa.so"
SOURCES = ["dsa_api.hip", "indexer.hip", "attention.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not Path(p).exists():
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libdsa.so")
    return p


# Per-source extras.  The indexer's scoring loop keeps its MFMA accumulators in VGPRs,
# where the ReLU/weight epilogue reads them without AGPR-to-VGPR copies.
SOURCE_FLAGS = {
    "indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, obj_dir: Path) -> Path:
    obj = obj_dir / (Path(src).stem + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), f"-I{INCLUDE}", "-c", str(CSRC / src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> Path:
    obj_dir = PKG / "_build"
    obj_dir.mkdir(exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir), SOURCES))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
