"""Build libdsa.so (gfx950 only) in-tree with hipcc.

    python -m dsa_sparse_attention_indexer_amd.build
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
INCLUDE = PKG.parent / "include"
LIB = PKG / "libdsa.so"
SOURCES = ["dsa_api.hip", "indexer.hip", "attention.hip", "retrieval.hip", "ceiling.hip"]

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
    "retrieval.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, obj_dir: Path) -> Path:
    obj = obj_dir / (Path(src).stem + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), f"-I{INCLUDE}", "-c", str(CSRC / src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


# Sources whose hand-written DPP instructions rely on the compiler's code around them for
# the wait states a DPP source operand needs after a VALU write of that register.
DPP_SOURCES = ["indexer.hip"]
DPP_WAIT_STATES = 2


def _vgprs(operand: str) -> set[int]:
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", operand)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", operand)
    return {int(m.group(1))} if m else set()


def dpp_hazards(asm: str) -> list[str]:
    """Places in gfx950 assembly where a DPP instruction reads its DPP source (src0) fewer
    than two wait states after a VALU instruction wrote that register.

    Straight-line order is checked (labels are ignored, so both sides of a branch join are
    covered by the preceding instructions); `s_nop N` counts as N + 1 wait states.
    """
    ins = []
    for line in asm.splitlines():
        t = line.split(";", 1)[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        ins.append(t)
    found = []
    for i, t in enumerate(ins):
        op, _, rest = t.partition(" ")
        if not op.endswith("_dpp"):
            continue
        ops = [x.strip() for x in rest.split(",")]
        src0 = _vgprs(ops[1].split()[0]) if len(ops) > 1 else set()
        waits, j = 0, i - 1
        while j >= 0 and waits < DPP_WAIT_STATES:
            u = ins[j]
            uop, _, urest = u.partition(" ")
            if uop == "s_nop":
                waits += int(urest.strip() or 0) + 1
            else:
                if uop.startswith("v_") and "_cmp" not in uop and _vgprs(urest.split(",")[0].strip()) & src0:
                    found.append(f"{u}  ->  {t}")
                    break
                waits += 1
            j -= 1
    return found


def _check_dpp(src: str) -> None:
    cmd = [hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), f"-I{INCLUDE}", "--cuda-device-only", "-S",
           str(CSRC / src), "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr}")
    bad = dpp_hazards(r.stdout)
    if bad:
        raise RuntimeError(f"{src}: DPP source read too soon after a VALU write:\n" + "\n".join(bad[:10]))


def build(verbose: bool = False) -> Path:
    obj_dir = PKG / "_build"
    obj_dir.mkdir(exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES) + len(DPP_SOURCES), os.cpu_count() or 1)) as ex:
        checks = [ex.submit(_check_dpp, s) for s in DPP_SOURCES]
        objs = list(ex.map(lambda s: _compile(s, obj_dir), SOURCES))
        for c in checks:
            c.result()
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
