"""Build libla.so (the HIP/gfx950 library) in-tree with hipcc.

    python -m gated_delta_rule_chunkwise_amd.build

Every .hip file under csrc/ is compiled for gfx950 into _build/ at the repository root
and linked into gated_delta_rule_chunkwise_amd/libla.so.  Packed fp32 instructions are
disabled for all device code.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = ROOT / "_build"
LIB = PKG / "libla.so"
ARCH = os.environ.get("LA_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{ROOT / 'include'}", f"-I{CSRC}",
]


def _compile(src: Path) -> Path:
    obj = BUILD / (src.stem + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", str(src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src.name}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(jobs: int = 8) -> Path:
    BUILD.mkdir(exist_ok=True)
    srcs = sorted(CSRC.glob("*.hip"))
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *map(str, objs), "-o", str(tmp)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
