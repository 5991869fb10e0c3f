"""Build liblmhead.so (gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIBRARY = PKG / "liblmhead.so"
SOURCES = [CSRC / "lmhead_kernels.hip", CSRC / "lmhead_abi.cpp"]
HEADERS = [ROOT / "include" / "lmhead.h", CSRC / "lmhead_internal.h"]

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    # one rounding per float operation everywhere: no FMA contraction, so the
    # same expression rounds the same way in every kernel instance
    "-ffp-contract=off",
    # no packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return str(Path(rocm) / "bin" / "hipcc")


def build(verbose: bool = False) -> Path:
    """Compile every HIP source into liblmhead.so (always recompiles)."""
    tmp = LIBRARY.with_name(LIBRARY.name + ".tmp%d" % os.getpid())
    cmd = [hipcc(), *FLAGS, f"-I{ROOT / 'include'}", f"-I{CSRC}",
           *map(str, SOURCES), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


def is_stale() -> bool:
    if not LIBRARY.exists():
        return True
    t = LIBRARY.stat().st_mtime
    return any(src.stat().st_mtime > t for src in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
