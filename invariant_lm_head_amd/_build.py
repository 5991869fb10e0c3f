"""Build liblmhead.so (gfx950) in-tree with hipcc.

The tile and fold kernels are instantiated one (mode, epilogue) pair per
object file (``csrc/lmhead_tiles.hip`` compiled once per pair), so the objects
compile in parallel; they are then linked into one shared library.  Object
files go to ``_build/`` beside this file (not shipped, not committed).
"""
from __future__ import annotations

import hashlib
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
OBJDIR = PKG / "_build"
LIBRARY = PKG / "liblmhead.so"
SOURCES = [CSRC / "lmhead_abi.cpp", CSRC / "lmhead_kernels.hip", CSRC / "lmhead_tiles.hip"]
HEADERS = [ROOT / "include" / "lmhead.h", CSRC / "lmhead_internal.h", CSRC / "lmhead_device.h"]

# (mode, epilogue) pairs of lmhead_tiles.hip: epilogue numbers as in
# lmhead_internal.h (0 store, 1 top-2, 2 log-softmax, 3 sampling, 4 integer
# log-softmax, int8 only)
TILE_INSTANCES = [(0, 0), (0, 1), (0, 2), (0, 3), (1, 0), (1, 1), (1, 2), (1, 3), (1, 4)]

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
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


def _units():
    """(source, extra flags, object path) of every object file."""
    inc = [f"-I{ROOT / 'include'}", f"-I{CSRC}"]
    digest = [f'-DLMH_SOURCE_DIGEST="{source_digest()}"']
    units = [(CSRC / "lmhead_abi.cpp", inc + digest, OBJDIR / "lmhead_abi.o"),
             (CSRC / "lmhead_kernels.hip", inc, OBJDIR / "lmhead_kernels.o")]
    for mode, epi in TILE_INSTANCES:
        units.append((CSRC / "lmhead_tiles.hip",
                      inc + [f"-DLMH_INST_MODE={mode}", f"-DLMH_INST_EPI={epi}"],
                      OBJDIR / f"lmhead_tiles_m{mode}_e{epi}.o"))
    return units


def build(verbose: bool = False, jobs: int | None = None) -> Path:
    """Compile every HIP source and link liblmhead.so (always recompiles)."""
    OBJDIR.mkdir(exist_ok=True)
    units = _units()
    tag = "%d" % os.getpid()

    def compile_one(unit):
        src, extra, obj = unit
        tmp = obj.with_name(obj.name + ".tmp" + tag)
        cmd = [hipcc(), *FLAGS, *extra, "-c", str(src), "-o", str(tmp)]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, obj)
        return obj

    n = jobs or min(len(units), max(1, min(os.cpu_count() or 1, 16)))
    with ThreadPoolExecutor(max_workers=n) as pool:
        objs = list(pool.map(compile_one, units))
    tmp = LIBRARY.with_name(LIBRARY.name + ".tmp" + tag)
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *map(str, objs), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


def source_digest() -> str:
    """SHA-256 (16 hex digits) over the library's sources and headers."""
    h = hashlib.sha256()
    for p in sorted(SOURCES + HEADERS, key=lambda q: q.name):
        h.update(p.name.encode())
        h.update(p.read_bytes())
    return h.hexdigest()[:16]


def is_stale() -> bool:
    """True when the library is missing or older than any of its sources."""
    if not LIBRARY.exists():
        return True
    t = LIBRARY.stat().st_mtime
    return any(src.stat().st_mtime > t for src in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
