"""Oracle outputs of the full-size workloads, stored for the GPU parity tests.

    python tests/golden/make_oracle_golden.py [--threads N] [--only NAME]

The float64 / int64 oracle (``oracle/``) is run here on every row the GPU
tests compare, and its outputs are written to ``tests/golden/oracle_<name>.npz``
(plain numpy arrays, no pickles), so the GPU host does not spend minutes of CPU
time recomputing them.  This script calls only ``oracle/`` and the seeded input
generators in ``synth/``; no value comes from the HIP path.

Each file records the SHA-256 of the inputs it was computed from (``inputs``),
and ``tests/test_golden_files.py`` recomputes sampled rows with the live oracle
on the CPU, so a file that no longer matches the generators or the oracle
fails there.

Files:
  oracle_int8.npz     int8 head 4096 x 128256, rows 0..511: greedy top-2 (ids,
                      exact raw values, scaled float32 values and margin), the
                      float log-prob of the target, the exact int32 logits of
                      64 rows (one every 8) as per-row digests, and the integer
                      front and back: per-token quantisation of the int32
                      hidden rows (q digest, M, E) and the Q.24 log-prob.
  oracle_logprob.npz  float head 4096 x 151936: log p(target) of rows 0..255
                      and of every 64th row of the 16384 (508 rows).
  oracle_neartie.npz  float head 2048 x 32000 with planted near ties, all 4096
                      rows: top-2 of the float64 logits and of the logits
                      rounded to bf16 (the bf16-output head).
"""
from __future__ import annotations

import argparse
import hashlib
import sys
import time
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
ROOT = HERE.parents[1]
sys.path.insert(0, str(ROOT))

import oracle  # noqa: E402
import synth  # noqa: E402


def digest(*arrays) -> str:
    """SHA-256 over the little-endian bytes of the arrays, in order."""
    h = hashlib.sha256()
    for a in arrays:
        a = np.ascontiguousarray(a)
        h.update(a.astype(a.dtype.newbyteorder("<"), copy=False).tobytes())
    return h.hexdigest()


def row_digests(z: np.ndarray) -> np.ndarray:
    """SHA-256 (hex) of each row's little-endian int32 values."""
    return np.array([hashlib.sha256(np.ascontiguousarray(r, dtype="<i4").tobytes()).hexdigest()
                     for r in z], dtype="U64")


LOGPROB_ROWS = np.union1d(np.arange(256), np.arange(0, 16384, 64)).astype(np.int64)
INT8_LOGIT_ROWS = np.arange(0, 512, 8).astype(np.int64)


def make_int8(o, nt):
    d = synth.make_inputs("int8")
    x, w, s, t, hid = d["x"], d["w"], d["scale"], d["target"], d["hidden"]
    out = {"inputs": np.array(digest(x, w, s, t, hid)), "rows": np.arange(512)}
    out["ids"], out["raw"], out["vals"], out["margin"] = o.greedy_i8(x, w, s, nthreads=nt)
    out["logprob"] = o.logprob_i8(x, w, t, s, nthreads=nt)
    out["logit_rows"] = INT8_LOGIT_ROWS
    out["logit_digests"] = row_digests(o.logits_i8(x[INT8_LOGIT_ROWS], w, nthreads=nt))
    q, M, E = o.quantize_rows(hid)
    out["q_digests"] = row_digests(q.astype(np.int32))
    out["step_m"], out["step_e"] = M, E
    out["logprob_q"] = o.logprob_int(q, w, *d["unit"], M, E, t, nthreads=nt)
    return out


def make_logprob(o, nt):
    d = synth.make_inputs("logprob")
    x, w, t = d["x"], d["w"], d["target"]
    rows = LOGPROB_ROWS
    return {"inputs": np.array(digest(x, w, t)), "rows": rows,
            "logprob": o.logprob_bf16(x[rows], w, t[rows], nthreads=nt)}


def make_neartie(o, nt):
    d = synth.make_inputs("neartie")
    x, w = d["x"], d["w"]
    out = {"inputs": np.array(digest(x, w)), "rows": np.arange(x.shape[0])}
    out["ids"], out["vals"], out["margin"] = o.greedy_bf16(x, w, nthreads=nt)
    out["ids16"], out["vals16"], out["margin16"] = o.greedy_bf16(x, w, round_bf16=True,
                                                                 nthreads=nt)
    return out


MAKERS = {"int8": make_int8, "logprob": make_logprob, "neartie": make_neartie}


def path_of(name: str) -> Path:
    return HERE / f"oracle_{name}.npz"


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--threads", type=int, default=None)
    ap.add_argument("--only", choices=sorted(MAKERS), default=None)
    args = ap.parse_args()
    o = oracle.default()
    for name, make in MAKERS.items():
        if args.only and name != args.only:
            continue
        t0 = time.perf_counter()
        arrays = make(o, args.threads)
        np.savez_compressed(path_of(name), **arrays)
        print(f"{path_of(name).name}: {time.perf_counter() - t0:.1f} s", flush=True)


if __name__ == "__main__":
    main()
