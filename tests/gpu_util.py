"""Helpers shared by the GPU tests: host <-> device copies, the comparison
rules of the head against the oracle, the stored oracle outputs of the
full-size workloads and the result files (not collected as tests)."""
from __future__ import annotations

import json
import os
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle
import synth

ROOT = Path(__file__).resolve().parents[1]
GOLDEN = ROOT / "tests" / "golden"

DEV = "cuda:0"
TOL = 1e-4          # float32 logits / log-probs vs the float64 oracle (absolute)
GAP_EXEMPT = 1e-4   # rows whose oracle top-2 gap is below this may pick either of the two


def gpu_bf16(a) -> torch.Tensor:
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)


def gpu(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def bits(t: torch.Tensor) -> torch.Tensor:
    """Reinterpret a float32/int32 tensor as int32 bit patterns."""
    return t.contiguous().view(torch.int32)


def check_greedy_bf16(ids, vals, margin, o_ids, o_vals, o_margin, tol=TOL, report=None):
    """float32-head top-2 against the oracle; returns the number of exempt rows.

    report: (result file, key) under which the comparison is recorded: rows,
    exempt rows and their oracle gaps in bf16 ulps, the largest errors.

    Values are order statistics, so they must match within tol on every row;
    the top-1 id must match on every row whose oracle gap is >= 1e-4; on exempt
    rows the GPU's top-1 must be one of the oracle's top-2.
    """
    ids, vals, margin = host(ids), host(vals).astype(np.float64), host(margin).astype(np.float64)
    assert np.all(np.abs(vals - o_vals) <= tol), np.max(np.abs(vals - o_vals))
    assert np.all(np.abs(margin - o_margin) <= 2 * tol), np.max(np.abs(margin - o_margin))
    assert np.all(vals[:, 0] >= vals[:, 1]) and np.all(margin >= 0)
    exempt = o_margin < GAP_EXEMPT
    bad = (ids[:, 0] != o_ids[:, 0]) & ~exempt
    assert not bad.any(), f"top-1 differs on {bad.sum()} non-exempt rows: {np.nonzero(bad)[0][:10]}"
    ok_exempt = (ids[:, 0] == o_ids[:, 0]) | (ids[:, 0] == o_ids[:, 1])
    assert np.all(ok_exempt[exempt])
    if report is not None:
        gaps = bf16_ulps(o_margin[exempt], o_vals[exempt, 0])
        record(*report, {
            "rows": int(len(ids)), "exempt_rows": int(exempt.sum()),
            "exempt_gap_bf16_ulps": [round(float(g), 4) for g in gaps],
            "exempt_rows_top1_differs": int((ids[exempt, 0] != o_ids[exempt, 0]).sum()),
            "max_abs_err_values": float(np.max(np.abs(vals - o_vals))),
            "max_abs_err_margin": float(np.max(np.abs(margin - o_margin)))})
    # where the 2nd and 3rd cannot be confused the second id must match too:
    # its value sits clear of the first by >= gap and the GPU agrees on the first
    return int(exempt.sum())


# ------------------------------------------------------- shared workloads
@pytest.fixture(scope="session")
def o():
    return oracle.default()


@pytest.fixture(scope="session")
def tl(o):
    """The 2048 x 32000 head, 512 rows, with the oracle's greedy result."""
    d = synth.make_inputs("tinyllama")
    d["o_greedy"] = o.greedy_bf16(d["x"], d["w"])
    d["gx"], d["gw"] = gpu_bf16(d["x"]), gpu_bf16(d["w"])
    return d


@pytest.fixture(scope="session")
def i8(o):
    """The 4096 x 128256 int8 head, 512 rows, with the oracle's stored outputs
    for every row (tests/golden/oracle_int8.npz)."""
    d = synth.make_inputs("int8")
    d["gx"], d["gw"], d["gs"] = gpu(d["x"]), gpu(d["w"]), gpu(d["scale"])
    d["golden"] = golden("int8", d["x"], d["w"], d["scale"], d["target"], d["hidden"])
    return d


# ------------------------------------------------- stored oracle outputs
def golden(name: str, *inputs) -> dict:
    """The oracle outputs tests/golden/make_oracle_golden.py stored for a
    workload, after checking that they were computed from these inputs."""
    from tests.golden.make_oracle_golden import digest
    with np.load(GOLDEN / f"oracle_{name}.npz", allow_pickle=False) as f:
        g = {k: f[k] for k in f.files}
    assert str(g["inputs"]) == digest(*inputs), \
        f"oracle_{name}.npz was made from other inputs: run tests/golden/make_oracle_golden.py"
    return g


def row_digests(z) -> list:
    """SHA-256 (hex) of each row's little-endian int32 values."""
    import hashlib
    return [hashlib.sha256(np.ascontiguousarray(r, dtype="<i4").tobytes()).hexdigest()
            for r in z]


# ------------------------------------------------------- result files
def results_dir() -> Path:
    """Where the GPU tests write their result files: results/ (the committed
    ones), or LMHEAD_RESULTS_DIR."""
    d = Path(os.environ.get("LMHEAD_RESULTS_DIR", ROOT / "results"))
    d.mkdir(parents=True, exist_ok=True)
    return d


def record(name: str, key: str, value) -> None:
    """Merge value under key into the JSON result file <results>/<name>.json."""
    path = results_dir() / f"{name}.json"
    data = json.loads(path.read_text()) if path.exists() else {}
    data[key] = value
    path.write_text(json.dumps(data, indent=1, sort_keys=True) + "\n")


def bf16_ulps(gap, z1):
    """A top-2 gap in bf16 units in the last place of the top logit:
    gap / 2^(floor(log2 |z1|) - 7)."""
    z1 = np.abs(np.asarray(z1, dtype=np.float64))
    ulp = np.exp2(np.floor(np.log2(np.where(z1 > 0, z1, 1.0))) - 7)
    return np.asarray(gap, dtype=np.float64) / ulp
