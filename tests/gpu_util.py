"""Helpers shared by the GPU tests: host <-> device copies and the comparison
rules of the head against the oracle (not collected as tests)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth

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


def check_greedy_bf16(ids, vals, margin, o_ids, o_vals, o_margin, tol=TOL):
    """float32-head top-2 against the oracle; returns the number of exempt rows.

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
    """The 4096 x 128256 int8 head, 512 rows, oracle greedy on sampled rows."""
    d = synth.make_inputs("int8")
    d["gx"], d["gw"], d["gs"] = gpu(d["x"]), gpu(d["w"]), gpu(d["scale"])
    rows = np.array([0, 1, 2, 7, 8, 15, 16, 63, 64, 100, 255, 256, 300, 511])
    d["rows"] = rows
    d["o_greedy"] = o.greedy_i8(d["x"][rows], d["w"], d["scale"][rows])
    return d
