"""Seeded synthetic inputs for the batch-invariant LM head.

This module only *makes inputs*: it holds none of the head's arithmetic (no
logits, argmax or softmax).  Both the CPU oracle (``oracle/``) and the HIP path
(``invariant_lm_head_amd``) are fed from here, and nothing else is shared
between them.

Recipe (the pages train and score real checkpoints on GSM8K/HumanEval/MBPP,
WikiText2/C4 and GRPO rollouts; none of that is reproduced, head-shaped
synthetic rows stand in for it):

* numpy ``default_rng`` (PCG64); seed = 100*c + j for workload c (1..5) and
  stream j (1 W, 2 hidden rows, 3 target ids, 4 row scales, 5 near-tie
  construction).  Large arrays are drawn in fixed row blocks, each block from
  ``default_rng([seed, block])``, so a prefix of rows is the same whatever the
  total row count: a row's bits are identical at batch 1 and batch 512.
* bf16 values are produced from float32 by round-to-nearest-even on the bit
  pattern; the data contain no NaN or Inf.
* "RMS-normalised" hidden rows: x ~ N(0,1) in float64, h = x / sqrt(mean(x^2))
  (gain 1, eps 0), cast to float32 then rounded to bf16.
* int8 tensors are uniform integers in [-127, 127]; per-row scales are
  float32(2^-18 * U[0.5, 2]).
* integer hidden rows (the input of the int8 head's per-token quantisation,
  stream 6): x ~ N(0,1) with 8 outlier channels (drawn once per seed) scaled
  by 12, RMS-normalised per row in float64, then round(h * 2^10) as int32.
  Their tensor unit: one unit of hidden (2^-10) times one unit of W,
  1 / (32 * 73.6) (73.6 = the standard deviation of uniform integers in
  [-127, 127]), so a logit has a standard deviation near 2; given as a
  31-bit dyadic INT_UNIT = (m, e), real value m 2^e.

Workloads (sizes from the head shapes the pages discuss: a TinyLlama-sized
head, a 151,936-token vocabulary for teacher-forced scoring, a 128,256-token
integer head):

  tiny      H=64,   V=1000,   B=4      bf16, hidden ~ N(0,1), W ~ N(0, 0.02)
  tinyllama H=2048, V=32000,  B<=512   bf16, RMS-normalised hidden, W ~ N(0, 0.02)
  neartie   H=2048, V=32000,  B=4096   tinyllama W with planted top-2 near ties
  logprob   H=4096, V=151936, B=16384  bf16 as tinyllama, target ids uniform
  int8      H=4096, V=128256, B<=512   int8 x int8, per-row fp32 scale
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "bf16_from_f32", "bf16_to_f32", "bf16_to_f64",
    "normal_bf16", "hidden_rms_bf16", "target_ids", "int8_uniform",
    "row_scales", "near_tie", "make_inputs", "hidden_int32", "INT_UNIT",
]

ROW_BLOCK = 4096  # rows per independently seeded block


@dataclass(frozen=True)
class Workload:
    name: str
    c: int          # workload number used in the seed layout
    H: int
    V: int
    B: int          # largest batch (rows)
    mode: str       # "bf16" or "int8"
    batches: tuple  # batch sizes swept (prefixes of the B rows)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 64, 1000, 4, "bf16", (4,)),
    "tinyllama": Workload("tinyllama", 2, 2048, 32000, 512, "bf16",
                          (1, 8, 64, 256, 512)),
    "neartie": Workload("neartie", 3, 2048, 32000, 4096, "bf16", (4096,)),
    "logprob": Workload("logprob", 4, 4096, 151936, 16384, "bf16", (16384,)),
    "int8": Workload("int8", 5, 4096, 128256, 512, "int8",
                     (1, 8, 64, 256, 512)),
}


def seed_of(c: int, j: int) -> int:
    return 100 * c + j


# ----------------------------------------------------------------- bf16 bits
def bf16_from_f32(a) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(u) -> np.ndarray:
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(u) -> np.ndarray:
    return bf16_to_f32(u).astype(np.float64)


def _blocks(rows: int):
    for blk in range((rows + ROW_BLOCK - 1) // ROW_BLOCK):
        lo = blk * ROW_BLOCK
        yield blk, lo, min(rows, lo + ROW_BLOCK)


# ------------------------------------------------------------- generators
def normal_bf16(seed: int, rows: int, cols: int, std: float) -> np.ndarray:
    """bf16(float32(std * N(0,1))) as uint16 [rows, cols]."""
    out = np.empty((rows, cols), dtype=np.uint16)
    for blk, lo, hi in _blocks(rows):
        rng = np.random.default_rng([seed, blk])
        x = rng.standard_normal((hi - lo, cols), dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[lo:hi] = bf16_from_f32(x)
    return out


def hidden_rms_bf16(seed: int, rows: int, cols: int) -> np.ndarray:
    """RMS-normalised Gaussian rows (gain 1, eps 0), rounded to bf16."""
    out = np.empty((rows, cols), dtype=np.uint16)
    for blk, lo, hi in _blocks(rows):
        rng = np.random.default_rng([seed, blk])
        x = rng.standard_normal((hi - lo, cols))
        x /= np.sqrt(np.mean(x * x, axis=1, keepdims=True))
        out[lo:hi] = bf16_from_f32(x.astype(np.float32))
    return out


def target_ids(seed: int, rows: int, V: int) -> np.ndarray:
    out = np.empty(rows, dtype=np.int32)
    for blk, lo, hi in _blocks(rows):
        rng = np.random.default_rng([seed, blk])
        out[lo:hi] = rng.integers(0, V, size=hi - lo, dtype=np.int64)
    return out


def int8_uniform(seed: int, rows: int, cols: int) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.int8)
    for blk, lo, hi in _blocks(rows):
        rng = np.random.default_rng([seed, blk])
        out[lo:hi] = rng.integers(-127, 128, size=(hi - lo, cols), dtype=np.int8)
    return out


def hidden_int32(seed: int, rows: int, cols: int, frac_bits: int = 10,
                 outliers: int = 8, gain: float = 12.0) -> np.ndarray:
    """RMS-normalised Gaussian rows with a few outlier channels, in fixed
    point with ``frac_bits`` fractional bits, as int32 [rows, cols]."""
    chans = np.random.default_rng([seed, 1 << 20]).choice(cols, size=min(outliers, cols),
                                                          replace=False)
    out = np.empty((rows, cols), dtype=np.int32)
    for blk, lo, hi in _blocks(rows):
        rng = np.random.default_rng([seed, blk])
        x = rng.standard_normal((hi - lo, cols))
        x[:, chans] *= gain
        x /= np.sqrt(np.mean(x * x, axis=1, keepdims=True))
        out[lo:hi] = np.rint(x * 2.0 ** frac_bits).astype(np.int32)
    return out


def _dyadic31(v: float):
    """(m, e) with 2^30 <= m < 2^31 and m 2^e the nearest such value to v > 0."""
    e = math.floor(math.log2(v)) - 30
    m = round(v / 2.0 ** e)
    if m == 2 ** 31:
        m, e = 2 ** 30, e + 1
    return int(m), int(e)


INT_UNIT = _dyadic31(2.0 ** -10 / (32.0 * math.sqrt((255 ** 2 - 1) / 12.0)))


def row_scales(seed: int, rows: int) -> np.ndarray:
    out = np.empty(rows, dtype=np.float32)
    for blk, lo, hi in _blocks(rows):
        rng = np.random.default_rng([seed, blk])
        out[lo:hi] = (2.0 ** -18 * rng.uniform(0.5, 2.0, size=hi - lo)).astype(np.float32)
    return out


# ------------------------------------------------------- near-tie builder
def _shrink_bf16(bits: np.ndarray, steps: np.ndarray) -> np.ndarray:
    """Move bf16 values `steps` representable values toward zero (never past it)."""
    sign = bits & np.uint16(0x8000)
    mag = (bits & np.uint16(0x7FFF)).astype(np.int64)
    mag = np.maximum(mag - steps, 0)
    return (sign | mag.astype(np.uint16)).astype(np.uint16)


def near_tie(W: np.ndarray, X: np.ndarray, seed: int, max_ulps: float = 4.0,
             frac_exact: float = 0.125, logit: float = 6.0, max_steps: int = 16):
    """Plant a top-2 near tie in every hidden row.

    For row r a distinct vocab pair (a_r, b_r) is drawn.  The winner's W row is
    set to bf16(c * h_r) with c = logit / H, so its logit is ~``logit`` (well
    above the random logits); the loser's row is the same vector with the
    largest-|h| coordinates shrunk toward zero by whole bf16 steps until the
    exact gap z_win - z_lose reaches d_r bf16 ulps of the winner's logit, with
    d_r ~ U[0, max_ulps].  A fraction ``frac_exact`` of rows get d_r = 0 (two
    identical W rows: an exact tie).  Which id of the pair wins is random, so
    the winner is the higher id about half the time.

    The gap is recorded exactly: each coordinate's contribution h_k*(w_k - w'_k)
    is a product of a bf16 value and a difference of two nearby bf16 values,
    exact in float64, and the contributions are summed with math.fsum.

    Returns (W', info) where W' is a modified copy of W and info holds int32
    arrays ``win``, ``lose`` and float64 ``gap``, ``ulp``.
    """
    rng = np.random.default_rng(seed)
    W = W.copy()
    V, H = W.shape
    R = X.shape[0]
    assert 2 * R <= V
    perm = rng.permutation(V)[: 2 * R]
    a, b = perm[0::2], perm[1::2]
    d = rng.uniform(0.0, max_ulps, size=R)
    d[rng.random(R) < frac_exact] = 0.0
    hi_wins = rng.random(R) < 0.5
    lo_id, hi_id = np.minimum(a, b), np.maximum(a, b)
    win = np.where(hi_wins, hi_id, lo_id).astype(np.int32)
    lose = np.where(hi_wins, lo_id, hi_id).astype(np.int32)

    c = np.float32(logit / H)
    h32 = bf16_to_f32(X)
    base = bf16_from_f32(h32 * c)                      # [R, H] uint16
    hb = h32.astype(np.float64)
    gap = np.zeros(R)
    ulp = np.zeros(R)
    for r in range(R):
        wrow = base[r]
        z_win = math.fsum((hb[r] * bf16_to_f64(wrow)).tolist())
        e = math.floor(math.log2(abs(z_win)))
        ulp[r] = 2.0 ** (e - 7)
        target = d[r] * ulp[r]
        lrow = wrow.copy()
        if target > 0.0:
            order = np.argsort(-np.abs(hb[r]), kind="stable")
            full = _shrink_bf16(wrow[order], np.full(H, max_steps))
            gains = hb[r][order] * (bf16_to_f64(wrow[order]) - bf16_to_f64(full))
            csum = np.cumsum(gains)
            n = int(np.searchsorted(csum, target))      # coords fully shrunk: [0, n)
            assert n < H, "near-tie target gap not reachable"
            lrow[order[:n]] = full[:n]
            rest = target - (csum[n - 1] if n else 0.0)
            k = order[n]
            for s in range(1, max_steps + 1):
                cand = _shrink_bf16(wrow[k:k + 1], np.array([s]))[0]
                if hb[r][k] * (bf16_to_f64(wrow[k]) - bf16_to_f64(cand)) >= rest:
                    break
            lrow[k] = cand
        diff = hb[r] * (bf16_to_f64(wrow) - bf16_to_f64(lrow))
        gap[r] = math.fsum(diff.tolist())
        W[win[r]] = wrow
        W[lose[r]] = lrow
    return W, {"win": win, "lose": lose, "gap": gap, "ulp": ulp, "d": d}


# ---------------------------------------------------------------- workloads
def make_inputs(name: str, rows: int | None = None, with_weights: bool = True):
    """All inputs of a workload as numpy arrays (rows = prefix of the batch).

    bf16 tensors are uint16 bit patterns, int8 tensors int8, targets int32 and
    scales float32.
    """
    wl = WORKLOADS[name]
    B = wl.B if rows is None else rows
    c = wl.c
    out = {"H": wl.H, "V": wl.V, "B": B, "mode": wl.mode}
    if wl.mode == "int8":
        if with_weights:
            out["w"] = int8_uniform(seed_of(c, 1), wl.V, wl.H)
        out["x"] = int8_uniform(seed_of(c, 2), B, wl.H)
        out["scale"] = row_scales(seed_of(c, 4), B)
        out["hidden"] = hidden_int32(seed_of(c, 6), B, wl.H)
        out["unit"] = INT_UNIT
    elif name == "tiny":
        if with_weights:
            out["w"] = normal_bf16(seed_of(c, 1), wl.V, wl.H, 0.02)
        out["x"] = normal_bf16(seed_of(c, 2), B, wl.H, 1.0)
    elif name == "neartie":
        # always planted over all rows, so a prefix sees the same W and pairs
        x = hidden_rms_bf16(seed_of(c, 2), wl.B, wl.H)
        w = normal_bf16(seed_of(2, 1), wl.V, wl.H, 0.02)   # the tinyllama W
        w, info = near_tie(w, x, seed_of(c, 5))
        out.update(x=x[:B], tie={k: v[:B] for k, v in info.items()})
        if with_weights:
            out["w"] = w
    else:
        if with_weights:
            out["w"] = normal_bf16(seed_of(c, 1), wl.V, wl.H, 0.02)
        out["x"] = hidden_rms_bf16(seed_of(c, 2), B, wl.H)
    out["target"] = target_ids(seed_of(c, 3), B, wl.V)
    return out
