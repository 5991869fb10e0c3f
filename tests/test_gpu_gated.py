"""Margin-gated float32 recompute on the GPU (through the C-ABI): the bf16-output
head decides each row unless its top-2 margin is below tau; such rows re-rank
their two candidates on their float32-head logits."""
import math

import numpy as np
import pytest

import synth
from invariant_lm_head_amd import lmhead
from tests.gpu_util import GAP_EXEMPT, TOL, gpu_bf16, host, o, tl  # noqa: F401

pytestmark = pytest.mark.gpu


def _bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.int32)


@pytest.mark.parametrize("B", [1, 3, 17, 300, 512])
def test_gated_composition(tl, B):
    """Against the GPU's own heads, bit for bit: gated = (bf16 margin < tau);
    an ungated row is the bf16-output head's result; a gated row holds the same
    two candidates, valued by the float32 head exactly as lmhead_logits gives
    them, ranked (lowest id on a tie), margin = first - second."""
    x, w = tl["gx"][:B].contiguous(), tl["gw"]
    ids16, vals16, m16, _ = (host(a) if a is not None else None
                             for a in lmhead.greedy_top2(x, w, round_bf16=True))
    z = host(lmhead.logits(x, w))
    for tau in (0.0, 1e-3, 0.05, 0.3, math.inf):
        ids, vals, margin, gated = (host(a) for a in lmhead.greedy_gated(x, w, tau))
        g = gated.astype(bool)
        assert set(np.unique(gated)) <= {0, 1}
        assert np.array_equal(g, m16 < tau), tau
        u = ~g
        assert np.array_equal(ids[u], ids16[u])
        assert np.array_equal(_bits(vals[u]), _bits(vals16[u]))
        assert np.array_equal(_bits(margin[u]), _bits(m16[u]))
        for r in np.nonzero(g)[0]:
            assert sorted(ids[r]) == sorted(ids16[r]), r
            zr = z[r, ids[r]]
            assert np.array_equal(_bits(vals[r]), _bits(zr)), r      # the float32 head's bits
            assert zr[0] > zr[1] or (zr[0] == zr[1] and ids[r, 0] < ids[r, 1]), r
            assert _bits(np.float32(zr[0] - zr[1])) == _bits(margin[r]), r
        print(f"B={B} tau={tau}: {int(g.sum())} rows recomputed", flush=True)


def _fragile(zs):
    """True where a float64 logit lies within 1e-5 of a bf16 rounding midpoint:
    there the float32 accumulation may round to the other bf16 neighbour."""
    zs = np.abs(np.asarray(zs, dtype=np.float64))
    ulp = np.exp2(np.floor(np.log2(np.maximum(zs, 1e-30))) - 7)
    frac = zs / ulp - np.floor(zs / ulp)
    return np.any(np.abs(frac - 0.5) * ulp <= 1e-5)


@pytest.mark.parametrize("tau", [1e-3, 0.05])
def test_gated_vs_oracle(tl, o, tau):
    """Against the CPU oracle's gated head (bf16 rounding of float64 logits,
    float64 re-ranking): the gate decision, the ids and the values agree on
    every row, except rows where a candidate's logit sits within 1e-5 of a
    bf16 rounding midpoint (counted; the bf16 rounding may differ there) and,
    for the order of a recomputed pair, an exact gap below 1e-4."""
    B = 128                     # the oracle's bf16 head over 32,000 columns, a few seconds
    ids, vals, margin, gated = (host(a) for a in
                                lmhead.greedy_gated(tl["gx"][:B].contiguous(), tl["gw"], tau))
    o_ids, o_vals, o_margin, o_gated = o.greedy_gated_bf16(tl["x"][:B], tl["w"], tau)
    fragile = 0
    for r in range(B):
        cand = sorted(set(ids[r]) | set(o_ids[r]))
        zc = o.logits_bf16(tl["x"][r:r + 1], tl["w"][cand], nthreads=1)[0]
        if _fragile(zc):
            fragile += 1
            continue
        assert bool(gated[r]) == bool(o_gated[r]), r
        assert set(ids[r]) == set(o_ids[r]), r
        if o_gated[r]:
            assert np.all(np.abs(vals[r] - o_vals[r]) <= TOL), r
            if o_margin[r] >= GAP_EXEMPT:
                assert list(ids[r]) == list(o_ids[r]), r
        else:
            assert list(ids[r]) == list(o_ids[r]), r
            assert np.all(vals[r].astype(np.float64) == o_vals[r]), r   # both bf16-rounded
    print(f"tau={tau}: {int(gated.sum())} of {B} rows recomputed; {fragile} fragile rows", flush=True)
    assert fragile <= 3


def test_gated_neartie(o):
    """Planted near ties (0 to 4 bf16 ulps of 6.0), 4,096 rows, tau = 1e-3: the
    bf16-output head ties every gap below half an ulp (margin 0) and those rows
    are recomputed; the gated head then picks the planted winner on every row
    whose exact gap is >= 1e-4, like the float32 head.  Prints the agreement of
    the three heads with the planted winner, binned by the gap in bf16 ulps."""
    d = synth.make_inputs("neartie")
    x, w = gpu_bf16(d["x"]), gpu_bf16(d["w"])
    t = d["tie"]
    want = np.where(t["gap"] == 0.0, np.minimum(t["win"], t["lose"]), t["win"])
    ids32 = host(lmhead.greedy_top2(x, w)[0])
    ids16, _, m16, _ = (host(a) if a is not None else None
                        for a in lmhead.greedy_top2(x, w, round_bf16=True))
    ids, vals, margin, gated = (host(a) for a in lmhead.greedy_gated(x, w, 1e-3))
    g = gated.astype(bool)
    assert np.array_equal(g, m16 < 1e-3)
    clear = t["gap"] >= GAP_EXEMPT
    assert np.array_equal(ids[clear, 0], want[clear])
    assert np.array_equal(ids[clear, 0], ids32[clear, 0])
    ulps = t["gap"] / t["ulp"]
    print(f"recomputed {g.sum()} of {len(g)} rows ({100 * g.mean():.1f}%)", flush=True)
    print("gap (bf16 ulp)   rows   bf16-head  gated-head  fp32-head", flush=True)
    for lo, hi in [(0, 0), (0, 0.5), (0.5, 1), (1, 2), (2, 4.01)]:
        sel = (ulps == 0) if hi == 0 else (ulps > lo) & (ulps <= hi)
        print(f"  ({lo}, {hi}]  {sel.sum():6d}  {np.mean(ids16[sel, 0] == want[sel]):.4f}"
              f"      {np.mean(ids[sel, 0] == want[sel]):.4f}"
              f"      {np.mean(ids32[sel, 0] == want[sel]):.4f}", flush=True)
    assert np.mean(ids[:, 0] == want) > np.mean(ids16[:, 0] == want)


def test_gated_edges(o):
    """tau = 0 recomputes nothing (the bf16 head bit for bit); V = 2; a row of
    zeros (every logit 0: margin 0, recomputed, tie -> ids 0, 1)."""
    rng = np.random.default_rng(31)
    H, V = 64, 2
    xb = synth.bf16_from_f32(rng.standard_normal((4, H)).astype(np.float32))
    xb[3] = 0
    wb = synth.bf16_from_f32((0.05 * rng.standard_normal((V, H))).astype(np.float32))
    x, w = gpu_bf16(xb), gpu_bf16(wb)
    ids16, vals16, m16, _ = lmhead.greedy_top2(x, w, round_bf16=True)
    ids, vals, margin, gated = lmhead.greedy_gated(x, w, 0.0)
    assert not host(gated).any()
    assert np.array_equal(host(ids), host(ids16)) and np.array_equal(host(vals), host(vals16))
    ids, vals, margin, gated = (host(a) for a in lmhead.greedy_gated(x, w, math.inf))
    assert gated.all()
    o_ids, o_vals, o_margin, o_gated = o.greedy_gated_bf16(xb, wb, math.inf)
    assert np.array_equal(ids[3], [0, 1]) and margin[3] == 0.0
    ok = o_margin >= GAP_EXEMPT
    assert np.array_equal(ids[ok], o_ids[ok])
    assert np.all(np.abs(vals - o_vals) <= TOL)
