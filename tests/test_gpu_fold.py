"""The top-2 fold over many blocks (through the C-ABI): a vocabulary of 70,001
columns has 547 blocks of 128 (one round of 16 records per lane), and one of
140,001 columns has 1094 (two rounds).  Greedy and sampled draws against the CPU oracle, and the gated
head against the GPU's own bf16 and float32 heads, at batches of five plans
(5, 40, 100, 200 and 300; 200 and 300 both take 256 x 256 tiles, with one row
tile and with two)."""
import math

import numpy as np
import pytest
import torch

import synth
from invariant_lm_head_amd import lmhead
from tests.gpu_util import DEV, TOL, check_greedy_bf16, gpu, gpu_bf16, host, o  # noqa: F401

pytestmark = pytest.mark.gpu

H, V = 64, 70001
G_TOL = 1e-5   # float32 Gumbel noise against float64


@pytest.fixture(scope="module")
def big():
    rng = np.random.default_rng(4242)
    x = synth.bf16_from_f32(rng.standard_normal((300, H)).astype(np.float32))
    w = synth.bf16_from_f32((0.1 * rng.standard_normal((V, H))).astype(np.float32))
    return {"x": x, "w": w, "gx": gpu_bf16(x), "gw": gpu_bf16(w)}


@pytest.mark.parametrize("B", [5, 40, 100, 200, 300])
def test_greedy_many_blocks(big, o, B):
    ids, vals, margin, _ = lmhead.greedy_top2(big["gx"][:B].contiguous(), big["gw"])
    ex = check_greedy_bf16(ids, vals, margin, *o.greedy_bf16(big["x"][:B], big["w"]))
    print(f"B={B}: {ex} exempt rows", flush=True)


@pytest.mark.parametrize("B", [5, 40, 100, 200, 300])
def test_sample_many_blocks(big, o, B):
    rng = np.random.default_rng(B)
    sd = rng.integers(0, 2 ** 63, B, dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    ps = rng.integers(0, 2 ** 40, B).astype(np.int64)
    T = 0.8
    tok, val, gap = (host(a) for a in lmhead.sample_gumbel(
        big["gx"][:B].contiguous(), big["gw"], T,
        torch.from_numpy(sd.view(np.int64)).to(DEV), gpu(ps)))
    o_tok, o_val, o_gap = o.sample_bf16(big["x"][:B], big["w"], T, sd, ps)
    tol = TOL / T + G_TOL
    assert np.all(np.abs(val.astype(np.float64) - o_val) <= tol)
    assert np.all(np.abs(gap.astype(np.float64) - o_gap) <= 2 * tol)
    exempt = o_gap < 2 * tol
    assert not ((tok != o_tok) & ~exempt).any()


def _bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.int32)


@pytest.mark.parametrize("B", [5, 40, 100, 200, 300])
def test_gated_many_blocks(big, B):
    """Bit for bit against the GPU's own heads: a row is recomputed iff its
    bf16-head margin is below tau; an ungated row is the bf16 head's result; a
    gated row holds the same two candidates valued by lmhead_logits."""
    x, w = big["gx"][:B].contiguous(), big["gw"]
    ids16, vals16, m16, _ = (host(a) if a is not None else None
                             for a in lmhead.greedy_top2(x, w, round_bf16=True))
    z = host(lmhead.logits(x, w))
    for tau in (0.02, math.inf):
        ids, vals, margin, gated = (host(a) for a in lmhead.greedy_gated(x, w, tau))
        g = gated.astype(bool)
        assert np.array_equal(g, m16 < tau), tau
        u = ~g
        assert np.array_equal(ids[u], ids16[u])
        assert np.array_equal(_bits(vals[u]), _bits(vals16[u]))
        for r in np.nonzero(g)[0]:
            assert sorted(ids[r]) == sorted(ids16[r]), r
            zr = z[r, ids[r]]
            assert np.array_equal(_bits(vals[r]), _bits(zr)), r
            assert zr[0] > zr[1] or (zr[0] == zr[1] and ids[r, 0] < ids[r, 1]), r
            assert _bits(np.float32(zr[0] - zr[1])) == _bits(margin[r]), r
        print(f"B={B} tau={tau}: {int(g.sum())} rows recomputed", flush=True)


V2 = 140001   # 1094 blocks: the fold takes two rounds of 16 records per lane


@pytest.fixture(scope="module")
def huge():
    rng = np.random.default_rng(4343)
    x = synth.bf16_from_f32(rng.standard_normal((300, H)).astype(np.float32))
    w = synth.bf16_from_f32((0.1 * rng.standard_normal((V2, H))).astype(np.float32))
    return {"x": x, "w": w, "gx": gpu_bf16(x), "gw": gpu_bf16(w)}


@pytest.mark.parametrize("B", [5, 300])
def test_greedy_two_fold_rounds(huge, o, B):
    """Rows of more than 1024 blocks: the greedy fold's second round."""
    ids, vals, margin, _ = lmhead.greedy_top2(huge["gx"][:B].contiguous(), huge["gw"])
    check_greedy_bf16(ids, vals, margin, *o.greedy_bf16(huge["x"][:B], huge["w"]))


def test_sample_two_fold_rounds(huge, o):
    B, T = 40, 0.8
    rng = np.random.default_rng(77)
    sd = rng.integers(0, 2 ** 63, B, dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    ps = rng.integers(0, 2 ** 40, B).astype(np.int64)
    tok, val, gap = (host(a) for a in lmhead.sample_gumbel(
        huge["gx"][:B].contiguous(), huge["gw"], T,
        torch.from_numpy(sd.view(np.int64)).to(DEV), gpu(ps)))
    o_tok, o_val, o_gap = o.sample_bf16(huge["x"][:B], huge["w"], T, sd, ps)
    tol = TOL / T + G_TOL
    assert np.all(np.abs(val.astype(np.float64) - o_val) <= tol)
    exempt = o_gap < 2 * tol
    assert not ((tok != o_tok) & ~exempt).any()
