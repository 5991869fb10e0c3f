"""Seeded Gumbel-max sampling on the GPU (through the C-ABI) against the CPU
oracle: the same draws (float32 rounding aside), the softmax distribution, and
a row's draw independent of the batch it is drawn in."""
import numpy as np
import pytest
import torch

import synth
from invariant_lm_head_amd import lmhead
from tests.gpu_util import DEV, TOL, gpu, gpu_bf16, host, i8, o, record, tl  # noqa: F401

pytestmark = pytest.mark.gpu

G_TOL = 1e-5   # float32 Gumbel noise against float64 (hardware log2, series near U = 1)


def keys(B, seed=51):
    rng = np.random.default_rng(seed)
    return (rng.integers(0, 2 ** 63, B, dtype=np.uint64) * np.uint64(2) + np.uint64(1),
            rng.integers(0, 2 ** 40, B).astype(np.int64))


def dkeys(seed_np, pos_np):
    return (torch.from_numpy(seed_np.view(np.int64)).to(DEV), gpu(pos_np))


def check_draws(tok, val, gap, o_tok, o_val, o_gap, tol):
    """Tokens equal wherever the oracle's winning lead is >= 2 tol (else the
    GPU's token must be the oracle's winner or runner-up by value); values and
    gaps within tol.  Returns the number of exempt rows."""
    h = lambda a: host(a) if isinstance(a, torch.Tensor) else np.asarray(a)  # noqa: E731
    tok, val, gap = h(tok), h(val).astype(np.float64), h(gap).astype(np.float64)
    assert np.all(np.abs(val - o_val) <= tol), np.max(np.abs(val - o_val))
    assert np.all(np.abs(gap - o_gap) <= 2 * tol), np.max(np.abs(gap - o_gap))
    exempt = o_gap < 2 * tol
    bad = (tok != o_tok) & ~exempt
    assert not bad.any(), np.nonzero(bad)[0][:10]
    return int(exempt.sum())


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_sample_vs_oracle(tl, o, T):
    B = 128
    sd, ps = keys(B)
    tok, val, gap = lmhead.sample_gumbel(tl["gx"][:B].contiguous(), tl["gw"], T, *dkeys(sd, ps))
    o_tok, o_val, o_gap = o.sample_bf16(tl["x"][:B], tl["w"], T, sd, ps)
    ex = check_draws(tok, val, gap, o_tok, o_val, o_gap, TOL / T + G_TOL)
    err = float(np.max(np.abs(host(val).astype(np.float64) - o_val)))
    record("sampling", f"tinyllama_128_rows_T{T}", {
        "rows": B, "tokens_equal": int((host(tok) == o_tok).sum()), "exempt_rows": ex,
        "max_value_error": err, "tolerance": TOL / T + G_TOL})


def test_sample_int8(i8, o):
    rows = np.array([0, 1, 2, 7, 8, 15, 16, 63, 64, 100, 255, 256, 300, 511])
    B = len(rows)
    sd, ps = keys(B, seed=52)
    scale = i8["scale"][rows].copy()
    scale[3] = -1.0                               # an invalid scale draws -1
    x = gpu(i8["x"][rows])
    tok, val, gap = (host(a) for a in lmhead.sample_gumbel(x, i8["gw"], 1.0, *dkeys(sd, ps),
                                                            row_scale=gpu(scale)))
    o_tok, o_val, o_gap = o.sample_i8(i8["x"][rows], i8["w"], 1.0, sd, ps, scale=scale)
    ok = np.arange(B) != 3
    assert tok[3] == -1 and np.isnan(val[3]) and o_tok[3] == -1
    # scaled logits |z s| <~ 20: float32 product and sum keep ~2e-6 relative
    check_draws(tok[ok], val[ok], gap[ok], o_tok[ok], o_val[ok], o_gap[ok], 1e-4)


def test_sample_row_invariance(tl):
    """A row's draw is bitwise the same alone, in a batch of 512, at another
    position in the batch and next to other rows (keys travel with the rows)."""
    B = 512
    sd, ps = keys(B, seed=53)
    x, w = tl["gx"], tl["gw"]
    tok, val, gap = (host(a) for a in lmhead.sample_gumbel(x, w, 1.0, *dkeys(sd, ps)))
    perm = np.random.default_rng(54).permutation(B)
    tp, vp, gp = (host(a) for a in lmhead.sample_gumbel(x[perm].contiguous(), w, 1.0,
                                                         *dkeys(sd[perm], ps[perm])))
    assert np.array_equal(tp, tok[perm]) and np.array_equal(vp.view(np.int32), val[perm].view(np.int32))
    for B1 in (1, 7, 33, 65, 200):
        t1, v1, _ = (host(a) for a in lmhead.sample_gumbel(x[:B1].contiguous(), w, 1.0,
                                                            *dkeys(sd[:B1], ps[:B1])))
        assert np.array_equal(t1, tok[:B1]) and np.array_equal(v1.view(np.int32),
                                                               val[:B1].view(np.int32)), B1


def _one_row_head(z_cols, n):
    V, H = len(z_cols), 64
    x = np.zeros((n, H), np.uint16)
    x[:, 0] = synth.bf16_from_f32(np.float32(1.0))
    w = np.zeros((V, H), np.uint16)
    w[:, 0] = synth.bf16_from_f32(np.asarray(z_cols, np.float32))
    return x, w


def test_sample_distribution():
    """65,536 draws from one logit row (positions 0..65535) follow softmax(z / T):
    chi-square p > 1e-6 at T = 1 and 0.5."""
    from scipy.stats import chi2
    z = np.array([1.0, 0.5, 0.0, -0.5, 2.0, 1.0, -1.0, 0.25])
    n = 65536
    x, w = _one_row_head(z, n)
    gx, gw = gpu_bf16(x), gpu_bf16(w)
    for T in (1.0, 0.5):
        sd = np.full(n, 12345, np.uint64)
        tok, _, _ = lmhead.sample_gumbel(gx, gw, T, *dkeys(sd, np.arange(n, dtype=np.int64)))
        p = np.exp(z / T - np.max(z / T))
        p /= p.sum()
        cnt = np.bincount(host(tok), minlength=len(z))
        stat = float(np.sum((cnt - n * p) ** 2 / (n * p)))
        record("sampling", f"distribution_T{T}", {"draws": n, "chi2": stat, "dof": len(z) - 1,
                                                   "p_value": float(chi2.sf(stat, len(z) - 1))})
        assert chi2.sf(stat, len(z) - 1) > 1e-6, (cnt, n * p)


def test_gumbel_noise_accuracy(o):
    """With every logit 0 the scores are the noise itself: V = 2 exposes both
    noise values of a row (value and value - gap).  120,000 of them against
    the float64 definition, within 1e-5."""
    n = 60000
    x, w = _one_row_head(np.zeros(2), n)
    sd = np.random.default_rng(55).integers(0, 2 ** 62, n, dtype=np.uint64)
    ps = np.arange(n, dtype=np.int64) * 977
    tok, val, gap = (host(a) for a in lmhead.sample_gumbel(gpu_bf16(x), gpu_bf16(w), 1.0,
                                                            *dkeys(sd, ps)))
    o_tok, o_val, o_gap = o.sample_bf16(x, w, 1.0, sd, ps)
    g_hi, g_lo = val.astype(np.float64), (val - gap).astype(np.float64)
    o_hi, o_lo = o_val, o_val - o_gap
    err = max(np.max(np.abs(g_hi - o_hi)), np.max(np.abs(g_lo - o_lo)))
    record("sampling", "gumbel_noise_accuracy", {
        "values": 2 * n, "max_abs_error": float(err), "tolerance": G_TOL,
        "noise_min": float(o_lo.min()), "noise_max": float(o_hi.max())})
    assert err <= G_TOL
    close = o_gap < 2 * G_TOL
    assert np.array_equal(tok[~close], o_tok[~close])


def test_sample_edges(o):
    """T -> 0 is the greedy head's argmax; a ragged V (1000) and a tiny V (2)."""
    d = synth.make_inputs("tiny")
    x, w = gpu_bf16(d["x"]), gpu_bf16(d["w"])
    sd, ps = keys(d["B"], seed=56)
    ids, _, margin, _ = lmhead.greedy_top2(x, w)
    tok, _, _ = lmhead.sample_gumbel(x, w, 1e-6, *dkeys(sd, ps))
    clear = host(margin) > 1e-3
    assert np.array_equal(host(tok)[clear], host(ids)[clear, 0])
    tok, val, gap = lmhead.sample_gumbel(x, w, 1.0, *dkeys(sd, ps))
    o_tok, o_val, o_gap = o.sample_bf16(d["x"], d["w"], 1.0, sd, ps)
    check_draws(tok, val, gap, o_tok, o_val, o_gap, TOL + G_TOL)
