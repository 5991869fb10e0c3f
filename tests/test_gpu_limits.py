"""The boundary's largest shapes (through the C-ABI): the most rows a call
accepts (B = 2^24), the longest k chain of the float head (H = 2^20) and of
the int8 head (H = 131008, the largest multiple of 64 whose extreme sums still
fit int32).  Sampled or whole outputs against the oracle."""
import numpy as np
import pytest
import torch

import synth
from invariant_lm_head_amd import lmhead
from tests.gpu_util import DEV, TOL, check_greedy_bf16, gpu, gpu_bf16, host, o  # noqa: F401

pytestmark = pytest.mark.gpu


def test_max_rows(o):
    """B = 2^24 rows (H = 64, V = 300): greedy top-2 and log-prob of 48 rows,
    the first, middle and last among them, against the oracle."""
    B, H, V = 1 << 24, 64, 300
    g = torch.Generator(device=DEV).manual_seed(11)
    x = torch.empty((B, H), dtype=torch.bfloat16, device=DEV)
    for r0 in range(0, B, 1 << 22):               # bounded fp32 staging
        x[r0:r0 + (1 << 22)] = torch.randn((1 << 22, H), device=DEV, generator=g).to(torch.bfloat16)
    rng = np.random.default_rng(12)
    wb = synth.bf16_from_f32((0.1 * rng.standard_normal((V, H))).astype(np.float32))
    w = gpu_bf16(wb)
    t = torch.randint(0, V, (B,), device=DEV, generator=g, dtype=torch.int32)
    ids, vals, margin, _ = lmhead.greedy_top2(x, w)
    lp = lmhead.logprob(x, w, t)
    rows = np.unique(np.concatenate([[0, 1, B // 2, B - 2, B - 1], rng.integers(0, B, 43)]))
    ri = torch.from_numpy(rows).to(DEV)
    xr = host(x[ri].contiguous().view(torch.int16)).view(np.uint16)
    check_greedy_bf16(ids[ri], vals[ri], margin[ri], *o.greedy_bf16(xr, wb))
    tr = host(t[ri])
    assert np.max(np.abs(host(lp[ri]) - o.logprob_bf16(xr, wb, tr))) <= TOL
    del x, ids, vals, margin, lp, t
    torch.cuda.empty_cache()


def test_max_hidden_float_exact(o):
    """H = 2^20 (the longest chain the boundary accepts) with entries in
    {-1, 0, 1}: every float32 partial sum is an integer below 2^24, so the
    logits are exact and equal the oracle's; ids follow, ties included."""
    B, H, V = 3, 1 << 20, 130
    rng = np.random.default_rng(13)
    one = np.array([0xBF80, 0x0000, 0x3F80], dtype=np.uint16)   # bf16 -1, 0, 1
    xb = one[rng.integers(0, 3, (B, H))]
    wb = one[rng.integers(0, 3, (V, H))]
    x, w = gpu_bf16(xb), gpu_bf16(wb)
    z = host(lmhead.logits(x, w)).astype(np.float64)
    zo = o.logits_bf16(xb, wb)
    assert np.array_equal(z, zo)
    ids, vals, margin, _ = lmhead.greedy_top2(x, w)
    o_ids, o_vals, o_margin = o.greedy_bf16(xb, wb)
    assert np.array_equal(host(ids), o_ids)
    assert np.array_equal(host(vals).astype(np.float64), o_vals)
    t = rng.integers(0, V, B).astype(np.int32)
    lp = host(lmhead.logprob(x, w, gpu(t)))
    assert np.max(np.abs(lp - o.logprob_bf16(xb, wb, t))) <= TOL


# H = 131008 int8 rows and vocabulary rows whose sums reach both ends of int32
H_I8_MAX = 131008
S_I8_MAX = np.float32(2.0 ** -26)   # scale that maps a 2^32 logit span to about 64 nats


def _int8_extremes(V):
    """Row 0 all -128 against vocabulary row 0 all -128 (z = 16384 H =
    2,146,435,072) and row 1 all +127 (z = -16256 H = -2,129,666,048); the
    other entries random.  Row 1 of x random."""
    rng = np.random.default_rng(14)
    x = rng.integers(-128, 128, (2, H_I8_MAX)).astype(np.int8)
    x[0] = -128
    w = rng.integers(-128, 128, (V, H_I8_MAX)).astype(np.int8)
    w[0] = -128
    w[1] = 127
    return x, w


@pytest.mark.parametrize("V", [2, 129])
def test_max_hidden_int8_exact(o, V):
    """H = 131008 int8: the logits of row 0 reach +2^31 - 2^20 and -2^31 + 2^24,
    so their differences exceed the int32 range (V = 2: the margin is 32640 H =
    4,276,101,120).  Logits, ids, raw and scaled top values and the margin
    bit-exact; the float log-prob of every target within 1e-4 (scale 2^-26)."""
    x, w = _int8_extremes(V)
    B = x.shape[0]
    gx, gw = gpu(x), gpu(w)
    z = host(lmhead.logits(gx, gw)).astype(np.int64)
    zo = o.logits_i8(x, w)
    assert zo[0, 0] == 16384 * H_I8_MAX and zo[0, 1] == -16256 * H_I8_MAX
    assert np.array_equal(z, zo)
    for s in (np.ones(B, dtype=np.float32), np.full(B, S_I8_MAX, dtype=np.float32)):
        ids, vals, margin, raw = lmhead.greedy_top2(gx, gw, row_scale=gpu(s))
        o_ids, o_raw, o_vals, o_margin = o.greedy_i8(x, w, s)
        assert np.array_equal(host(ids), o_ids) and np.array_equal(host(raw), o_raw)
        assert np.array_equal(host(vals).view(np.int32), o_vals.view(np.int32))
        assert np.array_equal(host(margin).view(np.int32), o_margin.view(np.int32))
        if V == 2:
            assert o_raw[0, 0] - o_raw[0, 1] == 32640 * H_I8_MAX > 2 ** 32 - 2 ** 25
            assert host(margin)[0] > 0
    s = np.full(B, S_I8_MAX, dtype=np.float32)
    for t in range(min(V, 4)):
        tgt = np.full(B, t, dtype=np.int32)
        lp = host(lmhead.logprob(gx, gw, gpu(tgt), row_scale=gpu(s)))
        lo = o.logprob_i8(x, w, tgt, s)
        assert np.all(np.isfinite(lp)), lp
        assert np.max(np.abs(lp - lo)) <= TOL, (t, lp, lo)
