"""HIP path against the CPU oracle, element by element, on the seeded workloads,
plus the edge cases of the method (all through the C-ABI)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from invariant_lm_head_amd import lmhead
from tests.gpu_util import (DEV, GAP_EXEMPT, TOL, bf16_ulps, check_greedy_bf16, golden,  # noqa: F401
                            gpu, gpu_bf16, host, i8, o, record, row_digests, tl)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ tiny
def test_tiny_all_calls(o):
    d = synth.make_inputs("tiny")
    x, w = gpu_bf16(d["x"]), gpu_bf16(d["w"])
    z = o.logits_bf16(d["x"], d["w"])
    zg = host(lmhead.logits(x, w)).astype(np.float64)
    assert np.max(np.abs(zg - z)) <= TOL
    # bf16-output head: within half a bf16 ulp (+ the float32 error) of the exact logit
    z16 = host(lmhead.logits(x, w, round_bf16=True).float()).astype(np.float64)
    ulp = np.exp2(np.floor(np.log2(np.abs(z))) - 7)
    assert np.all(np.abs(z16 - z) <= 0.5 * ulp + TOL)
    ids, vals, margin, raw = lmhead.greedy_top2(x, w)
    assert raw is None
    check_greedy_bf16(ids, vals, margin, *o.greedy_bf16(d["x"], d["w"]))
    lp = host(lmhead.logprob(x, w, gpu(d["target"])))
    assert np.max(np.abs(lp - o.logprob_bf16(d["x"], d["w"], d["target"]))) <= TOL


# ------------------------------------------------------------ tinyllama
@pytest.mark.parametrize("B", [1, 8, 64, 256, 512])
def test_tinyllama_greedy(tl, B):
    """Every row of every swept batch against the oracle; the exempt rows
    (oracle top-2 gap below 1e-4) are counted into the result file."""
    ids, vals, margin, _ = lmhead.greedy_top2(tl["gx"][:B].contiguous(), tl["gw"])
    o_ids, o_vals, o_margin = (a[:B] for a in tl["o_greedy"])
    exempt = check_greedy_bf16(ids, vals, margin, o_ids, o_vals, o_margin,
                               report=("parity_tinyllama_greedy", f"batch_{B}"))
    print(f"B={B}: {exempt} rows with oracle top-2 gap < {GAP_EXEMPT}", flush=True)


@pytest.mark.parametrize("B", [3, 16, 17, 65, 129, 300])
def test_tinyllama_logits(tl, o, B):
    """Full float32 logits of ragged batches (every tile variant) vs the oracle."""
    zg = host(lmhead.logits(tl["gx"][:B].contiguous(), tl["gw"]))
    rows = sorted({0, B // 2, B - 1})
    z = o.logits_bf16(tl["x"][rows], tl["w"])
    assert np.max(np.abs(zg[rows].astype(np.float64) - z)) <= TOL


def test_tinyllama_logprob(tl, o):
    """All 512 rows against the oracle."""
    B = 512
    t = tl["target"][:B]
    lp = host(lmhead.logprob(tl["gx"], tl["gw"], gpu(t)))
    ref = o.logprob_bf16(tl["x"], tl["w"], t)
    err = float(np.max(np.abs(lp - ref)))
    record("parity_tinyllama_logprob", "batch_512", {"rows": B, "max_abs_err": err})
    assert err <= TOL


# --------------------------------------------------------------- near tie
def test_neartie_fp32_vs_bf16_head():
    """Planted top-2 near ties (0 to 4 bf16 ulps), all 4,096 rows: the float32
    head against the oracle's float64 top-2 on every row (exempt rows counted);
    the planted winner on every row whose gap is >= 1e-4; the bf16-output head
    against the oracle's bf16-rounded top-2, and both heads' agreement with the
    planted winner binned by the gap in bf16 ulps, written to the result file."""
    d = synth.make_inputs("neartie")
    g = golden("neartie", d["x"], d["w"])
    x, w = gpu_bf16(d["x"]), gpu_bf16(d["w"])
    t = d["tie"]
    ids, vals, margin, _ = lmhead.greedy_top2(x, w)
    ids16, vals16, margin16, _ = lmhead.greedy_top2(x, w, round_bf16=True)
    check_greedy_bf16(ids, vals, margin, g["ids"], g["vals"], g["margin"],
                      report=("parity_neartie", "float32_head_vs_oracle"))
    ids, ids16 = host(ids), host(ids16)
    v16 = host(vals16).astype(np.float64)
    # bf16-output head: its values are bf16(float32 logit); against bf16(float64
    # logit) they differ only where the float32 logit sits within its error of
    # a bf16 rounding midpoint (counted), and then by one bf16 ulp
    ulp16 = np.exp2(np.floor(np.log2(np.maximum(np.abs(g["vals16"]), 1e-30))) - 7)
    dv = np.abs(v16 - g["vals16"])
    assert np.all((dv == 0) | (dv <= ulp16 * 1.0001))
    same16 = (ids16[:, 0] == g["ids16"][:, 0])
    want = np.where(t["gap"] == 0.0, np.minimum(t["win"], t["lose"]), t["win"])
    clear = t["gap"] >= GAP_EXEMPT
    assert np.array_equal(ids[clear, 0], want[clear])
    assert np.all(np.isin(ids[~clear, 0], np.stack([t["win"], t["lose"]])[:, ~clear]))
    ulps = t["gap"] / t["ulp"]
    table = []
    print("gap (bf16 ulp)   rows   fp32-head agree   bf16-head agree", flush=True)
    for lo, hi in [(0, 0), (0, 0.5), (0.5, 1), (1, 2), (2, 4.01)]:
        sel = (ulps == 0) if hi == 0 else (ulps > lo) & (ulps <= hi)
        a32, a16 = float(np.mean(ids[sel, 0] == want[sel])), float(np.mean(ids16[sel, 0] == want[sel]))
        table.append({"gap_bf16_ulps": [lo, hi], "rows": int(sel.sum()),
                      "float32_head_agrees": a32, "bf16_head_agrees": a16})
        print(f"  ({lo}, {hi}]  {sel.sum():6d}  {a32:.4f}  {a16:.4f}", flush=True)
    record("parity_neartie", "agreement_with_planted_winner", table)
    record("parity_neartie", "bf16_head_vs_oracle_bf16_rounding", {
        "rows": int(len(ids16)), "top1_differs": int((~same16).sum()),
        "values_differ_by_one_bf16_ulp": int((dv > 0).sum())})
    assert np.mean(ids[:, 0] == want) >= np.mean(ids16[:, 0] == want)
    # the bf16 head ties every pair whose gap is below half an ulp -> lowest id
    half = (ulps > 0) & (ulps < 0.45)
    assert np.mean(ids16[half, 0] == np.minimum(t["win"], t["lose"])[half]) > 0.95


# ------------------------------------------------------- logprob scoring
def test_logprob_full_size():
    """16,384 x 151,936 x 4,096 scoring batch (fused log-softmax, logits never
    stored) against the oracle on rows 0..255 and every 64th row."""
    d = synth.make_inputs("logprob")
    g = golden("logprob", d["x"], d["w"], d["target"])
    x, w, t = gpu_bf16(d["x"]), gpu_bf16(d["w"]), gpu(d["target"])
    lp = host(lmhead.logprob(x, w, t))
    rows = g["rows"]          # rows 0..255 and every 64th row (508 rows)
    assert np.all(np.isfinite(lp))
    err = float(np.max(np.abs(lp[rows] - g["logprob"])))
    record("parity_logprob_scoring", "rows_0_255_and_every_64th",
           {"rows": int(len(rows)), "max_abs_err": err})
    assert err <= TOL
    # batch invariance at full size: prefixes give the same bits (batches 1, 17
    # and 40 run the 256-column tiles chosen for large vocabularies)
    for B in (1, 17, 40, 512):
        lpb = host(lmhead.logprob(x[:B].contiguous(), w, t[:B].contiguous()))
        assert np.array_equal(lpb.view(np.int32), lp[:B].view(np.int32)), B


# ------------------------------------------------------------------ int8
@pytest.mark.parametrize("B", [1, 8, 64, 256, 512])
def test_int8_greedy_bit_exact(i8, B):
    """Every row of every swept batch: ids, exact raw values, scaled values and
    margin bit for bit against the oracle."""
    ids, vals, margin, raw = lmhead.greedy_top2(i8["gx"][:B].contiguous(), i8["gw"],
                                                row_scale=i8["gs"][:B].contiguous())
    g = i8["golden"]
    assert np.array_equal(host(ids), g["ids"][:B])
    assert np.array_equal(host(raw).astype(np.int64), g["raw"][:B])
    assert np.array_equal(host(vals).view(np.int32), g["vals"][:B].view(np.int32))
    assert np.array_equal(host(margin).view(np.int32), g["margin"][:B].view(np.int32))
    record("parity_int8", f"greedy_batch_{B}", {"rows": B, "bit_exact": True})


def test_int8_logits_exact(i8, o):
    """int32 logits of a 512-row call: 64 rows, one every 8 (every row tile and
    position class), equal the oracle's exact sums (per-row digests); 4 rows
    compared value by value."""
    z = lmhead.logits(i8["gx"], i8["gw"])
    g = i8["golden"]
    rows = torch.from_numpy(g["logit_rows"]).to(DEV)
    zr = host(z[rows])
    assert zr.dtype == np.int32
    assert row_digests(zr) == list(g["logit_digests"])
    assert np.array_equal(host(z[:4]).astype(np.int64), o.logits_i8(i8["x"][:4], i8["w"]))
    record("parity_int8", "logits_rows_compared", int(len(rows)))


def test_int8_logprob(i8):
    """Float log-prob of the scaled int8 logits, all 512 rows within 1e-4."""
    t = i8["target"]
    lp = host(lmhead.logprob(i8["gx"], i8["gw"], gpu(t), row_scale=i8["gs"]))
    err = float(np.max(np.abs(lp - i8["golden"]["logprob"])))
    record("parity_int8", "float_logprob_batch_512", {"rows": 512, "max_abs_err": err})
    assert err <= TOL


def test_int8_extremes_exact(o):
    """The int32 bound: all-127 rows against +-127 and -128 W rows (H = 4096)."""
    H, V = 4096, 300
    rng = np.random.default_rng(7)
    x = np.stack([np.full(H, 127, np.int8), np.full(H, -128, np.int8),
                  rng.integers(-128, 128, H).astype(np.int8)])
    w = rng.integers(-128, 128, (V, H)).astype(np.int8)
    w[0], w[1], w[2] = 127, -128, -127
    zg = host(lmhead.logits(gpu(x), gpu(w)))
    assert np.array_equal(zg.astype(np.int64), o.logits_i8(x, w))
    assert zg[0, 0] == 4096 * 127 * 127 and zg[1, 1] == 4096 * 128 * 128
    ids, vals, margin, raw = lmhead.greedy_top2(gpu(x), gpu(w))
    o_ids, o_raw, o_vals, o_margin = o.greedy_i8(x, w)
    assert np.array_equal(host(ids), o_ids) and np.array_equal(host(raw), o_raw)


# ---------------------------------------------------------------- edges
@pytest.mark.parametrize("mode", ["bf16", "int8"])
@pytest.mark.parametrize("B,H,V", [(1, 64, 2), (2, 64, 3), (5, 128, 17), (17, 64, 129),
                                   (70, 192, 130), (300, 64, 1000), (1, 4096, 257),
                                   (5, 64, 70001), (40, 128, 70001), (48, 192, 1000),
                                   (64, 256, 1000), (5, 64, 32768), (40, 64, 32769),
                                   (3, 64, 131072), (3, 64, 131073)])
def test_edge_shapes(o, mode, B, H, V):
    """Degenerate and ragged shapes through every entry point against the
    oracle.  V = 32768 and 32769 (256 and 257 blocks of 128) sit on either side
    of the folds' switch from 4 to 16 records per lane in flight; V = 131072
    and 131073 (1024 and 1025 blocks) on either side of their switch from one
    round of record loads to two."""
    rng = np.random.default_rng(B * 1000 + V)
    t = rng.integers(0, V, B).astype(np.int32)
    if mode == "bf16":
        x = synth.bf16_from_f32(rng.standard_normal((B, H)).astype(np.float32))
        w = synth.bf16_from_f32((0.1 * rng.standard_normal((V, H))).astype(np.float32))
        gx, gw = gpu_bf16(x), gpu_bf16(w)
        assert np.max(np.abs(host(lmhead.logits(gx, gw)) - o.logits_bf16(x, w))) <= TOL
        ids, vals, margin, _ = lmhead.greedy_top2(gx, gw)
        check_greedy_bf16(ids, vals, margin, *o.greedy_bf16(x, w))
        lp = host(lmhead.logprob(gx, gw, gpu(t)))
        assert np.max(np.abs(lp - o.logprob_bf16(x, w, t))) <= TOL
    else:
        x = rng.integers(-127, 128, (B, H)).astype(np.int8)
        w = rng.integers(-127, 128, (V, H)).astype(np.int8)
        s = (2.0 ** -12 * rng.uniform(0.5, 2, B)).astype(np.float32)
        gx, gw, gs = gpu(x), gpu(w), gpu(s)
        assert np.array_equal(host(lmhead.logits(gx, gw)).astype(np.int64), o.logits_i8(x, w))
        ids, vals, margin, raw = lmhead.greedy_top2(gx, gw, row_scale=gs)
        o_ids, o_raw, o_vals, o_margin = o.greedy_i8(x, w, s)
        assert np.array_equal(host(ids), o_ids) and np.array_equal(host(raw), o_raw)
        assert np.array_equal(host(vals).view(np.int32), o_vals.view(np.int32))
        assert np.array_equal(host(margin).view(np.int32), o_margin.view(np.int32))
        lp = host(lmhead.logprob(gx, gw, gpu(t), row_scale=gs))
        assert np.max(np.abs(lp - o.logprob_i8(x, w, t, s))) <= TOL


def test_wide_plans_batch_invariant():
    """At 70,001 columns (more than 256 blocks of 256) the float head runs
    32- and 64-row tiles of 128 columns at batches up to 64, 128 x 256 tiles at
    100 and 256 x 256 tiles at 200 (one row tile) and 300 (two): greedy,
    log-prob and sampled draws of every row have the same bits at batch 1, 17,
    40, 100, 200 and 300."""
    rng = np.random.default_rng(77)
    B, H, V = 300, 128, 70001
    x = gpu_bf16(synth.bf16_from_f32(rng.standard_normal((B, H)).astype(np.float32)))
    w = gpu_bf16(synth.bf16_from_f32((0.1 * rng.standard_normal((V, H))).astype(np.float32)))
    t = gpu(rng.integers(0, V, B).astype(np.int32))
    seed = gpu(rng.integers(0, 2 ** 62, B, dtype=np.int64).astype(np.uint64).view(np.int64))
    pos = gpu(np.arange(B, dtype=np.int64))

    def run(n):
        ids, vals, margin, _ = lmhead.greedy_top2(x[:n].contiguous(), w)
        lp = lmhead.logprob(x[:n].contiguous(), w, t[:n].contiguous())
        tok, val, gap = lmhead.sample_gumbel(x[:n].contiguous(), w, 0.7, seed[:n].contiguous(),
                                             pos[:n].contiguous())
        return [host(a).view(np.int32) for a in (ids, vals, margin, lp, tok, val, gap)]

    full = run(B)
    for n in (1, 17, 40, 100, 200):
        for got, ref in zip(run(n), full):
            assert np.array_equal(got, ref[:n]), n


def test_wide_plans_batch_invariant_int8():
    """The int8 head at 70,001 columns runs 512-column tiles at batches up to
    64 and the usual tiles above: every row's top-2 ids, exact raw values and
    log-prob have the same bits at batch 1, 17, 40, 100, 200 and 300."""
    rng = np.random.default_rng(78)
    B, H, V = 300, 128, 70001
    x = gpu(rng.integers(-127, 128, (B, H)).astype(np.int8))
    w = gpu(rng.integers(-127, 128, (V, H)).astype(np.int8))
    s = gpu((2.0 ** -12 * rng.uniform(0.5, 2, B)).astype(np.float32))
    t = gpu(rng.integers(0, V, B).astype(np.int32))

    def run(n):
        ids, vals, margin, raw = lmhead.greedy_top2(x[:n].contiguous(), w, row_scale=s[:n].contiguous())
        lp = lmhead.logprob(x[:n].contiguous(), w, t[:n].contiguous(), row_scale=s[:n].contiguous())
        return [host(a).view(np.int32) for a in (ids, raw, vals, margin, lp)]

    full = run(B)
    for n in (1, 17, 40, 100, 200):
        for got, ref in zip(run(n), full):
            assert np.array_equal(got, ref[:n]), n


def test_exact_ties_go_to_lowest_id():
    """Identical W rows tie exactly on the GPU too (same arithmetic wherever the
    column sits): the lowest id wins and the margin is exactly 0."""
    rng = np.random.default_rng(3)
    H, V = 256, 1000
    x = synth.bf16_from_f32(rng.standard_normal((40, H)).astype(np.float32))
    w = synth.bf16_from_f32((0.02 * rng.standard_normal((V, H))).astype(np.float32))
    for r in range(40):
        # the row's best direction planted at 3 ids: same tile, other tile, other block
        a = rng.choice(V, 3, replace=False)
        w[a] = synth.bf16_from_f32(synth.bf16_to_f32(x[r]) * np.float32(0.1))
        ids, vals, margin, _ = lmhead.greedy_top2(gpu_bf16(x[r:r + 1]), gpu_bf16(w))
        s = np.sort(a)
        assert list(host(ids)[0]) == [s[0], s[1]], (r, a)
        assert host(margin)[0] == 0.0
    xi = rng.integers(-127, 128, (1, H)).astype(np.int8)
    wi = rng.integers(-3, 4, (V, H)).astype(np.int8)
    wi[[900, 17, 400]] = xi[0]
    ids, vals, margin, raw = lmhead.greedy_top2(gpu(xi), gpu(wi))
    assert list(host(ids)[0]) == [17, 400] and host(margin)[0] == 0.0


def test_invalid_target_and_scale_give_nan(o):
    rng = np.random.default_rng(5)
    H, V, B = 64, 300, 6
    x = synth.bf16_from_f32(rng.standard_normal((B, H)).astype(np.float32))
    w = synth.bf16_from_f32((0.1 * rng.standard_normal((V, H))).astype(np.float32))
    t = np.array([-1, 0, V, 299, 2 ** 31 - 1, 5], np.int32)
    lp = host(lmhead.logprob(gpu_bf16(x), gpu_bf16(w), gpu(t)))
    assert np.isnan(lp[[0, 2, 4]]).all() and np.isfinite(lp[[1, 3, 5]]).all()
    xi = rng.integers(-127, 128, (B, H)).astype(np.int8)
    wi = rng.integers(-127, 128, (V, H)).astype(np.int8)
    s = np.array([1e-4, 0.0, -1.0, np.inf, np.nan, 2e-4], np.float32)
    ids, vals, margin, raw = lmhead.greedy_top2(gpu(xi), gpu(wi), row_scale=gpu(s))
    o_ids, o_raw, _, _ = o.greedy_i8(xi, wi, s)
    assert np.array_equal(host(ids), o_ids) and np.array_equal(host(raw), o_raw)
    v = host(vals)
    assert np.isnan(v[1:5]).all() and np.isfinite(v[[0, 5]]).all()
    lp = host(lmhead.logprob(gpu(xi), gpu(wi), gpu(np.full(B, 3, np.int32)), row_scale=gpu(s)))
    assert np.isnan(lp[1:5]).all() and np.isfinite(lp[[0, 5]]).all()


def test_workspace_contents_do_not_matter(tl):
    """One workspace, filled with junk first, serves consecutive greedy and
    log-prob calls of different sizes; results equal those of a fresh zeroed
    workspace."""
    n = lmhead.workspace_bytes(0, 512, 2048, 32000)
    ws = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=torch.Generator().manual_seed(5)).to(DEV)
    t = torch.from_numpy(np.arange(512, dtype=np.int32) * 61 % 32000).to(DEV)
    runs = []
    for B in (512, 7, 512, 1, 300):
        g = lmhead.greedy_top2(tl["gx"][:B].contiguous(), tl["gw"], ws=ws)
        lp = lmhead.logprob(tl["gx"][:B].contiguous(), tl["gw"], t[:B].contiguous(), ws=ws)
        runs.append((*g[:3], lp))
    fresh = lmhead.greedy_top2(tl["gx"], tl["gw"], ws=torch.zeros_like(ws))
    fresh_lp = lmhead.logprob(tl["gx"], tl["gw"], t, ws=torch.zeros_like(ws))
    for B, r in zip((512, 7, 512, 1, 300), runs):
        for a, b in zip(r, (*fresh[:3], fresh_lp)):
            assert torch.equal(a, b[:B])


def test_self_check_reports_no_mismatch(tl, i8):
    assert lmhead.self_check(tl["gx"][:6].contiguous(), tl["gw"]) == 0
    assert lmhead.self_check(i8["gx"][:5].contiguous(), i8["gw"]) == 0


def test_load_time_self_check_ran(tl):
    """The binding ran the device self-check in both modes and from the packed
    bf16 layout before the first call on this device, and found no logit whose
    bits depend on the batch."""
    lmhead.greedy_top2(tl["gx"][:2].contiguous(), tl["gw"])
    res = lmhead.ensure_self_check(DEV)
    assert res == {lmhead.MODE_BF16: 0, lmhead.MODE_INT8: 0, lmhead.MODE_BF16_PACKED: 0}


def test_bad_arguments_raise_before_launch(tl):
    x, w = tl["gx"][:4].contiguous(), tl["gw"]
    small = torch.zeros(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(lmhead.LMHeadError) as e:
        lmhead.greedy_top2(x, w, ws=small)
    assert e.value.status == 6
    with pytest.raises(lmhead.LMHeadError) as e:
        lmhead.logits(x[:, :100].contiguous(), w[:, :100].contiguous())
    assert e.value.status == 2
    # caller buffers the kernels would overrun are refused by the binding
    with pytest.raises(ValueError):
        lmhead.logits(x, w, out=torch.empty((4, 100), dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError):
        lmhead.logits(x, w, out=torch.empty((4, w.shape[0]), dtype=torch.bfloat16, device=DEV))
    xi, wi = torch.zeros((4, 64), dtype=torch.int8, device=DEV), torch.zeros((8, 64), dtype=torch.int8, device=DEV)
    with pytest.raises(ValueError):
        lmhead.greedy_top2(xi, wi, row_scale=torch.ones(3, device=DEV))
    with pytest.raises(ValueError):
        lmhead.greedy_top2(xi, wi, row_scale=torch.ones(4, dtype=torch.float64, device=DEV))
    with pytest.raises(ValueError):
        lmhead.greedy_top2(x, w, ws=torch.zeros((2, 1 << 20), dtype=torch.uint8, device=DEV)[:, ::2])
