"""Pins of the CPU oracle against what mathematics and the pages fix.

Every pin takes an ``oracle.Oracle`` and raises AssertionError when it
disagrees.  None of them re-types the oracle's formula or re-calls its code:
they compare with exact rational arithmetic (``fractions``), 50-digit
``decimal`` arithmetic, an independent BLAS (numpy float64 / int64 matmul),
brute-force sorting, closed forms and invariants.  ``FAST`` pins also run
against copies of the oracle with a planted mistake (test_oracle_mutants.py).
"""
from __future__ import annotations

import json
import math
from decimal import Decimal, getcontext
from fractions import Fraction
from pathlib import Path

import numpy as np

import synth

GOLDEN = Path(__file__).resolve().parent / "golden"


# ------------------------------------------------------------- helpers
def rand_bf16(rng, shape, emin=-8, emax=3):
    """Random bf16 bit patterns: random sign, exponent in [emin, emax], mantissa."""
    sign = rng.integers(0, 2, shape).astype(np.uint32) << 15
    expo = rng.integers(127 + emin, 127 + emax + 1, shape).astype(np.uint32) << 7
    mant = rng.integers(0, 128, shape).astype(np.uint32)
    return (sign | expo | mant).astype(np.uint16)


def bf16_const(v: float, shape):
    return np.full(shape, synth.bf16_from_f32(np.float32(v)).item(), dtype=np.uint16)


def fracs(a):
    return [[Fraction(float(v)) for v in row] for row in a]


def dec(fr: Fraction) -> Decimal:
    return Decimal(fr.numerator) / Decimal(fr.denominator)


def float32_rne(fr: Fraction) -> float:
    """Nearest float32 (ties to even) of an exact rational (normal range)."""
    if fr == 0:
        return 0.0
    sgn = -1 if fr < 0 else 1
    a = abs(fr)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = a / Fraction(2) ** (e - 23)          # in [2^23, 2^24)
    n = math.floor(q)
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sgn * float(Fraction(n) * Fraction(2) ** (e - 23))


# ------------------------------------------------------------ logits
def pin_logits_bruteforce(o):
    """Float64 logits equal the exact rational dot products within the
    sequential-summation bound H * 2^-52 * sum|terms|."""
    rng = np.random.default_rng(11)
    for _ in range(40):
        B, H, V = int(rng.integers(1, 5)), int(rng.integers(1, 9)), int(rng.integers(2, 17))
        x, w = rand_bf16(rng, (B, H)), rand_bf16(rng, (V, H))
        z = o.logits_bf16(x, w)
        xf, wf = fracs(synth.bf16_to_f64(x)), fracs(synth.bf16_to_f64(w))
        for r in range(B):
            for v in range(V):
                terms = [xf[r][k] * wf[v][k] for k in range(H)]
                exact = sum(terms)
                bound = Fraction(H) * Fraction(2) ** -52 * sum(abs(t) for t in terms)
                assert abs(Fraction(float(z[r, v])) - exact) <= bound, (r, v)


def pin_logits_one_hot(o):
    """x = e_k picks column k of W: z[k, v] == W[v, k] exactly (V != H, so a
    transposed or mis-strided operand cannot pass)."""
    rng = np.random.default_rng(12)
    H, V = 24, 37
    x = np.zeros((H, H), np.uint16)
    x[np.arange(H), np.arange(H)] = bf16_const(1.0, ()).item()
    w = rand_bf16(rng, (V, H))
    z = o.logits_bf16(x, w)
    assert np.array_equal(z, synth.bf16_to_f64(w).T)
    xi = np.eye(H, dtype=np.int8)
    wi = rng.integers(-128, 128, (V, H)).astype(np.int8)
    assert np.array_equal(o.logits_i8(xi, wi), wi.astype(np.int64).T)


def pin_logits_closed_forms(o):
    """W = 0 gives z = 0; constant rows give z = H * c * d exactly."""
    H, V = 64, 9
    rng = np.random.default_rng(13)
    x = rand_bf16(rng, (3, H))
    assert np.all(o.logits_bf16(x, np.zeros((V, H), np.uint16)) == 0.0)
    c, ds = 0.375, [-1.25, 0.5, 3.0, -0.0078125, 2.0, 1.5, -6.0, 0.25, 1.0]
    xc = bf16_const(c, (2, H))
    wd = np.stack([bf16_const(d, (H,)) for d in ds])
    z = o.logits_bf16(xc, wd)
    assert np.array_equal(z[0], np.array([H * c * d for d in ds]))
    xi = np.full((2, H), -7, np.int8)
    wi = np.stack([np.full(H, d, np.int8) for d in (5, -128, 127, 0)])
    assert np.array_equal(o.logits_i8(xi, wi)[1], np.array([H * -7 * d for d in (5, -128, 127, 0)]))


def pin_int_logits_bruteforce(o):
    """int8 logits equal Python's arbitrary-precision integer dot products."""
    rng = np.random.default_rng(14)
    for _ in range(20):
        B, H, V = int(rng.integers(1, 5)), int(rng.integers(1, 40)), int(rng.integers(2, 17))
        x = rng.integers(-128, 128, (B, H)).astype(np.int8)
        w = rng.integers(-128, 128, (V, H)).astype(np.int8)
        z = o.logits_i8(x, w)
        for r in range(B):
            for v in range(V):
                assert int(z[r, v]) == sum(int(x[r, k]) * int(w[v, k]) for k in range(H))


def pin_int_overflow_bound(o):
    """An all-127 row against an all-127 W row at H = 4096 hits the stated bound
    4096 * 127^2 = 66,064,384 < 2^31 exactly; -128 squared at H = 131,071 stays
    below 2^31 too."""
    x = np.full((1, 4096), 127, np.int8)
    w = np.stack([np.full(4096, 127, np.int8), np.full(4096, -127, np.int8)])
    assert o.logits_i8(x, w).tolist() == [[66064384, -66064384]]
    H = 131071
    z = o.logits_i8(np.full((1, H), -128, np.int8), np.full((1, H), -128, np.int8))
    assert int(z[0, 0]) == H * 128 * 128 < 2 ** 31


def pin_logits_vs_blas(o):
    """float64 logits agree with an independent BLAS (numpy float64 matmul)
    within 1e-9 on the tiny workload and eight rows of the 2048 x 32000 head."""
    d = synth.make_inputs("tiny")
    ref = synth.bf16_to_f64(d["x"]) @ synth.bf16_to_f64(d["w"]).T
    assert np.max(np.abs(o.logits_bf16(d["x"], d["w"]) - ref)) <= 1e-9
    d = synth.make_inputs("tinyllama", rows=8)
    ref = synth.bf16_to_f64(d["x"]) @ synth.bf16_to_f64(d["w"]).T
    assert np.max(np.abs(o.logits_bf16(d["x"], d["w"]) - ref)) <= 1e-9


def pin_int_logits_vs_numpy(o):
    """int8-workload rows: int64 logits equal numpy's exact int64 matmul on a
    slice of 8,192 vocabulary rows."""
    d = synth.make_inputs("int8", rows=4)
    w = d["w"][-8192:]
    ref = d["x"].astype(np.int64) @ w.astype(np.int64).T
    assert np.array_equal(o.logits_i8(d["x"], w), ref)


# ------------------------------------------------------------- greedy
def _brute_top2(z):
    order = sorted(range(len(z)), key=lambda v: (-z[v], v))
    return order[:2]


def pin_top2_bruteforce(o):
    """Top-2 ids equal brute-force sorting by (value desc, id asc), with many
    exact ties (values from a small set)."""
    rng = np.random.default_rng(21)
    for _ in range(300):
        V = int(rng.integers(2, 13))
        zi = rng.integers(-3, 4, V)
        ids, vals = o.top2_f64(zi.astype(np.float64))
        assert list(ids) == _brute_top2(list(zi)), zi
        assert list(vals) == [float(zi[i]) for i in _brute_top2(list(zi))]
        ids, vals = o.top2_i64(zi.astype(np.int64))
        assert list(ids) == _brute_top2(list(zi)), zi


def pin_top2_hand_ties(o):
    """The maximum at ids 5, 2 and 9: top-1 = 2 and top-2 = 5, margin 0
    (lowest-id tie rule)."""
    z = np.zeros(12)
    z[[5, 2, 9]] = 4.0
    z[7] = 3.9
    ids, vals = o.top2_f64(z)
    assert list(ids) == [2, 5] and vals[0] - vals[1] == 0.0
    ids, _ = o.top2_i64(z.astype(np.int64) * 0 + np.where(z == 4.0, 7, 1))
    assert list(ids) == [2, 5]


def pin_greedy_identical_rows(o):
    """Two identical dominant W rows (ids 3 and 7) tie exactly: top-1 = 3,
    top-2 = 7, margin 0, whatever their order in memory."""
    rng = np.random.default_rng(22)
    H, V = 64, 16
    x = rand_bf16(rng, (2, H), emin=-2, emax=1)
    w = rand_bf16(rng, (V, H), emin=-12, emax=-9)
    w[3] = w[7] = synth.bf16_from_f32(synth.bf16_to_f32(x[0]) * np.float32(0.5))
    ids, vals, margin = o.greedy_bf16(x[:1], w)
    assert list(ids[0]) == [3, 7] and margin[0] == 0.0
    xi = rng.integers(-127, 128, (1, H)).astype(np.int8)
    wi = rng.integers(-3, 4, (V, H)).astype(np.int8)
    wi[3] = wi[7] = xi[0]
    ids, raw, vals, margin = o.greedy_i8(xi, wi)
    assert list(ids[0]) == [3, 7] and raw[0, 0] == raw[0, 1] and margin[0] == 0.0


def pin_greedy_permutation(o):
    """Permuting W's rows permutes the chosen ids (tie-free data)."""
    d = synth.make_inputs("tiny")
    rng = np.random.default_rng(23)
    perm = rng.permutation(d["V"])
    ids, vals, _ = o.greedy_bf16(d["x"], d["w"])
    ids_p, vals_p, _ = o.greedy_bf16(d["x"], d["w"][perm])
    assert np.array_equal(perm[ids_p], ids) and np.array_equal(vals, vals_p)


def pin_greedy_near_ties(o):
    """Hand-built gaps from exact bf16 edits: 0, one float64 ulp of 6.0, 2^-17,
    2^-14 (< 1e-4), 2^-13 (> 1e-4) and one bf16 ulp of 6.0 (1/32).  Rows a (id
    9) and b (id 4) share the logit 6.0; a's last coordinate adds the gap.  The
    float64 head resolves every gap exactly (winner 9, margin == gap; tie ->
    id 4); the bf16-output head ties every gap below half a bf16 ulp."""
    H, V = 64, 12
    gaps = [0.0, 2.0 ** -50, 2.0 ** -17, 2.0 ** -14, 2.0 ** -13, 2.0 ** -5]
    rng = np.random.default_rng(24)
    for g in gaps:
        x = bf16_const(1.0, (1, H))
        w = rand_bf16(rng, (V, H), emin=-14, emax=-12)
        w[4] = w[9] = 0
        w[4, 0] = w[9, 0] = bf16_const(6.0, ()).item()
        w[9, H - 1] = synth.bf16_from_f32(np.float32(g)).item()
        assert float(synth.bf16_to_f64(w[9, H - 1:])[0]) == g
        ids, vals, margin = o.greedy_bf16(x, w)
        if g == 0.0:
            assert list(ids[0]) == [4, 9] and margin[0] == 0.0
        else:
            assert list(ids[0]) == [9, 4] and margin[0] == g
        exempt = margin[0] < 1e-4                 # the 1e-4 argmax exemption rule
        assert exempt == (g < 1e-4)
        ids16, vals16, margin16 = o.greedy_bf16(x, w, round_bf16=True)
        if g < 2.0 ** -6:
            assert list(ids16[0]) == [4, 9] and margin16[0] == 0.0 and vals16[0, 0] == 6.0
        else:
            assert list(ids16[0]) == [9, 4] and margin16[0] == g


def pin_gated_hand_cases(o):
    """The margin-gated head on the near-tie rows of pin_greedy_near_ties (ids
    9 and 4 share the logit 6.0; id 9 adds the gap g), one row per gap in one
    batch.  The bf16-output head ties every gap below half a bf16 ulp of 6.0
    (margin 0, id 4 first); with tau = 1e-3 those rows are recomputed and the
    exact float64 logits decide (6 + g against 6, id 4 on g = 0).  The one-ulp
    gap (1/32 >= tau) keeps the bf16 decision and its rounded values; tau = 0
    recomputes nothing; tau = 0.05 recomputes the one-ulp row as well."""
    H, V = 64, 12
    gaps = [0.0, 2.0 ** -50, 2.0 ** -17, 2.0 ** -14, 2.0 ** -13, 2.0 ** -5]
    rng = np.random.default_rng(26)
    x = bf16_const(1.0, (len(gaps), H))
    # one W per gap: rows are processed independently, so stack the cases as
    # separate calls over the same x row and check the batch call row by row
    ws = []
    for g in gaps:
        w = rand_bf16(rng, (V, H), emin=-14, emax=-12)
        w[4] = w[9] = 0
        w[4, 0] = w[9, 0] = bf16_const(6.0, ()).item()
        w[9, H - 1] = synth.bf16_from_f32(np.float32(g)).item()
        ws.append(w)
    for tau in (0.0, 1e-3, 0.05):
        for g, w in zip(gaps, ws):
            ids, vals, margin, gated = o.greedy_gated_bf16(x[:1], w, tau)
            bf16_tie = g < 2.0 ** -6
            bf16_margin = 0.0 if bf16_tie else g
            assert gated[0] == (bf16_margin < tau), (tau, g)
            if gated[0]:
                want = [4, 9] if g == 0.0 else [9, 4]
                assert list(ids[0]) == want and vals[0, 0] == 6.0 + g and vals[0, 1] == 6.0
                assert margin[0] == g
            elif bf16_tie:
                assert list(ids[0]) == [4, 9] and list(vals[0]) == [6.0, 6.0] and margin[0] == 0.0
            else:
                assert list(ids[0]) == [9, 4] and margin[0] == g and vals[0, 0] == 6.0 + g
    # several rows of one call are gated independently: rows 0..2 share one W
    w = ws[2]                                     # gap 2^-17: a bf16 tie
    xx = np.concatenate([x[:1], bf16_const(2.0, (1, H)), bf16_const(0.0, (1, H))])
    ids, vals, margin, gated = o.greedy_gated_bf16(xx, w, 1e-3)
    assert list(gated) == [True, True, True]     # row 2: every logit is 0 -> margin 0
    assert list(ids[0]) == [9, 4] and list(ids[1]) == [9, 4] and margin[1] == 2 * 2.0 ** -17
    assert list(ids[2]) == [0, 1] and margin[2] == 0.0


def pin_gated_rerank_bruteforce(o):
    """tau = inf recomputes every row: the ids are the bf16-output head's two
    candidates, ranked by their exact rational logits (lowest id on a tie),
    and the values are those logits (brute force with fractions)."""
    rng = np.random.default_rng(27)
    for trial in range(4):
        B, H, V = 3, 64, 10
        x = rand_bf16(rng, (B, H), emin=-3, emax=0)
        w = rand_bf16(rng, (V, H), emin=-3, emax=0)
        ids16, _, _ = o.greedy_bf16(x, w, round_bf16=True)
        ids, vals, margin, gated = o.greedy_gated_bf16(x, w, float("inf"))
        assert gated.all()
        xf, wf = fracs(synth.bf16_to_f64(x)), fracs(synth.bf16_to_f64(w))
        for r in range(B):
            cand = sorted(int(c) for c in ids16[r])
            z = {c: sum(a * b for a, b in zip(xf[r], wf[c])) for c in cand}
            order = sorted(cand, key=lambda c: (-z[c], c))
            assert list(ids[r]) == order, (trial, r)
            assert vals[r, 0] == float(z[order[0]]) and vals[r, 1] == float(z[order[1]])


# ------------------------------------------------------------ sampling
def _chi2_sf(stat, dof):
    """Survival function of the chi-square distribution (scipy's routine)."""
    from scipy.stats import chi2
    return float(chi2.sf(stat, dof))


_ROCRAND_TOOL: list = []


def rocrand_philox_blocks(triples):
    """Philox4x32-10 blocks from rocRAND's engine header (an independent
    implementation of the published generator), built host-only once per
    process: block of (seed, subsequence, n) = counter (n lo, n hi,
    subsequence lo, subsequence hi) under key (seed lo, seed hi)."""
    import subprocess
    import tempfile
    if not _ROCRAND_TOOL:
        src = Path(__file__).resolve().parent / "philox_rocrand.cpp"
        exe = Path(tempfile.mkdtemp(prefix="philox_rocrand_")) / "philox_rocrand"
        subprocess.run(["/opt/rocm/llvm/bin/clang++", "-x", "hip", "--offload-host-only", "-O1",
                        "-I/opt/rocm/include", str(src), "-o", str(exe)], check=True)
        _ROCRAND_TOOL.append(exe)
    inp = "".join(f"{s} {q} {n}\n" for s, q, n in triples)
    out = subprocess.run([str(_ROCRAND_TOOL[0])], input=inp, capture_output=True, text=True,
                         check=True).stdout.split()
    return np.array(out, dtype=np.uint64).astype(np.uint32).reshape(-1, 4)


def pin_philox_vs_rocrand(o):
    """Philox4x32-10 against rocRAND's engine on 64 random (counter, key) pairs
    covering all four counter words (the second below 2^30) and both key words,
    plus the zero block and single set bits."""
    rng = np.random.default_rng(41)
    triples = [(0, 0, 0), (1, 0, 0), (0, 1, 0), (0, 0, 1)]
    for _ in range(64):   # n < 2^62: the engine takes the offset 4 n in 64 bits
        seed, sub = (int(v) for v in rng.integers(0, 2 ** 63, 2, dtype=np.uint64) * 2 + 1)
        triples.append((seed, sub, int(rng.integers(0, 2 ** 62))))
    ref = rocrand_philox_blocks(triples)
    m = (1 << 32) - 1
    for (seed, sub, n), want in zip(triples, ref):
        ctr = [n & m, n >> 32, sub & m, sub >> 32]
        got = o.philox4x32(ctr, [seed & m, seed >> 32])
        assert np.array_equal(got, want), (seed, sub, n)


def pin_gumbel_decimal(o):
    """G = -ln(-ln U) to 50 digits, with U = (2u + 1) 2^-24 from the top 23
    bits u of rocRAND's Philox4x32-10 block: word (v >> 5) & 3 of counter
    (32 (v >> 7) + (v & 31), 0, position lo, position hi) under key (seed lo,
    seed hi)."""
    getcontext().prec = 50
    rng = np.random.default_rng(42)
    cases = [(int(rng.integers(0, 2 ** 63)) * 2 + 1, int(rng.integers(0, 2 ** 40)),
              int(rng.integers(0, 200000))) for _ in range(40)]
    blocks = rocrand_philox_blocks([(seed, pos, 32 * (v >> 7) + (v & 31)) for seed, pos, v in cases])
    for (seed, pos, v), blk in zip(cases, blocks):
        u = int(blk[(v >> 5) & 3]) >> 9
        U = Decimal(2 * u + 1) / Decimal(2 ** 24)
        g = -(-(U.ln())).ln()
        assert abs(Decimal(o.gumbel(seed, pos, v)) - g) < Decimal("1e-12"), (seed, pos, v)


def _sample_rows(o, z_cols, T, n, seed=7):
    """n draws from one fixed logit row z_cols (exact in bf16; x = e_0, W[:, 0]
    = z), keyed by (seed, position = draw index)."""
    V, H = len(z_cols), 64
    x = np.zeros((n, H), np.uint16)
    x[:, 0] = bf16_const(1.0, ()).item()
    w = np.zeros((V, H), np.uint16)
    w[:, 0] = synth.bf16_from_f32(np.asarray(z_cols, np.float32))
    assert np.array_equal(synth.bf16_to_f64(w[:, 0]), np.asarray(z_cols, np.float64))
    return o.sample_bf16(x, w, T, np.full(n, seed, np.uint64), np.arange(n, dtype=np.int64))


def pin_sample_distribution(o):
    """Gumbel-max draws follow softmax(z / T): chi-square of 40,000 draws over
    6 tokens at T = 1 and T = 0.5 (p > 1e-6), and a uniform draw when all
    logits are equal."""
    z = np.array([1.0, 0.5, 0.0, -0.5, 2.0, 1.0])
    n = 40000
    for T in (1.0, 0.5):
        tok, val, gap = _sample_rows(o, z, T, n)
        p = np.exp(z / T - np.max(z / T))
        p /= p.sum()
        cnt = np.bincount(tok, minlength=len(z))
        stat = float(np.sum((cnt - n * p) ** 2 / (n * p)))
        assert _chi2_sf(stat, len(z) - 1) > 1e-6, (T, cnt, n * p)
        assert np.all(gap >= 0)
    tok, _, _ = _sample_rows(o, np.zeros(8), 1.0, n, seed=8)
    cnt = np.bincount(tok, minlength=8)
    assert _chi2_sf(float(np.sum((cnt - n / 8) ** 2 / (n / 8))), 7) > 1e-6, cnt


def pin_sample_limits_and_keys(o):
    """T -> 0 is the greedy argmax (logit gaps of 2^-4 against noise in
    [-2.9, 16.7] at T = 2^-16); the same (seed, position) draws the same token
    in any row order; int8 and bf16 rows with equal logits draw equally; an
    invalid int8 scale draws -1."""
    rng = np.random.default_rng(43)
    H, V, B = 64, 40, 30
    x = np.zeros((B, H), np.uint16)
    x[:, 0] = bf16_const(1.0, ()).item()
    z = rng.permutation(V).astype(np.float64) / 16.0        # distinct, gaps >= 1/16
    w = np.zeros((V, H), np.uint16)
    w[:, 0] = synth.bf16_from_f32(z.astype(np.float32))
    seed = rng.integers(0, 2 ** 63, B, dtype=np.uint64)
    pos = rng.integers(0, 2 ** 31, B).astype(np.int64)
    tok, _, _ = o.sample_bf16(x, w, 2.0 ** -16, seed, pos)
    assert np.all(tok == int(np.argmax(z)))
    tok, val, gap = o.sample_bf16(x, w, 1.0, seed, pos)
    perm = rng.permutation(B)
    tok_p, val_p, _ = o.sample_bf16(x[perm], w, 1.0, seed[perm], pos[perm])
    assert np.array_equal(tok_p, tok[perm]) and np.array_equal(val_p, val[perm])
    assert len(set(tok.tolist())) > 1                       # different keys, different draws
    # int8: x = e_0, W[:, 0] = small integers, scale 1 -> the same logits
    zi = rng.integers(-40, 41, V)
    xi = np.zeros((B, H), np.int8)
    xi[:, 0] = 1
    wi = np.zeros((V, H), np.int8)
    wi[:, 0] = zi
    wb = np.zeros((V, H), np.uint16)
    wb[:, 0] = synth.bf16_from_f32(zi.astype(np.float32))
    t8, v8, g8 = o.sample_i8(xi, wi, 0.7, seed, pos, scale=np.ones(B, np.float32))
    tb, vb, gb = o.sample_bf16(x, wb, 0.7, seed, pos)
    assert np.array_equal(t8, tb) and np.array_equal(v8, vb) and np.array_equal(g8, gb)
    sc = np.ones(B, np.float32)
    sc[3], sc[5] = 0.0, np.nan
    t8, v8, _ = o.sample_i8(xi, wi, 0.7, seed, pos, scale=sc)
    assert t8[3] == -1 and t8[5] == -1 and np.isnan(v8[3]) and t8[4] == tb[4]


def pin_int_scaled_values(o):
    """int8 top-2 values and margin are the nearest float32 of the exact
    rational raw * scale; a non-positive scale gives NaN values but valid ids."""
    d = synth.make_inputs("int8", rows=6, with_weights=False)
    rng = np.random.default_rng(25)
    w = rng.integers(-127, 128, (257, d["H"])).astype(np.int8)
    scale = d["scale"].copy()
    scale[5] = -1.0
    ids, raw, vals, margin = o.greedy_i8(d["x"], w, scale)
    z = d["x"].astype(np.int64) @ w.astype(np.int64).T
    for r in range(6):
        assert list(ids[r]) == _brute_top2(list(z[r]))
        assert list(raw[r]) == [int(z[r, i]) for i in ids[r]]
        if r == 5:
            assert np.isnan(vals[r]).all() and np.isnan(margin[r])
            continue
        s = Fraction(float(scale[r]))
        assert [float(v) for v in vals[r]] == [float32_rne(int(q) * s) for q in raw[r]]
        assert float(margin[r]) == float32_rne(int(raw[r, 0] - raw[r, 1]) * s)
    # logits above 2^24 (not float32-representable): the scaled value must still
    # be one rounding of the exact product
    H = d["H"]
    xb = np.full((1, H), 127, np.int8)
    for r in range(48):
        wb = rng.integers(100, 128, (2, H)).astype(np.int8)
        sb = np.array([2.0 ** -18 * rng.uniform(0.5, 2.0)], np.float32)
        ids, raw, vals, margin = o.greedy_i8(xb, wb, sb)
        s = Fraction(float(sb[0]))
        assert raw[0, 0] > 2 ** 24
        assert [float(v) for v in vals[0]] == [float32_rne(int(q) * s) for q in raw[0]]


# ----------------------------------------------------------- log-prob
def pin_logsoftmax_sums_to_one(o):
    """sum_v exp(log p_v) = 1 within 1e-6 (logsumexp identity), and the
    per-target log-prob is that vector's entry."""
    d = synth.make_inputs("tiny")
    z = o.logits_bf16(d["x"], d["w"])
    lp = o.logprob_bf16(d["x"], d["w"], d["target"])
    for r in range(d["B"]):
        lsm = o.logsoftmax_f64(z[r])
        assert abs(math.fsum(np.exp(lsm).tolist()) - 1.0) <= 1e-6
        assert abs(lsm[d["target"][r]] - lp[r]) <= 1e-12
    rng = np.random.default_rng(31)
    zz = rng.normal(0, 20, 5000)
    assert abs(math.fsum(np.exp(o.logsoftmax_f64(zz)).tolist()) - 1.0) <= 1e-6


def pin_logprob_closed_forms(o):
    """W = 0: log p = -ln V for every target.  V = 2: log p_0 = -log1p(exp(z1 - z0))."""
    rng = np.random.default_rng(32)
    H, V = 64, 50
    x = rand_bf16(rng, (3, H))
    lp = o.logprob_bf16(x, np.zeros((V, H), np.uint16), np.array([0, 17, 49], np.int32))
    assert np.allclose(lp, -math.log(V), rtol=0, atol=1e-14)
    x = rand_bf16(rng, (4, H), emin=-3, emax=0)
    w = rand_bf16(rng, (2, H), emin=-3, emax=0)
    xf, wf = fracs(synth.bf16_to_f64(x)), fracs(synth.bf16_to_f64(w))
    for t in (0, 1):
        lp = o.logprob_bf16(x, w, np.full(4, t, np.int32))
        for r in range(4):
            z = [float(sum(a * b for a, b in zip(xf[r], wf[v]))) for v in (0, 1)]
            assert abs(lp[r] + math.log1p(math.exp(z[1 - t] - z[t]))) <= 1e-12


def pin_logprob_shift_invariance(o):
    """Appending a coordinate x_H = 1 with W[:, H] = c adds c to every logit
    and leaves every log-prob unchanged (1e-12); in int8 mode exactly."""
    d = synth.make_inputs("tiny")
    x2 = np.concatenate([d["x"], bf16_const(1.0, (d["B"], 1))], axis=1)
    w2 = np.concatenate([d["w"], bf16_const(3.5, (d["V"], 1))], axis=1)
    a = o.logprob_bf16(d["x"], d["w"], d["target"])
    b = o.logprob_bf16(x2, w2, d["target"])
    assert np.max(np.abs(a - b)) <= 1e-12
    rng = np.random.default_rng(33)
    x = rng.integers(-127, 128, (3, 64)).astype(np.int8)
    w = rng.integers(-127, 128, (300, 64)).astype(np.int8)
    t = np.array([0, 150, 299], np.int32)
    s = np.full(3, 2.0 ** -12, np.float32)
    a = o.logprob_i8(x, w, t, s)
    b = o.logprob_i8(np.concatenate([x, np.ones((3, 1), np.int8)], 1),
                     np.concatenate([w, np.full((300, 1), 99, np.int8)], 1), t, s)
    assert np.array_equal(a, b)


def pin_logprob_decimal(o):
    """50-digit decimal log-softmax of the exact rational logits agrees within
    1e-12 (bf16 mode) and for the scaled int8 logits."""
    getcontext().prec = 50
    rng = np.random.default_rng(34)
    H, V = 16, 23
    x = rand_bf16(rng, (3, H), emin=-2, emax=1)
    w = rand_bf16(rng, (V, H), emin=-3, emax=0)
    t = np.array([0, 11, 22], np.int32)
    lp = o.logprob_bf16(x, w, t)
    xf, wf = fracs(synth.bf16_to_f64(x)), fracs(synth.bf16_to_f64(w))
    for r in range(3):
        z = [dec(sum(a * b for a, b in zip(xf[r], wf[v]))) for v in range(V)]
        ref = z[t[r]] - sum(zv.exp() for zv in z).ln()
        assert abs(Decimal(float(lp[r])) - ref) <= Decimal("1e-12")
    xi = rng.integers(-127, 128, (3, 64)).astype(np.int8)
    wi = rng.integers(-127, 128, (40, 64)).astype(np.int8)
    s = np.array([2.0 ** -10, 3.0e-4, 1.0e-3], np.float32)
    lp = o.logprob_i8(xi, wi, t % 40, s)
    for r in range(3):
        zr = [sum(int(a) * int(b) for a, b in zip(xi[r], wi[v])) for v in range(40)]
        sr = dec(Fraction(float(s[r])))
        y = [sr * zv for zv in zr]
        ref = y[t[r] % 40] - sum(yv.exp() for yv in y).ln()
        assert abs(Decimal(float(lp[r])) - ref) <= Decimal("1e-12")


def pin_logprob_out_of_range(o):
    """A target outside [0, V) gives NaN (and only for that row)."""
    d = synth.make_inputs("tiny")
    t = np.array([-1, 3, d["V"], 999], np.int32)
    lp = o.logprob_bf16(d["x"], d["w"], t)
    assert np.isnan(lp[0]) and np.isnan(lp[2]) and np.isfinite(lp[1]) and np.isfinite(lp[3])
    xi = np.ones((2, 64), np.int8)
    wi = np.ones((5, 64), np.int8)
    lp = o.logprob_i8(xi, wi, np.array([5, 4], np.int32), np.ones(2, np.float32))
    assert np.isnan(lp[0]) and abs(lp[1] + math.log(5)) < 1e-14


# ------------------------------------------------------ bf16 rounding
def pin_round_bf16(o):
    """Rounding float64 -> bf16 is nearest-even: it matches the bit-level RNE
    of float32 inputs, exact halfway cases go to the even neighbour, and random
    doubles match an exact rational rounding."""
    rng = np.random.default_rng(41)
    f32 = (rng.standard_normal(2000) * np.exp2(rng.integers(-20, 20, 2000))).astype(np.float32)
    ref = synth.bf16_to_f32(synth.bf16_from_f32(f32)).astype(np.float64)
    got = np.array([o.round_bf16(float(v)) for v in f32])
    assert np.array_equal(got, ref)
    assert o.round_bf16(1.0 + 2.0 ** -8) == 1.0
    assert o.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert o.round_bf16(-(1.0 + 2.0 ** -8)) == -1.0
    assert o.round_bf16(6.0 + 2.0 ** -6) == 6.0 and o.round_bf16(6.0 + 3 * 2.0 ** -6) == 6.0 + 2.0 ** -4
    for v in rng.standard_normal(500) * 50:
        a = Fraction(float(v))
        e = math.floor(math.log2(abs(a)))
        q = a / Fraction(2) ** (e - 7)
        n = math.floor(q)
        rem = q - n
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2):
            n += 1
        assert o.round_bf16(float(v)) == float(n * Fraction(2) ** (e - 7))


# --------------------------------------------- the pages' own numbers
def pin_pages_float_examples(o):
    """The printed float examples (golden file) hold in IEEE arithmetic, and a
    crafted row shows the two summation orders a split-K kernel can pick give
    different float32 results while the oracle's float64 logit is exact."""
    g = json.loads((GOLDEN / "pages_float_examples.json").read_text())
    for case in g["cases"]:
        t = {"float64": np.float64, "float32": np.float32}[case["dtype"]]
        a, b, c = (t(case[k]) for k in ("a", "b", "c"))
        got = t(t(a + b) + c) if case["order"] == "(a+b)+c" else t(a + t(b + c))
        assert float(got) == float(case["value"]), case
    H = 8
    x = bf16_const(1.0, (1, H))
    vals = [2.0 ** 24, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0]
    w = synth.bf16_from_f32(np.array([vals], np.float32))
    seq = np.float32(0)
    for v in vals:
        seq = np.float32(seq + np.float32(v))
    halves = np.float32(0)
    for part in (vals[:4], vals[4:]):
        acc = np.float32(0)
        for v in part:
            acc = np.float32(acc + np.float32(v))
        halves = np.float32(halves + acc)
    assert seq == 2.0 ** 24 and halves == 2.0 ** 24 + 4
    assert o.logits_bf16(x, w)[0, 0] == 2.0 ** 24 + 7


# --------------------------------------------------- near-tie workload
def pin_neartie_builder(o, rows=48):
    """On the planted near-tie rows the oracle's top-2 is the planted pair, the
    winner is the planted winner (lowest id on an exact tie) and its margin
    equals the builder's exact gap within 1e-9."""
    d = synth.make_inputs("neartie", rows=rows)
    ids, vals, margin = o.greedy_bf16(d["x"], d["w"])
    t = d["tie"]
    for r in range(rows):
        win, lose, gap = int(t["win"][r]), int(t["lose"][r]), float(t["gap"][r])
        assert set(ids[r]) == {win, lose}, r
        assert ids[r, 0] == (min(win, lose) if gap == 0.0 else win), r
        assert abs(margin[r] - gap) <= 1e-9, r


# -------------------------------------------- integer front and back
# The algorithm is ours (the pages name its ingredients only); it is pinned to
# exact rationals, 50-digit decimals, an independent int64 matmul and the
# invariants the integer arithmetic guarantees.
Q24, Q30 = 2 ** 24, 2 ** 30


def _dec_exp(fr: Fraction) -> Decimal:
    getcontext().prec = 50
    return dec(fr).exp()


def _dec_ln(fr: Fraction) -> Decimal:
    getcontext().prec = 50
    return dec(fr).ln()


def pin_int_quantize(o):
    """Per-token int8 quantisation: the step D = M 2^E has a 15-bit mantissa,
    127 D covers max|x| and no smaller 15-bit-mantissa step does; q is the
    exact round-half-away of x / D (Fraction); the largest |x| maps to +-127;
    |x - q D| <= D / 2; quantising -x gives -q; x * 2^j gives the same q and M
    with E + j; a zero row gives q = 0, D = 1."""
    rng = np.random.default_rng(71)
    rows = []
    for mag in (1, 3, 100, 2 ** 12, 2 ** 20, 2 ** 30):
        for _ in range(3):
            rows.append(rng.integers(-mag, mag + 1, 24))
    rows.append(np.array([2 ** 31 - 1, -(2 ** 31 - 1)] + [5] * 22))
    rows.append(np.array([-(2 ** 31)] + [7] * 23))
    rows.append(np.array([0] * 23 + [1]))
    rows.append(np.array([127 * 2 ** k for k in range(24)]))       # exact steps
    x = np.array(rows, dtype=np.int64).astype(np.int32)
    q, M, E = o.quantize_rows(x)
    for r in range(x.shape[0]):
        a = max(abs(int(v)) for v in x[r])
        m, e = int(M[r]), int(E[r])
        assert 2 ** 14 <= m < 2 ** 15, r
        D = Fraction(m) * Fraction(2) ** e
        assert 127 * D >= a, r
        prev = (Fraction(m - 1) * Fraction(2) ** e if m > 2 ** 14
                else Fraction(2 ** 15 - 1) * Fraction(2) ** (e - 1))
        assert 127 * prev < a, r
        for k in range(x.shape[1]):
            v = Fraction(int(x[r, k]))
            want = math.floor(abs(v) / D + Fraction(1, 2)) * (1 if v >= 0 else -1)
            assert int(q[r, k]) == want, (r, k)
            assert abs(v - int(q[r, k]) * D) <= D / 2, (r, k)
        big = [k for k in range(x.shape[1]) if abs(int(x[r, k])) == a]
        assert all(abs(int(q[r, k])) == 127 for k in big), r
    ok = np.all(x != -(2 ** 31), axis=1)
    qn, Mn, En = o.quantize_rows(-x[ok])
    assert np.array_equal(qn, -q[ok]) and np.array_equal(Mn, M[ok]) and np.array_equal(En, E[ok])
    small = np.all(np.abs(x.astype(np.int64)) < 2 ** 24, axis=1)
    for j in (1, 5):
        q2, M2, E2 = o.quantize_rows(x[small] * 2 ** j)
        assert np.array_equal(q2, q[small]) and np.array_equal(M2, M[small])
        assert np.array_equal(E2, E[small] + j)
    q0, M0, E0 = o.quantize_rows(np.zeros((1, 8), np.int32))
    assert not q0.any() and Fraction(int(M0[0])) * Fraction(2) ** int(E0[0]) == 1


def pin_int_exp(o):
    """Integer exp against 50-digit e^(-T / 2^24) * 2^30: within 3 units of
    2^-30 on boundaries of the ln 2 reduction and on random T; exactly 2^30 at
    T = 0; non-increasing in T; 0 far out.  The bound: Horner roundings
    0.5 (1 + 0.7 + 0.7^2 + ...) < 1.7, series truncation (ln 2)^11 / 11! <
    0.5, the rounded ln 2 (1.9e-9 relative per halving) < 1.1, and the final
    shift 0.5."""
    rng = np.random.default_rng(72)
    L = round(math.log(2) * Q24)
    Ts = [0, 1, 2, L - 1, L, L + 1, 7 * L - 1, 7 * L, 31 * L + 3, 33 * L]
    Ts += [int(t) for t in rng.integers(0, 40 * Q24, 300)]
    Ts += [int(t) for t in rng.integers(0, Q24, 100)]
    worst = 0.0
    for T in Ts:
        got = o.iexp_q30(T)
        want = _dec_exp(Fraction(-T, Q24)) * Q30
        worst = max(worst, abs(float(Decimal(got) - want)))
    assert worst <= 3.0, worst
    assert o.iexp_q30(0) == Q30
    assert o.iexp_q30(2 ** 62) == 0 and o.iexp_q30(64 * Q24) == 0
    ts = sorted(set(Ts))
    vals = [o.iexp_q30(t) for t in ts]
    assert all(a >= b for a, b in zip(vals, vals[1:]))


def pin_int_ln(o):
    """Integer ln against 50-digit ln(S / 2^30) * 2^30: within 12 units of
    2^-30 for S from 2^30 to 2^50, and 0 at S = 2^30.  The bound: the 30-bit
    mantissa 0.5, the rounded ln 2 0.05 per octave (0.85), u rounded 0.5
    times 2 / (1 - u^2) <= 2.25 (1.2), and 2 x (0.5 + a carried 0.2) for each
    of at most 9 series terms above one unit (8.6); below 2^-26 nats, so under
    one unit of the Q.24 result."""
    rng = np.random.default_rng(73)
    Ss = [Q30, Q30 + 1, 2 * Q30 - 1, 2 * Q30, 3 * Q30, 2 ** 47 + 12345, 2 ** 50 - 1]
    Ss += [int(Q30 * float(f)) for f in np.exp(rng.uniform(0.0, 13.8, 300))]
    for S in Ss:
        got = o.iln_q30(S)
        want = _dec_ln(Fraction(S, Q30)) * Q30
        assert abs(Decimal(got) - want) <= 12, (S, got, want)
    assert o.iln_q30(Q30) == 0


def pin_int_row_scale(o):
    """The row's logit scale m / 2^k equals um 2^ue * M 2^E within half a unit
    of m's last bit, with 2^30 <= m < 2^31; out-of-range exponents and
    non-positive mantissas are refused."""
    rng = np.random.default_rng(74)
    for _ in range(200):
        um = int(rng.integers(1, 2 ** 31))
        M = int(rng.integers(2 ** 14, 2 ** 15))
        ue, E = int(rng.integers(-70, -20)), int(rng.integers(-21, 12))
        res = o.int_row_scale(um, ue, M, E)
        exact = Fraction(um * M) * Fraction(2) ** (ue + E)
        if res is None:
            kk = 30 - math.floor(math.log2(exact))
            assert kk < 24 or kk > 86 or kk in (23, 87), (um, ue, M, E)
            continue
        m, k = res
        assert 2 ** 30 <= m < 2 ** 31
        assert abs(Fraction(m, 2 ** k) - exact) <= Fraction(1, 2 ** (k + 1)), (um, ue, M, E)
    assert o.int_row_scale(0, -40, 2 ** 14, 0) is None
    assert o.int_row_scale(2 ** 30, -40, -5, 0) is None
    assert o.int_row_scale(2 ** 30, 0, 2 ** 14, 0) is None          # k < 24: too coarse


def _int_logsoftmax_check(o, z, m, k, targets):
    """Integer log-prob of row z against the 50-digit log-softmax of the real
    logits z m / 2^k, within a bound derived from the arithmetic: 3 output
    units (2^-24: the rounded T of the target, the rounded ln, the ln error),
    3 units of 2^-30 per element exp and per block rescale relative to the
    exact sum of exps, and 15 units of 2^-30 for the rescale factors and the
    integer ln."""
    s = Fraction(m, 2 ** k)
    zmax = max(z)
    getcontext().prec = 50
    es = [_dec_exp(s * (int(v) - zmax)) for v in z]
    S = sum(es)
    V = len(z)
    nb = (V + 127) // 128
    bound = Decimal(3) / Q24 + Decimal(3 * (V + nb)) / Q30 / S + Decimal(15) / Q30
    for t in targets:
        got = Decimal(o.logprob_int_row(z, m, k, t)) / Q24
        want = dec(s * (int(z[t]) - zmax)) - S.ln()
        assert abs(got - want) <= bound, (V, t, float(got), float(want))


def pin_int_logsoftmax(o):
    """Integer log-softmax: random rows (V across block edges) within the
    derived bound of the exact log-softmax; uniform logits give -ln V; V = 2;
    adding a constant to every logit changes no bit; invalid targets and
    scales give the sentinel."""
    rng = np.random.default_rng(75)
    for V in (2, 127, 128, 129, 300, 1000):
        z = rng.integers(-2 ** 26, 2 ** 26, V)
        m, k = int(rng.integers(2 ** 30, 2 ** 31)), int(rng.integers(52, 57))
        _int_logsoftmax_check(o, z, m, k, [0, V - 1, int(rng.integers(0, V))])
    z = np.full(1000, 12345)
    _int_logsoftmax_check(o, z, 2 ** 30, 50, [0, 999])
    got = Decimal(o.logprob_int_row(z, 2 ** 30, 50, 3)) / Q24
    assert abs(got + Decimal(1000).ln()) <= Decimal(3) / Q24
    z = np.array([0, 40000], np.int64)                       # V = 2, s (z1 - z0) = 1.2207
    m, k = 2 ** 30, 45                                       # s = 2^-15
    got = Decimal(o.logprob_int_row(z, m, k, 0)) / Q24
    want = -Decimal(math.log1p(math.exp(40000 / 2 ** 15)))
    assert abs(got - want) <= Decimal(3) / Q24 + Decimal(10) / Q30
    z = rng.integers(-2 ** 24, 2 ** 24, 700)
    base = [o.logprob_int_row(z, 1500000000, 50, t) for t in range(0, 700, 37)]
    for c in (-(2 ** 28), 1, 987654321):
        moved = [o.logprob_int_row(z + c, 1500000000, 50, t) for t in range(0, 700, 37)]
        assert moved == base, c
    bad = o.LOGP_INVALID
    assert o.logprob_int_row(z, 1500000000, 50, -1) == bad
    assert o.logprob_int_row(z, 1500000000, 50, 700) == bad
    assert o.logprob_int_row(z, 0, 50, 3) == bad
    assert o.logprob_int_row(z, 1500000000, 23, 3) == bad


def pin_int_logprob_head(o):
    """The whole integer path on tiny int8 heads: logits from an independent
    int64 matmul, the row scale from exact rationals, the log-prob within the
    derived bound of the exact log-softmax; the sum over every target of
    exp(log p) is 1 within V times that bound."""
    rng = np.random.default_rng(76)
    B, H, V = 3, 64, 260
    x = rng.integers(-127, 128, (B, H)).astype(np.int8)
    w = rng.integers(-127, 128, (V, H)).astype(np.int8)
    um, ue = 1_400_000_000, -58
    M = rng.integers(2 ** 14, 2 ** 15, B).astype(np.int32)
    E = np.array([-3, 0, 4], np.int32)
    t = np.array([5, 0, V - 1], np.int32)
    got = o.logprob_int(x, w, um, ue, M, E, t)
    z = x.astype(np.int64) @ w.astype(np.int64).T
    getcontext().prec = 50
    for r in range(B):
        s = Fraction(um) * Fraction(2) ** ue * int(M[r]) * Fraction(2) ** int(E[r])
        mk = o.int_row_scale(um, ue, int(M[r]), int(E[r]))
        assert mk is not None and abs(Fraction(mk[0], 2 ** mk[1]) - s) <= s / 2 ** 30
        zmax = int(z[r].max())
        S = sum(_dec_exp(s * (int(v) - zmax)) for v in z[r])
        want = dec(s * (int(z[r, t[r]]) - zmax)) - S.ln()
        # the 31-bit scale moves a logit difference d by at most d s 2^-30
        slack = Decimal(float(s) * float(zmax - z[r].min()) / 2 ** 29)
        bound = Decimal(3) / Q24 + Decimal(3 * (V + 3)) / Q30 / S + slack
        assert abs(Decimal(int(got[r])) / Q24 - want) <= bound, r
        every = [o.logprob_int_row(z[r], mk[0], mk[1], v) for v in range(V)]
        total = sum(math.exp(v / Q24) for v in every)
        assert abs(total - 1.0) <= V * float(bound), (r, total)


FAST = [
    pin_logits_bruteforce, pin_logits_one_hot, pin_logits_closed_forms,
    pin_int_logits_bruteforce, pin_int_overflow_bound, pin_top2_bruteforce,
    pin_top2_hand_ties, pin_greedy_identical_rows, pin_greedy_permutation,
    pin_greedy_near_ties, pin_gated_hand_cases, pin_gated_rerank_bruteforce,
    pin_philox_vs_rocrand, pin_gumbel_decimal, pin_sample_distribution, pin_sample_limits_and_keys,
    pin_int_scaled_values, pin_logsoftmax_sums_to_one,
    pin_logprob_closed_forms, pin_logprob_shift_invariance, pin_logprob_decimal,
    pin_logprob_out_of_range, pin_round_bf16, pin_pages_float_examples,
    pin_int_quantize, pin_int_exp, pin_int_ln, pin_int_row_scale, pin_int_logsoftmax,
    pin_int_logprob_head,
]
SLOW = [pin_logits_vs_blas, pin_int_logits_vs_numpy, pin_neartie_builder]
ALL = FAST + SLOW
