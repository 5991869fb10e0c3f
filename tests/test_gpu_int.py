"""The all-integer front and back of the int8 head on the GPU (through the
C-ABI), bit for bit against the oracle: per-token int8 quantisation with a
dyadic step, and the fixed-point log-softmax (Q.24 nats) of the exact int32
logits ("Eliminating Nondeterminism in LLM Inference with Integer-Only
Arithmetic", section "DetLLM")."""
import math

import numpy as np
import pytest
import torch

import synth
from invariant_lm_head_amd import lmhead
from tests.gpu_util import DEV, gpu, host, i8, o, record, row_digests  # noqa: F401

pytestmark = pytest.mark.gpu

Q24 = 2 ** 24


@pytest.fixture(scope="module")
def hid(i8):  # noqa: F811
    """int32 hidden rows of the int8 workload, quantised on the GPU."""
    h = i8["hidden"]
    q, sm, se = lmhead.quantize_rows(gpu(h))
    return {"h": h, "q": q, "sm": sm, "se": se, "unit": i8["unit"]}


def test_quantize_bit_exact(hid, o, i8):  # noqa: F811
    """512 hidden rows of 4096: q, M and E equal the oracle's bit for bit
    (live oracle, and the stored per-row digests of q)."""
    q, M, E = o.quantize_rows(hid["h"])
    assert np.array_equal(host(hid["q"]), q)
    assert np.array_equal(host(hid["sm"]), M) and np.array_equal(host(hid["se"]), E)
    g = i8["golden"]
    assert row_digests(host(hid["q"]).astype(np.int32)) == list(g["q_digests"])
    assert np.array_equal(host(hid["sm"]), g["step_m"]) and np.array_equal(host(hid["se"]), g["step_e"])


@pytest.mark.parametrize("B", [1, 8, 64, 256, 512])
def test_logprob_int_all_rows(i8, hid, B):  # noqa: F811
    """Every row of every swept batch: log p in Q.24 equals the oracle's
    (stored) bit for bit."""
    t = i8["target"][:B]
    got = host(lmhead.logprob_int(hid["q"][:B].contiguous(), i8["gw"], hid["unit"],
                                  hid["sm"][:B].contiguous(), hid["se"][:B].contiguous(),
                                  gpu(t)))
    want = i8["golden"]["logprob_q"][:B]
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:10]
    record("parity_int8", f"integer_logprob_batch_{B}", {"rows": B, "bit_exact": True})


@pytest.mark.parametrize("H", [1, 63, 100, 257, 4096])
def test_quantize_edges(o, H):  # noqa: F811
    """Ragged widths, a zero row, INT32_MIN and INT32_MAX, tiny values, exact
    powers of two: bit-exact against the oracle."""
    rng = np.random.default_rng(H)
    rows = [rng.integers(-2 ** 31, 2 ** 31, H), np.zeros(H), rng.integers(-2, 3, H),
            np.full(H, -2 ** 31), np.full(H, 2 ** 31 - 1), np.full(H, 127 << 9),
            rng.integers(-2 ** 12, 2 ** 12, H)]
    x = np.stack(rows).astype(np.int64).astype(np.int32)
    q, M, E = (host(t) for t in lmhead.quantize_rows(gpu(x)))
    oq, oM, oE = o.quantize_rows(x)
    assert np.array_equal(q, oq) and np.array_equal(M, oM) and np.array_equal(E, oE)


def _oracle_rows(o, i8, hid, rows, t):  # noqa: F811
    qh = host(hid["q"])[rows]
    return o.logprob_int(qh, i8["w"], *hid["unit"], host(hid["sm"])[rows], host(hid["se"])[rows],
                         t)


@pytest.mark.parametrize("B", [1, 5, 33])
def test_logprob_int_bit_exact(i8, hid, o, B):  # noqa: F811
    """The 4096 x 128256 head on the GPU-quantised rows: log p in Q.24 equals
    the oracle's bit for bit (32- and 64-row tiles; the fold reads each row's
    1002 block records in four rounds)."""
    t = i8["target"][:B]
    got = host(lmhead.logprob_int(hid["q"][:B].contiguous(), i8["gw"], hid["unit"],
                                  hid["sm"][:B].contiguous(), hid["se"][:B].contiguous(),
                                  gpu(t)))
    want = _oracle_rows(o, i8, hid, np.arange(B), t)
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:10]
    print(f"B={B}: log p / nats in [{got.min() / Q24:.3f}, {got.max() / Q24:.3f}]", flush=True)


@pytest.mark.parametrize("B", [64, 200, 512])
def test_logprob_int_sampled_rows(i8, hid, o, B):  # noqa: F811
    """Larger batches (the 64-, 256- and 256 x 256-row tilings): sampled rows
    bit-exact against the oracle."""
    t = i8["target"][:B]
    got = host(lmhead.logprob_int(hid["q"][:B].contiguous(), i8["gw"], hid["unit"],
                                  hid["sm"][:B].contiguous(), hid["se"][:B].contiguous(),
                                  gpu(t)))
    rows = np.array(sorted({0, 1, 31, 32, B // 2, B - 2, B - 1}))
    want = _oracle_rows(o, i8, hid, rows, t[rows])
    assert np.array_equal(got[rows], want)


def test_logprob_int_batch_invariant(i8, hid):  # noqa: F811
    """Every row's bits are the same at batch 1, 8, 300 and 512."""
    t = gpu(i8["target"])
    full = host(lmhead.logprob_int(hid["q"], i8["gw"], hid["unit"], hid["sm"], hid["se"], t))
    for B in (300, 8):
        part = host(lmhead.logprob_int(hid["q"][:B].contiguous(), i8["gw"], hid["unit"],
                                       hid["sm"][:B].contiguous(), hid["se"][:B].contiguous(),
                                       t[:B].contiguous()))
        assert np.array_equal(part, full[:B]), B
    for r in (0, 7, 299, 511):
        one = host(lmhead.logprob_int(hid["q"][r:r + 1].contiguous(), i8["gw"], hid["unit"],
                                      hid["sm"][r:r + 1].contiguous(),
                                      hid["se"][r:r + 1].contiguous(), t[r:r + 1].contiguous()))
        assert one[0] == full[r], r


def test_logprob_int_close_to_float(i8, hid, o):  # noqa: F811
    """Against the float64 log-softmax of the real logits z * m / 2^k (z from
    the oracle's exact int64 logits): within 1e-6 nats on 4 rows."""
    B = 4
    t = i8["target"][:B]
    got = host(lmhead.logprob_int(hid["q"][:B].contiguous(), i8["gw"], hid["unit"],
                                  hid["sm"][:B].contiguous(), hid["se"][:B].contiguous(),
                                  gpu(t))) / Q24
    z = o.logits_i8(host(hid["q"])[:B], i8["w"])
    for r in range(B):
        m, k = o.int_row_scale(*hid["unit"], int(host(hid["sm"])[r]), int(host(hid["se"])[r]))
        y = (z[r] - z[r].max()).astype(np.float64) * (m / 2.0 ** k)
        want = y[t[r]] - math.log(np.exp(y).sum())
        assert abs(got[r] - want) <= 1e-6, (r, got[r], want)


@pytest.mark.parametrize("B,H,V", [(3, 64, 2), (40, 192, 1000), (300, 128, 333), (7, 64, 129),
                                   (5, 64, 32768), (5, 64, 32769)])
def test_logprob_int_edges(o, B, H, V):  # noqa: F811
    """Ragged V (blocks of 128 cut short), V = 2, a zero hidden row (every logit
    0: log p = -ln V), an invalid target and an invalid step: bit-exact
    against the oracle, sentinels where the header says.  V = 32768 and 32769
    give 256 and 257 blocks: the fold's last single-round row and its first
    row read in two rounds."""
    rng = np.random.default_rng(B * 1000 + V)
    x = rng.integers(-127, 128, (B, H)).astype(np.int8)
    x[0] = 0
    w = rng.integers(-127, 128, (V, H)).astype(np.int8)
    M = rng.integers(2 ** 14, 2 ** 15, B).astype(np.int32)
    E = rng.integers(-4, 4, B).astype(np.int32)
    M[-1] = 0                                   # not a valid step
    t = rng.integers(0, V, B).astype(np.int32)
    t[1 % B] = V                                # out of range
    unit = synth.INT_UNIT
    got = host(lmhead.logprob_int(gpu(x), gpu(w), unit, gpu(M), gpu(E), gpu(t)))
    want = o.logprob_int(x, w, *unit, M, E, t)
    assert np.array_equal(got, want)
    assert got[-1] == lmhead.LOGP_INVALID and got[1 % B] == lmhead.LOGP_INVALID
    if B > 2:
        assert abs(got[0] / Q24 + math.log(V)) <= 4 / Q24


def test_logprob_int_scale_out_of_range(o):  # noqa: F811
    """A unit so large that k < 24 (coarser than the Q.24 grid) is refused per
    row with the sentinel, like the oracle."""
    rng = np.random.default_rng(5)
    x = rng.integers(-127, 128, (2, 64)).astype(np.int8)
    w = rng.integers(-127, 128, (300, 64)).astype(np.int8)
    M, E = np.array([2 ** 14, 2 ** 14], np.int32), np.array([0, -60], np.int32)
    t = np.array([3, 4], np.int32)
    got = host(lmhead.logprob_int(gpu(x), gpu(w), (2 ** 30, -20), gpu(M), gpu(E), gpu(t)))
    want = o.logprob_int(x, w, 2 ** 30, -20, M, E, t)
    assert np.array_equal(got, want)
    assert got[0] == lmhead.LOGP_INVALID and got[1] != lmhead.LOGP_INVALID
