"""Bitwise batch invariance of the HIP path: a row's logits, top-2 and log-prob
bits do not depend on the batch size, the row's position or its neighbours.
("12 Exactness", section 12.2; "batch-logprob-gap", table T1: fp32 gives 0.00%
of importance ratios outside [0.9, 1.1] between batch 1 and batch 8, and its
rerun control is bit-exact.)"""
import hashlib

import numpy as np
import pytest
import torch

from invariant_lm_head_amd import lmhead
from tests.gpu_util import bits, gpu, host, i8, o, record, tl  # noqa: F401

pytestmark = pytest.mark.gpu

# every batch size of the sweep range: all tile variants and their boundaries
SIZES = list(range(1, 512))


def test_logits_bits_equal_for_every_batch_size(tl):
    """Batches 1..511 against batch 512: every logit of every row, bit for bit."""
    full = lmhead.logits(tl["gx"], tl["gw"])
    for B in SIZES:
        z = lmhead.logits(tl["gx"][:B].contiguous(), tl["gw"])
        assert torch.equal(bits(z), bits(full[:B])), B
    record("invariance", "logits_batches_1_to_512", {"batches": len(SIZES) + 1,
                                                     "rows_compared": sum(SIZES)})


def test_greedy_and_logprob_bits_equal_for_every_batch_size(tl):
    """Batches 1..511 against batch 512: top-2 ids, values, margin and log-prob."""
    t = gpu(tl["target"])
    g512 = lmhead.greedy_top2(tl["gx"], tl["gw"])
    l512 = lmhead.logprob(tl["gx"], tl["gw"], t)
    for B in SIZES:
        x = tl["gx"][:B].contiguous()
        g = lmhead.greedy_top2(x, tl["gw"])
        for a, b in zip(g[:3], g512[:3]):
            assert torch.equal(bits(a), bits(b[:B])), B
        lp = lmhead.logprob(x, tl["gw"], t[:B].contiguous())
        assert torch.equal(bits(lp), bits(l512[:B])), B
    record("invariance", "greedy_logprob_batches_1_to_512", {"batches": len(SIZES) + 1})


def test_packed_w_greedy_bits_equal_for_every_batch_size(tl):
    """The packed W layout (lmhead_pack_w), batches 1..512, against the
    row-major batch-512 call: top-2 ids, values and margin, bit for bit, with
    both rankings (float32 logits and the bf16-output head)."""
    pw = lmhead.pack_w(tl["gw"])
    for round_bf16 in (False, True):
        g512 = lmhead.greedy_top2(tl["gx"], tl["gw"], round_bf16=round_bf16)
        for B in SIZES + [512]:
            g = lmhead.greedy_top2(tl["gx"][:B].contiguous(), pw, round_bf16=round_bf16)
            for a, b in zip(g[:3], g512[:3]):
                assert torch.equal(bits(a), bits(b[:B])), (B, round_bf16)
    record("invariance", "packed_greedy_batches_1_to_512", {"batches": len(SIZES) + 1,
                                                            "rows_compared": sum(SIZES) + 512})


def test_row_position_and_neighbours_do_not_matter(tl):
    """A permuted batch (every row at another position with other neighbours)
    and one row repeated B times give the same bits per row."""
    x, w = tl["gx"], tl["gw"]
    t = gpu(tl["target"])
    z = lmhead.logits(x, w)
    g = lmhead.greedy_top2(x, w)
    lp = lmhead.logprob(x, w, t)
    perm = torch.randperm(512, generator=torch.Generator().manual_seed(0)).to(x.device)
    assert torch.equal(bits(lmhead.logits(x[perm].contiguous(), w)), bits(z[perm]))
    gp = lmhead.greedy_top2(x[perm].contiguous(), w)
    for a, b in zip(gp[:3], g[:3]):
        assert torch.equal(bits(a), bits(b[perm]))
    assert torch.equal(bits(lmhead.logprob(x[perm].contiguous(), w, t[perm].contiguous())),
                       bits(lp[perm]))
    for r, B in [(0, 16), (5, 64), (300, 257), (511, 512)]:
        rep = x[r:r + 1].repeat(B, 1).contiguous()
        zr = lmhead.logits(rep, w)
        assert torch.equal(bits(zr), bits(z[r:r + 1]).expand(B, -1)), (r, B)
        lr = lmhead.logprob(rep, w, t[r:r + 1].repeat(B).contiguous())
        assert torch.equal(bits(lr), bits(lp[r:r + 1]).expand(B)), (r, B)


def test_reruns_are_bit_exact(tl):
    t = gpu(tl["target"])
    for B in (1, 64, 512):
        x = tl["gx"][:B].contiguous()
        a = [lmhead.logprob(x, tl["gw"], t[:B].contiguous()) for _ in range(3)]
        assert all(torch.equal(bits(a[0]), bits(b)) for b in a[1:])


def test_importance_ratio_out_of_band_is_zero(tl):
    """exp(logp at batch B - logp at batch 1) stays exactly 1 for every row."""
    t = gpu(tl["target"])
    lp1 = torch.cat([lmhead.logprob(tl["gx"][r:r + 1].contiguous(), tl["gw"], t[r:r + 1].contiguous())
                     for r in range(32)])
    for B in (8, 32):
        lpb = lmhead.logprob(tl["gx"][:B].contiguous(), tl["gw"], t[:B].contiguous())
        ratio = torch.exp(lpb.double() - lp1[:B].double())
        out_of_band = ((ratio < 0.9) | (ratio > 1.1)).float().mean().item()
        assert out_of_band == 0.0 and torch.equal(ratio, torch.ones_like(ratio))


def test_int8_logit_hash_identical_across_batches(i8):
    """A per-row digest of the int32 logits (SHA-256, 12 hex digits) is the same
    at batch 1, 8 and 64 and in a reversed batch."""
    x, w = i8["gx"], i8["gw"]

    def digests(z):
        return [hashlib.sha256(host(r).astype("<i4").tobytes()).hexdigest()[:12] for r in z]

    ref = digests(lmhead.logits(x[:8].contiguous(), w))
    assert digests(lmhead.logits(x[:1].contiguous(), w)) == ref[:1]
    assert digests(lmhead.logits(x[:64].contiguous(), w))[:8] == ref
    assert digests(lmhead.logits(x[:8].flip(0).contiguous(), w))[::-1] == ref


def test_int8_greedy_every_batch_size_against_oracle(i8):
    """The int8 head at every batch 1..512 (every plan, every short last row
    tile): ids, exact raw values, scaled values and margins bit for bit equal
    to the oracle's stored outputs for those rows."""
    g = i8["golden"]
    for B in range(1, 513):
        ids, vals, margin, raw = lmhead.greedy_top2(i8["gx"][:B].contiguous(), i8["gw"],
                                                    row_scale=i8["gs"][:B].contiguous())
        assert np.array_equal(host(ids), g["ids"][:B]), B
        assert np.array_equal(host(raw).astype(np.int64), g["raw"][:B]), B
        assert np.array_equal(host(vals).view(np.int32), g["vals"][:B].view(np.int32)), B
        assert np.array_equal(host(margin).view(np.int32), g["margin"][:B].view(np.int32)), B
    record("invariance", "int8_greedy_batches_1_to_512_vs_oracle",
           {"batches": 512, "rows_compared": 512 * 513 // 2})
