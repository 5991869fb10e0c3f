"""The float head's small-batch plan (512 bytes of each row per stage, X and W
rings of equal depth) at the pipeline's degenerate lengths: one stage (H = 256),
two (512), three (768) and nine (2304), with a ragged last vocabulary block
(V = 1000).  Logits, greedy top-2 and log-prob against the oracle, and every
row bitwise equal to the same row computed at batch 40, whose plan stages 256
bytes per row."""
import numpy as np
import pytest

import synth
from invariant_lm_head_amd import lmhead
from tests.gpu_util import TOL, check_greedy_bf16, gpu, gpu_bf16, host, o  # noqa: F401

pytestmark = pytest.mark.gpu

V = 1000


@pytest.mark.parametrize("H", [256, 512, 768, 2304])
def test_small_batch_stage_lengths(o, H):
    rng = np.random.default_rng(H)
    xb = synth.bf16_from_f32(rng.standard_normal((40, H)).astype(np.float32))
    wb = synth.bf16_from_f32((0.05 * rng.standard_normal((V, H))).astype(np.float32))
    t = rng.integers(0, V, 40).astype(np.int32)
    x, w, gt = gpu_bf16(xb), gpu_bf16(wb), gpu(t)

    def run(n):
        z = lmhead.logits(x[:n].contiguous(), w)
        ids, vals, margin, _ = lmhead.greedy_top2(x[:n].contiguous(), w)
        lp = lmhead.logprob(x[:n].contiguous(), w, gt[:n].contiguous())
        return z, ids, vals, margin, lp

    ref = [host(a) for a in run(40)]
    for n in (1, 7, 32):
        z, ids, vals, margin, lp = run(n)
        assert np.max(np.abs(host(z) - o.logits_bf16(xb[:n], wb))) <= TOL
        check_greedy_bf16(ids, vals, margin, *o.greedy_bf16(xb[:n], wb))
        assert np.max(np.abs(host(lp) - o.logprob_bf16(xb[:n], wb, t[:n]))) <= TOL
        for got, full in zip((z, ids, vals, margin, lp), ref):
            got = host(got)
            assert np.array_equal(got.view(np.int32), full[:n].view(np.int32)), (H, n)
