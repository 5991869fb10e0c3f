"""Batch-variance demonstrator ("batch-logprob-gap": the importance ratio
exp(logp_new - logp_old) of an unchanged policy leaves [0.9, 1.1] when only the
batch shape changes; repeating the same batch is bit-exact).  Without a model:
log p(target) of the same 512 rows scored as one batch of 512, as 64 batches of
8 and one row at a time, by this head and by batch-variant comparators built
from library GEMMs, and the ratio between them.  This head must give the same
bits at every batch size; the comparators are measured and printed."""
import numpy as np
import pytest
import torch

from invariant_lm_head_amd import lmhead
from tests.gpu_util import DEV, gpu, host, o, record, tl  # noqa: F401

pytestmark = pytest.mark.gpu

BAND = (0.9, 1.1)


def score_in_batches(fn, n_rows, bsz):
    return torch.cat([fn(r, min(r + bsz, n_rows)) for r in range(0, n_rows, bsz)])


def ratio_stats(lp_b, lp_1):
    """Share of rows whose log-prob bits differ, max |dlogp|, out-of-band share."""
    a, b = host(lp_b).astype(np.float64), host(lp_1).astype(np.float64)
    changed = np.mean(host(lp_b).view(np.int32) != host(lp_1).view(np.int32))
    ratio = np.exp(a - b)
    out = np.mean((ratio < BAND[0]) | (ratio > BAND[1]))
    return float(changed), float(np.max(np.abs(a - b))), float(out)


def comparators(x, w, t):
    """log p(target) functions (rows r0..r1) of batch-variant heads."""
    wt_bf = w.t()
    wf = w.float()

    def lib_bf16(r0, r1):                      # library bf16 GEMM, bf16 logits
        z = torch.matmul(x[r0:r1], wt_bf).float()
        return torch.log_softmax(z, dim=-1).gather(1, t[r0:r1, None].long())[:, 0]

    def lib_fp32(r0, r1):                      # library float32 GEMM
        z = torch.matmul(x[r0:r1].float(), wf.t())
        return torch.log_softmax(z, dim=-1).gather(1, t[r0:r1, None].long())[:, 0]

    def split_k(r0, r1):                       # float32 split-K, split count chosen by batch
        xs = x[r0:r1].float()
        s = 1 if r1 - r0 <= 8 else 4
        H = xs.shape[1]
        z = sum(torch.matmul(xs[:, k:k + H // s], wf[:, k:k + H // s].t())
                for k in range(0, H, H // s))
        return torch.log_softmax(z, dim=-1).gather(1, t[r0:r1, None].long())[:, 0]

    return {"library bf16 GEMM": lib_bf16, "library fp32 GEMM": lib_fp32,
            "fp32 split-K by batch": split_k}


def measure(tl, n=512):
    """{name: {(B, 1): (changed, max|dlogp|, out-of-band)}} for this head and the
    comparators, plus the rerun control (the same batch twice)."""
    x, w = tl["gx"][:n].contiguous(), tl["gw"]
    t = gpu(tl["target"][:n])

    def ours(r0, r1):
        return lmhead.logprob(x[r0:r1].contiguous(), w, t[r0:r1].contiguous())

    heads = {"this head": ours, **comparators(x, w, t)}
    res = {}
    for name, fn in heads.items():
        lp1 = score_in_batches(fn, n, 1)
        lp8 = score_in_batches(fn, n, 8)
        lpn = score_in_batches(fn, n, n)
        rerun = score_in_batches(fn, n, n)
        res[name] = {"b8_vs_b1": ratio_stats(lp8, lp1), "b512_vs_b1": ratio_stats(lpn, lp1),
                     "rerun": ratio_stats(rerun, lpn)}
    return res


def test_batch_variance_demonstrator(tl):
    res = measure(tl)
    print(f"{'head':24s} {'compare':11s} {'bits differ':>11s} {'max|dlogp|':>11s} "
          f"{'ratio out of [0.9,1.1]':>23s}", flush=True)
    for name, r in res.items():
        for k, (ch, mx, out) in r.items():
            print(f"{name:24s} {k:11s} {100 * ch:10.2f}% {mx:11.2e} {100 * out:22.2f}%", flush=True)
            record("batch_variance", f"{name} | {k}", {"bits_differ": ch, "max_abs_dlogp": mx,
                                                        "ratio_out_of_band": out})
    for k in ("b8_vs_b1", "b512_vs_b1", "rerun"):
        assert res["this head"][k] == (0.0, 0.0, 0.0), k
    for name in res:
        assert res[name]["rerun"][0] == 0.0, name       # every head is bit-exact on a rerun
