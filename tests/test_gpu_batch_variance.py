"""Batch-variance demonstrator ("batch-logprob-gap": the importance ratio
exp(logp_new - logp_old) of an unchanged policy leaves [0.9, 1.1] when only the
batch shape changes; repeating the same batch is bit-exact).  Without a model:
log p(target) of the same 512 rows scored as one batch of 512, as 64 batches of
8 and one row at a time, by this head and by batch-variant comparators built
from library GEMMs, and the ratio between them.

Two row sets: the TinyLlama-shaped head (logit std 0.9), and the same rows with
W scaled by 3.5 (logit std 3.2, the spread of a trained model's logits).  The
comparators with bf16 engine numerics (bf16 logits and a bf16 log-softmax, as
an inference engine keeps them) quantise log p to 2^-3 nats at |log p| >= 16,
so a batch-dependent rounding flip moves the ratio by 13%: at the wider spread
they leave the band on a few percent of rows, the shape of the pages' table,
while this head gives the same bits at every batch size."""
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

    def engine_bf16(r0, r1):                   # library bf16 GEMM, bf16 log-softmax
        z = torch.matmul(x[r0:r1], wt_bf)
        return torch.log_softmax(z, dim=-1).gather(1, t[r0:r1, None].long())[:, 0].float()

    H = x.shape[1]
    # k slices of W, transposed and contiguous, for one and four splits
    w_k = {s: [w[:, k:k + H // s].t().contiguous() for k in range(0, H, H // s)] for s in (1, 4)}

    def split_k_bf16(r0, r1):                  # bf16 partials, split count by batch, bf16 log-softmax
        s = 1 if r1 - r0 <= 8 else 4
        z = None
        for i, wk in enumerate(w_k[s]):
            part = torch.matmul(x[r0:r1, i * (H // s):(i + 1) * (H // s)].contiguous(), wk)
            z = part if z is None else z + part
        return torch.log_softmax(z, dim=-1).gather(1, t[r0:r1, None].long())[:, 0].float()

    return {"library bf16 GEMM": lib_bf16, "library fp32 GEMM": lib_fp32,
            "fp32 split-K by batch": split_k, "bf16 engine (bf16 log-softmax)": engine_bf16,
            "bf16 split-K by batch (bf16 log-softmax)": split_k_bf16}


def measure(tl, n=512, w_scale=1.0):
    """{name: {(B, 1): (changed, max|dlogp|, out-of-band)}} for this head and the
    comparators, plus the rerun control (the same batch twice)."""
    x, w = tl["gx"][:n].contiguous(), tl["gw"]
    if w_scale != 1.0:
        w = (w.float() * w_scale).to(torch.bfloat16).contiguous()
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


ROW_SETS = {"tinyllama": 1.0, "tinyllama, W x 3.5": 3.5}


@pytest.mark.parametrize("rows", list(ROW_SETS))
def test_batch_variance_demonstrator(tl, rows):
    res = measure(tl, w_scale=ROW_SETS[rows])
    for name, r in res.items():
        for k, (ch, mx, out) in r.items():
            record("batch_variance", f"{rows} | {name} | {k}",
                   {"bits_differ": ch, "max_abs_dlogp": mx, "ratio_out_of_band": out})
    for k in ("b8_vs_b1", "b512_vs_b1", "rerun"):
        assert res["this head"][k] == (0.0, 0.0, 0.0), k
    for name in res:
        assert res[name]["rerun"][0] == 0.0, name       # every head is bit-exact on a rerun
    if ROW_SETS[rows] > 1.0:
        # the demonstrator shows the effect: a batch-dependent split with bf16
        # numerics leaves the band on some rows at a trained model's spread
        assert res["bf16 split-K by batch (bf16 log-softmax)"]["b512_vs_b1"][2] > 0.0
