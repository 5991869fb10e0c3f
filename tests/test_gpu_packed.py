"""The packed bf16 weight layout (lmhead_pack_w, LMHEAD_MODE_BF16_PACKED) on the
GPU, through the C-ABI.  Packing moves bytes and changes no arithmetic, so:

- the packed bytes equal the layout's formula in the header, applied here in
  numpy (rows past V zero);
- every entry point with the packed W returns the bits it returns with the
  row-major W, at batch sizes that run every tile plan of the float head
  (including the gated head's float32 recompute, which reads W rows itself);
- one case against the oracle directly.
"""
import math

import numpy as np
import pytest
import torch

import synth
from invariant_lm_head_amd import lmhead
from tests.gpu_util import DEV, TOL, check_greedy_bf16, gpu, gpu_bf16, host, o  # noqa: F401

pytestmark = pytest.mark.gpu


def packed_reference(wb: np.ndarray) -> np.ndarray:
    """The header's formula: byte k of row v at (v / 128) (128 R + 16384) +
    (k / 128) 16384 + (v % 128) 128 + k % 128, R = 2H; rows from V to the end
    of the last group of 128 and each group's unused last block are zero."""
    V, H = wb.shape
    R = 2 * H
    C = 128
    group = 128 * R + 128 * C
    src = np.ascontiguousarray(wb, dtype=np.uint16).view(np.uint8).reshape(V, R)
    out = np.zeros((V + 127) // 128 * group, dtype=np.uint8)
    v = np.arange(V, dtype=np.int64)[:, None]
    k = np.arange(R, dtype=np.int64)[None, :]
    off = (v // 128) * group + (k // C) * 128 * C + (v % 128) * C + k % C
    out[off] = src
    return out


def bf16_w(rng, V, H, scale=0.1):
    return synth.bf16_from_f32((scale * rng.standard_normal((V, H))).astype(np.float32))


@pytest.mark.parametrize("V,H", [(1000, 64), (130, 192), (3000, 2048), (257, 256), (2, 64)])
def test_pack_layout(V, H):
    """Row lengths of one block (128 bytes), three (384), 32 (4096) and four
    (512), and ragged last groups."""
    rng = np.random.default_rng(V + H)
    wb = bf16_w(rng, V, H)
    pw = lmhead.pack_w(gpu_bf16(wb))
    got = host(pw.data)
    want = packed_reference(wb)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


def _bits(t):
    a = host(t) if not isinstance(t, np.ndarray) else t
    return a.view(np.int32) if a.dtype == np.float32 else a


def _same(a, b, what):
    if a is None or b is None:
        assert a is None and b is None, what
        return
    ha, hb = _bits(a), _bits(b)
    assert ha.dtype == hb.dtype and np.array_equal(ha, hb), what


# (H, V): row bytes 4096 (the float head's 512-byte stages when row-major),
# 384 (128-byte stages), 1536, 128 (one block per row) with a ragged last
# group, and a vocabulary wide enough for the 128 x 256 and 256 x 256 tiles at
# batches 65-128 and 129-256
SHAPES = [(2048, 32000), (192, 1000), (768, 1000), (64, 1001), (128, 70001)]
BATCHES = [1, 7, 33, 64, 65, 129, 200, 257, 300]


@pytest.fixture(scope="module")
def heads():
    out = {}
    for H, V in SHAPES:
        rng = np.random.default_rng(H * 7 + V)
        x = gpu_bf16(synth.bf16_from_f32(rng.standard_normal((max(BATCHES), H)).astype(np.float32)))
        w = gpu_bf16(bf16_w(rng, V, H))
        t = gpu(rng.integers(0, V, max(BATCHES)).astype(np.int32))
        seed = gpu(rng.integers(0, 2 ** 62, max(BATCHES), dtype=np.int64))
        pos = gpu(rng.integers(0, 2 ** 40, max(BATCHES), dtype=np.int64))
        out[(H, V)] = (x, w, lmhead.pack_w(w), t, seed, pos)
    return out


@pytest.mark.parametrize("H,V", SHAPES)
def test_packed_bitwise_equal_row_major(heads, H, V):
    x_all, w, pw, t_all, seed_all, pos_all = heads[(H, V)]
    for B in BATCHES:
        x, t = x_all[:B].contiguous(), t_all[:B].contiguous()
        seed, pos = seed_all[:B].contiguous(), pos_all[:B].contiguous()
        for name, f in [
            ("logits", lambda ww: (lmhead.logits(x, ww),)),
            ("logits bf16", lambda ww: (lmhead.logits(x, ww, round_bf16=True).view(torch.int16),)),
            ("greedy", lambda ww: lmhead.greedy_top2(x, ww)),
            ("greedy bf16", lambda ww: lmhead.greedy_top2(x, ww, round_bf16=True)),
            ("logprob", lambda ww: (lmhead.logprob(x, ww, t),)),
            ("gated 1e-3", lambda ww: lmhead.greedy_gated(x, ww, 1e-3)),
            ("gated all rows", lambda ww: lmhead.greedy_gated(x, ww, math.inf)),
            ("sample", lambda ww: lmhead.sample_gumbel(x, ww, 0.8, seed, pos)),
        ]:
            for a, b in zip(f(w), f(pw)):
                _same(a, b, (H, V, B, name))
        if lmhead.workspace_bytes(0, B, H, V) <= lmhead.STATIC_WORKSPACE_BYTES:
            for a, b in zip(lmhead.greedy_top2_noalloc(x, w), lmhead.greedy_top2_noalloc(x, pw)):
                _same(a, b, (H, V, B, "noalloc"))


def test_packed_self_check(heads):
    x, w, pw, *_ = heads[(192, 1000)]
    assert lmhead.self_check(x[:300].contiguous(), pw) == 0


def test_packed_against_oracle(o):
    """Packed W against the oracle itself: greedy top-2 and log-prob."""
    rng = np.random.default_rng(5)
    B, H, V = 40, 256, 1001
    xb = synth.bf16_from_f32(rng.standard_normal((B, H)).astype(np.float32))
    wb = bf16_w(rng, V, H)
    t = rng.integers(0, V, B).astype(np.int32)
    pw = lmhead.pack_w(gpu_bf16(wb))
    x = gpu_bf16(xb)
    ids, vals, margin, _ = lmhead.greedy_top2(x, pw)
    check_greedy_bf16(ids, vals, margin, *o.greedy_bf16(xb, wb))
    lp = host(lmhead.logprob(x, pw, gpu(t)))
    assert np.max(np.abs(lp - o.logprob_bf16(xb, wb, t))) <= TOL


def test_packed_binding_refuses_int8():
    """The packed layout is a bf16 layout: int8 rows with it are refused."""
    w = gpu_bf16(np.zeros((130, 64), dtype=np.uint16))
    pw = lmhead.pack_w(w)
    x8 = gpu(np.zeros((2, 64), dtype=np.int8))
    with pytest.raises(TypeError):
        lmhead.greedy_top2(x8, pw)
