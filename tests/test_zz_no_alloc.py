"""The entry point that allocates nothing (lmhead_greedy_top2_noalloc, through
the C-ABI) against lmhead_greedy_top2 with a caller workspace: bitwise equal
outputs on two calls in a row, the second with a smaller input, in every
mode (bf16, bf16 from packed W, int8); a shape beyond the static workspace is
refused."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from invariant_lm_head_amd import lmhead
from tests.gpu_util import DEV, gpu, gpu_bf16

pytestmark = pytest.mark.gpu


def _noalloc(lib, mode, x, w, B, H, V, scale=None, round_bf16=0):
    """Direct C-ABI call; returns the four outputs as host arrays."""
    ids = torch.full((B, 2), -7, dtype=torch.int32, device=DEV)
    vals = torch.full((B, 2), -7.0, dtype=torch.float32, device=DEV)
    margin = torch.full((B,), -7.0, dtype=torch.float32, device=DEV)
    raw = torch.full((B, 2), -7, dtype=torch.int32, device=DEV) if mode == 1 else None
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    st = lib.lmhead_greedy_top2_noalloc(mode, round_bf16, P(x), P(w), B, H, V, P(scale), P(ids),
                                        P(vals), P(margin), P(raw), stream)
    assert st == 0, lib.lmhead_status_string(st)
    torch.cuda.synchronize()
    return [None if t is None else t.cpu().numpy().view(np.int32) for t in (ids, vals, margin, raw)]


def _with_workspace(x, w, scale=None, round_bf16=False):
    out = lmhead.greedy_top2(x, w, row_scale=scale, round_bf16=round_bf16)
    torch.cuda.synchronize()
    return [None if t is None else t.cpu().numpy().view(np.int32) for t in out]


def _same(a, b):
    for u, v in zip(a, b):
        assert (u is None) == (v is None)
        if u is not None:
            assert np.array_equal(u, v)


def test_noalloc_matches_workspace_entry_point():
    lib = lmhead.library()
    d = synth.make_inputs("tinyllama")
    x, w = gpu_bf16(d["x"]), gpu_bf16(d["w"])
    H, V = d["x"].shape[1], d["w"].shape[0]
    # batch 512 (two row tiles, 2 MB of records), then batch 5 (one row tile):
    # the second call runs on what the first left in the static array
    for B, rnd in ((512, 0), (5, 0), (300, 1), (1, 1)):
        xb = x[:B].contiguous()
        got = _noalloc(lib, 0, xb, w, B, H, V, round_bf16=rnd)
        _same(got, _with_workspace(xb, w, round_bf16=bool(rnd)))
    # the packed W layout (mode 2): batch 257 (a one-row last tile), then 3
    pw = lmhead.pack_w(w)
    for B in (257, 3):
        xb = x[:B].contiguous()
        got = _noalloc(lib, lmhead.MODE_BF16_PACKED, xb, pw.data, B, H, V)
        _same(got, _with_workspace(xb, pw))
    # int8 head (4096 x 128256 would need 4 MB at batch 512; a smaller vocabulary
    # keeps the test short): batch 64, then 3
    rng = np.random.default_rng(31)
    H8, V8 = 1024, 20000
    x8 = gpu(rng.integers(-127, 128, (64, H8)).astype(np.int8))
    w8 = gpu(rng.integers(-127, 128, (V8, H8)).astype(np.int8))
    s8 = gpu((2.0 ** -18 * rng.uniform(0.5, 2.0, 64)).astype(np.float32))
    for B in (64, 3):
        xb, sb = x8[:B].contiguous(), s8[:B].contiguous()
        got = _noalloc(lib, 1, xb, w8, B, H8, V8, scale=sb)
        _same(got, _with_workspace(xb, w8, scale=sb))


def test_noalloc_refuses_oversized_workspace():
    lib = lmhead.library()
    B, H, V = 16384, 4096, 151936          # 311 MB of records
    assert lib.lmhead_workspace_bytes(0, B, H, V) > lmhead.STATIC_WORKSPACE_BYTES
    x = torch.empty((1, 16), dtype=torch.uint8, device=DEV)
    P = ctypes.c_void_p(x.data_ptr())
    st = lib.lmhead_greedy_top2_noalloc(0, 0, P, P, B, H, V, None, P, P, P, None, None)
    assert st == 6   # LMHEAD_E_WORKSPACE, before anything is queued
