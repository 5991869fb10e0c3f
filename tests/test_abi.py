"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and its host-side validation returns the documented status
codes before queueing anything (no pointer is dereferenced, no HIP call made)."""
import ctypes
import re
from pathlib import Path

import pytest

from invariant_lm_head_amd import _build, lmhead

HEADER = Path(__file__).resolve().parents[1] / "include" / "lmhead.h"

OK, E_NULL, E_SHAPE, E_ALIGN, E_MODE, E_OVERFLOW, E_WORKSPACE, E_HIP, E_VALUE = range(9)
A = ctypes.c_void_p(0x10000)      # aligned, never dereferenced
A2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10008)    # 8-byte aligned only
ODD = ctypes.c_void_p(0x10002)    # 2-byte aligned only
S = ctypes.c_void_p(0)            # default stream (never reached)


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(lmhead_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return lmhead.library()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) == 16
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(lmhead.SIGNATURES)


def test_library_matches_its_sources(lib):
    """The loaded library was built from the sources beside it (the binding
    refuses a library whose recorded digest differs)."""
    assert lib.lmhead_source_digest().decode() == _build.source_digest()


def test_stale_library_is_refused(monkeypatch):
    """A library whose recorded digest is not the sources' is not loaded."""
    monkeypatch.setattr(lmhead, "_lib", None)
    monkeypatch.setattr(_build, "source_digest", lambda: "0" * 16)
    with pytest.raises(lmhead.StaleLibraryError):
        lmhead.library()


def test_library_is_gfx950_only():
    out = _build.FLAGS
    assert "--offload-arch=gfx950" in out and "-ffp-contract=off" in out


def test_status_strings(lib):
    for st in range(8):
        assert lib.lmhead_status_string(st)
    assert b"unknown" in lib.lmhead_status_string(99)
    assert lib.lmhead_last_error()


def test_workspace_bytes_layout(lib):
    # target logits (B x 4 B) | B x ceil(V/128) 16-byte records, the first
    # region rounded up to 256 bytes
    def up(n):
        return (n + 255) // 256 * 256

    for (B, H, V) in [(1, 2048, 32000), (512, 2048, 32000), (4, 64, 1000), (16384, 4096, 151936)]:
        want = up(4 * B) + 16 * B * ((V + 127) // 128)
        assert lib.lmhead_workspace_bytes(0, B, H, V) == want
        assert lib.lmhead_workspace_bytes(1, B, H, V) == want
        assert lib.lmhead_workspace_bytes(2, B, H, V) == want     # packed W: same workspace
    assert lib.lmhead_workspace_bytes(0, 0, 2048, 32000) == 0
    assert lib.lmhead_workspace_bytes(0, 1, 100, 32000) == 0
    assert lib.lmhead_workspace_bytes(3, 1, 2048, 32000) == 0
    # B and V each within bounds but together beyond one launch grid (2^32 threads)
    assert lib.lmhead_workspace_bytes(0, 1 << 24, 64, 151936) == 0
    assert lib.lmhead_workspace_bytes(0, 1 << 24, 64, 32000) > 0      # 2^32 - 2^24 threads: fits
    assert lib.lmhead_workspace_bytes(0, 512, 64, 1 << 30) == 0
    assert lib.lmhead_workspace_bytes(0, 32, 64, 1 << 30) > 0


def logits_status(lib, mode=0, rnd=0, x=A, w=A, B=4, H=64, V=1000, out=A2):
    return lib.lmhead_logits(mode, rnd, x, w, B, H, V, out, S)


def test_logits_validation(lib):
    assert logits_status(lib, mode=3) == E_MODE
    assert logits_status(lib, mode=-1) == E_MODE
    assert logits_status(lib, rnd=2) == E_MODE
    assert logits_status(lib, mode=2, x=None) == E_NULL         # packed W: a bf16 mode
    assert logits_status(lib, mode=2, rnd=1, out=None) == E_NULL
    assert logits_status(lib, mode=2, w=MIS) == E_ALIGN
    assert logits_status(lib, mode=2, H=96) == E_SHAPE
    assert logits_status(lib, mode=1, rnd=1) == E_MODE          # bf16 rounding needs bf16 mode
    assert logits_status(lib, x=None) == E_NULL
    assert logits_status(lib, w=None) == E_NULL
    assert logits_status(lib, out=None) == E_NULL
    for B, H, V in [(0, 64, 1000), (4, 0, 1000), (4, 96, 1000), (4, 64, 1), (4, 64, 0),
                    (-1, 64, 10), ((1 << 24) + 1, 64, 10)]:
        assert logits_status(lib, B=B, H=H, V=V) == E_SHAPE, (B, H, V)
    assert logits_status(lib, mode=1, H=131072) == E_OVERFLOW
    assert logits_status(lib, mode=1, H=131008) != E_OVERFLOW
    assert logits_status(lib, x=MIS) == E_ALIGN
    assert logits_status(lib, w=MIS) == E_ALIGN
    assert logits_status(lib, out=ODD) == E_ALIGN


def test_greedy_validation(lib):
    ws_need = lib.lmhead_workspace_bytes(0, 4, 64, 1000)

    def call(mode=0, rnd=0, x=A, w=A, B=4, H=64, V=1000, scale=None, ids=A, vals=A, margin=A,
             raw=None, ws=A2, nws=ws_need):
        return lib.lmhead_greedy_top2(mode, rnd, x, w, B, H, V, scale, ids, vals, margin, raw,
                                      ws, nws, S)

    assert call(mode=7) == E_MODE
    assert call(mode=1, rnd=1) == E_MODE
    assert call(ids=None) == E_NULL
    assert call(vals=None) == E_NULL
    assert call(margin=None) == E_NULL
    assert call(V=1) == E_SHAPE
    assert call(H=65) == E_SHAPE
    assert call(ids=ODD) == E_ALIGN
    assert call(vals=ODD) == E_ALIGN
    assert call(mode=1, raw=ODD) == E_ALIGN
    assert call(mode=1, scale=ODD) == E_ALIGN
    assert call(x=MIS) == E_ALIGN
    assert call(ws=None) == E_WORKSPACE
    assert call(nws=ws_need - 1) == E_WORKSPACE
    assert call(ws=MIS) == E_ALIGN
    assert call(mode=1, H=1 << 17) == E_OVERFLOW
    assert call(B=1 << 24, V=151936) == E_SHAPE        # grid beyond 2^32 threads


def test_logprob_validation(lib):
    ws_need = lib.lmhead_workspace_bytes(0, 4, 64, 1000)

    def call(mode=0, x=A, w=A, B=4, H=64, V=1000, scale=None, tgt=A, out=A, ws=A2, nws=ws_need):
        return lib.lmhead_logprob(mode, x, w, B, H, V, scale, tgt, out, ws, nws, S)

    assert call(mode=5) == E_MODE
    assert call(tgt=None) == E_NULL
    assert call(out=None) == E_NULL
    assert call(B=0) == E_SHAPE
    assert call(tgt=ODD) == E_ALIGN
    assert call(out=ODD) == E_ALIGN
    assert call(w=MIS) == E_ALIGN
    assert call(nws=16) == E_WORKSPACE
    assert call(mode=1, H=1 << 18) == E_OVERFLOW


def test_gated_validation(lib):
    ws_need = lib.lmhead_workspace_bytes(0, 4, 64, 1000)

    def call(mode=0, x=A, w=A, B=4, H=64, V=1000, tau=1e-3, ids=A, vals=A, margin=A, gated=A,
             ws=A2, nws=ws_need):
        return lib.lmhead_greedy_gated(mode, x, w, B, H, V, tau, ids, vals, margin, gated, ws,
                                       nws, S)

    assert call(mode=1) == E_MODE              # the float32 recompute is a bf16-mode step
    assert call(mode=3) == E_MODE
    assert call(gated=None) == E_NULL
    assert call(gated=ODD) == E_ALIGN
    assert call(tau=-1.0) == E_VALUE
    assert call(tau=float("nan")) == E_VALUE
    assert call(tau=-0.0, ids=None) == E_NULL  # -0 is a valid tau; the inner call refuses
    assert call(ids=None) == E_NULL
    assert call(margin=ODD) == E_ALIGN
    assert call(nws=ws_need - 1) == E_WORKSPACE
    assert call(V=1) == E_SHAPE
    assert lib.lmhead_status_string(E_VALUE) == b"a scalar argument is out of range"


def test_sample_validation(lib):
    ws_need = lib.lmhead_workspace_bytes(0, 4, 64, 1000)
    A8 = ctypes.c_void_p(0x30000)

    def call(mode=0, x=A, w=A, B=4, H=64, V=1000, T=1.0, scale=None, seed=A8, pos=A8, tok=A,
             val=None, gap=None, ws=A2, nws=ws_need):
        return lib.lmhead_sample_gumbel(mode, x, w, B, H, V, T, scale, seed, pos, tok, val, gap,
                                        ws, nws, S)

    assert call(mode=3) == E_MODE
    assert call(mode=2, seed=None) == E_NULL
    assert call(seed=None) == E_NULL
    assert call(pos=None) == E_NULL
    assert call(tok=None) == E_NULL
    assert call(seed=ctypes.c_void_p(0x30004)) == E_ALIGN   # 4-byte aligned only
    assert call(tok=ODD) == E_ALIGN
    assert call(val=ODD) == E_ALIGN
    assert call(T=0.0) == E_VALUE
    assert call(T=-1.0) == E_VALUE
    assert call(T=float("inf")) == E_VALUE
    assert call(T=float("nan")) == E_VALUE
    assert call(nws=ws_need - 1) == E_WORKSPACE
    assert call(V=1) == E_SHAPE
    assert call(mode=1, H=1 << 17) == E_OVERFLOW


def test_packed_w_layout_size_and_validation(lib):
    """lmhead_packed_w_bytes: ceil(V / 128) groups of 128 rows of 2H bytes and
    one unused 16 KB block; no int8 bound on H (a bf16 layout).  lmhead_pack_w
    refuses what the other calls refuse, and a destination whose range meets
    w's, before anything is queued."""
    for H, V in [(2048, 32000), (64, 2), (64, 129), (4096, 151936), (131072, 1000)]:
        assert lib.lmhead_packed_w_bytes(H, V) == (V + 127) // 128 * (128 * 2 * H + 16384), (H, V)
    for H, V in [(100, 1000), (0, 1000), (64, 1), (64, (1 << 30) + 1), ((1 << 20) + 64, 10)]:
        assert lib.lmhead_packed_w_bytes(H, V) == 0, (H, V)

    def call(w=A, H=64, V=1000, out=A2):
        return lib.lmhead_pack_w(w, H, V, out, S)

    assert call(w=None) == E_NULL
    assert call(out=None) == E_NULL
    assert call(w=MIS) == E_ALIGN
    assert call(out=MIS) == E_ALIGN
    assert call(H=96) == E_SHAPE
    assert call(V=1) == E_SHAPE
    # packing in place, or into a range that meets w's, is refused
    w0 = 0x100000
    nw = 1000 * 2 * 64
    assert call(w=ctypes.c_void_p(w0), out=ctypes.c_void_p(w0)) == E_VALUE
    assert call(w=ctypes.c_void_p(w0), out=ctypes.c_void_p(w0 + nw - 16)) == E_VALUE
    assert call(w=ctypes.c_void_p(w0 + 16), out=ctypes.c_void_p(w0)) == E_VALUE


def test_quantize_validation(lib):
    def call(x=A, B=4, H=100, q=A2, m=A, e=A):
        return lib.lmhead_quantize_rows(x, B, H, q, m, e, S)

    assert call(x=None) == E_NULL
    assert call(q=None) == E_NULL
    assert call(m=None) == E_NULL
    assert call(e=None) == E_NULL
    assert call(B=0) == E_SHAPE
    assert call(H=0) == E_SHAPE
    assert call(B=(1 << 24) + 1) == E_SHAPE
    assert call(x=ODD) == E_ALIGN
    assert call(m=ODD) == E_ALIGN
    assert call(e=ODD) == E_ALIGN


def test_logprob_int_validation(lib):
    ws_need = lib.lmhead_workspace_bytes(1, 4, 64, 1000)

    def call(x=A, w=A, B=4, H=64, V=1000, um=1 << 30, ue=-40, sm=A, se=A, tgt=A, out=A2,
             ws=A2, nws=ws_need):
        return lib.lmhead_logprob_int(x, w, B, H, V, um, ue, sm, se, tgt, out, ws, nws, S)

    assert call(x=None) == E_NULL
    assert call(sm=None) == E_NULL
    assert call(se=None) == E_NULL
    assert call(tgt=None) == E_NULL
    assert call(out=None) == E_NULL
    assert call(V=1) == E_SHAPE
    assert call(H=65) == E_SHAPE
    assert call(H=1 << 17) == E_OVERFLOW
    assert call(x=MIS) == E_ALIGN
    assert call(sm=ODD) == E_ALIGN
    assert call(out=ctypes.c_void_p(0x20004)) == E_ALIGN     # int64 output: 8-byte aligned
    assert call(um=0) == E_VALUE
    assert call(um=-5) == E_VALUE
    assert call(ws=None) == E_WORKSPACE
    assert call(nws=ws_need - 1) == E_WORKSPACE


def test_self_check_validation(lib):
    need = lib.lmhead_self_check_bytes(0, 4, 64, 1000)
    # batch logits + one-row logits + reversed logits + reversed rows, 256-byte aligned regions
    up = lambda n: (n + 255) // 256 * 256  # noqa: E731
    assert need == 2 * up(4 * 4 * 1000) + up(4 * 1000) + up(4 * 64 * 2)
    assert lib.lmhead_self_check(0, A, A, 4, 64, 1000, None, need, A2, S) == E_NULL
    assert lib.lmhead_self_check(0, A, A, 4, 64, 1000, A2, need, None, S) == E_NULL
    assert lib.lmhead_self_check(0, A, A, 4, 64, 1000, A2, need - 1, A, S) == E_WORKSPACE
    assert lib.lmhead_self_check(0, A, A, 4, 64, 1000, MIS, need, A, S) == E_ALIGN
    # the mismatch counter is a 64-bit device atomic: 4-byte alignment is refused
    assert lib.lmhead_self_check(0, A, A, 4, 64, 1000, A2, need, ctypes.c_void_p(0x20004),
                                 S) == E_ALIGN


def test_binding_refuses_mixed_dtypes():
    import torch
    with pytest.raises(TypeError):
        lmhead._mode_of(torch.zeros(1, 64, dtype=torch.bfloat16), torch.zeros(2, 64, dtype=torch.int8))


def test_binding_checks_caller_arrays():
    """Per-row arrays and workspaces the kernels would read past are refused
    before any call (CPU tensors stand in for device ones here)."""
    import torch
    cpu = torch.device("cpu")
    assert lmhead._vec(None, "row_scale", 4, torch.float32, cpu) is None
    ok = torch.ones(4)
    assert lmhead._vec(ok, "row_scale", 4, torch.float32, cpu) is ok
    for bad in (torch.ones(3), torch.ones(4, dtype=torch.float64), torch.ones(8)[::2]):
        with pytest.raises(ValueError):
            lmhead._vec(bad, "row_scale", 4, torch.float32, cpu)
    with pytest.raises(ValueError):
        lmhead._ws(torch.zeros(2, 64, dtype=torch.uint8)[:, ::2], cpu)
    assert lmhead._ws(None, cpu) is None


def test_self_check_switch(monkeypatch):
    """LMHEAD_SELF_CHECK=0 (false/no/off) turns the binding's load-time device
    self-check off; anything else, or unset, leaves it on."""
    for v, on in (("0", False), ("false", False), ("Off", False), ("no", False), ("1", True),
                  ("yes", True)):
        monkeypatch.setenv("LMHEAD_SELF_CHECK", v)
        assert lmhead.self_check_enabled() is on
    monkeypatch.delenv("LMHEAD_SELF_CHECK")
    assert lmhead.self_check_enabled()


def test_abi_from_plain_c(tmp_path):
    """tests/abi_c_check.c, built as C99 with gcc against the library: the
    header is valid C and the validation paths answer from C (no GPU)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    root = HEADER.parents[1]
    exe = tmp_path / "abi_c_check"
    lib_dir = _build.LIBRARY.parent
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    f"-I{root / 'include'}", str(root / "tests" / "abi_c_check.c"),
                    f"-L{lib_dir}", "-llmhead", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
