"""Python binding of liblmhead.so (the C-ABI in include/lmhead.h).

Argument marshalling only: every step of the head runs in the HIP kernels.
PyTorch provides device memory and the current stream.  There is no CPU or
PyTorch fallback: if the library cannot be loaded, every call raises.

Before the first call on a device the binding runs the library's device
self-check (lmhead_self_check) in both arithmetic modes, and from the packed
bf16 layout, on a fixed synthetic batch: every row's logits alone, in the batch and in the reversed batch must
have the same bits, or every call on that device raises SelfCheckError
("12 Exactness", section 12.8: a load-time self-check of the row property on
the device).  Set LMHEAD_SELF_CHECK=0 to skip it.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

from . import _build

MODE_BF16, MODE_INT8, MODE_BF16_PACKED = 0, 1, 2
ROUND_F32, ROUND_BF16 = 0, 1

_STATUS = {0: "LMHEAD_OK", 1: "LMHEAD_E_NULL", 2: "LMHEAD_E_SHAPE", 3: "LMHEAD_E_ALIGN",
           4: "LMHEAD_E_MODE", 5: "LMHEAD_E_OVERFLOW", 6: "LMHEAD_E_WORKSPACE",
           7: "LMHEAD_E_HIP", 8: "LMHEAD_E_VALUE"}

# every function the header declares, with its C signature
_P, _I, _I64, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "lmhead_workspace_bytes": ([_I, _I64, _I64, _I64], _SZ),
    "lmhead_logits": ([_I, _I, _P, _P, _I64, _I64, _I64, _P, _P], _I),
    "lmhead_greedy_top2": ([_I, _I, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P], _I),
    "lmhead_greedy_top2_noalloc": ([_I, _I, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P],
                                   _I),
    "lmhead_logprob": ([_I, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _SZ, _P], _I),
    "lmhead_greedy_gated": ([_I, _P, _P, _I64, _I64, _I64, ctypes.c_float, _P, _P, _P, _P, _P,
                             _SZ, _P], _I),
    "lmhead_sample_gumbel": ([_I, _P, _P, _I64, _I64, _I64, ctypes.c_float, _P, _P, _P, _P, _P,
                              _P, _P, _SZ, _P], _I),
    "lmhead_quantize_rows": ([_P, _I64, _I64, _P, _P, _P, _P], _I),
    "lmhead_logprob_int": ([_P, _P, _I64, _I64, _I64, ctypes.c_int32, ctypes.c_int32, _P, _P, _P,
                            _P, _P, _SZ, _P], _I),
    "lmhead_self_check_bytes": ([_I, _I64, _I64, _I64], _SZ),
    "lmhead_self_check": ([_I, _P, _P, _I64, _I64, _I64, _P, _SZ, _P, _P], _I),
    "lmhead_packed_w_bytes": ([_I64, _I64], _SZ),
    "lmhead_pack_w": ([_P, _I64, _I64, _P, _P], _I),
    "lmhead_status_string": ([_I], ctypes.c_char_p),
    "lmhead_last_error": ([], ctypes.c_char_p),
    "lmhead_source_digest": ([], ctypes.c_char_p),
}


class LMHeadError(RuntimeError):
    def __init__(self, fn: str, status: int, lib):
        msg = lib.lmhead_status_string(status).decode()
        if status == 7:
            msg += " (" + lib.lmhead_last_error().decode() + ")"
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None
_lock = threading.Lock()


class StaleLibraryError(RuntimeError):
    pass


def library():
    """Load liblmhead.so, building it first only if it does not exist.

    A library built from other sources than the ones beside it (its
    lmhead_source_digest() differs from the sources' digest) is refused: run
    the build again (``python -m invariant_lm_head_amd._build``)."""
    global _lib
    with _lock:
        if _lib is None:
            if not _build.LIBRARY.exists():
                _build.build()
            lib = ctypes.CDLL(str(_build.LIBRARY))
            for name, (args, res) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.argtypes, fn.restype = args, res
            built, now = lib.lmhead_source_digest().decode(), _build.source_digest()
            if built != now:
                raise StaleLibraryError(
                    f"{_build.LIBRARY} was built from sources with digest {built}, but the "
                    f"sources now hash to {now}: rebuild it (python -m invariant_lm_head_amd._build)")
            _lib = lib
    return _lib


class SelfCheckError(RuntimeError):
    pass


_self_checked: dict = {}
SELF_CHECK_SHAPES = ((MODE_BF16, 300, 128, 2000), (MODE_INT8, 300, 128, 2000),
                     (MODE_BF16_PACKED, 300, 128, 2000))


def self_check_enabled() -> bool:
    """LMHEAD_SELF_CHECK=0 (or false/no/off) skips the load-time self-check."""
    return os.environ.get("LMHEAD_SELF_CHECK", "1").strip().lower() not in ("0", "false", "no", "off")


def ensure_self_check(device) -> dict:
    """Run the device self-check once per device (both arithmetic modes and
    the packed bf16 layout, 300 rows: the batch spans two 256-row tiles, each
    row alone runs the 32-row tile) and raise SelfCheckError if any logit's
    bits differ.  Returns {mode:
    mismatches} (empty when the check is switched off)."""
    dev = torch.device(device)
    key = dev.index if dev.index is not None else torch.cuda.current_device()
    if key in _self_checked:
        res = _self_checked[key]
    elif not self_check_enabled():
        res = _self_checked[key] = {}
    else:
        res = {}
        g = torch.Generator().manual_seed(12)
        for mode, B, H, V in SELF_CHECK_SHAPES:
            if mode == MODE_INT8:
                x = torch.randint(-127, 128, (B, H), generator=g, dtype=torch.int8)
                w = torch.randint(-127, 128, (V, H), generator=g, dtype=torch.int8)
            else:
                x = torch.randn((B, H), generator=g).to(torch.bfloat16)
                w = (0.05 * torch.randn((V, H), generator=g)).to(torch.bfloat16)
            with torch.cuda.device(dev):
                wd = w.to(dev)
                res[mode] = self_check(x.to(dev), pack_w(wd) if mode == MODE_BF16_PACKED else wd)
        _self_checked[key] = res
    if any(res.values()):
        raise SelfCheckError(f"device self-check on {dev}: logits whose bits depend on the "
                             f"batch (mismatches per mode {res}); refusing to run")
    return res


def _check(fn: str, status: int):
    if status != 0:
        raise LMHeadError(fn, status, library())


class PackedW:
    """A bf16 vocabulary matrix [V, H] in the library's packed layout (written
    by pack_w, read by every call in MODE_BF16_PACKED).  `data` holds the
    packed bytes; shape, dtype and device describe the matrix it came from."""

    def __init__(self, data: torch.Tensor, V: int, H: int):
        self.data, self.shape = data, torch.Size((V, H))
        self.dtype, self.device, self.is_cuda = torch.bfloat16, data.device, data.is_cuda

    def dim(self) -> int:
        return 2

    def is_contiguous(self) -> bool:
        return True

    def data_ptr(self) -> int:
        return self.data.data_ptr()


def pack_w(w: torch.Tensor) -> PackedW:
    """Pack a contiguous bf16 device matrix [V, H] once for MODE_BF16_PACKED
    calls (lmhead_pack_w): every output keeps the bits of the row-major call."""
    if w.dtype != torch.bfloat16 or w.dim() != 2 or not w.is_cuda or not w.is_contiguous():
        raise ValueError("w must be a contiguous 2-D bfloat16 device tensor")
    V, H = w.shape
    nbytes = int(library().lmhead_packed_w_bytes(H, V))
    if nbytes == 0:
        raise ValueError(f"no packed layout for w of shape {tuple(w.shape)}")
    data = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    st = library().lmhead_pack_w(_ptr(w), H, V, _ptr(data), _stream(w.device))
    _check("lmhead_pack_w", st)
    return PackedW(data, V, H)


def _mode_of(x: torch.Tensor, w) -> int:
    if x.dtype == torch.bfloat16 and isinstance(w, PackedW):
        return MODE_BF16_PACKED
    if x.dtype == torch.bfloat16 and w.dtype == torch.bfloat16:
        return MODE_BF16
    if x.dtype == torch.int8 and w.dtype == torch.int8 and not isinstance(w, PackedW):
        return MODE_INT8
    raise TypeError(f"x and w must both be bfloat16 or both int8, got {x.dtype}, {w.dtype}")


def _dims(x: torch.Tensor, w, checked: bool = True):
    if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
        raise ValueError(f"x must be [B, H] and w [V, H], got {tuple(x.shape)}, {tuple(w.shape)}")
    if not (x.is_cuda and w.is_cuda and x.is_contiguous() and w.is_contiguous()):
        raise ValueError("x and w must be contiguous device tensors")
    if x.device != w.device:
        raise ValueError(f"x and w must be on one device, got {x.device}, {w.device}")
    if checked:
        ensure_self_check(x.device)
    return x.shape[0], x.shape[1], w.shape[0]


def _vec(t, name: str, B: int, dtype, dev):
    """A caller's per-row array: None, or a contiguous [B] tensor of dtype on dev
    (the kernels read B elements of it)."""
    if t is None:
        return None
    if t.dtype != dtype or t.shape != (B,) or t.device != dev or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape ({B},) on {dev}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")
    return t


def _ws(ws, dev):
    if ws is not None and (ws.device != dev or not ws.is_contiguous()):
        raise ValueError(f"ws must be a contiguous tensor on {dev}")
    return ws


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


# ---------------------------------------------------------------- workspace
_ws_cache: dict = {}


def workspace_bytes(mode: int, B: int, H: int, V: int) -> int:
    return int(library().lmhead_workspace_bytes(mode, B, H, V))


def workspace(nbytes: int, device) -> torch.Tensor:
    """A workspace of at least nbytes for the current stream, reused by all
    calls ordered on that stream (calls on one stream never overlap)."""
    dev = torch.device(device)
    key = (dev.index, torch.cuda.current_stream(dev).cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 1 << 16), dtype=torch.uint8, device=dev)
        _ws_cache[key] = ws
    return ws


# ---------------------------------------------------------------- calls
def logits(x: torch.Tensor, w: torch.Tensor, round_bf16: bool = False,
           out: torch.Tensor | None = None) -> torch.Tensor:
    """Z = x @ w.T as float32 (bf16 mode), bf16 (round_bf16) or int32 (int8 mode)."""
    mode = _mode_of(x, w)
    B, H, V = _dims(x, w)
    dt = torch.int32 if mode == MODE_INT8 else (torch.bfloat16 if round_bf16 else torch.float32)
    if out is None:
        out = torch.empty((B, V), dtype=dt, device=x.device)
    elif out.dtype != dt or out.shape != (B, V) or out.device != x.device or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous {dt} tensor of shape ({B}, {V}) on {x.device}")
    st = library().lmhead_logits(mode, ROUND_BF16 if round_bf16 else ROUND_F32, _ptr(x), _ptr(w),
                                 B, H, V, _ptr(out), _stream(x.device))
    _check("lmhead_logits", st)
    return out


def greedy_top2(x: torch.Tensor, w: torch.Tensor, row_scale: torch.Tensor | None = None,
                round_bf16: bool = False, ws: torch.Tensor | None = None):
    """Per-row top-2 ids [B,2] int32, values [B,2] float32, margin [B] float32 and,
    in int8 mode, the exact int32 logits of the two [B,2] (None in bf16 mode)."""
    mode = _mode_of(x, w)
    B, H, V = _dims(x, w)
    dev = x.device
    ids = torch.empty((B, 2), dtype=torch.int32, device=dev)
    vals = torch.empty((B, 2), dtype=torch.float32, device=dev)
    margin = torch.empty((B,), dtype=torch.float32, device=dev)
    raw = torch.empty((B, 2), dtype=torch.int32, device=dev) if mode == MODE_INT8 else None
    rs = _vec(row_scale, "row_scale", B, torch.float32, dev)
    need = workspace_bytes(mode, B, H, V)
    if _ws(ws, dev) is None:
        ws = workspace(need, dev)
    st = library().lmhead_greedy_top2(mode, ROUND_BF16 if round_bf16 else ROUND_F32,
                                      _ptr(x), _ptr(w), B, H, V, _ptr(rs), _ptr(ids),
                                      _ptr(vals), _ptr(margin), _ptr(raw), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(dev))
    _check("lmhead_greedy_top2", st)
    return ids, vals, margin, raw


STATIC_WORKSPACE_BYTES = 16 << 20   # LMHEAD_STATIC_WORKSPACE_BYTES


def greedy_top2_noalloc(x: torch.Tensor, w: torch.Tensor, row_scale: torch.Tensor | None = None,
                        round_bf16: bool = False, out=None):
    """greedy_top2 through the entry point that allocates nothing: the library
    takes its workspace from a static device array (shapes whose workspace
    exceeds STATIC_WORKSPACE_BYTES are refused).  out: optional preallocated
    (ids, vals, margin, raw) to write into (raw None in bf16 mode)."""
    mode = _mode_of(x, w)
    B, H, V = _dims(x, w)
    dev = x.device
    if out is None:
        out = (torch.empty((B, 2), dtype=torch.int32, device=dev),
               torch.empty((B, 2), dtype=torch.float32, device=dev),
               torch.empty((B,), dtype=torch.float32, device=dev),
               torch.empty((B, 2), dtype=torch.int32, device=dev) if mode == MODE_INT8 else None)
    ids, vals, margin, raw = out
    rs = _vec(row_scale, "row_scale", B, torch.float32, dev)
    st = library().lmhead_greedy_top2_noalloc(mode, ROUND_BF16 if round_bf16 else ROUND_F32,
                                              _ptr(x), _ptr(w), B, H, V, _ptr(rs), _ptr(ids),
                                              _ptr(vals), _ptr(margin), _ptr(raw), _stream(dev))
    _check("lmhead_greedy_top2_noalloc", st)
    return ids, vals, margin, raw


def logprob(x: torch.Tensor, w: torch.Tensor, target: torch.Tensor,
            row_scale: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """log p(target[b]) [B] float32 under the softmax of row b's logits."""
    mode = _mode_of(x, w)
    B, H, V = _dims(x, w)
    dev = x.device
    if target.dtype != torch.int32 or target.numel() != B or target.device != dev:
        raise ValueError(f"target must be an int32 tensor of B ids on {dev}")
    rs = _vec(row_scale, "row_scale", B, torch.float32, dev)
    out = torch.empty((B,), dtype=torch.float32, device=dev)
    need = workspace_bytes(mode, B, H, V)
    if _ws(ws, dev) is None:
        ws = workspace(need, dev)
    st = library().lmhead_logprob(mode, _ptr(x), _ptr(w), B, H, V, _ptr(rs),
                                  _ptr(target.contiguous()), _ptr(out), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(dev))
    _check("lmhead_logprob", st)
    return out


LOGP_FRAC = 24             # lmhead_logprob_int: log-probs in units of 2^-24 nats
LOGP_INVALID = -2 ** 63    # its value for a target out of range or an invalid scale


def quantize_rows(x: torch.Tensor):
    """Per-token int8 quantisation of int32 rows [B, H]: q [B, H] int8 and the
    row steps D = step_m 2^step_e ([B] int32 each)."""
    if x.dtype != torch.int32 or x.dim() != 2 or not x.is_cuda:
        raise ValueError("x must be a 2-D int32 device tensor")
    x = x.contiguous()
    B, H = x.shape
    dev = x.device
    ensure_self_check(dev)
    q = torch.empty((B, H), dtype=torch.int8, device=dev)
    step_m = torch.empty((B,), dtype=torch.int32, device=dev)
    step_e = torch.empty((B,), dtype=torch.int32, device=dev)
    st = library().lmhead_quantize_rows(_ptr(x), B, H, _ptr(q), _ptr(step_m), _ptr(step_e),
                                        _stream(dev))
    _check("lmhead_quantize_rows", st)
    return q, step_m, step_e


def logprob_int(x: torch.Tensor, w: torch.Tensor, unit: tuple, step_m: torch.Tensor,
                step_e: torch.Tensor, target: torch.Tensor, ws: torch.Tensor | None = None):
    """All-integer log p(target[b]) [B] int64 in units of 2^-24 nats of the
    int8 head; row b's logit scale is unit[0] 2^unit[1] * step_m[b] 2^step_e[b]."""
    if _mode_of(x, w) != MODE_INT8:
        raise ValueError("logprob_int takes int8 x and w")
    B, H, V = _dims(x, w)
    dev = x.device
    for name, t in (("step_m", step_m), ("step_e", step_e), ("target", target)):
        if t.dtype != torch.int32 or t.numel() != B or t.device != dev:
            raise ValueError(f"{name} must be an int32 tensor of B values on {dev}")
    out = torch.empty((B,), dtype=torch.int64, device=dev)
    need = workspace_bytes(MODE_INT8, B, H, V)
    if _ws(ws, dev) is None:
        ws = workspace(need, dev)
    st = library().lmhead_logprob_int(_ptr(x), _ptr(w), B, H, V, int(unit[0]), int(unit[1]),
                                      _ptr(step_m.contiguous()), _ptr(step_e.contiguous()),
                                      _ptr(target.contiguous()), _ptr(out), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(dev))
    _check("lmhead_logprob_int", st)
    return out


def greedy_gated(x: torch.Tensor, w: torch.Tensor, tau: float,
                 ws: torch.Tensor | None = None):
    """bf16-output greedy top-2 whose rows with margin < tau are re-ranked on
    their two candidates' float32 logits: ids [B,2] int32, values [B,2] float32,
    margin [B] float32, gated [B] int32 (1 = recomputed)."""
    mode = _mode_of(x, w)
    B, H, V = _dims(x, w)
    dev = x.device
    ids = torch.empty((B, 2), dtype=torch.int32, device=dev)
    vals = torch.empty((B, 2), dtype=torch.float32, device=dev)
    margin = torch.empty((B,), dtype=torch.float32, device=dev)
    gated = torch.empty((B,), dtype=torch.int32, device=dev)
    need = workspace_bytes(mode, B, H, V)
    if _ws(ws, dev) is None:
        ws = workspace(need, dev)
    st = library().lmhead_greedy_gated(mode, _ptr(x), _ptr(w), B, H, V, float(tau), _ptr(ids),
                                       _ptr(vals), _ptr(margin), _ptr(gated), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream(dev))
    _check("lmhead_greedy_gated", st)
    return ids, vals, margin, gated


def sample_gumbel(x: torch.Tensor, w: torch.Tensor, temperature: float, seed: torch.Tensor,
                  position: torch.Tensor, row_scale: torch.Tensor | None = None,
                  ws: torch.Tensor | None = None):
    """Seeded Gumbel-max draw of every row: token [B] int32, winning score [B]
    float32 and its gap to the runner-up [B] float32.  seed: [B] uint64 bits
    (any 64-bit integer tensor), position: [B] int64."""
    mode = _mode_of(x, w)
    B, H, V = _dims(x, w)
    dev = x.device
    for name, t in (("seed", seed), ("position", position)):
        if t.numel() != B or t.device != dev or t.element_size() != 8:
            raise ValueError(f"{name} must be a tensor of B 64-bit integers on {dev}")
    rs = _vec(row_scale, "row_scale", B, torch.float32, dev)
    token = torch.empty((B,), dtype=torch.int32, device=dev)
    value = torch.empty((B,), dtype=torch.float32, device=dev)
    gap = torch.empty((B,), dtype=torch.float32, device=dev)
    need = workspace_bytes(mode, B, H, V)
    if _ws(ws, dev) is None:
        ws = workspace(need, dev)
    st = library().lmhead_sample_gumbel(mode, _ptr(x), _ptr(w), B, H, V, float(temperature),
                                        _ptr(rs), _ptr(seed.contiguous()),
                                        _ptr(position.contiguous()), _ptr(token), _ptr(value),
                                        _ptr(gap), _ptr(ws), ws.numel() * ws.element_size(),
                                        _stream(dev))
    _check("lmhead_sample_gumbel", st)
    return token, value, gap


def self_check(x: torch.Tensor, w: torch.Tensor) -> int:
    """Number of logits whose bits differ between batch, single-row and reversed
    runs of x (0 proves the row property on this device for these rows)."""
    mode = _mode_of(x, w)
    B, H, V = _dims(x, w, checked=False)
    dev = x.device
    nbytes = int(library().lmhead_self_check_bytes(mode, B, H, V))
    scratch = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    count = torch.zeros(1, dtype=torch.int64, device=dev)
    st = library().lmhead_self_check(mode, _ptr(x), _ptr(w), B, H, V, _ptr(scratch), nbytes,
                                     _ptr(count), _stream(dev))
    _check("lmhead_self_check", st)
    return int(count.item())
