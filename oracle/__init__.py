"""CPU oracle of the batch-invariant LM head (float64 / exact int64).

TEST INFRASTRUCTURE, NOT PRODUCT.  Only ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s cpu_baseline leg may import this package.  The HIP library
(``invariant_lm_head_amd``) never imports it, and the two share no code; only
the seeded input generators in ``synth`` feed both.

The arithmetic lives in ``oracle.c`` (plain loops, one sequential float64 or
int64 accumulator per logit); this module compiles it with gcc (no FMA
contraction, no fast-math, no vectorisation) and wraps it with ctypes.  The
sources of each definition are cited in ``oracle.c``.

``Oracle(path)`` loads any build of the source (the tests load copies with a
planted mistake to show that the pins catch it); the module-level functions
use the default build ``liblmhead_oracle.so``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_DIR = Path(__file__).resolve().parent
SOURCE = _DIR / "oracle.c"
LIBRARY = _DIR / "liblmhead_oracle.so"

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
          "-ffp-contract=off", "-fno-fast-math", "-fno-tree-vectorize"]


def compile_source(src: Path, out: Path) -> Path:
    tmp = out.with_name(out.name + ".tmp%d" % os.getpid())
    subprocess.run(["gcc", *CFLAGS, str(src), "-o", str(tmp), "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> Path:
    """Compile oracle.c into liblmhead_oracle.so (always when force)."""
    global _default
    if force or not LIBRARY.exists() or LIBRARY.stat().st_mtime < SOURCE.stat().st_mtime:
        compile_source(SOURCE, LIBRARY)
        _default = None
    return LIBRARY


def default_threads() -> int:
    """Worker threads when none are given: OMP_NUM_THREADS if set, else the
    online CPUs, at most 16."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    n = int(env) if env.isdigit() and int(env) > 0 else (os.cpu_count() or 1)
    return max(1, min(n, 16))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _nt(n):
    return default_threads() if n is None else n


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _shape(x, w):
    B, H = x.shape
    V, H2 = w.shape
    assert H == H2, "hidden width of x and w differ"
    return B, H, V


class Oracle:
    """ctypes wrapper of one build of oracle.c."""

    def __init__(self, path: Path):
        lib = ctypes.CDLL(str(path))
        i64, i32, P, D = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_double
        sig = {
            "oracle_logits_bf16": ([P, P, i64, i64, i64, P, i32], ctypes.c_int),
            "oracle_logits_i8": ([P, P, i64, i64, i64, P, i32], ctypes.c_int),
            "oracle_greedy_bf16": ([P, P, i64, i64, i64, i32, P, P, P, i32], ctypes.c_int),
            "oracle_greedy_i8": ([P, P, i64, i64, i64, P, P, P, P, P, i32], ctypes.c_int),
            "oracle_logprob_bf16": ([P, P, i64, i64, i64, P, P, i32], ctypes.c_int),
            "oracle_logprob_i8": ([P, P, i64, i64, i64, P, P, P, i32], ctypes.c_int),
            "oracle_top2_f64": ([P, i64, P, P], None),
            "oracle_top2_i64": ([P, i64, P, P], None),
            "oracle_logsoftmax_f64": ([P, i64, P], None),
            "oracle_logprob_i64_row": ([P, i64, D, i64], D),
            "oracle_round_bf16": ([D], D),
            "oracle_philox4x32": ([P, P, P], None),
            "oracle_gumbel": ([ctypes.c_uint64, i64, i64], D),
            "oracle_sample_bf16": ([P, P, i64, i64, i64, D, P, P, P, P, P, i32], ctypes.c_int),
            "oracle_sample_i8": ([P, P, i64, i64, i64, P, D, P, P, P, P, P, i32], ctypes.c_int),
            "oracle_threads": ([i32], ctypes.c_int),
            "oracle_iexp_q30": ([ctypes.c_uint64], ctypes.c_uint64),
            "oracle_iln_q30": ([ctypes.c_uint64], i64),
            "oracle_int_row_scale": ([ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int32, P, P], ctypes.c_int),
            "oracle_quantize_rows": ([P, i64, i64, P, P, P], ctypes.c_int),
            "oracle_logprob_int_row": ([P, i64, i64, ctypes.c_int32, i64], i64),
            "oracle_logprob_int": ([P, P, i64, i64, i64, ctypes.c_int32, ctypes.c_int32, P, P,
                                    P, P, i32], ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            fn = getattr(lib, name)
            fn.argtypes, fn.restype = args, res
        self.lib = lib

    def threads(self, n: int = 0) -> int:
        """Worker threads used for n (0 = all online CPUs)."""
        return self.lib.oracle_threads(n)

    # -------------------------------------------------------- logits
    def logits_bf16(self, x, w, nthreads: int | None = None) -> np.ndarray:
        """z[r, v] = sum_k x[r, k] * w[v, k] in float64, k ascending (bf16 bits in)."""
        x, w = _c(x, np.uint16), _c(w, np.uint16)
        B, H, V = _shape(x, w)
        z = np.empty((B, V), np.float64)
        assert self.lib.oracle_logits_bf16(_ptr(x), _ptr(w), B, H, V, _ptr(z), _nt(nthreads)) == 0
        return z

    def logits_i8(self, x, w, nthreads: int | None = None) -> np.ndarray:
        """z[r, v] = sum_k x[r, k] * w[v, k] exactly in int64."""
        x, w = _c(x, np.int8), _c(w, np.int8)
        B, H, V = _shape(x, w)
        z = np.empty((B, V), np.int64)
        assert self.lib.oracle_logits_i8(_ptr(x), _ptr(w), B, H, V, _ptr(z), _nt(nthreads)) == 0
        return z

    # -------------------------------------------------------- greedy
    def greedy_bf16(self, x, w, round_bf16: bool = False, nthreads: int | None = None):
        """Top-2 ids, values and margin of each row's float64 logits.

        Ties go to the lowest id.  With ``round_bf16`` the logits are first
        rounded to bf16 (nearest-even): the ordinary 16-bit head's output.
        Returns (ids[B,2] int32, vals[B,2] float64, margin[B] float64).
        """
        x, w = _c(x, np.uint16), _c(w, np.uint16)
        B, H, V = _shape(x, w)
        ids = np.empty((B, 2), np.int32)
        vals = np.empty((B, 2), np.float64)
        margin = np.empty(B, np.float64)
        rc = self.lib.oracle_greedy_bf16(_ptr(x), _ptr(w), B, H, V, int(round_bf16),
                                         _ptr(ids), _ptr(vals), _ptr(margin), _nt(nthreads))
        assert rc == 0
        return ids, vals, margin

    def greedy_i8(self, x, w, scale=None, nthreads: int | None = None):
        """Top-2 on exact int64 logits, then the per-row scale.

        Returns (ids[B,2] int32, raw[B,2] int64, vals[B,2] float32, margin[B]
        float32) with vals = float32(raw * scale), margin = float32((raw1 -
        raw2) * scale): one rounding of an exact float64 product each (NaN
        when the scale is not a positive finite number).
        """
        x, w = _c(x, np.int8), _c(w, np.int8)
        B, H, V = _shape(x, w)
        s = None if scale is None else _c(scale, np.float32)
        ids = np.empty((B, 2), np.int32)
        raw = np.empty((B, 2), np.int64)
        vals = np.empty((B, 2), np.float32)
        margin = np.empty(B, np.float32)
        rc = self.lib.oracle_greedy_i8(_ptr(x), _ptr(w), B, H, V,
                                       None if s is None else _ptr(s),
                                       _ptr(ids), _ptr(raw), _ptr(vals), _ptr(margin), _nt(nthreads))
        assert rc == 0
        return ids, raw, vals, margin

    # --------------------------------------------------- gated recompute
    def greedy_gated_bf16(self, x, w, tau: float, nthreads: int | None = None):
        """The margin-gated head ("Greedy Decoding Has a Precision Clause",
        section "Correct the vulnerable token decisions, not every calculation").

        The bf16-output head (float64 logits rounded to bf16, lowest id on a
        tie) decides every row whose top-2 margin is at least tau.  A row whose
        margin is below tau re-ranks its two candidates on their unrounded
        float64 logits, lowest id on a tie.  Returns (ids[B,2] int32,
        vals[B,2] float64, margin[B] float64, gated[B] bool).
        """
        x, w = _c(x, np.uint16), _c(w, np.uint16)
        ids, vals, margin = self.greedy_bf16(x, w, round_bf16=True, nthreads=nthreads)
        gated = margin < tau
        for r in np.nonzero(gated)[0]:
            cand = ids[r].copy()
            z = self.logits_bf16(x[r:r + 1], w[cand], nthreads=1)[0]
            if z[1] > z[0] or (z[1] == z[0] and cand[1] < cand[0]):
                cand, z = cand[::-1], z[::-1]
            ids[r], vals[r], margin[r] = cand, z, z[0] - z[1]
        return ids, vals, margin, gated

    # ------------------------------------------------------- sampling
    def philox4x32(self, ctr, key):
        """Philox4x32-10 of a 4-word counter under a 2-word key (4 uint32 words)."""
        c = np.ascontiguousarray(ctr, dtype=np.uint32)
        k = np.ascontiguousarray(key, dtype=np.uint32)
        out = np.empty(4, np.uint32)
        self.lib.oracle_philox4x32(_ptr(c), _ptr(k), _ptr(out))
        return out

    def gumbel(self, seed: int, position: int, v: int) -> float:
        """Gumbel noise of token v for the draw keyed by (seed, position)."""
        return self.lib.oracle_gumbel(int(seed) & (2 ** 64 - 1), int(position), int(v))

    def sample_bf16(self, x, w, temperature: float, seed, position, nthreads: int | None = None):
        """Seeded Gumbel-max draw of every row ("12 Exactness", section 12.5):
        token = argmax_v z_v / T + G(seed[r], position[r], v), lowest id on a
        tie.  Returns (token[B] int32, value[B] float64 (the winning score),
        gap[B] float64 (its lead over the runner-up))."""
        x, w = _c(x, np.uint16), _c(w, np.uint16)
        B, H, V = _shape(x, w)
        sd, ps = _c(seed, np.uint64), _c(position, np.int64)
        tok, val, gap = np.empty(B, np.int32), np.empty(B, np.float64), np.empty(B, np.float64)
        assert self.lib.oracle_sample_bf16(_ptr(x), _ptr(w), B, H, V, float(temperature),
                                           _ptr(sd), _ptr(ps), _ptr(tok), _ptr(val), _ptr(gap),
                                           _nt(nthreads)) == 0
        return tok, val, gap

    def sample_i8(self, x, w, temperature: float, seed, position, scale=None,
                  nthreads: int | None = None):
        """As sample_bf16 on the scaled int8 logits raw * scale[r]; a row whose
        scale is not a positive finite number draws token -1 (value, gap NaN)."""
        x, w = _c(x, np.int8), _c(w, np.int8)
        B, H, V = _shape(x, w)
        sd, ps = _c(seed, np.uint64), _c(position, np.int64)
        sc = None if scale is None else _c(scale, np.float32)
        tok, val, gap = np.empty(B, np.int32), np.empty(B, np.float64), np.empty(B, np.float64)
        assert self.lib.oracle_sample_i8(_ptr(x), _ptr(w), B, H, V,
                                         None if sc is None else _ptr(sc), float(temperature),
                                         _ptr(sd), _ptr(ps), _ptr(tok), _ptr(val), _ptr(gap),
                                         _nt(nthreads)) == 0
        return tok, val, gap

    # ------------------------------------------------------ log-prob
    def logprob_bf16(self, x, w, target, nthreads: int | None = None) -> np.ndarray:
        """log p(target[r]) under softmax of row r's float64 logits (NaN if out of range)."""
        x, w = _c(x, np.uint16), _c(w, np.uint16)
        B, H, V = _shape(x, w)
        t = _c(target, np.int32)
        out = np.empty(B, np.float64)
        assert self.lib.oracle_logprob_bf16(_ptr(x), _ptr(w), B, H, V, _ptr(t), _ptr(out),
                                            _nt(nthreads)) == 0
        return out

    def logprob_i8(self, x, w, target, scale=None, nthreads: int | None = None) -> np.ndarray:
        """log p(target[r]) under softmax of scale[r] * z (exact int differences)."""
        x, w = _c(x, np.int8), _c(w, np.int8)
        B, H, V = _shape(x, w)
        t = _c(target, np.int32)
        s = None if scale is None else _c(scale, np.float32)
        out = np.empty(B, np.float64)
        assert self.lib.oracle_logprob_i8(_ptr(x), _ptr(w), B, H, V,
                                          None if s is None else _ptr(s), _ptr(t), _ptr(out),
                                          _nt(nthreads)) == 0
        return out

    # ------------------------------------------- per-row definitions
    def top2_f64(self, z):
        """(ids[2], vals[2]) of one float64 logit row; ties to the lowest id."""
        z = _c(z, np.float64)
        ids = np.empty(2, np.int32)
        vals = np.empty(2, np.float64)
        self.lib.oracle_top2_f64(_ptr(z), z.size, _ptr(ids), _ptr(vals))
        return ids, vals

    def top2_i64(self, z):
        z = _c(z, np.int64)
        ids = np.empty(2, np.int32)
        vals = np.empty(2, np.int64)
        self.lib.oracle_top2_i64(_ptr(z), z.size, _ptr(ids), _ptr(vals))
        return ids, vals

    def logsoftmax_f64(self, z) -> np.ndarray:
        """Full log-softmax vector of one float64 logit row."""
        z = _c(z, np.float64)
        out = np.empty_like(z)
        self.lib.oracle_logsoftmax_f64(_ptr(z), z.size, _ptr(out))
        return out

    def logprob_i64_row(self, z, scale: float, t: int) -> float:
        z = _c(z, np.int64)
        return self.lib.oracle_logprob_i64_row(_ptr(z), z.size, float(scale), int(t))

    # ------------------------------------------ integer front and back
    # ("Eliminating Nondeterminism in LLM Inference with Integer-Only
    # Arithmetic", section "DetLLM": dyadic scales with one rounding rule,
    # integer exp and softmax, per-token quantisation; the algorithm itself is
    # stated in oracle.c, "integer front and back")
    NATS_FRAC = 24            # fractional bits of a log-prob (Q.24 nats)
    LOGP_INVALID = -2 ** 63   # target out of range or scale not valid

    def iexp_q30(self, T: int) -> int:
        """e^(-T / 2^24) in Q.30 for T >= 0 in Q.24 nats."""
        return int(self.lib.oracle_iexp_q30(int(T)))

    def iln_q30(self, S: int) -> int:
        """ln(S / 2^30) in Q.30 for S >= 2^30."""
        return int(self.lib.oracle_iln_q30(int(S)))

    def int_row_scale(self, um: int, ue: int, M: int, E: int):
        """(m, k) with m / 2^k = um 2^ue * M 2^E, m of 31 bits, or None when
        the scale is not valid (um, M <= 0 or k outside [24, 86])."""
        m, k = ctypes.c_int64(), ctypes.c_int32()
        ok = self.lib.oracle_int_row_scale(int(um), int(ue), int(M), int(E),
                                           ctypes.byref(m), ctypes.byref(k))
        return (m.value, k.value) if ok else None

    def quantize_rows(self, x):
        """Per-token int8 quantisation of int32 rows: (q[B,H] int8, M[B] int32,
        E[B] int32) with the row's step D = M 2^E."""
        x = _c(x, np.int32)
        B, H = x.shape
        q = np.empty((B, H), np.int8)
        M, E = np.empty(B, np.int32), np.empty(B, np.int32)
        assert self.lib.oracle_quantize_rows(_ptr(x), B, H, _ptr(q), _ptr(M), _ptr(E)) == 0
        return q, M, E

    def logprob_int_row(self, z, m: int, k: int, t: int) -> int:
        """Integer log-softmax of one row of exact integer logits with the
        logit scale m / 2^k: log p(t) in Q.24 (LOGP_INVALID if invalid)."""
        z = _c(z, np.int64)
        return int(self.lib.oracle_logprob_int_row(_ptr(z), z.size, int(m), int(k), int(t)))

    def logprob_int(self, x, w, um: int, ue: int, M, E, target,
                    nthreads: int | None = None) -> np.ndarray:
        """log p(target[r]) in Q.24 (int64) of the int8 head with the integer
        log-softmax; row r's logit scale is um 2^ue * M[r] 2^E[r]."""
        x, w = _c(x, np.int8), _c(w, np.int8)
        B, H, V = _shape(x, w)
        M, E, t = _c(M, np.int32), _c(E, np.int32), _c(target, np.int32)
        out = np.empty(B, np.int64)
        assert self.lib.oracle_logprob_int(_ptr(x), _ptr(w), B, H, V, int(um), int(ue),
                                           _ptr(M), _ptr(E), _ptr(t), _ptr(out),
                                           _nt(nthreads)) == 0
        return out

    def round_bf16(self, v: float) -> float:
        """Nearest bf16 value (ties to even) of a float64, as float64."""
        return self.lib.oracle_round_bf16(float(v))


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        build(force=False)
        _default = Oracle(LIBRARY)
    return _default


def __getattr__(name):
    # module-level access to the default build: oracle.logits_bf16(...), ...
    if not name.startswith("_") and hasattr(Oracle, name):
        return getattr(default(), name)
    raise AttributeError(name)
