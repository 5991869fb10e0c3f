"""Benchmark of the batch-invariant LM head on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extras]

Workload (the metric's): the TinyLlama-shaped head, H = 2048, V = 32000, bf16
hidden rows (RMS-normalised Gaussian) and W ~ N(0, 0.02) in bf16, synthetic and
seeded.  One step = one greedy top-2 call (float32 head, logits never
stored) at each batch size 1, 8, 64, 256 and 512: 841 rows.  value = rows /
second over the K timed steps.  Inputs are resident in HBM before timing; four
copies of W (524 MB, more than the 256 MB Infinity Cache) rotate from call to
call, so W is read from HBM, not from the cache.  W is packed once, before
timing, into the library's packed layout (lmhead_pack_w: the same bytes in
another order, every output bit the same as with the row-major W); the
row-major W's times are reported beside it (per_batch_row_major).

Printed as ONE JSON line on stdout, with:
  roofline      the dominant call (the largest batch: its tile kernel plus the
                row-fold kernel) against MI355X's peak, from HIP events on the
                stream the kernels run on; traffic = HBM bytes per call from the
                committed rocprofv3 counter summary (null once the kernel
                sources differ from the ones it was taken on);
  per_batch     every batch size: us per call, rows/s, GB/s, TFLOP/s, roofline;
  per_batch_row_major  the same calls reading the row-major W;
  cpu_baseline  the float64 CPU oracle timed on this host on a bounded sample;
  other         the other workloads (log-prob scoring at H = 4096, V = 151936;
                int8 head at H = 4096, V = 128256; near-tie stress; full logits);
                the float head's read packed W like the sweep, the int8 head's
                row-major W.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
DOCS = [ROOT / "README.md", ROOT / "DESIGN.md"]  # documents with generated tables
sys.path.insert(0, str(ROOT))

HBM_PEAK = 8.0e12           # bytes/s, MI355X HBM3E
MFMA_PEAK = {"bf16": 2.5e15, "int8": 5.0e15}   # dense, per second
METRIC = "LM-head rows/s + % of HBM/MFMA roofline, V=32000 H=2048, batch 1..512"
SWEEP = (1, 8, 64, 256, 512)
NCOPIES = 4
PACKED = 2                  # LMHEAD_MODE_BF16_PACKED


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def roofline(B, H, V, t, esize=2, out_bytes_per_row=20, mode="bf16", extra_bytes=0):
    """Algorithmic bytes (W once + X + outputs) and flops (2 B V H) against t seconds."""
    nbytes = V * H * esize + B * H * esize + B * out_bytes_per_row + extra_bytes
    flops = 2.0 * B * V * H
    t_hbm, t_mfma = nbytes / HBM_PEAK, flops / MFMA_PEAK[mode]
    if t_hbm >= t_mfma:
        return {"bound": "hbm", "achieved": nbytes / t / 1e9, "peak": HBM_PEAK / 1e9,
                "unit": "GB/s", "frac": t_hbm / t, "bytes": nbytes, "flops": flops}
    return {"bound": "mfma", "achieved": flops / t / 1e12, "peak": MFMA_PEAK[mode] / 1e12,
            "unit": "TFLOP/s" if mode == "bf16" else "TOP/s", "frac": t_mfma / t,
            "bytes": nbytes, "flops": flops}


class Caller:
    """Direct ctypes calls with pre-built arguments (keeps Python overhead per
    launch well under the kernel time; torch allocates nothing in the loop)."""

    def __init__(self, torch, lmhead, x_list, w_list, B, H, V, mode=0, kind="greedy",
                 target=None, scale=None, round_bf16=0, tau=0.0, steps=None, unit=None):
        self.torch = torch
        lib = lmhead.library()
        dev = x_list[0].device
        self.stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        ws_bytes = lmhead.workspace_bytes(mode, B, H, V)
        self.ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
        self.calls = []
        if kind == "greedy":
            ids = torch.empty((B, 2), dtype=torch.int32, device=dev)
            vals = torch.empty((B, 2), dtype=torch.float32, device=dev)
            margin = torch.empty((B,), dtype=torch.float32, device=dev)
            raw = torch.empty((B, 2), dtype=torch.int32, device=dev) if mode == 1 else None
            self.keep = (ids, vals, margin, raw)
            for xx, ww in zip(x_list, w_list):
                self.calls.append((lib.lmhead_greedy_top2, (
                    mode, round_bf16, P(xx), P(ww), B, H, V, P(scale), P(ids), P(vals), P(margin),
                    P(raw), P(self.ws), ws_bytes, self.stream)))
        elif kind == "sample":
            token = torch.empty((B,), dtype=torch.int32, device=dev)
            value = torch.empty((B,), dtype=torch.float32, device=dev)
            gap = torch.empty((B,), dtype=torch.float32, device=dev)
            g = torch.Generator().manual_seed(B)
            seed = torch.randint(0, 2 ** 62, (B,), generator=g, dtype=torch.int64).to(dev)
            pos = torch.arange(B, dtype=torch.int64).to(dev)
            self.keep = (token, value, gap, seed, pos)
            for xx, ww in zip(x_list, w_list):
                self.calls.append((lib.lmhead_sample_gumbel, (
                    mode, P(xx), P(ww), B, H, V, ctypes.c_float(tau or 1.0), P(scale), P(seed),
                    P(pos), P(token), P(value), P(gap), P(self.ws), ws_bytes, self.stream)))
        elif kind == "gated":
            ids = torch.empty((B, 2), dtype=torch.int32, device=dev)
            vals = torch.empty((B, 2), dtype=torch.float32, device=dev)
            margin = torch.empty((B,), dtype=torch.float32, device=dev)
            gated = torch.empty((B,), dtype=torch.int32, device=dev)
            self.keep = (ids, vals, margin, gated)
            for xx, ww in zip(x_list, w_list):
                self.calls.append((lib.lmhead_greedy_gated, (
                    mode, P(xx), P(ww), B, H, V, ctypes.c_float(tau), P(ids), P(vals), P(margin),
                    P(gated), P(self.ws), ws_bytes, self.stream)))
        elif kind == "logprob":
            out = torch.empty((B,), dtype=torch.float32, device=dev)
            self.keep = (out,)
            for xx, ww in zip(x_list, w_list):
                self.calls.append((lib.lmhead_logprob, (
                    mode, P(xx), P(ww), B, H, V, P(scale), P(target), P(out), P(self.ws),
                    ws_bytes, self.stream)))
        elif kind == "logprob_int":
            out = torch.empty((B,), dtype=torch.int64, device=dev)
            sm, se = steps
            self.keep = (out, sm, se)
            for xx, ww in zip(x_list, w_list):
                self.calls.append((lib.lmhead_logprob_int, (
                    P(xx), P(ww), B, H, V, int(unit[0]), int(unit[1]), P(sm), P(se), P(target),
                    P(out), P(self.ws), ws_bytes, self.stream)))
        elif kind == "quantize":
            q = torch.empty((B, H), dtype=torch.int8, device=dev)
            sm = torch.empty((B,), dtype=torch.int32, device=dev)
            se = torch.empty((B,), dtype=torch.int32, device=dev)
            self.keep = (q, sm, se)
            for xx in x_list:
                self.calls.append((lib.lmhead_quantize_rows, (P(xx), B, H, P(q), P(sm), P(se),
                                                              self.stream)))
        elif kind == "logits":
            out = torch.empty((B, V), dtype=torch.float32 if mode == 0 else torch.int32, device=dev)
            self.keep = (out,)
            for xx, ww in zip(x_list, w_list):
                self.calls.append((lib.lmhead_logits, (mode, 0, P(xx), P(ww), B, H, V, P(out),
                                                       self.stream)))
        self.i = 0

    def __call__(self, i=None):
        """Launch once; i picks the W copy (default: this caller's own rotation)."""
        if i is None:
            i = self.i
            self.i = (self.i + 1) % len(self.calls)
        fn, args = self.calls[i % len(self.calls)]
        st = fn(*args)
        if st != 0:
            raise RuntimeError(f"lmhead call failed with status {st}")


def time_calls(torch, caller, n, warmup=3):
    """Average seconds per launch from HIP events on the current stream."""
    for _ in range(warmup):
        caller()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(n):
        caller()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / 1e3 / n


def source_digest() -> str:
    """Digest of the library's sources (the one the library records at build)."""
    from invariant_lm_head_amd import _build
    return _build.source_digest()


def traffic_from_profile(kernel_tag: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources (else None)."""
    path = ROOT / "profiles" / f"counters_{kernel_tag}.md"
    if not path.exists():
        return None
    src, val = None, None
    for line in path.read_text().splitlines():
        if line.startswith("source_digest:"):
            src = line.split(":", 1)[1].strip()
        if line.startswith("hbm_bytes_per_launch:"):
            val = float(line.split(":", 1)[1].strip())
    return val if src == source_digest() else None


def host_facts() -> dict:
    """The host the CPU leg runs on: online CPUs and the CPU model."""
    model = None
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"online_cpus": os.cpu_count(), "cpu_model": model,
            "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def cpu_baseline():
    """The float64 / int64 oracle on the host's cores (threads: OMP_NUM_THREADS
    if set, else the online CPUs, at most 16).  The metric's workload: greedy
    top-2 of the H=2048, V=32000 head, chunks of 256 rows until about 8 s have
    passed (at most 2048 rows), then 64 rows on one thread.  The other
    workloads on bounded samples (a few seconds each): the tiny head in full,
    64 near-tie rows, 8 rows of the 16384 x 151936 scoring batch, 16 rows of the
    int8 head (greedy, and the integer log-softmax of 16 quantised rows)."""
    import oracle
    import synth
    o = oracle.default()
    d = synth.make_inputs("tinyllama", rows=2048)
    n = oracle.default_threads()
    rows = 0
    t0 = time.perf_counter()
    while rows < 2048 and time.perf_counter() - t0 < 8.0:
        o.greedy_bf16(d["x"][rows:rows + 256], d["w"], nthreads=n)
        rows += 256
    dt = time.perf_counter() - t0
    t1 = time.perf_counter()
    o.greedy_bf16(d["x"][:64], d["w"], nthreads=1)
    dt1 = time.perf_counter() - t1
    del d

    def timed(f):
        t = time.perf_counter()
        f()
        return time.perf_counter() - t

    other = {}
    dt_ = synth.make_inputs("tiny")
    t = timed(lambda: o.greedy_bf16(dt_["x"], dt_["w"], nthreads=n))
    other["tiny_greedy_4x64x1000"] = {"rows": 4, "s": t, "rows_per_s": 4 / t}
    nt = synth.make_inputs("neartie", rows=64)
    t = timed(lambda: o.greedy_bf16(nt["x"], nt["w"], nthreads=n))
    other["neartie_greedy_2048x32000"] = {"rows": 64, "s": t, "rows_per_s": 64 / t}
    del nt
    lp = synth.make_inputs("logprob", rows=8)
    t = timed(lambda: o.logprob_bf16(lp["x"], lp["w"], lp["target"], nthreads=n))
    other["logprob_4096x151936"] = {"rows": 8, "s": t, "rows_per_s": 8 / t}
    del lp
    i8 = synth.make_inputs("int8", rows=16)
    t = timed(lambda: o.greedy_i8(i8["x"], i8["w"], i8["scale"], nthreads=n))
    other["int8_greedy_4096x128256"] = {"rows": 16, "s": t, "rows_per_s": 16 / t}
    q, M, E = o.quantize_rows(i8["hidden"])
    t = timed(lambda: o.logprob_int(q, i8["w"], *i8["unit"], M, E, i8["target"], nthreads=n))
    other["int8_integer_logprob_4096x128256"] = {"rows": 16, "s": t, "rows_per_s": 16 / t}
    del i8
    return {"value": rows / dt, "unit": "rows/s", "cores": n, "kind": "oracle",
            "sample": f"float64 greedy top-2 of rows 0..{rows - 1} of the H=2048, V=32000 head "
                      f"({dt:.1f} s wall on {n} threads)",
            "threads": n, "host": host_facts(),
            "single_thread_rows_per_s": 64 / dt1,
            "single_thread_sample": f"rows 0..63 on one thread ({dt1:.1f} s)",
            "other": other}


def output_digests(torch, lmhead, synth, bf16, dev) -> dict:
    """SHA-256 (16 hex digits) of the outputs of fixed scenarios, one per mode
    and call: a result, so that two runs or two builds can be compared bit for
    bit (the integer head's bits are also those of the stored oracle outputs
    the tests compare with)."""
    def h(*ts):
        m = hashlib.sha256()
        for t in ts:
            m.update(t.detach().contiguous().cpu().numpy().tobytes())
        return m.hexdigest()[:16]

    d = synth.make_inputs("tinyllama")
    x, w = bf16(d["x"]), bf16(d["w"])
    t = torch.from_numpy(d["target"]).to(dev)
    seed = torch.arange(512, dtype=torch.int64, device=dev) * 7919 + 1
    pos = torch.arange(512, dtype=torch.int64, device=dev)
    out = {"float_logits_512x2048x32000": h(lmhead.logits(x, w)),
           "float_greedy_512": h(*lmhead.greedy_top2(x, w)[:3]),
           "float_logprob_512": h(lmhead.logprob(x, w, t)),
           "bf16_output_gated_tau1e-3_512": h(*lmhead.greedy_gated(x, w, 1e-3)),
           "float_sample_T0.7_512": h(*lmhead.sample_gumbel(x, w, 0.7, seed, pos))}
    del x, w
    i8 = synth.make_inputs("int8")
    xi, wi = torch.from_numpy(i8["x"]).to(dev), torch.from_numpy(i8["w"]).to(dev)
    si, ti = torch.from_numpy(i8["scale"]).to(dev), torch.from_numpy(i8["target"]).to(dev)
    out["int8_logits_8x4096x128256"] = h(lmhead.logits(xi[:8].contiguous(), wi))
    out["int8_greedy_512"] = h(*lmhead.greedy_top2(xi, wi, row_scale=si))
    q, sm, se = lmhead.quantize_rows(torch.from_numpy(i8["hidden"]).to(dev))
    out["int8_integer_logprob_512"] = h(lmhead.logprob_int(q, wi, i8["unit"], sm, se, ti))
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extras", action="store_true", help="skip the other workloads")
    ap.add_argument("--counters", action="store_true",
                    help="only launch what the counter runs read: a 512 MiB device copy "
                         "(calibration), greedy top-2 at batch 1, 256 and 512 and the int8 "
                         "head at batch 512")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DB",
                    help="print the markdown summary of rocprofv3 --pmc databases of "
                         "--counters runs (no GPU needed)")
    ap.add_argument("--summarize-trace", metavar="DB",
                    help="print the per-kernel durations of a rocprofv3 --kernel-trace database")
    ap.add_argument("--write-tables", action="store_true",
                    help="regenerate the generated tables of the repository's documents from "
                         "results/ and profiles/ (no GPU)")
    args = ap.parse_args()
    if args.write_tables:
        write_tables(ROOT / "results", DOCS)
        return
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters))
        return
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(rows shard across GPUs with no exchange).", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from invariant_lm_head_amd import lmhead

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    if args.counters:
        counters_run(torch, lmhead, synth, dev)
        return

    wl = synth.WORKLOADS["tinyllama"]
    H, V = wl.H, wl.V
    d = synth.make_inputs("tinyllama")
    x = bf16(d["x"])
    ws_ = [bf16(d["w"]) for _ in range(NCOPIES)]
    wp_ = [lmhead.pack_w(w) for w in ws_]   # once, before anything is timed
    torch.cuda.synchronize()

    callers = {B: Caller(torch, lmhead, [x[:B].contiguous()] * NCOPIES, wp_, B, H, V, mode=PACKED)
               for B in SWEEP}

    # ---- the timed steps (whole sweep per step)
    # consecutive calls always read different W copies (global rotation)
    k = 0
    for _ in range(args.warmup):
        for B in SWEEP:
            callers[B](k)
            k += 1
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    s.record()
    for _ in range(args.steps):
        for B in SWEEP:
            callers[B](k)
            k += 1
    e.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    step_s = s.elapsed_time(e) / 1e3 / args.steps
    rows = sum(SWEEP)
    value = rows / step_s
    log(f"step: {step_s * 1e6:.1f} us for {rows} rows -> {value / 1e6:.3f} M rows/s "
        f"(wall {t_wall:.3f} s for {args.steps} steps)")

    # ---- per-batch kernel times (HIP events, cold W) and warm (one W copy)
    per_batch = []
    for B in SWEEP:
        t = time_calls(torch, callers[B], 200)
        warm = Caller(torch, lmhead, [x[:B].contiguous()], wp_[:1], B, H, V, mode=PACKED)
        tw = time_calls(torch, warm, 200)
        rf = roofline(B, H, V, t)
        per_batch.append({"batch": B, "us_per_call": t * 1e6, "rows_per_s": B / t,
                          "roofline": {k: rf[k] for k in ("bound", "achieved", "peak", "unit", "frac")},
                          "gbps": rf["bytes"] / t / 1e9, "tflops": rf["flops"] / t / 1e12,
                          "us_per_call_warm_mall": tw * 1e6})
        log(f"B={B:4d}: {t * 1e6:8.2f} us  {B / t / 1e6:8.3f} M rows/s  {rf['bound']} "
            f"{rf['achieved']:8.1f} {rf['unit']} = {100 * rf['frac']:5.1f}% "
            f"(warm MALL {tw * 1e6:.2f} us)")

    dom = max(per_batch, key=lambda r: r["us_per_call"])
    rf = dict(dom["roofline"])
    traffic = traffic_from_profile(f"greedy_tinyllama_b{dom['batch']}")
    rf["traffic"] = traffic
    rf["kernel"] = (f"one greedy top-2 call at batch {dom['batch']} (tile kernel + fold kernel), "
                    "packed W")

    out = {
        "metric": METRIC, "value": value, "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": step_s * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "TinyLlama-shaped head H=2048 V=32000, fused greedy top-2 "
                               "(float32 head), one call per batch 1,8,64,256,512",
                   "H": H, "V": V, "batches": list(SWEEP), "rows_per_step": rows,
                   "w_copies_rotated": NCOPIES, "w_layout": "packed once (lmhead_pack_w)",
                   "parallelism": "single GPU"},
        "roofline": rf,
        "per_batch": per_batch,
        "source_digest": source_digest(),
    }

    # ---- other workloads (reported, not in value)
    if not args.no_extras:
        # the same sweep's calls reading the row-major W (bits identical)
        out["per_batch_row_major"] = []
        for B in SWEEP:
            c = Caller(torch, lmhead, [x[:B].contiguous()] * NCOPIES, ws_, B, H, V)
            t = time_calls(torch, c, 200)
            rfr = roofline(B, H, V, t)
            out["per_batch_row_major"].append({
                "batch": B, "us_per_call": t * 1e6, "rows_per_s": B / t,
                "roofline": {k: rfr[k] for k in ("bound", "achieved", "peak", "unit", "frac")}})
            log(f"row-major W, B={B:4d}: {t * 1e6:8.2f} us")
        del c
        out["other"] = extras(torch, lmhead, synth, bf16, x, wp_, d)
        del wp_
        out["output_digests"] = output_digests(torch, lmhead, synth, bf16, dev)
    del callers
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline()
        cb = out["cpu_baseline"]
        log(f"cpu oracle: {cb['value']:.1f} rows/s on {cb['cores']} threads "
            f"({cb['host']['online_cpus']} online CPUs, {cb['host']['cpu_model']})")
    print(json.dumps(out), flush=True)


def counters_run(torch, lmhead, synth, dev):
    """Launch sequence for the rocprofv3 --pmc runs (one counter set per run):
    3 copies of 512 MiB (read 512 MiB + write 512 MiB each: the calibration of
    the HBM byte counters), then 5 greedy top-2 calls at each batch 1, 256 and
    512 of the H=2048, V=32000 head (four rotating packed W copies), then 5 greedy
    top-2 calls of the int8 head H=4096, V=128256 at batch 512."""
    src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    d = synth.make_inputs("tinyllama")

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    x = bf16(d["x"])
    w = [lmhead.pack_w(bf16(d["w"])) for _ in range(NCOPIES)]   # as the timed sweep reads W
    torch.cuda.synchronize()
    for B in (1, 256, 512):
        c = Caller(torch, lmhead, [x[:B].contiguous()] * NCOPIES, w, B, 2048, 32000, mode=PACKED)
        for _ in range(5):
            c()
        torch.cuda.synchronize()
        log(f"counter launches: greedy 2048 x 32000 batch {B} done")
    del x, w, c
    i8 = synth.make_inputs("int8", rows=512)
    xi = torch.from_numpy(i8["x"]).to(dev)
    wi = torch.from_numpy(i8["w"]).to(dev)
    si = torch.from_numpy(i8["scale"]).to(dev)
    c = Caller(torch, lmhead, [xi], [wi], 512, i8["H"], i8["V"], mode=1, scale=si)
    for _ in range(5):
        c()
    torch.cuda.synchronize()
    log("counter launches: int8 greedy 4096 x 128256 batch 512 done")


# ------------------------------------------------------------ profile summaries
# Kernels of the launch sequence of --counters, by (template arguments, mode,
# epilogue, threads in the grid): the workload each one belongs to.
COUNTER_CONFIGS = [
    ("Tile<32, 128, 1, 4, 256, 2, 3, false, false>, 0, 1>", 64000, "tinyllama greedy, batch 1, tile kernel"),
    ("lmhead_merge_top2_kernel<0, 1>", 256, "tinyllama greedy, batch 1, fold kernel"),
    ("Tile<256, 128, 4, 2, 128, 2, 4, false, false>, 0, 1>", 128000, "tinyllama greedy, batch 256, tile kernel"),
    ("lmhead_merge_top2_kernel<0, 1>", 16384, "tinyllama greedy, batch 256, fold kernel"),
    ("Tile<256, 256, 4, 2, 128, 2, 3, false, true>, 0, 1>", 128000, "tinyllama greedy, batch 512, tile kernel"),
    ("lmhead_merge_top2_kernel<0, 1>", 32768, "tinyllama greedy, batch 512, fold kernel"),
    ("Tile<256, 256, 4, 2, 128, 2, 3, false, true>, 1, 1>", 513024, "int8 4096x128256 greedy, batch 512, tile kernel"),
    ("lmhead_merge_top2_kernel<1, 1>", 32768, "int8 4096x128256 greedy, batch 512, fold kernel"),
]
COPY_KERNEL = ("__amd_rocclr_copyBuffer", 131072)   # the 512 MiB calibration copy


def _rocpd(db):
    """(per-dispatch rows {name, grid, dur_ns, counters}) of a rocprofv3 database."""
    import sqlite3
    con = sqlite3.connect(str(db))
    cur = con.cursor()
    out = {}
    for d, name, dur, grid in cur.execute(
            "select dispatch_id, name, duration, grid_x * grid_y * grid_z from kernels"):
        out[d] = {"name": name, "grid": grid, "dur_ns": dur, "c": {}}
    try:
        for d, cn, v in cur.execute("select dispatch_id, counter_name, value from counters_collection"):
            if d in out:
                out[d]["c"][cn] = v
    except sqlite3.OperationalError:
        pass
    return list(out.values())


def _label(name, grid):
    for key, g, label in COUNTER_CONFIGS:
        if key in name and g == grid:
            return label
    return None


def _median(v):
    v = sorted(v)
    return v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])


def _pmc_names(db):
    import sqlite3
    con = sqlite3.connect(str(db))
    try:
        return sorted({r[0] for r in con.execute("select distinct counter_name from counters_collection")})
    except sqlite3.OperationalError:
        return []


def summarize_counters(dbs) -> str:
    """Markdown summary of --counters runs: per workload kernel, the median of
    each counter over its dispatches, and derived figures (HBM bytes from the
    calibrated FETCH_SIZE / WRITE_SIZE, MFMA busy cycles against the time the
    kernel took at the 2.4 GHz peak clock, LDS, TA and TD busy shares)."""
    per = {}
    calib = {}
    for db in dbs:
        for r in _rocpd(db):
            if COPY_KERNEL[0] in r["name"] and r["grid"] == COPY_KERNEL[1]:
                for cn, v in r["c"].items():
                    calib.setdefault(cn, []).append(v)
                continue
            lab = _label(r["name"], r["grid"])
            if lab is None:
                continue
            e = per.setdefault(lab, {"name": r["name"], "dur": [], "c": {}})
            e["dur"].append(r["dur_ns"])
            for cn, v in r["c"].items():
                e["c"].setdefault(cn, []).append(v)
    fetch_f = 524288.0 / _median(calib["FETCH_SIZE"]) if "FETCH_SIZE" in calib else None
    write_f = 524288.0 / _median(calib["WRITE_SIZE"]) if "WRITE_SIZE" in calib else None
    lines = ["| kernel | counter | median per dispatch |", "|---|---|---|"]
    derived = ["| kernel | duration us (profiled) | MFMA busy at 2.4 GHz | MFMA busy / active cycles | "
               "LDS active | TA busy | TD busy | read MB | written MB |",
               "|---|---|---|---|---|---|---|---|---|"]
    traffic = {}
    for key, _g, lab in COUNTER_CONFIGS:
        if lab not in per:
            continue
        e = per[lab]
        c = {cn: _median(v) for cn, v in e["c"].items()}
        for cn in sorted(c):
            lines.append(f"| {lab} | {cn} | {c[cn]:.6g} |")
        dur = _median(e["dur"]) / 1e3
        # GRBM_GUI_ACTIVE: busy cycles summed over the 8 XCDs (its window is a
        # few microseconds longer than the dispatch, so shares over it are
        # lower bounds)
        cyc = c["GRBM_GUI_ACTIVE"] / 8 if "GRBM_GUI_ACTIVE" in c else None
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES")
        peak = busy / (1024 * dur * 1e3 * 2.4) if busy is not None else None
        mfma = busy / (1024 * cyc) if cyc and busy is not None else None
        lds = 4 * c["SQ_LDS_IDX_ACTIVE"] / (256 * cyc) if cyc and "SQ_LDS_IDX_ACTIVE" in c else None
        ta = c["TA_TA_BUSY_sum"] / (256 * cyc) if cyc and "TA_TA_BUSY_sum" in c else None
        td = c["TD_TD_BUSY_sum"] / (256 * cyc) if cyc and "TD_TD_BUSY_sum" in c else None
        rd = c["FETCH_SIZE"] * 1024 * fetch_f / 1e6 if fetch_f and "FETCH_SIZE" in c else None
        wr = c["WRITE_SIZE"] * 1024 * write_f / 1e6 if write_f and "WRITE_SIZE" in c else None
        if rd is not None and wr is not None:
            traffic[lab] = (rd + wr) * 1e6
        f = lambda v, fmt: "" if v is None else format(v, fmt)  # noqa: E731
        derived.append(f"| {lab} | {dur:.2f} | {f(peak, '.1%')} | {f(mfma, '.1%')} | {f(lds, '.1%')} | "
                       f"{f(ta, '.1%')} | {f(td, '.1%')} | {f(rd, '.2f')} | {f(wr, '.2f')} |")
    cal = []
    if fetch_f:
        cal.append(f"| FETCH_SIZE | {_median(calib['FETCH_SIZE']):.1f} KiB | {fetch_f:.3f} |")
    if write_f:
        cal.append(f"| WRITE_SIZE | {_median(calib['WRITE_SIZE']):.1f} KiB | {write_f:.3f} |")
    call = [traffic.get("tinyllama greedy, batch 512, " + k) for k in ("tile kernel", "fold kernel")]
    head = [f"source_digest: {source_digest()}"]
    if None not in call:
        head.append(f"hbm_bytes_per_launch: {sum(call):.0f}")
    head += ["", "Commands (from the repository root on the GPU host, one rocprofv3 run per "
             "counter set):", "", "    cd /tmp && export TMPDIR=/tmp"]
    for db in dbs:
        names = [n for n in _pmc_names(db)]
        d = Path(db).parent
        d = d if d.is_absolute() else Path("/root/repo") / d
        head.append(f"    timeout -s KILL 120 rocprofv3 --pmc {' '.join(names)} -d {d} -o pmc -- "
                    f"python3 /root/repo/bench.py --counters")
    out = head + ["", "## Derived per kernel (medians over its dispatches)", ""] + derived + [""]
    if cal:
        out += ["## Calibration: a plain copy of 512 MiB (524288 KiB read, 524288 KiB written)", "",
                "| counter | copy reads as | factor |", "|---|---|---|"] + cal + [""]
    out += ["## Raw counters", ""] + lines + [""]
    return "\n".join(out)


def summarize_trace(db) -> str:
    """Markdown table of a rocprofv3 --kernel-trace database: calls and
    average / min / max duration per kernel."""
    per = {}
    for r in _rocpd(db):
        per.setdefault(r["name"], []).append(r["dur_ns"] / 1e3)
    rows = ["| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for name, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        if "lmhead" not in name and "quantize" not in name:
            continue
        short = name.replace("lmh::(anonymous namespace)::", "").replace("void ", "")
        short = short.replace("(lmh::Params)", "")
        rows.append(f"| `{short}` | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    return "\n".join(rows) + "\n"


# ------------------------------------------------------- generated tables
def _fmt_roof(r):
    return f"{100 * r['frac']:.1f}% of {'HBM' if r['bound'] == 'hbm' else 'MFMA'} peak"


def render_tables(results: Path) -> dict:
    """Markdown tables from the committed result files: the bench line
    (results/bench_full.json) and the GPU tests' parity files."""
    b = json.loads((results / "bench_full.json").read_text())
    t = {}
    rows = ["| batch | us / call (packed W from HBM) | rows/s | roofline | "
            "us / call (row-major W from HBM) | us / call (packed W in the Infinity Cache) |",
            "|---|---|---|---|---|---|"]
    rm = {r["batch"]: r for r in b.get("per_batch_row_major", [])}
    for r in b["per_batch"]:
        rmaj = f"{rm[r['batch']]['us_per_call']:.2f}" if r["batch"] in rm else ""
        rows.append(f"| {r['batch']} | {r['us_per_call']:.2f} | {r['rows_per_s'] / 1e6:.3f} M | "
                    f"{_fmt_roof(r['roofline'])} | {rmaj} | {r['us_per_call_warm_mall']:.2f} |")
    rows.append(f"| sweep step (841 rows) | {b['ms_per_step'] * 1e3:.1f} | "
                f"{b['value'] / 1e6:.3f} M | dominant call: {_fmt_roof(b['roofline'])} | "
                f"{sum(r['us_per_call'] for r in rm.values()):.1f} (sum of the calls) | |")
    t["per_batch"] = "\n".join(rows)
    o = b.get("other", {})
    # the performance targets of this head on MI355X (70% of the HBM roofline
    # where W's stream bounds a call, 50% of MFMA peak at large batches)
    # against this run
    pb = {r["batch"]: r for r in b["per_batch"]}
    rows = ["| workload | target | measured | met |", "|---|---|---|---|"]

    def tgt(label, want, got, ok):
        rows.append(f"| {label} | {want} | {got} | {'yes' if ok else 'no'} |")

    if 1 in pb:
        u = pb[1]["us_per_call"]
        tgt("greedy 2048 x 32000, batch 1", "<= 23.4 us (70% of HBM)",
            f"{u:.2f} us ({_fmt_roof(pb[1]['roofline'])})", u <= 23.4)
    for B, lim in ((256, 26.7), (512, 53.3)):
        if B in pb:
            u = pb[B]["us_per_call"]
            tgt(f"greedy 2048 x 32000, batch {B}", f"<= {lim} us (50% of MFMA)",
                f"{u:.2f} us ({100 * 2 * B * 32000 * 2048 / (u * 1e-6) / 2.5e15:.1f}% of MFMA)",
                u <= lim)
    if "logprob_16384x151936x4096" in o:
        r = o["logprob_16384x151936x4096"]
        tgt("log-prob scoring 4096 x 151936, 16384 rows", "<= 16.2 ms (50% of MFMA)",
            f"{r['ms_per_call']:.2f} ms ({_fmt_roof(r['roofline'])})", r["ms_per_call"] <= 16.2)
    if "int8_b1" in o:
        r = o["int8_b1"]
        tgt("int8 greedy 4096 x 128256, batch 1", "<= 93.8 us (70% of HBM)",
            f"{r['us_per_call']:.1f} us ({_fmt_roof(r['roofline'])})", r["us_per_call"] <= 93.8)
    if "int8_b512" in o:
        r = o["int8_b512"]
        tgt("int8 greedy 4096 x 128256, batch 512", ">= 2.4 M rows/s (50% of MFMA)",
            f"{r['rows_per_s'] / 1e6:.2f} M rows/s ({_fmt_roof(r['roofline'])})",
            r["rows_per_s"] >= 2.4e6)
    t["targets"] = "\n".join(rows)
    names = {
        "tinyllama_logprob_b512": "log-prob, 2048 x 32000, batch 512",
        "tinyllama_logits_b512": "float32 logits stored, 2048 x 32000, batch 512",
        "neartie_4096": "near-tie set, 2048 x 32000, 4096 rows",
        "logprob_16384x151936x4096": "log-prob scoring, 4096 x 151936, 16384 rows",
        "greedy_4096x151936_b1": "greedy, 4096 x 151936 (1.24 GB of W), row-major W, batch 1",
        "greedy_4096x151936_b64": "greedy, 4096 x 151936, row-major W, batch 64",
        "greedy_4096x151936_packed_b1": "greedy, 4096 x 151936, packed W, batch 1",
        "greedy_4096x151936_packed_b64": "greedy, 4096 x 151936, packed W, batch 64",
        "int8_b1": "int8 greedy, 4096 x 128256, batch 1",
        "int8_b8": "int8 greedy, batch 8",
        "int8_b64": "int8 greedy, batch 64",
        "int8_b256": "int8 greedy, batch 256",
        "int8_b512": "int8 greedy, batch 512",
        "int_logprob_b1": "integer log-prob (Q.24), 4096 x 128256, batch 1",
        "int_logprob_b512": "integer log-prob (Q.24), batch 512",
    }
    rows = ["| workload | time / call | rows/s | roofline |", "|---|---|---|---|"]
    for k, label in names.items():
        if k not in o:
            continue
        r = o[k]
        tt = f"{r['ms_per_call']:.2f} ms" if "ms_per_call" in r else f"{r['us_per_call']:.1f} us"
        roof = _fmt_roof(r["roofline"])
        if "float_logprob_us" in r:
            roof += (f"; {100 * (r['us_per_call'] / r['float_logprob_us'] - 1):+.1f}% against the "
                     f"float log-prob of the int8 head ({r['float_logprob_us']:.1f} us)")
        rows.append(f"| {label} | {tt} | {r['rows_per_s'] / 1e6:.3f} M | {roof} |")
    for B in (1, 512):
        g, sm = o.get(f"gated_tau1e-3_b{B}"), o.get(f"sample_gumbel_b{B}")
        if g:
            rows.append(f"| margin-gated head (tau 1e-3), batch {B} | {g['us_per_call']:.1f} us | | "
                        f"{100 * g['overhead']:+.1f}% against the bf16-output head, "
                        f"{100 * g['gate_rate']:.2f}% of rows recomputed |")
        if sm:
            rows.append(f"| seeded Gumbel-max sampling, batch {B} | {sm['us_per_call']:.1f} us | "
                        f"{sm['rows_per_s'] / 1e6:.3f} M | {100 * sm['overhead']:+.1f}% against greedy |")
    if "tiny_b4" in o:
        tb = o["tiny_b4"]
        rows.append(f"| tiny 4 x 64 x 1000: greedy / log-prob / logits | {tb['greedy_us_per_call']:.1f} / "
                    f"{tb['logprob_us_per_call']:.1f} / {tb['logits_us_per_call']:.1f} us | | latency |")
    t["other"] = "\n".join(rows)
    c = b.get("cpu_baseline")
    if c:
        h = c.get("host", {})
        rows = [f"Host: {h.get('cpu_model')}, {h.get('online_cpus')} online CPUs; the oracle ran on "
                f"{c['threads']} threads.", "",
                "| oracle workload | rows | rows/s |", "|---|---|---|",
                f"| float64 greedy, 2048 x 32000 (the metric's) | {c['sample'].split('rows ')[1].split(' ')[0]} | "
                f"{c['value']:.1f} ({c['single_thread_rows_per_s']:.1f} on one thread) |"]
        for k, r in c.get("other", {}).items():
            rows.append(f"| {k} | {r['rows']} | {r['rows_per_s']:.1f} |")
        t["cpu"] = "\n".join(rows)
    par = {}
    for f in (sorted(results.glob("parity_*.json")) + sorted(results.glob("invariance.json"))
              + sorted(results.glob("batch_variance.json"))):
        par[f.stem] = json.loads(f.read_text())
    rows = ["| check | rows | result |", "|---|---|---|"]
    g = par.get("parity_tinyllama_greedy", {})
    for B in (1, 8, 64, 256, 512):
        e = g.get(f"batch_{B}")
        if e:
            rows.append(f"| float32 greedy, 2048 x 32000, batch {B}, against the oracle | {e['rows']} | "
                        f"{e['exempt_rows']} exempt rows (oracle gap < 1e-4); max error of values "
                        f"{e['max_abs_err_values']:.1e} |")
    e = par.get("parity_tinyllama_logprob", {}).get("batch_512")
    if e:
        rows.append(f"| float32 log-prob, 2048 x 32000 | {e['rows']} | max error {e['max_abs_err']:.1e} |")
    e = par.get("parity_logprob_scoring", {}).get("rows_0_255_and_every_64th")
    if e:
        rows.append(f"| float32 log-prob, 4096 x 151936 (16384-row batch) | {e['rows']} | "
                    f"max error {e['max_abs_err']:.1e} |")
    nt = par.get("parity_neartie", {})
    e = nt.get("float32_head_vs_oracle")
    if e:
        gaps = e["exempt_gap_bf16_ulps"]
        rows.append(f"| float32 greedy, near-tie set | {e['rows']} | {e['exempt_rows']} exempt rows "
                    f"(gaps {min(gaps, default=0):.2f}-{max(gaps, default=0):.2f} bf16 ulps), "
                    f"{e['exempt_rows_top1_differs']} of them with the other top-1 |")
    e = nt.get("bf16_head_vs_oracle_bf16_rounding")
    if e:
        rows.append(f"| bf16-output head against the oracle's bf16-rounded logits | {e['rows']} | "
                    f"{e['top1_differs']} top-1 differ, {e['values_differ_by_one_bf16_ulp']} values one bf16 ulp apart |")
    i8 = par.get("parity_int8", {})
    n = sum(v["rows"] for k, v in i8.items() if k.startswith("greedy_batch") and v.get("bit_exact"))
    if n:
        rows.append(f"| int8 greedy (ids, raw, values, margin), batches 1/8/64/256/512 | {n} | bit-exact |")
    n = sum(v["rows"] for k, v in i8.items() if k.startswith("integer_logprob") and v.get("bit_exact"))
    if n:
        rows.append(f"| integer log-prob (Q.24), batches 1/8/64/256/512 | {n} | bit-exact |")
    if "logits_rows_compared" in i8:
        rows.append(f"| int8 logits of a 512-row call | {i8['logits_rows_compared']} | bit-exact |")
    e = i8.get("float_logprob_batch_512")
    if e:
        rows.append(f"| float log-prob of the int8 head | {e['rows']} | max error {e['max_abs_err']:.1e} |")
    inv = par.get("invariance", {})
    if "logits_batches_1_to_512" in inv:
        rows.append(f"| bitwise invariance: logits, top-2, log-prob at every batch 1..512 | "
                    f"{inv['logits_batches_1_to_512']['rows_compared']} rows x 32000 logits | identical |")
    if "int8_greedy_batches_1_to_512_vs_oracle" in inv:
        rows.append(f"| int8 greedy at every batch 1..512 against the oracle's stored rows | "
                    f"{inv['int8_greedy_batches_1_to_512_vs_oracle']['rows_compared']} rows | "
                    f"bit-exact |")
    if "packed_greedy_batches_1_to_512" in inv:
        rows.append(f"| bitwise invariance, packed W: top-2 at every batch 1..512 against the "
                    f"row-major batch-512 call, both rankings | "
                    f"{inv['packed_greedy_batches_1_to_512']['rows_compared']} rows x 2 | identical |")
    t["parity"] = "\n".join(rows)
    bv = par.get("batch_variance")
    if bv:
        rows = ["| rows | head | compared | log-prob bits differ | max abs dlog p | "
                "ratio outside [0.9, 1.1] |", "|---|---|---|---|---|---|"]
        for key, r in bv.items():
            parts = key.split(" | ")
            if len(parts) != 3:
                continue
            rset, head, cmp_ = parts
            rows.append(f"| {rset} | {head} | {cmp_.replace('_', ' ')} | "
                        f"{100 * r['bits_differ']:.2f}% | {r['max_abs_dlogp']:.1e} | "
                        f"{100 * r['ratio_out_of_band']:.2f}% |")
        t["batch_variance"] = "\n".join(rows)
    nt_tab = nt.get("agreement_with_planted_winner")
    if nt_tab:
        rows = ["| planted gap (bf16 ulps) | rows | float32 head picks the planted winner | bf16-output head |",
                "|---|---|---|---|"]
        for r in nt_tab:
            lo, hi = r["gap_bf16_ulps"]
            rows.append(f"| {'0 (exact tie)' if hi == 0 else f'({lo}, {hi}]'} | {r['rows']} | "
                        f"{100 * r['float32_head_agrees']:.2f}% | {100 * r['bf16_head_agrees']:.2f}% |")
        t["neartie"] = "\n".join(rows)
    return t


def render_counter_table(profile: Path) -> dict:
    """The tile kernels' rows of the committed counter summary's derived table."""
    if not profile.exists():
        return {}
    label = {"tinyllama greedy, batch 1, tile kernel": "batch 1 (32 × 128 tile)",
             "tinyllama greedy, batch 256, tile kernel": "batch 256 (256 × 128)",
             "tinyllama greedy, batch 512, tile kernel": "batch 512 (256 × 256)",
             "int8 4096x128256 greedy, batch 512, tile kernel":
                 "int8 4096 × 128256, batch 512 (256 × 256)"}
    rows = ["| kernel | MFMA busy at 2.4 GHz | MFMA busy / active cycles | LDS active | TA busy | "
            "TD busy |", "|---|---|---|---|---|---|"]
    for line in profile.read_text().splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 9 and cells[0] in label:
            rows.append(f"| {label[cells[0]]} | " + " | ".join(cells[2:7]) + " |")
    return {"counters": "\n".join(rows)} if len(rows) > 2 else {}


def write_tables(results: Path, docs) -> None:
    """Replace every <!-- generated:NAME --> ... <!-- /generated:NAME --> block
    of the docs with the table NAME."""
    import re
    tabs = render_tables(results)
    tabs.update(render_counter_table(ROOT / "profiles" / "counters_greedy_tinyllama_b512.md"))
    for doc in docs:
        text = doc.read_text()
        for name, md in tabs.items():
            text = re.sub(rf"(<!-- generated:{name} -->).*?(<!-- /generated:{name} -->)",
                          lambda m: m.group(1) + "\n" + md + "\n" + m.group(2), text, flags=re.S)
        doc.write_text(text)


def extras(torch, lmhead, synth, bf16, x, w_copies, d):
    """The other workloads.  w_copies: the TinyLlama head's W copies, packed;
    the float head's workloads read packed W like the sweep (the 4096 x 151936
    head both ways), the int8 head row-major W."""
    H, V = 2048, 32000
    P2 = PACKED
    res = {}
    B = 512
    t = torch.from_numpy(d["target"][:B]).to(x.device)
    c = Caller(torch, lmhead, [x[:B].contiguous()] * NCOPIES, w_copies, B, H, V, mode=P2,
               kind="logprob", target=t)
    tt = time_calls(torch, c, 100)
    res["tinyllama_logprob_b512"] = {"us_per_call": tt * 1e6, "rows_per_s": B / tt,
                                     "roofline": roofline(B, H, V, tt, out_bytes_per_row=8)}
    c = Caller(torch, lmhead, [x[:B].contiguous()] * NCOPIES, w_copies, B, H, V, mode=P2,
               kind="logits")
    tt = time_calls(torch, c, 100)
    res["tinyllama_logits_b512"] = {"us_per_call": tt * 1e6, "rows_per_s": B / tt,
                                    "roofline": roofline(B, H, V, tt, out_bytes_per_row=4 * V)}
    del c
    log("tinyllama logprob/logits B=512: "
        f"{res['tinyllama_logprob_b512']['us_per_call']:.1f} / "
        f"{res['tinyllama_logits_b512']['us_per_call']:.1f} us")

    # the tiny workload (H=64, V=1000, batch 4; W stays in L2): latency per call
    dt = synth.make_inputs("tiny")
    xt, wt = bf16(dt["x"]), bf16(dt["w"])
    tt_t = torch.from_numpy(dt["target"]).to(x.device)
    tiny = {}
    for kind in ("greedy", "logprob", "logits"):
        c = Caller(torch, lmhead, [xt], [wt], 4, 64, 1000, kind=kind, target=tt_t)
        tiny[f"{kind}_us_per_call"] = time_calls(torch, c, 200) * 1e6
    res["tiny_b4"] = tiny
    log("tiny 4 x 64 x 1000: greedy / logprob / logits "
        f"{tiny['greedy_us_per_call']:.1f} / {tiny['logprob_us_per_call']:.1f} / "
        f"{tiny['logits_us_per_call']:.1f} us")

    # margin-gated float32 recompute (tau = 1e-3) against the plain bf16-output head
    for B in (1, 512):
        xb = [x[:B].contiguous()] * NCOPIES
        plain = Caller(torch, lmhead, xb, w_copies, B, H, V, mode=P2, round_bf16=1)
        gated = Caller(torch, lmhead, xb, w_copies, B, H, V, mode=P2, kind="gated", tau=1e-3)
        tp, tg = time_calls(torch, plain, 100), time_calls(torch, gated, 100)
        rate = float(gated.keep[3].float().mean().item())
        res[f"gated_tau1e-3_b{B}"] = {"us_per_call": tg * 1e6, "us_bf16_head": tp * 1e6,
                                       "overhead": tg / tp - 1.0, "gate_rate": rate}
        log(f"gated B={B}: {tg * 1e6:.1f} us vs bf16 head {tp * 1e6:.1f} us "
            f"({100 * (tg / tp - 1):+.1f}%), gate rate {100 * rate:.2f}%")

    # seeded Gumbel-max sampling (T = 1) against the float32 greedy head
    for B in (1, 512):
        xb = [x[:B].contiguous()] * NCOPIES
        greedy = Caller(torch, lmhead, xb, w_copies, B, H, V, mode=P2)
        samp = Caller(torch, lmhead, xb, w_copies, B, H, V, mode=P2, kind="sample", tau=1.0)
        tgr, tsa = time_calls(torch, greedy, 100), time_calls(torch, samp, 100)
        res[f"sample_gumbel_b{B}"] = {"us_per_call": tsa * 1e6, "us_greedy": tgr * 1e6,
                                      "overhead": tsa / tgr - 1.0, "rows_per_s": B / tsa}
        log(f"sample B={B}: {tsa * 1e6:.1f} us vs greedy {tgr * 1e6:.1f} us "
            f"({100 * (tsa / tgr - 1):+.1f}%)")

    # near-tie stress, 4096 rows
    nt = synth.make_inputs("neartie")
    xn, wn = bf16(nt["x"]), lmhead.pack_w(bf16(nt["w"]))
    c = Caller(torch, lmhead, [xn], [wn], 4096, H, V, mode=P2)
    tt = time_calls(torch, c, 30)
    res["neartie_4096"] = {"us_per_call": tt * 1e6, "rows_per_s": 4096 / tt,
                           "roofline": roofline(4096, H, V, tt)}
    c = Caller(torch, lmhead, [xn], [wn], 4096, H, V, mode=P2, kind="gated", tau=1e-3)
    tg = time_calls(torch, c, 30)
    res["neartie_4096_gated_tau1e-3"] = {"us_per_call": tg * 1e6,
                                         "gate_rate": float(c.keep[3].float().mean().item())}
    del c, xn, wn, nt
    log(f"near-tie 4096 rows: {tt * 1e6:.1f} us")

    # log-prob scoring, 16384 x 151936 x 4096
    lp = synth.make_inputs("logprob")
    Hl, Vl, Bl = lp["H"], lp["V"], lp["B"]
    xl, wl_ = bf16(lp["x"]), bf16(lp["w"])
    tl = torch.from_numpy(lp["target"]).to(x.device)
    del lp
    wlp = lmhead.pack_w(wl_)   # kept alive while its callers run
    c = Caller(torch, lmhead, [xl], [wlp], Bl, Hl, Vl, mode=P2, kind="logprob", target=tl)
    tt = time_calls(torch, c, 5, warmup=1)
    res["logprob_16384x151936x4096"] = {"ms_per_call": tt * 1e3, "rows_per_s": Bl / tt,
                                        "roofline": roofline(Bl, Hl, Vl, tt, out_bytes_per_row=8),
                                        "exp_per_s": Bl * Vl / tt}
    log(f"log-prob 16384x151936x4096: {tt * 1e3:.2f} ms = "
        f"{100 * res['logprob_16384x151936x4096']['roofline']['frac']:.1f}% of MFMA peak")
    # greedy on the same 1.24 GB head (five times the Infinity Cache, so W
    # comes from HBM on every call) at batch 1 and 64
    for B in (1, 64):
        c = Caller(torch, lmhead, [xl[:B].contiguous()], [wl_], B, Hl, Vl)
        tt = time_calls(torch, c, 30)
        key = f"greedy_4096x151936_b{B}"
        res[key] = {"us_per_call": tt * 1e6, "rows_per_s": B / tt, "roofline": roofline(B, Hl, Vl, tt)}
        log(f"greedy 4096x151936 B={B}: {tt * 1e6:.1f} us, "
            f"{res[key]['roofline']['bound']} {100 * res[key]['roofline']['frac']:.1f}%")
    # the same with W packed once (lmhead_pack_w)
    for B in (1, 64):
        c = Caller(torch, lmhead, [xl[:B].contiguous()], [wlp], B, Hl, Vl, mode=PACKED)
        tt = time_calls(torch, c, 30)
        key = f"greedy_4096x151936_packed_b{B}"
        res[key] = {"us_per_call": tt * 1e6, "rows_per_s": B / tt, "roofline": roofline(B, Hl, Vl, tt)}
        log(f"greedy 4096x151936 packed W B={B}: {tt * 1e6:.1f} us, "
            f"{res[key]['roofline']['bound']} {100 * res[key]['roofline']['frac']:.1f}%")
    del c, xl, wl_, wlp, tl
    torch.cuda.empty_cache()

    # int8 head, 4096 x 128256, batch 1 .. 512
    i8 = synth.make_inputs("int8")
    Hi, Vi = i8["H"], i8["V"]
    xi = torch.from_numpy(i8["x"]).to(x.device)
    wi = [torch.from_numpy(i8["w"]).to(x.device)]
    si = torch.from_numpy(i8["scale"]).to(x.device)
    del i8
    for B in (1, 8, 64, 256, 512):
        c = Caller(torch, lmhead, [xi[:B].contiguous()], wi, B, Hi, Vi, mode=1, scale=si[:B])
        tt = time_calls(torch, c, 50)
        res[f"int8_b{B}"] = {"us_per_call": tt * 1e6, "rows_per_s": B / tt,
                             "roofline": roofline(B, Hi, Vi, tt, esize=1, out_bytes_per_row=28,
                                                  mode="int8")}
        r = res[f"int8_b{B}"]["roofline"]
        log(f"int8 B={B}: {tt * 1e6:.1f} us, {r['bound']} {100 * r['frac']:.1f}%")

    # the all-integer path at the same shape: per-token quantisation of int32
    # hidden rows, then the integer log-softmax (log p in Q.24), and the float
    # log-prob of the int8 head for comparison
    hid = torch.from_numpy(synth.hidden_int32(synth.seed_of(5, 6), 512, Hi)).to(x.device)
    ti = torch.from_numpy(synth.target_ids(synth.seed_of(5, 3), 512, Vi)).to(x.device)
    cq = Caller(torch, lmhead, [hid], [None], 512, Hi, Vi, mode=1, kind="quantize")
    tq = time_calls(torch, cq, 50)
    res["int_quantize_b512"] = {"us_per_call": tq * 1e6,
                                "gbps": 512 * Hi * 5 / tq / 1e9}
    log(f"int quantize 512 x {Hi}: {tq * 1e6:.1f} us")
    qi, smi, sei = cq.keep
    for B in (1, 512):
        c = Caller(torch, lmhead, [qi[:B].contiguous()], wi, B, Hi, Vi, mode=1,
                   kind="logprob_int", target=ti[:B].contiguous(),
                   steps=(smi[:B].contiguous(), sei[:B].contiguous()), unit=synth.INT_UNIT)
        tt = time_calls(torch, c, 50)
        cf = Caller(torch, lmhead, [xi[:B].contiguous()], wi, B, Hi, Vi, mode=1, kind="logprob",
                    target=ti[:B].contiguous(), scale=si[:B])
        tf = time_calls(torch, cf, 50)
        res[f"int_logprob_b{B}"] = {"us_per_call": tt * 1e6, "rows_per_s": B / tt,
                                    "float_logprob_us": tf * 1e6,
                                    "roofline": roofline(B, Hi, Vi, tt, esize=1,
                                                         out_bytes_per_row=20, mode="int8")}
        r = res[f"int_logprob_b{B}"]["roofline"]
        log(f"integer log-prob B={B}: {tt * 1e6:.1f} us ({r['bound']} {100 * r['frac']:.1f}%), "
            f"float log-prob of the int8 head {tf * 1e6:.1f} us")
    return res


if __name__ == "__main__":
    main()
