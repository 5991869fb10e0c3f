"""Float guard of the integer head, checked on the built gfx950 code (no GPU).

"Eliminating Nondeterminism in LLM Inference with Integer-Only Arithmetic",
section "DetLLM": the integer forward pass must hold no floating-point
arithmetic (a guard there turns any float tensor into an error).  Here the
guard reads the library's own gfx950 machine code: the code objects are taken
out of liblmhead.so's offload bundles and disassembled, and

* every int8 tile kernel that decides a top-2 (greedy) or an integer softmax
  partial, the integer log-softmax fold and the per-token quantisation kernel
  contain no floating-point instruction at all;
* the int8 greedy fold, which ranks exact int32 keys and only then scales the
  two winners, uses floating point only for that scaling: integer-to-float64
  conversions, one float64 product, its rounding to float32 and the scale's
  validity test.
"""
import re
import subprocess
from pathlib import Path

import pytest

from invariant_lm_head_amd import _build, lmhead

LLVM = Path("/opt/rocm/llvm/bin")
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
FLOAT_OP = re.compile(r"^\s*(v_[a-z0-9_]*?(?:f16|f32|f64|bf16|xf32)[a-z0-9_]*)\b")
# what the int8 greedy fold may do in floating point: scale the two exact
# winners, one float64 product rounded once to float32, and test the scale
SCALING_OPS = re.compile(r"^v_(cvt_f64_(i32|u32|f32)|cvt_f32_f64|mul_f64|cmp_\w*_f32|"
                         r"cmp_class_f32|cndmask_b32|ldexp_f64|mul_f32)")


def code_objects(lib: Path, out: Path):
    """gfx950 code objects of every offload bundle in the library."""
    sec = out / "fatbin.bin"
    subprocess.run([str(LLVM / "llvm-objcopy"), "--dump-section", f".hip_fatbin={sec}",
                    str(lib), str(out / "stripped.so")], check=True)
    data = sec.read_bytes()
    objs = []
    pos = data.find(MAGIC)
    while pos >= 0:
        n = int.from_bytes(data[pos + 24:pos + 32], "little")
        p = pos + 32
        for _ in range(n):
            off, size, tlen = (int.from_bytes(data[p + 8 * i:p + 8 * i + 8], "little")
                               for i in range(3))
            triple = data[p + 24:p + 24 + tlen].decode()
            p += 24 + tlen
            if "gfx950" in triple and size:
                f = out / f"co{len(objs)}.o"
                f.write_bytes(data[pos + off:pos + off + size])
                objs.append(f)
        pos = data.find(MAGIC, pos + 1)
    return objs


def kernels(objs):
    """{demangled kernel name: [instruction mnemonics]} over all code objects."""
    out = {}
    for f in objs:
        txt = subprocess.run([str(LLVM / "llvm-objdump"), "-d", "-C", "--mcpu=gfx950",
                              "--no-show-raw-insn", str(f)], check=True, capture_output=True,
                             text=True).stdout
        name = None
        for line in txt.splitlines():
            m = re.match(r"^[0-9a-f]+ <(.*)>:$", line)
            if m:
                name = m.group(1)
                out.setdefault(name, [])
            elif name and line.startswith("\t"):
                ins = line.strip().split(" ")[0]
                if ins:
                    out[name].append(ins)
    return out


@pytest.fixture(scope="module")
def disasm(tmp_path_factory):
    if not (LLVM / "llvm-objdump").exists():
        pytest.skip("ROCm LLVM tools not installed")
    lmhead.library()   # builds the library if it is missing; refuses a stale one
    return kernels(code_objects(_build.LIBRARY, tmp_path_factory.mktemp("co")))


def float_ops(ins):
    return sorted({m.group(1) for i in ins for m in [FLOAT_OP.match(i)] if m})


def select(disasm, pattern):
    ks = {k: v for k, v in disasm.items() if re.search(pattern, k)}
    assert ks, f"no kernel matches {pattern}"
    return ks


def test_code_objects_found(disasm):
    assert any("lmhead_tile_kernel" in k for k in disasm)
    # the bf16 head does use float arithmetic: the guard sees it there
    bf16_top2 = select(disasm, r"lmhead_tile_kernel<.*>, 0, 1>\(")
    assert all(float_ops(v) for v in bf16_top2.values())


def test_int8_tile_kernels_have_no_float_instruction(disasm):
    # MODE 1 (int8) with the top-2 (1) or integer log-softmax (4) epilogue
    ks = select(disasm, r"lmhead_tile_kernel<.*>, 1, [14]>\(")
    for name, ins in ks.items():
        assert any(i.startswith("v_mfma_i32") for i in ins), name
        assert not float_ops(ins), (name, float_ops(ins))


def test_integer_front_and_back_have_no_float_instruction(disasm):
    for pat in (r"quantize_rows_kernel", r"lmhead_merge_kernel<1, 4>"):
        for name, ins in select(disasm, pat).items():
            assert not float_ops(ins), (name, float_ops(ins))


def test_int8_greedy_fold_floats_only_scale_the_winners(disasm):
    for name, ins in select(disasm, r"lmhead_merge_top2_kernel<1, 1>").items():
        extra = [op for op in float_ops(ins) if not SCALING_OPS.match(op)]
        assert not extra, (name, extra)
