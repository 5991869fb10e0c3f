"""The CPU oracle's fast pins again, against a build of oracle.c with
AddressSanitizer and UndefinedBehaviorSanitizer (halting on the first report),
in a child process: an out-of-bounds access, a signed overflow or an
over-wide shift anywhere the pins reach fails this test."""
import os
import shutil
import subprocess
import sys
from pathlib import Path

import pytest

import oracle

ROOT = Path(__file__).resolve().parent.parent


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_pins_under_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("sanitizer runtimes not available")
    lib = tmp_path / "liblmhead_oracle_san.so"
    flags = [f for f in oracle.CFLAGS if not f.startswith("-O")]
    subprocess.run(["gcc", "-O1", "-g", *flags, "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    str(oracle.SOURCE), "-o", str(lib), "-lm"], check=True)
    code = (
        "import sys\n"
        f"sys.path.insert(0, {str(ROOT)!r})\n"
        "import oracle\n"
        "from tests import oracle_pins\n"
        f"o = oracle.Oracle({str(lib)!r})\n"
        "for pin in oracle_pins.FAST:\n"
        "    pin(o)\n"
        "print('pins passed:', len(oracle_pins.FAST), flush=True)\n"
    )
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "pins passed" in r.stdout
