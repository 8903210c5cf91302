"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: a copy of
oracle/oracle.c is built with -fsanitize=address,undefined (every report
fatal) and the whole pin suite runs against it in a subprocess, through
LOWBIT_ORACLE_LIB_OVERRIDE, with the ASan runtime preloaded (the Python
interpreter itself is not instrumented).  A read or write past an array,
an overflowing signed shift or similar in the oracle fails this test.
Host code only; CPU."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None or _runtime("libasan.so") is None,
                    reason="gcc with the ASan runtime is not installed")
def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = tmp_path / "liboracle_asan.so"
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                    "-ffp-contract=off", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-o", str(lib), SRC, "-lm"], check=True)
    env = dict(os.environ, LOWBIT_ORACLE_LIB_OVERRIDE=str(lib),
               LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, f"pin suite under ASan/UBSan: status {r.returncode}\n{out}"
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
