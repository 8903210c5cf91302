"""The pins catch planted mistakes: each case below builds a copy of
oracle/oracle.c with one deliberate error and runs tests/test_oracle_pins.py
against it (in a subprocess, through LOWBIT_ORACLE_LIB_OVERRIDE); at least
one pin must fail.  CPU only; the real oracle is untouched."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTATIONS = {
    "q1 bit rule >= becomes >": (
        "if (v >= 0.0) codes[code_byte(ORC_Q1, k, row, col)]",
        "if (v > 0.0) codes[code_byte(ORC_Q1, k, row, col)]"),
    "bit order inside a byte (reader)": (
        "int bit = (int)(col % 8);", "int bit = 7 - (int)(col % 8);"),
    "row order inside a cell": (
        "return cell * (fmt == ORC_Q1 ? 16 : 32) + r;",
        "return cell * (fmt == ORC_Q1 ? 16 : 32) + (15 - r);"),
    "scale element index": (
        "return ((row / 16) * (k / 128) + group) * 16 + row % 16;",
        "return ((row / 16) * (k / 128) + group) * 16 + (15 - row % 16);"),
    "bf16 subnormal range": ("if (E < -126) E = -126;", "if (E < -127) E = -127;"),
    "fp16 ties away from zero": (
        "double res = rint(a / ulp) * ulp;", "double res = round(a / ulp) * ulp;"),
    "silu sign": ("return v / (1.0 + exp(-v));", "return v / (1.0 + exp(v));"),
    "ffn gate read from the up half": (
        "double gate = hbuf[i * 2 * f + j];", "double gate = hbuf[i * 2 * f + f + j];"),
    "ternary ties away from zero": (
        "if (2.0 * fabs(v) > s) t =", "if (2.0 * fabs(v) >= s) t ="),
    "base-3 digit weight": ("p *= 3;", "p *= 4;"),
    "gemv group scale dropped": (
        "total += orc_fp16_to_f64(scales[scale_elem(k, row, g)]) * part;", "total += part;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not unique: {old}"
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                    "-ffp-contract=off", "-o", str(lib), str(mutant), "-lm"], check=True)
    env = dict(os.environ, LOWBIT_ORACLE_LIB_OVERRIDE=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    # exit status 1 = some test failed (not a collection or usage error)
    assert r.returncode == 1, f"{name}: pins did not fail (status {r.returncode})\n{r.stdout[-800:]}"
