"""Host-side checks of bench.py's bookkeeping (no GPU).

The HBM traffic that bench.py reports in its roofline object comes from
rocprofv3 counters recorded in profiles/traffic.json together with a
fingerprint of the GEMV's code; the figure must lapse when the code
changes and survive edits to comments or layout only.
"""
import json
import os
import subprocess
import sys

import bench


def _fp(tmp_path, name, text):
    p = tmp_path / name
    p.write_text(text)
    return bench.source_sha(str(p))


BASE = """// header comment
__global__ void k(float* y) {  /* inline note */
  y[0] = 1.0f;  // trailing
}
"""


def test_fingerprint_ignores_comments_and_whitespace(tmp_path):
    a = _fp(tmp_path, "a.hip", BASE)
    b = _fp(tmp_path, "b.hip", "// another header\n\n__global__   void k(float* y) {\n"
                               "  /* a different\n note */ y[0] = 1.0f;\n}\n")
    assert a == b


def test_fingerprint_changes_with_code(tmp_path):
    a = _fp(tmp_path, "a.hip", BASE)
    for edit in ("y[0] = 2.0f;", "y[1] = 1.0f;", "y[0] = 1.0;"):
        assert _fp(tmp_path, "c.hip", BASE.replace("y[0] = 1.0f;", edit)) != a, edit


def test_recorded_counters_match_the_current_gemv_source():
    """profiles/traffic.json was taken on the GEMV code in the tree (else
    bench.py would report traffic as null)."""
    src = os.path.join(bench.ROOT, "bit_matmul_lowbit_amd", "csrc", "gemv.hip")
    with open(os.path.join(bench.ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)[bench.MAIN_KERNEL]
    assert rec["source_sha"] == bench.source_sha(src)
    assert bench.traffic_record(src) == rec["hbm_bytes_per_launch"]
    # read + write, and read within 1 % of the algorithmic weight bytes
    assert rec["hbm_bytes_per_launch"] == rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
    assert abs(rec["hbm_read_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"] - 1) < 0.01


def test_cli_rejects_several_gpus_and_unknown_groups():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--secondary", "gemm,nope"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "nope" in r.stderr
