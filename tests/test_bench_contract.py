"""The bench's contract on the CPU: one GPU only, and the recorded HBM traffic
is reported only for the kernel source it was measured on."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"] and msg["n_gpus_requested"] == 2


def test_recorded_traffic_follows_the_kernel_source(monkeypatch, tmp_path):
    got = bench.measured_traffic("llama8b", "bf16", 16, -1, "planned")
    m = bench.MEASURED_TRAFFIC[("llama8b", "bf16", 16, -1, "planned")]
    want = int(round(1024 * (m["fetch_kib"] * m["fetch_scale"] + m["write_kib"] * m["write_scale"])))
    same = bench.device_source_sha256() == m["source_sha256"]
    assert got == (want if same else None)
    # an edit of the code of any device source voids the recorded figure; an
    # added comment or blank line does not (the compiled kernels are the same)
    sources = list(bench.DEVICE_SOURCES)
    for k in range(len(sources)):
        paths = list(sources)
        text = open(paths[k], "rb").read()
        other = tmp_path / f"commented_{k}"
        other.write_bytes(text + b"\n// a note\n\n/* another */\n")
        paths[k] = str(other)
        monkeypatch.setattr(bench, "DEVICE_SOURCES", paths)
        assert bench.measured_traffic("llama8b", "bf16", 16, -1, "planned") == got
        other = tmp_path / f"edited_{k}"
        other.write_bytes(text + b"\nstatic int pkv_edit_marker;\n")
        paths[k] = str(other)
        monkeypatch.setattr(bench, "DEVICE_SOURCES", paths)
        assert bench.measured_traffic("llama8b", "bf16", 16, -1, "planned") is None
    assert bench.measured_traffic("small", "bf16", 16, -1, "fused") is None       # never measured
    assert bench.measured_traffic("beam", "bf16", 8, -1, "planned") is None       # never measured


def test_code_only_keeps_literals_and_drops_comments():
    src = 'int a = 1; // x\n/* y\n z */ const char* s = "//not a comment";\n\n  char c = \'"\';  \n'
    assert bench._code_only(src) == 'int a = 1;\n const char* s = "//not a comment";\n  char c = \'"\';'
