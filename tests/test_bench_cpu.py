"""Host logic of bench.py (no GPU): the algorithmic byte and flop counts the roofline fractions divide by, the
refusal of more than one GPU, and the rule that a recorded HBM-traffic figure is used only for the kernel
source and workload it was measured on."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_quantize_bytes_per_element():
    L = object.__new__(bench.Linear)
    L.M, L.N, L.K = 256, 384, 512
    b = L.quant_bytes()
    # 1x128 or 128x1: 2 bytes in, 1 code out, one fp32 scale per 128 elements
    assert b["x_rows"] == 256 * 512 * 3.03125 and b["dy_cols_t"] == 256 * 384 * 3.03125
    # both groupings from one read: 2 in, 2 codes out, two scales per 128
    assert b["x_dual"] == 256 * 512 * 4.0625 and b["dy_dual"] == 256 * 384 * 4.0625
    # weight blocks with the transposed copy: 2 in, 2 codes out, one scale per 128x128 block
    assert abs(b["w_blocks_T"] - 384 * 512 * 4.0) == 384 * 512 * 4 / 16384
    # requantization of saved codes: 1 in, 1 out, two scales per 128
    assert b["x_requant_t"] == 256 * 512 * 2.0625


def test_decode_gemm_bytes():
    M, N, K = 32, 6144, 4096
    expect = N * K + (N // 128) * (K // 128) * 4 + M * K + (K // 128) * M * 4 + 2 * M * N
    assert bench.decode_gemm_bytes(M, N, K) == expect
    # the weight stream dominates at decode sizes
    assert N * K / expect > 0.97


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_recorded_traffic_needs_matching_source_and_workload(tmp_path):
    good = {"workload": "llama3_8b_train_m16384", "kernel_source_sha256": bench.source_digest(),
            "gemm_bytes_per_launch": 123}
    p = tmp_path / "t.json"
    p.write_text(json.dumps(good))
    assert bench.recorded_traffic(str(p), "llama3_8b_train_m16384") == 123
    assert bench.recorded_traffic(str(p), "llama3_8b_prefill_m16384") is None
    p.write_text(json.dumps(dict(good, kernel_source_sha256="0" * 64)))
    assert bench.recorded_traffic(str(p), "llama3_8b_train_m16384") is None
    assert bench.recorded_traffic(str(tmp_path / "missing.json"), "llama3_8b_train_m16384") is None


def test_source_digest_ignores_comments_only(tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("// header\nint f(int x) {\n    return x + 1;  // one more\n}\n")
    b.write_text("/* another\n   header */\n\nint f(int x) {\n    return x + 1;\n}\n// trailer\n")
    c.write_text("int f(int x) {\n    return x + 2;\n}\n")
    assert bench.source_digest([str(a)]) == bench.source_digest([str(b)])
    assert bench.source_digest([str(a)]) != bench.source_digest([str(c)])
