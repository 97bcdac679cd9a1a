"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic byte and FLOP counts
behind the roofline figure, and the validity rule of the committed HBM counter figures."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_decode_gate_up_algorithmic_bytes():
    # every routed expert selected at T = 128: 257 experts' W_g and W_u (2048 x 7168 bf16 each),
    # the 128 token rows once, and 128 x 9 rows of h written once
    cfg = W.config("decode_bf16")
    w = bench._work(cfg, np.full(256, 4))
    expected = 257 * 2 * 2048 * 7168 * 2 + 128 * 7168 * 2 + 128 * 9 * 2048 * 2
    assert w["gemm1_bytes"] == expected == 15_097_659_392
    assert w["gemm1_flops"] == 2 * 2 * 7168 * 2048 * 128 * 9
    assert w["n_selected"] == 256


def test_unselected_experts_are_not_counted():
    cfg = W.config("decode_bf16")
    counts = np.zeros(256, dtype=np.int64)
    counts[:100] = 1
    w = bench._work(cfg, counts)
    assert w["n_selected"] == 100
    assert w["gemm1_bytes"] == 101 * 2 * 2048 * 7168 * 2 + 128 * 7168 * 2 + 128 * 9 * 2048 * 2


def test_fp8_bytes_count_codes_and_block_scales():
    cfg = W.config("fp8")
    w = bench._work(cfg, np.full(256, 1))
    scales = 2 * (2048 // 128) * (7168 // 128) * 4      # W_g and W_u block scales of one expert
    T = cfg.T
    # h leaves the gate/up GEMM as E4M3 codes with one fp32 scale per 1x128 tile
    assert w["gemm1_bytes"] == 257 * (2 * 2048 * 7168 + scales) + T * 7168 + T * 9 * 2048 * (1 + 4 / 128)


def test_comment_edits_keep_the_source_hash():
    src = "int a; // note\n/* block\n comment */ int b;\n\n"
    assert bench._code_only(src) == bench._code_only("int a;\n int b;")
    assert bench._code_only(src) != bench._code_only("int a; int c;")


def test_counter_figures_are_dropped_when_the_kernels_change(monkeypatch, tmp_path):
    rec = {"decode_bf16": {"ffn1": {"source_hash": "abc", "hbm_bytes_per_launch": 1.5e10}}}
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    monkeypatch.setattr(bench, "_kernel_source_hash", lambda: "abc")
    assert bench._traffic("decode_bf16", "ffn1") == 1.5e10
    assert bench._traffic("prefill_bf16", "ffn1") is None
    monkeypatch.setattr(bench, "_kernel_source_hash", lambda: "def")
    assert bench._traffic("decode_bf16", "ffn1") is None


def test_committed_counter_figures_agree_with_the_algorithmic_bytes():
    t = bench._traffic("decode_bf16", "ffn1")
    if t is None:
        pytest.skip("the kernel sources changed since the counters were taken (the bench reports null)")
    # the gate/up GEMM reads each selected weight byte once: traffic within 2 % of the algorithmic bytes
    assert t == pytest.approx(15_097_659_392, rel=0.02)


def test_binding_roof_takes_the_larger_floor():
    # 2.5 TFLOP at the bf16 peak is 1 ms; 4 GB at 8 TB/s is 0.5 ms: MFMA binds, 2 ms reaches half
    r = bench.binding_roof(2.5e12, 4e9, 2.0)
    assert r["binding_roof"] == "mfma" and abs(r["roof_ms"] - 1.0) < 1e-12
    assert abs(r["frac_of_binding_roof"] - 0.5) < 1e-12
    # the same flops in FP8 take 0.5 ms; 16 GB take 2 ms at 8 TB/s: HBM binds, 4 ms reaches half
    r = bench.binding_roof(2.5e12, 16e9, 4.0, "fp8")
    assert r["binding_roof"] == "hbm" and abs(r["roof_ms"] - 2.0) < 1e-12
    assert abs(r["frac_of_binding_roof"] - 0.5) < 1e-12
