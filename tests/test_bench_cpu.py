"""bench.py's host logic without a GPU: the one-GPU guard, the algorithmic work it divides by, and the
staleness rule for committed HBM-traffic summaries."""

import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_touching_a_device():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def closed_form(cfg, n_act, es=2):
    """B_alg and F_alg of one layer: every active expert's three matrices, the shared expert's, the
    router, x read once and the output written once; flops 2 T d E + 6 (T k) d H + 6 T d Hs (the gated
    MLP's 6 rows d H form)."""
    T, d, E, k, H, Hs = cfg.T, cfg.d, cfg.E, cfg.k, cfg.H, cfg.Hs
    b = es * (n_act * 3 * d * H + 3 * d * Hs + E * d) + es * T * d + es * T * d
    f = 2 * T * d * E + 6 * T * k * d * H + 6 * T * d * Hs
    return b, f


@pytest.mark.parametrize("name,gb,tflop", [("dsv3_decode_t256", 22.65, 0.2039), ("dsv3_prefill_t8192", 22.88, 6.524)])
def test_layer_work_matches_the_closed_forms_with_every_expert_active(name, gb, tflop):
    cfg = synth.CONFIG_BY_NAME[name]
    w = bench.alg_bytes_and_flops(cfg, [np.ones(cfg.E, dtype=np.int64)], 2)
    b, f = closed_form(cfg, cfg.E)
    assert w["layer"] == b and w["flops_layer"] == f
    assert w["flops_gate_up"] + w["flops_down"] == f - 2 * cfg.T * cfg.d * cfg.E   # the experts' share
    assert abs(b / 1e9 - gb) < 0.005 and abs(f / 1e12 - tflop) < 0.0005           # the rounded table values


def test_layer_bytes_count_only_the_active_experts_and_average_over_batches():
    cfg = synth.CONFIG_BY_NAME["dsv3_decode_t8"]
    c1 = np.zeros(cfg.E, dtype=np.int64)
    c1[:60] = 1
    c2 = np.zeros(cfg.E, dtype=np.int64)
    c2[100:157] = 1
    w = bench.alg_bytes_and_flops(cfg, [c1, c2], 2)
    assert w["n_act"] == 58.5
    assert w["layer"] == (closed_form(cfg, 60)[0] + closed_form(cfg, 57)[0]) / 2


def test_int8_weights_count_one_byte_per_weight_plus_row_scales():
    cfg = synth.CONFIG_BY_NAME["dsv3_decode_t8"]
    counts = np.ones(cfg.E, dtype=np.int64)
    w16 = bench.alg_bytes_and_flops(cfg, [counts], 2)
    w8 = bench.alg_bytes_and_flops(cfg, [counts], 2, one_byte=True)
    weights = cfg.E * 3 * cfg.d * cfg.H + 3 * cfg.d * cfg.Hs
    rows = cfg.E * (2 * cfg.H + cfg.d) + 2 * cfg.Hs + cfg.d     # one float scale per weight row
    assert w16["layer"] - w8["layer"] == weights - 4 * rows


def test_traffic_summary_is_ignored_once_its_sources_change(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    src = tmp_path / "k.hip"
    src.write_text("__global__ void k() {}\n")
    kernel = "ffn_down_stream<1, 2>"
    summary = {"kernel": kernel, "sources": ["k.hip"], "source_sha": bench.source_sha(["k.hip"]),
               "bytes_per_launch": 12345}
    path = bench.traffic_path("w", kernel)
    assert os.path.basename(path) == "traffic_ffn_down_stream_1_2_w.json"
    with open(path, "w") as f:
        json.dump(summary, f)
    assert bench.traffic_for("w", kernel) == 12345
    assert bench.traffic_for("w", kernel.replace("<1, 2>", "<2, 2>")) is None   # another kernel: no file
    src.write_text("__global__ void k() { /* changed */ }\n")
    assert bench.traffic_for("w", kernel) is None


def test_gelu_expert_stage_bytes():
    """W1 and W2 of every active expert (bf16) with their fp32 biases, x read once, the hidden rows
    written and read back, the expert rows written."""
    cfg = synth.CONFIG_BY_NAME["dsv3_decode_t256"]
    T, d, E, k, H = cfg.T, cfg.d, cfg.E, cfg.k, cfg.H
    counts = np.ones(E, dtype=np.int64)
    counts[:6] = 0
    want = (E - 6) * (2 * H * d * 2 + 4 * (H + d)) + 2 * T * d + 2 * (2 * T * k * H) + 2 * T * k * d
    assert bench.gelu_alg_bytes(cfg, [counts]) == want


def test_gelu_bench_refuses_int8_weights_before_touching_a_device():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--expert", "gelu", "--layout", "int8"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "--expert gelu" in r.stderr


@pytest.mark.parametrize("extra", [["--layout", "int8"], ["--workload", "tiny_fp32"], ["--ep-share", "3"]])
def test_ep_share_refuses_what_it_cannot_split_before_touching_a_device(extra):
    """The expert-parallel share needs bf16 weights of a SwiGLU layer and a degree that divides E."""
    args = ["--ep-share", "8"] + extra if extra[0] != "--ep-share" else extra
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "--ep-share" in r.stderr
