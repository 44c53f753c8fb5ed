"""Host logic of bench.py (no GPU): the one-GPU rule, the algorithmic bytes and flops
of a call, and the rule that counter-measured traffic is reported only for the exact
kernel sources it was measured on."""
import json
import os
import subprocess
import sys

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, env=env, timeout=120)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run_bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    r = _run_bench(["--gpus", "1"], {"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_algorithmic_work_of_the_ling_lite_call():
    """bytes = D*3*I*H*b_w + 3*I_s*H*b_s + E*H*b_r + T*H*(b_x + b_y) and flops =
    2TEH + 6TkHI + 6THI_s, written out for the Ling-lite shape (bf16, no expert
    bias) with 50 of its 64 experts selected."""
    spec = synth.SPECS[2]
    T = 4096
    counts = np.zeros(64, dtype=np.int64)
    counts[:50] = 1
    w = bench.algorithmic(spec, T, counts)
    assert w["D"] == 50
    expect_bytes = 50 * 3 * 1408 * 2048 * 2 + 3 * 2816 * 2048 * 2 + 64 * 2048 * 2 + 4096 * 2048 * (2 + 2)
    expect_flops = 2 * 4096 * 64 * 2048 + 6 * 4096 * 6 * 2048 * 1408 + 6 * 4096 * 2048 * 2816
    assert w["bytes"] == expect_bytes
    assert w["flops"] == expect_flops
    assert w["up_flops"] == 4 * 4096 * 6 * 2048 * 1408


def test_algorithmic_work_of_quantised_and_biased_layers():
    """u8 and u4 experts store one fp16 scale and one fp16 zero point per 64 codes;
    the selection-only expert bias is E fp32 values."""
    T = 64
    counts = np.ones(512, dtype=np.int64)
    counts[100:] = 0
    for cid, code_bytes in ((5, 1.0), (6, 0.5)):
        spec = synth.SPECS[cid]
        assert spec.use_expert_bias and spec.quant_group == 64
        w = bench.algorithmic(spec, T, counts)
        per_expert = 3 * 1024 * 4096 * (code_bytes + 4 / 64)
        expect = (100 * per_expert + 3 * 1024 * 4096 * 2 + 512 * 4096 * 2 + 64 * 4096 * 4 + 4 * 512)
        assert w["D"] == 100
        assert abs(w["bytes"] - expect) < 1e-6 * expect


def test_recorded_traffic_only_for_matching_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"source_digest": "abc123",
                             "kernels": {"up_tiled_cfg2_T4096": {"hbm_bytes_per_launch": 1.5e9}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.recorded_traffic("up_tiled_cfg2_T4096", "abc123") == 1.5e9
    assert bench.recorded_traffic("up_tiled_cfg2_T4096", "def456") is None
    assert bench.recorded_traffic("up_stream_cfg2_T1", "abc123") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.recorded_traffic("up_tiled_cfg2_T4096", "abc123") is None


def test_source_digest_tracks_the_kernel_sources():
    d = bench.source_digest()
    assert len(d) == 16 and int(d, 16) >= 0
    assert bench.source_digest() == d
