"""Host logic of bench.py, on the CPU: the per-step roofline against a hand-worked case, the
HBM-traffic record that is reported only for the attention source it was measured on, and the
refusal of more than one GPU."""
import os
import shutil
import subprocess
import sys

import pytest

import bench
from synth import RLTConfig

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_step_roofline_hand_worked_case():
    # d = 64, one block, FFN 256, W = 4, one memory group, bf16, one sequence, one token.
    cfg = RLTConfig("hand", 64, 2, 32, 1, 256, 4, 1, 1.0, 1, 1, "bf16", 0.02)
    # weights per step: gate 2 d^2 = 8192, block 6 d^2 + 3 d F = 24576 + 49152 -> 81920 elements
    # bytes of token 1: 2 (81920 + window 1 x 2d + prefix 1 x 2d) + d (2 + 8) = 164992
    # flops of token 1: 2 x 81920 + 4 d (1 + 1) = 164352 -> bandwidth-bound at 8 TB/s
    # memory projection: 2 (d + 2d + 2 d^2) = 16768 bytes, 2 x 2 d^2 = 16384 flops
    want = 164992 / 8e12 + 16768 / 8e12
    assert bench.step_roofline_seconds(cfg, 1, 1) == pytest.approx(want, rel=1e-12)
    # one block: the shared prefix is read once per step either way
    assert bench.step_roofline_seconds(cfg, 1, 1, memory_once=True) == pytest.approx(want,
                                                                                    rel=1e-12)


def test_step_roofline_counts_every_layer_prefix_unless_memory_once():
    cfg = RLTConfig("deep", 64, 2, 32, 4, 256, 4, 1, 1.0, 2, 16, "bf16", 0.02)
    full = bench.step_roofline_seconds(cfg, 2, 16)
    once = bench.step_roofline_seconds(cfg, 2, 16, memory_once=True)
    assert once < full
    # the difference is (L - 1) prefix reads per token, all bandwidth-bound here
    d, L, es, B = 64, 4, 2, 2
    extra = sum(es * B * (L - 1) * t * 2 * d for t in range(1, 17)) / 8e12
    assert full - once == pytest.approx(extra, rel=1e-9)


def _copy_tree(dst):
    for sub in ("profiles", os.path.join("stateful_decoding_amd", "csrc")):
        shutil.copytree(os.path.join(ROOT, sub), os.path.join(dst, sub))


def test_traffic_record_only_for_the_measured_source(tmp_path, monkeypatch):
    rec = bench.traffic_record("s140m_bf16")
    assert isinstance(rec, int) and rec > 0
    assert bench.traffic_record("s50m_bf16") is None  # no record for another workload
    _copy_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_record("s140m_bf16") == rec  # same sources: same record
    for name in ("attention.hip", "internal.h", "common.h"):
        path = tmp_path / "stateful_decoding_amd" / "csrc" / name
        original = path.read_bytes()
        path.write_bytes(original + b"\n")  # any change to a hashed source
        assert bench.traffic_record("s140m_bf16") is None, name
        path.write_bytes(original)
    assert bench.traffic_record("s140m_bf16") == rec


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
