"""Host logic of bench.py (CPU only): the one-GPU contract, the algorithmic byte
counts the roofline divides by, and when the stored HBM traffic figure is used."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from block_diffusion_draft_proj_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_at_the_batched_workload():
    cfg = synth.CONFIGS["batched"]
    B, L, Hq, Hkv, d, V = 8, 8192, 32, 8, 128, 151936
    # attention: ctx K and V (bf16), block q, k, v (bf16), output (fp32), lengths
    attn = 2 * 2 * B * Hkv * L * d + 2 * B * 16 * Hq * d + 2 * 2 * B * 16 * Hkv * d + 4 * B * 16 * Hq * d + 4 * B
    assert bench.attn_bytes(cfg, np.full(B, L, np.int32)) == attn == 272_105_504
    # verify: logits, block tokens / posterior / commit positions, four per-sequence words
    assert bench.verify_bytes(cfg, B) == 2 * B * 16 * V + 4 * B * 16 * 3 + 4 * B * 4 == 38_897_280
    # draft tokens: the 15 mask rows of logits, staged tokens in, the block out
    assert bench.draft_bytes(cfg, B) == 2 * B * 15 * V + 4 * B + 4 * B * 16 == 36_465_184
    # block q/k/v: the fused weight, the hidden states, the three outputs
    n_out = (Hq + 2 * Hkv) * d
    assert bench.qkv_bytes(cfg, B) == 2 * (n_out * 4096 + 16 * B * 4096 + 16 * B * n_out) == 52_953_088


def test_sliding_window_bytes_at_the_batched_workload():
    # the window is half the longest context, in whole pages; only the last W positions
    # of each context are read
    cfg = synth.CONFIGS["batched"]
    B, Hq, Hkv, d = 8, 32, 8, 128
    W = bench.window_size(cfg, 8192)
    assert W == 4096 and bench.window_size(cfg, 40) == 16 and bench.window_size(cfg, 100) == 48
    win = 2 * 2 * B * Hkv * W * d + 2 * B * 16 * Hq * d + 2 * 2 * B * 16 * Hkv * d + 4 * B * 16 * Hq * d + 4 * B
    assert bench.attn_bytes(cfg, np.minimum(np.full(B, 8192, np.int32), W)) == win == 137_887_776


def test_traffic_figure_only_for_its_workload_and_sources():
    t = bench.ATTN_TRAFFIC
    assert bench.measured_traffic("ragged") is None
    saved = t["sha256"]
    try:
        t["sha256"] = "0" * 64                     # sources changed since the counters were taken
        assert bench.measured_traffic(t["workload"]) is None
    finally:
        t["sha256"] = saved
    if saved == bench.sources_sha256(bench.ATTN_TRAFFIC_SOURCES):
        assert bench.measured_traffic(t["workload"]) == t["read"] + t["write"]
