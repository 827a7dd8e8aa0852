"""Host-side checks of bench.py (no GPU): the one-GPU rule and the roofline arithmetic
behind its headline fraction."""
import os
import subprocess
import sys

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_headline_bytes_per_cycle():
    """Qwen3-8B-shaped drafter, batch 1, context 4096: every weight once (W_fuse 4096 x 20480,
    W_k | W_v and W_q | W_o of 5 layers, 3 MLP matrices of 12288 x 4096 per layer, the
    151936 x 4096 LM head), 5 layers of 8 kv heads x 4096 keys x 128 for K and V, bf16."""
    cfg = synth.get_config("C3")
    parts, total = bench.algorithmic_bytes(cfg, 1, 4096.0, 0.0)
    mb = {k: v / 1e6 for k, v in parts.items()}
    assert mb["w_fuse"] == pytest.approx(167.77, abs=0.01)
    assert mb["w_k_w_v"] == pytest.approx(83.89, abs=0.01)
    assert mb["w_q_w_o"] == pytest.approx(335.54, abs=0.01)
    assert mb["mlp"] == pytest.approx(1509.95, abs=0.01)
    assert mb["lm_head"] == pytest.approx(1244.66, abs=0.01)
    assert mb["ctx_kv"] == pytest.approx(83.89, abs=0.01)
    # with the planted mean accept length the bench uses: 3.426 GB, 2335 cycles/s at 8 TB/s
    _, total = bench.algorithmic_bytes(cfg, 1, 4096.0, 5.52)
    assert total / 1e9 == pytest.approx(3.426, abs=0.001)
    assert bench.HBM_PEAK_GBS * 1e9 / total == pytest.approx(2335, abs=1)


def test_batch32_gemm_flops():
    """LLaMA-3.1-8B shape, batch 32, gamma 16: the LM head alone is 2 x 512 x 128256 x 4096."""
    cfg = synth.get_config("C4").with_(batch=32)
    f = bench.gemm_flops(cfg, 32, 16, 0.0)
    H, L = cfg.hidden, cfg.n_layers
    lm = 2 * 512 * cfg.vocab * H
    blk = 2 * 512 * L * ((32 + 16) * 128 * H + 32 * 128 * H + 3 * cfg.inter * H)
    assert f == pytest.approx(lm + blk, rel=1e-12)
    assert lm / 1e9 == pytest.approx(538.0, abs=0.1)
