"""Host-side pieces of bench.py, checked on the CPU: the algorithmic byte and
flop counts it reports (against closed forms and the oracle's own masks), the
steps-per-graph choice, and the refusal of more than one GPU."""
import subprocess
import sys
from pathlib import Path

import numpy as np
import pytest

import bench
import oracle

ROOT = Path(__file__).resolve().parents[1]


def test_step_bytes_of_the_qwen_decode_step():
    # W 151936 x 2048 bf16 = 622.33 MB; prefix + block K/V 2 x 2 x 1296 x 128
    # x 2 = 1.33 MB; q, out, h 0.066 MB each; 623.85 MB in all.
    inp = dict(B=16, P=1280, Hq=16, Hkv=2, dh=128, d=2048, V=151936, dtype="bf16")
    b_lm, b_step = bench.step_bytes(inp)
    assert b_lm == 151936 * 2048 * 2 + 16 * 2048 * 2 + 16 * 8
    assert abs(b_step / 1e6 - 623.85) < 0.01
    inp8 = dict(inp, dtype="fp8")
    b_lm8, _ = bench.step_bytes(inp8)
    assert b_lm8 == 151936 * 2048 + 4 * 151936 + 16 * 2048 * 2 + 16 * 8


@pytest.mark.parametrize("n_vis,n_txt,block", [(4, 4, 2), (0, 5, 2), (3, 7, 3), (5, 9, 4),
                                               (2, 6, 6), (1, 1, 1)])
def test_dualstream_pairs_counts_the_oracle_mask(n_vis, n_txt, block):
    assert bench.dualstream_pairs(n_vis, n_txt, block) == \
        int(oracle.dualstream_mask(n_vis, n_txt, block).sum())


def test_dualstream_pairs_of_the_training_config():
    # 1024 visual + 2048 clean + 2048 noisy tokens, block 32: 8,980,992
    # visible pairs per head, i.e. 73.57 GFLOP over 16 heads of 128.
    n = bench.dualstream_pairs(1024, 2048, 32)
    assert n == 8_980_992
    assert abs(n * 16 * 4 * 128 / 1e9 - 73.57) < 0.01


def test_headline_steps_per_graph():
    # long runs keep 25 steps per replay; short ones time at least 4 replays
    assert bench.headline_steps_per_graph(500, 25) == 25
    assert bench.headline_steps_per_graph(20, 25) == 5
    assert bench.headline_steps_per_graph(24, 25) == 6
    assert bench.headline_steps_per_graph(3, 25) == 1
    for K in range(1, 300):
        S = bench.headline_steps_per_graph(K, 25)
        assert K % S == 0 and 1 <= S <= 25 and (S == 1 or K // S >= 4)


def test_graph_divisor():
    assert bench.graph_divisor(500, 25) == 25
    assert bench.graph_divisor(20, 25) == 20
    assert bench.graph_divisor(24, 25) == 24
    assert bench.graph_divisor(97, 25) == 1
    assert bench.graph_divisor(60, 25) == 20
    for K in range(1, 200):
        s = bench.graph_divisor(K, 25)
        assert K % s == 0 and 1 <= s <= 25
        assert all(K % t for t in range(s + 1, min(25, K) + 1))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)
    assert not r.stdout.strip().startswith("{")
