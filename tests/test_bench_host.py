"""Host checks of bench.py: the one-GPU contract and the algorithmic counts the
roofline figures divide by (no GPU needed)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from vision_transformer_attention_amd.workloads import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_counts_of_the_headline_and_swin():
    # DeiT-S iRPE-K: 64 x 6 units of 197 tokens (196 positioned), d 64, one
    # contextual term over 81 table rows: 4 T^2 d per unit for QK^T and PV plus
    # 2 n K d for the bucket scores; Q, K, V read and O written once, bf16.
    flop, nbytes = bench.flops_bytes(WORKLOADS["deit_s_irpe_k"])
    assert flop == 384 * (4 * 197 * 197 * 64 + 2 * 196 * 81 * 64) == 4_595_417_088
    assert nbytes == 4 * 64 * 6 * 197 * 64 * 2 == 38_731_776
    # Swin-T W7: 32 images x 3 heads x 64 windows of 49 tokens, d 32, bias only
    flop, nbytes = bench.flops_bytes(WORKLOADS["swin_t_w7"])
    assert flop == 32 * 3 * 64 * 4 * 49 * 49 * 32
    assert nbytes == 4 * 32 * 3 * 3136 * 32 * 2


def test_counts_of_the_wide_grid():
    # DETR-like 50 x 84 grid: 2 x 8 units of 4200 tokens, d 32, key term over 81 rows
    flop, nbytes = bench.flops_bytes(WORKLOADS["detr_wide_irpe_k"])
    assert flop == 16 * (4 * 4200 * 4200 * 32 + 2 * 4200 * 81 * 32)
    assert nbytes == 4 * 16 * 4200 * 32 * 2
