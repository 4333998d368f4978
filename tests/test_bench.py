"""bench.py's host-side contract (CPU only): the algorithmic byte and flop counts
its roofline divides by, checked against sizes worked out by hand for the
workloads, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("c,d,s,expected", [
    (410, 128, 2, 216_632),   # 32-layer OPT-6.7B stack, k = 205 + 205
    (104, 128, 2, 56_288),    # one OPT-6.7B layer, batch 16, k = 52 + 52
    (42, 128, 2, 23_800),     # OPT-30B, 4 % budget
    (2048, 128, 2, 1_074_944),  # 2048-slot cache (stream, 100 % budget)
    (52, 64, 4, 28_784),      # tiny fp32 workload
])
def test_decode_bytes_per_unit(c, d, s, expected):
    # K and V slots 2cds, score read + write 8c, positions 4c, new q/k/v 3ds,
    # new K/V slot write 2ds, fp32 output 4d
    assert bench.decode_bytes_per_unit(c, d, s) == expected


def test_decode_bytes_fixed_scores():
    # fixed scores are only read (4c instead of 8c) plus the new token's score (4 B)
    c, d, s = 410, 128, 2
    assert bench.decode_bytes_per_unit(c, d, s, fixed=True) == bench.decode_bytes_per_unit(c, d, s) - 4 * c + 4


def test_prefill_flops_per_unit():
    # two causal QK^T passes over the L(L+1)/2 pairs, 2d flops per pair each
    L, d = 2048, 128
    assert bench.prefill_flops_per_unit(L, d) == 2 * (2 * d) * (L * (L + 1) // 2)
    # the prompt's own output adds a PV product over the same pairs
    assert bench.prefill_flops_per_unit(L, d, with_out=True) == 3 * (2 * d) * (L * (L + 1) // 2)
    # the 32-layer stack: 65,536 units of 2048 tokens, 70.4 TFLOP per prefill
    assert abs(65_536 * bench.prefill_flops_per_unit(L, d) / 1e12 - 70.40) < 0.01


def test_prefill_bytes_per_unit():
    L, k, d, s = 2048, 410, 128, 2
    assert bench.prefill_bytes_per_unit(L, k, d, s) == 2 * L * d * s + 3 * k * d * s + 12 * k
    # a prompt shorter than the budget keeps (and moves) every row
    assert bench.prefill_bytes_per_unit(100, k, d, s) == 2 * 100 * d * s + 3 * 100 * d * s + 12 * 100


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 1" in r.stderr
    assert r.stdout == ""
