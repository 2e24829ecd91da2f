"""Host-side checks of the benchmark contract and of the workload FLOP counts
(no GPU needed)."""
import os
import subprocess
import sys

import numpy as np
import pytest

from fa_inputs import (BENCH_WORKLOAD, FP8_WORKLOADS, GENERAL_WORKLOADS, MASK_CAUSAL, WORKLOADS,
                       Workload, packed_lengths)
from oracle import visible_general

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_bench_workload_is_registered():
    assert BENCH_WORKLOAD in WORKLOADS
    names = list(WORKLOADS) + list(FP8_WORKLOADS) + list(GENERAL_WORKLOADS)
    assert len(names) == len(set(names))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", [-1, 0, 7, 150])
def test_flop_count_is_four_d_per_visible_pair(causal, window):
    """The metric's count (4*B*H*N^2*d, halved when causal) and its windowed
    form equal 4*d per visible (query, key) pair, counted from the oracle's
    visibility rule."""
    N, d, B, H = 100, 64, 2, 3
    wl = Workload("t", B, H, N, d, "bf16", MASK_CAUSAL if causal else 0, seed=0,
                  window_left=window)
    pairs = int(visible_general(N, N, causal, window, N).sum())
    if window < 0 and causal:
        # The metric's own convention: N^2 / 2, not N (N + 1) / 2.
        assert wl.flops() == 4.0 * B * H * d * N * N / 2
    else:
        assert wl.flops() == 4.0 * B * H * d * pairs


def test_packed_flops_sum_the_sequences():
    wl = GENERAL_WORKLOADS["bf16_varlen_b16h32_n512_4096_d128_causal"]
    n = packed_lengths(wl)
    assert len(n) == wl.B and n.max() == wl.N and n.min() >= wl.len_range[0]
    want = sum(4.0 * wl.H * wl.d * k * (k + 1) / 2 for k in n.tolist())
    assert wl.flops() == want
    assert np.array_equal(packed_lengths(wl), n)      # seeded
