"""bench.py host logic: the multi-GPU refusal, the algorithmic byte and FLOP
counts behind the two rooflines, and the committed counter summaries (CPU)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from chunk_gated_delta_carve_amd.workloads import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_headline_algorithmic_bytes():
    # per head-token: q, k, g, b_x (64 each), v and o (64 each), w (1), bf16;
    # plus the fp32 final state (64 x 64) and mean (64) of the 48 (batch, head) pairs
    per_tok = (4 * 64 + 64 + 64 + 1) * 2
    expect = 4 * 2048 * 12 * per_tok + 48 * 64 * 64 * 4 + 48 * 64 * 4
    assert bench.algorithmic_bytes(4, 2048, 12, 64, 64, 2) == expect == 76492800


def test_algorithmic_flops_counts_chunks_and_tail():
    # one chunk of L = 4 tokens, d_k = d_v = 2, no projection, counted term by term:
    # A and P 2 * 6 pairs * 2, inverse 4, W and U 10 * 4, 3 L d d = 48, P.Delta 6 * 2,
    # mean 4 * 2
    mac = 2 * 6 * 2 + 4 + 10 * 4 + 48 + 6 * 2 + 8
    assert bench.algorithmic_flops(1, 4, 1, 2, 2, 4) == 2 * mac
    # a ragged tail is a shorter chunk; batch and heads multiply
    assert bench.algorithmic_flops(3, 6, 5, 2, 2, 4) == 15 * (2 * mac + bench.algorithmic_flops(1, 2, 1, 2, 2, 2))
    # the headline shape: 4.56 GFLOP per call, far below the MFMA/HBM ridge
    f = bench.algorithmic_flops(4, 2048, 12, 64, 64, 64)
    assert 4.5e9 < f < 4.6e9
    intensity = f / bench.algorithmic_bytes(4, 2048, 12, 64, 64, 2)
    ridge = bench.MFMA_PEAK_TFLOPS["bf16"] * 1e12 / (bench.HBM_PEAK_GBS * 1e9)
    assert intensity < ridge / 4


@pytest.mark.parametrize("reader", ["measured_traffic", "measured_mfma"])
def test_committed_counter_summaries_match_the_sources(reader):
    """The committed rocprofv3 summaries of the headline shape are keyed to the
    current kernel sources (bench.py reports null figures otherwise)."""
    got = getattr(bench, reader)(WORKLOADS["init_equiv"])
    assert got is not None, f"{reader}: summary missing or taken from other kernel sources"
