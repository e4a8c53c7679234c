"""The algorithmic work bench.py divides by (every roofline figure rests on
it), pinned on the CPU: the key-pair counts against the oracle's key sets by
brute force, against the closed forms of full windows, and at the workloads'
sizes against the totals derived independently from the closed forms."""
import numpy as np
import pytest

import bench
import oracle.swa_oracle as so


@pytest.mark.parametrize("N,W,start,S", [(50, 20, 0, 0), (50, 20, 30, 3), (7, 1, 5, 0), (64, 100, 10, 2),
                                         (40, 8, 2, 4)])
def test_band_pairs_brute_force(N, W, start, S):
    q = np.arange(start, start + N)
    k = np.arange(0, start + N)
    assert bench.band_pairs(N, W, start, S) == int(so.key_mask(q, k, W, S).sum())


def test_band_pairs_closed_forms():
    # queries past the first W positions each see exactly W keys (plus the sinks)
    assert bench.band_pairs(4096, 4096, start=8192) == 4096 * 4096
    assert bench.band_pairs(4096, 4092, start=5000, n_sink=4) == 4096 * 4096
    # W >= N: plain causal attention, N (N + 1) / 2 pairs
    assert bench.band_pairs(16384, 16384) == 16384 * 16385 // 2
    # a window of 1: every query sees itself only
    assert bench.band_pairs(1000, 1, start=17) == 1000


def test_workload_totals():
    W = 4096
    # 8192 tokens from position 0: the first W queries see i + 1 keys, the rest W
    n8192 = W * (W + 1) // 2 + (8192 - W) * W
    assert bench.band_pairs(8192, W) == n8192 == 25_167_872
    assert bench.attn_flops(n8192) == 412_350_414_848
    # 16384 tokens (chunked or not, the key sets are the same)
    n16k = W * (W + 1) // 2 + (16384 - W) * W
    assert bench.band_pairs(16384, W) == n16k == 58_722_304
    assert sum(bench.band_pairs(4096, W, start=4096 * c) for c in range(4)) == n16k
    assert bench.attn_flops(bench.band_pairs(16384, 16384)) == 4 * 128 * 32 * 134_225_920
