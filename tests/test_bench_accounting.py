"""Host-side accounting of bench.py, checked on the CPU.

The algorithmic work that the reported rates divide by must match the
method's definitions: pairs by brute force over the causal + window mask, the
decode's K/V bytes by the visible rows, and the combine's bytes by the valid
splits of the oracle's split rule (FlashMLA patch stack page, section 3).
"""
import numpy as np
import pytest

import bench
import oracle


@pytest.mark.parametrize("L,W", [(1, 0), (7, 0), (64, 0), (100, 1), (100, 33), (100, 99),
                                 (100, 100), (100, 513), (1000, 513)])
def test_pairs_window_brute_force(L, W):
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    vis = (j <= i) & ((W <= 0) | (j > i - W))
    assert bench.pairs_window(L, W) == int(vis.sum())


@pytest.mark.parametrize("window", [0, 513, 5000])
def test_decode_and_combine_bytes_follow_the_split_rule(window):
    rng = np.random.default_rng(window + 1)
    B, Hq, Hkv, D = 23, 16, 4, 128
    seqlens = rng.integers(0, 40000, size=B)
    seqlens[:3] = [0, 1, 65]
    nsplits = rng.integers(1, 65, size=B)
    valid = sum(len(oracle.split_ranges(int(n), int(s), window)) for n, s in zip(seqlens, nsplits))
    want_comb = valid * Hq * (D + 1) * 4 + B * Hq * D * 2 + B * Hq * 4
    assert bench.combine_bytes(seqlens, nsplits, Hq, D, window) == want_comb
    rows = sum(min(int(n), window) if window > 0 else int(n) for n in seqlens)
    want_dec = rows * Hkv * D * 2 * 2 + 2 * B * Hq * D * 2 + B * Hq * 4 + Hq * 4
    assert bench.decode_bytes(seqlens, Hq, Hkv, D, window) == want_dec


def test_bench_refuses_more_than_one_gpu():
    # One process per GPU is the only mode: --gpus above 1 ends with an error
    # line before anything touches a device.
    import json
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    line = json.loads(res.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["n_gpus"] == 2
