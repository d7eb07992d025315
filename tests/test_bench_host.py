"""Host-side checks of the benchmark's accounting (no GPU): the algorithmic
bytes and flops its roofline figures divide by, and its one-GPU contract."""

import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("causal", [True, False])
def test_algorithmic_work_counts_the_visible_pairs(causal):
    """The flop count is 2176 per visible (query-head, key) pair, where the
    oracle's masking decides visibility; rows with no key and rows with more
    queries than keys included."""
    rng = np.random.default_rng(3)
    w = W.make_workload("accounting", 0, [0, 5, 37, 100, 64], [1, 3, 7, 120, 64], 16, 16,
                        causal=causal, rng=rng)
    nbytes, flops = bench.algorithmic(w)
    lens = oracle.kv_lengths(w.kv_indptr, w.kv_last_page_len, w.page_size)
    pairs = sum(oracle.visible_keys(i, int(q), int(n), causal)
                for q, n in zip(w.qo_lens(), lens) for i in range(int(q)))
    assert flops == 2176 * w.num_heads * pairs
    # latent rows once, query in, output and LSE out, the four index arrays
    T, H, B = w.num_tokens, w.num_heads, w.batch
    index_bytes = 4 * (len(w.qo_indptr) + len(w.kv_indptr) + len(w.kv_last_page_len)
                       + int(w.kv_indptr[-1]))
    assert nbytes == 1152 * int(lens.sum()) + T * H * 2 * (576 + 512) + 4 * T * H + index_bytes


def test_decode_batch_accounting():
    """The decode batch (64 rows, 128 heads, page 64, seed 1002): 141,622
    keys, 181.0 MB and 39.4 GFLOP per step; HBM-bound at the published
    peaks."""
    w = W.decode_batch()
    assert int(w.kv_lens().sum()) == 141_622
    nbytes, flops = bench.algorithmic(w)
    assert (nbytes, flops) == (181_016_868, 39_445_692_416)
    e = bench.roofline_entry(w, 0.0741, nbytes, flops)
    assert e["bound"] == "hbm" and abs(e["frac"] - nbytes / 0.0741e-3 / 8e12) < 1e-4


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
