"""Host-only checks of the benchmark's bookkeeping (no GPU).

* ``kept_flops`` (the numerator of the roofline fraction: 4·d per kept
  (query, key) token pair, ragged tail blocks counting only their real rows
  and columns) against a brute-force count over the token-level mask that a
  block CSR expands to;
* ``bench.py --gpus N`` with N > 1 exits with a message and status 2 before
  touching a GPU (one GPU is measured; the path shards by head).
"""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _random_csr(rng, G, nq, nk, density):
    rows, cols = [0], []
    for _ in range(G * nq):
        keep = np.flatnonzero(rng.random(nk) < density)
        cols.extend(keep.tolist())
        rows.append(len(cols))
    return np.array(rows, np.int32), np.array(cols, np.int32)


def _brute(row_ptr, col_idx, G, N, Bq, Bk, d):
    nq = (N + Bq - 1) // Bq
    pairs = 0
    for g in range(G):
        m = np.zeros((N, N), bool)
        for i in range(nq):
            r = g * nq + i
            for j in col_idx[row_ptr[r]:row_ptr[r + 1]]:
                m[i * Bq:(i + 1) * Bq, j * Bk:(j + 1) * Bk] = True
        pairs += int(m.sum())
    return 4.0 * d * pairs


@pytest.mark.parametrize("N,Bq,Bk", [(1000, 128, 64), (1024, 64, 64), (777, 128, 128), (40, 64, 64)])
def test_kept_flops_counts_real_token_pairs(N, Bq, Bk):
    rng = np.random.Generator(np.random.PCG64(N + Bq + Bk))
    G, d = 3, 128
    nq, nk = (N + Bq - 1) // Bq, (N + Bk - 1) // Bk
    row_ptr, col_idx = _random_csr(rng, G, nq, nk, 0.4)
    assert bench.kept_flops(row_ptr, col_idx, G, N, Bq, Bk, d) == _brute(row_ptr, col_idx, G, N, Bq, Bk, d)


def test_kept_flops_full_density_is_dense_attention():
    G, N, Bq, Bk, d = 2, 700, 128, 64, 64
    nq, nk = (N + Bq - 1) // Bq, (N + Bk - 1) // Bk
    row_ptr = np.arange(G * nq + 1, dtype=np.int32) * nk
    col_idx = np.tile(np.arange(nk, dtype=np.int32), G * nq)
    assert bench.kept_flops(row_ptr, col_idx, G, N, Bq, Bk, d) == 4.0 * d * N * N * G


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout
