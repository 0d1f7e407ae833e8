"""The compression figures bench.py reports, against the oracle's definition
(CPU).

bench.py computes the storage ratios of the Master-Mirror record with its own
code; the oracle's ``compression`` is pinned to the notes' printed table and
to its closed form (test_oracle.py).  Both must agree on the same diff-block
counts, for every ratio bench.py prints.
"""

import numpy as np
import pytest

import bench
import oracle as O


@pytest.mark.parametrize("seed,N,L,T,H,D,eb,master", [
    (0, 3, 1, 192, 2, 64, 4, 1),        # the tiny round's shape, fp32
    (1, 10, 28, 3200, 4, 128, 2, 7),    # 7B-shaped round
    (2, 10, 48, 4912, 8, 128, 2, 0),    # 14B-shaped round
    (3, 64, 28, 5536, 4, 128, 2, 63),   # 64 agents
])
def test_bench_compression_equals_oracle(seed, N, L, T, H, D, eb, master):
    rng = np.random.default_rng(seed)
    nb = T // 16
    counts = rng.integers(0, nb + 1, size=(N, L))
    counts[master] = 0
    priv_len = rng.integers(0, 4096, size=N)
    got = bench.compression(counts, master, T, H, D, eb, priv_len, L)
    ref = O.compression(counts, master, T, H, D, eb, priv_len=priv_len)
    assert got["per_mirror_ratio_mean"] == pytest.approx(ref["per_mirror_ratio_mean"], rel=1e-12)
    assert got["group_ratio"] == pytest.approx(ref["group_ratio"], rel=1e-12)
    assert got["footprint_with_private_ratio"] == pytest.approx(ref["footprint_ratio"], rel=1e-12)
    assert got["dense_shared_GB"] * 1e9 == pytest.approx(ref["dense_shared_bytes"], rel=1e-12)
    assert got["master_plus_diff_GB"] * 1e9 == pytest.approx(ref["stored_shared_bytes"], rel=1e-12)
    assert got["dense_total_GB"] * 1e9 == pytest.approx(ref["dense_total_bytes"], rel=1e-12)
    assert got["stored_total_GB"] * 1e9 == pytest.approx(ref["stored_total_bytes"], rel=1e-12)


def test_bench_compression_without_diffs_is_one_copy():
    # every Mirror equal to the Master: the record holds only row offsets, and
    # the group stores one cache (plus 4 bytes per row)
    N, L, T, H, D, eb = 4, 3, 64, 2, 64, 2
    counts = np.zeros((N, L), dtype=np.int64)
    got = bench.compression(counts, 0, T, H, D, eb, np.zeros(N, dtype=np.int64), L)
    dense_one = L * T * H * D * 2 * eb
    assert got["master_plus_diff_GB"] * 1e9 == dense_one + (N - 1) * L * 4
    assert got["group_ratio"] == pytest.approx(N * dense_one / (dense_one + (N - 1) * L * 4))
