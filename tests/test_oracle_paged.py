"""Pins of the paged-layout oracle (CPU).

A paged call is the contiguous call on the sequences gathered out of their
pages.  Pinned here by: the identity page table reducing to a reshape of the
pool, scatter/gather round trips, permutation invariance of the whole
restore-attention against the contiguous oracle on the original arrays, the
paged deviation against the contiguous deviation at the check layer, the
content of every diff entry's page, untouched pages staying untouched, and
clamping of out-of-range page IDs.
"""

import numpy as np
import pytest

import oracle as O

P = O.paged


def _pool(rng, L, n_pages, H, D):
    return rng.standard_normal((L, n_pages, 16, H, D)).astype(np.float32)


def test_identity_table_is_a_reshape():
    rng = np.random.default_rng(0)
    pool = _pool(rng, 2, 5, 2, 8)
    seq = P.gather(pool, [0, 1, 2, 3, 4], 70)
    want = pool.reshape(2, 80, 2, 8)[:, :70]
    np.testing.assert_array_equal(seq, want)


def test_scatter_then_gather_round_trip_and_untouched_pages():
    rng = np.random.default_rng(1)
    pool = _pool(rng, 3, 9, 2, 8)
    before = pool.copy()
    seq = rng.standard_normal((3, 37, 2, 8)).astype(np.float32)
    row = [7, 2, 5]
    P.scatter(pool, row, seq)
    np.testing.assert_array_equal(P.gather(pool, row, 37), seq)
    for p in set(range(9)) - set(row):
        np.testing.assert_array_equal(pool[:, p], before[:, p])
    # the last page is partial: its rows past the sequence keep their values
    np.testing.assert_array_equal(pool[:, 5, 5:], before[:, 5, 5:])


def test_out_of_range_ids_are_clamped():
    rng = np.random.default_rng(2)
    pool = _pool(rng, 1, 4, 1, 8)
    np.testing.assert_array_equal(P.gather(pool, [-3, 99], 32),
                                  np.concatenate([pool[:, 0], pool[:, 3]], axis=1))


def test_deviation_paged_reads_each_agents_pages_at_the_check_layer():
    # three agents' reused K (two layers, 40 tokens: a partial last page) laid
    # into shuffled pages of one pool by plain indexing, one used entry out of
    # range (it clamps to the last page, which holds that page's rows); the
    # paged deviation equals the contiguous one on the original arrays at the
    # check layer.  A wrong layer, agent row, page or in-page row changes it.
    rng = np.random.default_rng(31)
    N, L, T, H, D = 3, 2, 40, 2, 8
    npg = 3
    n_pages = N * npg + 2
    kr = O.f64_to_bf16(rng.standard_normal((N, L, T, H, D)))
    kx = O.f64_to_bf16(rng.standard_normal((N, T, H, D)))
    pool = O.f64_to_bf16(rng.standard_normal((L, n_pages, 16, H, D)))
    perm = rng.permutation(n_pages - 1)  # page n_pages - 1 is placed by hand
    pages = np.full((N, npg + 1), -7, np.int64)  # the spare column is never read
    k = 0
    for i in range(N):
        for j in range(npg):
            pid = n_pages - 1 if (i, j) == (1, 2) else int(perm[k])
            k += (i, j) != (1, 2)
            pages[i, j] = n_pages + 5 if (i, j) == (1, 2) else pid
            n = min(16, T - 16 * j)
            pool[:, pid, :n] = kr[i, :, 16 * j:16 * j + n]
    for check in (0, 1):
        got = P.deviation_paged(pool, pages, check, kx, T)
        want = O.deviation(kr[:, check], kx)
        for g, w in zip(got, want):
            np.testing.assert_array_equal(g, w)
    # the other layer's deviation is a different answer (the pin can fail)
    assert not np.array_equal(P.deviation_paged(pool, pages, 0, kx, T)[0], O.deviation(kr[:, 1], kx)[0])


def _round(rng, N=3, L=2, H=2, D=8, lens=(16, 32, 16)):
    bs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(bs[-1])
    src = bs[:-1].copy()
    dst = np.stack([rng.permutation(len(lens)) * 50 + rng.integers(0, 40) for _ in range(N)]).astype(np.int32)
    return bs, src, dst, T


def test_rerotate_paged_equals_contiguous_on_permuted_pages():
    rng = np.random.default_rng(3)
    N, L, H, D = 3, 2, 2, 8
    bs, src, dst, T = _round(rng, N, L, H, D)
    kc = rng.standard_normal((L, T, H, D)).astype(np.float32)
    npg = T // 16
    perm = rng.permutation(40)
    kc_row = perm[:npg]
    out_pages = perm[npg:npg + N * npg].reshape(N, npg)
    kc_pool = _pool(rng, L, 40, H, D)
    P.scatter(kc_pool, kc_row, kc)
    out_pool = _pool(rng, L, 40, H, D)
    res = P.rerotate_paged(kc_pool, kc_row, out_pool, out_pages, bs, src, dst, 1e4)
    want = O.rerotate(kc, bs, src, dst, 1e4)
    for i in range(N):
        np.testing.assert_array_equal(P.gather(res, out_pages[i], T), want[i])
    used = set(out_pages.reshape(-1).tolist())
    for p in set(range(40)) - used:
        np.testing.assert_array_equal(res[:, p], out_pool[:, p])


def test_paged_encode_entries_name_pages_holding_the_values():
    rng = np.random.default_rng(4)
    N, L, T, H, D = 4, 2, 64, 2, 8
    base = rng.standard_normal((L, T, H, D)).astype(np.float32)
    ak = np.stack([base.copy() for _ in range(N)])
    av = np.stack([base.copy() * 2 for _ in range(N)])
    ak[1, 0, 20] += 1.0   # agent 1, layer 0, block 1
    av[3, 1, 63] -= 1.0   # agent 3, layer 1, block 3
    ak[2, :, 0:16] += 0.5  # agent 2, both layers, block 0
    pages = rng.permutation(30)[:N * 4].reshape(N, 4)
    kp, vp = _pool(rng, L, 30, H, D), _pool(rng, L, 30, H, D)
    for i in range(N):
        P.scatter(kp, pages[i], ak[i])
        P.scatter(vp, pages[i], av[i])
    off, idx, page, dk, dv = P.diff_encode_paged(kp, vp, pages, 0, N, T)
    assert np.diff(off).tolist() == [0, 0, 1, 0, 1, 1, 0, 1]
    assert idx.tolist() == [1, 0, 0, 3]
    assert page.tolist() == [pages[1][1], pages[2][0], pages[2][0], pages[3][3]]
    for r in range(N * L):
        for e in range(off[r], off[r + 1]):
            np.testing.assert_array_equal(kp[r % L, page[e]], dk[e])
            np.testing.assert_array_equal(vp[r % L, page[e]], dv[e])


def test_paged_restore_attn_equals_contiguous_oracle():
    rng = np.random.default_rng(5)
    N, L, H, Hq, D = 3, 2, 2, 4, 8
    bs, src, dst, T = _round(rng, N, L, H, D)
    priv_len = np.array([5, 0, 37], np.int32)
    priv_off = np.concatenate([[0], np.cumsum(priv_len)]).astype(np.int32)
    base_k = rng.standard_normal((L, T, H, D)).astype(np.float32)
    base_v = rng.standard_normal((L, T, H, D)).astype(np.float32)
    ak = np.stack([base_k.copy() for _ in range(N)])
    av = np.stack([base_v.copy() for _ in range(N)])
    ak[0, 1, 16:32] += 0.3
    av[2, 0, 40] -= 0.2
    pk = rng.standard_normal((L, int(priv_off[-1]), H, D)).astype(np.float32)
    pv = rng.standard_normal((L, int(priv_off[-1]), H, D)).astype(np.float32)
    q = rng.standard_normal((N, L, Hq, D)).astype(np.float32)
    master = 1
    npg = T // 16
    ids = rng.permutation(60)
    pages = ids[:N * npg].reshape(N, npg)
    ppg = 3  # >= ceil(37 / 16)
    priv_pages = ids[N * npg:N * npg + N * ppg].reshape(N, ppg)
    kp, vp = _pool(rng, L, 60, H, D), _pool(rng, L, 60, H, D)
    for i in range(N):
        P.scatter(kp, pages[i], ak[i])
        P.scatter(vp, pages[i], av[i])
        P.scatter(kp, priv_pages[i], pk[:, priv_off[i]:priv_off[i + 1]])
        P.scatter(vp, priv_pages[i], pv[:, priv_off[i]:priv_off[i + 1]])
    off, idx, page, _, _ = P.diff_encode_paged(kp, vp, pages, master, N, T)
    got = P.restore_attn_paged(q, priv_off, kp, vp, priv_pages, kp, vp, pages, master, off, idx, page,
                               bs, src, dst, 1e4, 0.35)
    off_c, idx_c, dk_c, dv_c = O.diff_encode(ak, av, master)
    want = O.restore_attn(q, priv_off, pk, pv, ak[master], av[master], off_c, idx_c, dk_c, dv_c,
                          bs, src, dst, 1e4, 0.35)
    np.testing.assert_array_equal(got, want)
