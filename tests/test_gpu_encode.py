"""a4 parity: tdx_diff_encode against the oracle (GPU).  Integer outputs and
copied values must be bit-exact."""

import numpy as np
import pytest
import torch

import oracle as O
from collective_kv_cache_amd import tdx
from workload import CONFIGS, make_layout, cached_kv, agent_caches, mirror_blocks, to_numpy_bits

from gpu_common import DEV, Round, assert_close, dlayout, host, shape_of

pytestmark = pytest.mark.gpu


def _encode(cfg, lay, ak, av, master, cap=None, n_layers=None):
    shape = shape_of(cfg, n_layers)
    m = torch.tensor([master], dtype=torch.int32, device=DEV)
    return tdx.diff_encode(shape, dlayout(lay), m, ak.to(DEV), av.to(DEV), cap_blocks=cap, check=False)


def _compare(ds, ref, L, cap=None):
    off, idx, dk, dv = ref
    nnz = ds.nnz()
    assert nnz == int(off[-1])
    # row offsets are clamped to the capacity; nnz keeps the true total
    want_off = off if cap is None else np.minimum(off, cap)
    np.testing.assert_array_equal(host(ds.off).astype(np.int64), want_off)
    n = nnz if cap is None else min(nnz, cap)
    np.testing.assert_array_equal(host(ds.idx)[:n], idx[:n])
    np.testing.assert_array_equal(host(ds.k)[:n], dk[:n])
    np.testing.assert_array_equal(host(ds.v)[:n], dv[:n])


@pytest.mark.parametrize("name,n_layers", [("tiny", 1), ("qwen7b_round", 2), ("qwen14b_round", 2),
                                           ("qwen7b_scaleout", 1)])
def test_encode_matches_oracle(name, n_layers):
    cfg = CONFIGS[name].scaled(n_layers=n_layers)
    lay = make_layout(cfg)
    kc, vc = cached_kv(cfg, lay)
    master = 1
    ak, av = agent_caches(cfg, lay, kc, vc, master)
    ds = _encode(cfg, lay, ak, av, master)
    ref = O.diff_encode(to_numpy_bits(ak), to_numpy_bits(av), master)
    _compare(ds, ref, n_layers)
    np.testing.assert_array_equal(host(ds.master_k), to_numpy_bits(kc))
    np.testing.assert_array_equal(host(ds.master_v), to_numpy_bits(vc))


def test_encode_zero_and_all_blocks():
    cfg = CONFIGS["tiny"].scaled(n_layers=2)
    lay = make_layout(cfg)
    kc, vc = cached_kv(cfg, lay)
    same_k = kc.unsqueeze(0).repeat(cfg.n_agents, 1, 1, 1, 1)
    same_v = vc.unsqueeze(0).repeat(cfg.n_agents, 1, 1, 1, 1)
    ds = _encode(cfg, lay, same_k, same_v, 2)
    assert ds.nnz() == 0
    assert host(ds.off).tolist() == [0] * (cfg.n_agents * 2 + 1)
    nb = lay.n_tokens // 16
    ak, av = agent_caches(cfg, lay, kc, vc, 0, blocks=[np.arange(nb)] * cfg.n_agents)
    ds = _encode(cfg, lay, ak, av, 0)
    ref = O.diff_encode(to_numpy_bits(ak), to_numpy_bits(av), 0)
    assert ds.nnz() == (cfg.n_agents - 1) * 2 * nb
    _compare(ds, ref, 2)


def test_encode_sign_of_zero_counts_as_a_difference():
    cfg = CONFIGS["tiny"]
    lay = make_layout(cfg)
    k = torch.zeros((cfg.n_agents, 1, lay.n_tokens, cfg.n_kv_heads, cfg.head_dim))
    v = torch.zeros_like(k)
    k[2, 0, 17, 1, 5] = -0.0
    v[1, 0, lay.n_tokens - 1, 0, 0] = 1e-40  # an fp32 subnormal
    ds = _encode(cfg, lay, k, v, 0)
    ref = O.diff_encode(to_numpy_bits(k), to_numpy_bits(v), 0)
    _compare(ds, ref, 1)
    assert ds.nnz() == 2


def test_encode_capacity_overflow_reports_true_total():
    cfg = CONFIGS["qwen7b_round"].scaled(n_layers=2)
    lay = make_layout(cfg)
    kc, vc = cached_kv(cfg, lay)
    ak, av = agent_caches(cfg, lay, kc, vc, 3)
    ref = O.diff_encode(to_numpy_bits(ak), to_numpy_bits(av), 3)
    total = int(ref[0][-1])
    cap = total // 3
    ds = _encode(cfg, lay, ak, av, 3, cap=cap)
    _compare(ds, ref, 2, cap=cap)
    with pytest.raises(tdx.TdxError):
        tdx.diff_encode(shape_of(cfg), dlayout(lay), torch.tensor([3], dtype=torch.int32, device=DEV),
                        ak.to(DEV), av.to(DEV), cap_blocks=cap, check=True)


@pytest.mark.parametrize("capped", [False, True])
def test_encode_more_than_4096_rows(capped):
    # 700 agents x 6 layers = 4200 CSR rows: past 4096 rows the row offsets
    # come from one workgroup's scan of the row counts instead of each row's
    # own sum of the earlier counts; both clamp the offsets to the capacity
    cfg = CONFIGS["tiny"].scaled(n_agents=700, n_layers=6, n_blocks=3, blk_len=(16, 32), priv=("uniform", 0, 40))
    lay = make_layout(cfg)
    kc, vc = cached_kv(cfg, lay)
    ak, av = agent_caches(cfg, lay, kc, vc, 5)
    ref = O.diff_encode(to_numpy_bits(ak), to_numpy_bits(av), 5)
    cap = int(ref[0][-1]) // 2 if capped else None
    ds = _encode(cfg, lay, ak, av, 5, cap=cap)
    _compare(ds, ref, 6, cap=cap)


def test_overflowed_record_restores_as_truncated():
    # a record whose blocks overflow the capacity names only written entries
    # (offsets clamped), so the fused and dense restores and the transfer
    # restore read inside it; their outputs equal the oracle run on the
    # truncated record (the first cap entries, offsets min(off, cap))
    import math

    cfg = CONFIGS["qwen7b_round"].scaled(n_layers=2, n_agents=5)
    lay = make_layout(cfg)
    r = Round(cfg, lay, master=2)
    h = {k: to_numpy_bits(v) for k, v in r.host.items()}
    off, idx, dk, dv = O.diff_encode(h["ak"], h["av"], 2)
    cap = int(off[-1]) // 2
    m = torch.tensor([2], dtype=torch.int32, device=DEV)
    ds = tdx.diff_encode(r.shape, r.dl, m, r.dev["ak"], r.dev["av"], cap_blocks=cap, check=False)
    assert ds.nnz() == int(off[-1]) > cap
    toff = np.minimum(off, cap)
    np.testing.assert_array_equal(host(ds.off).astype(np.int64), toff)
    d = r.dev
    fused = tdx.restore_attn(r.shape, r.dl, d["q"], d["po"], d["pk"], d["pv"], r.max_priv, ds.master_k,
                             ds.master_v, ds)
    kd, vd = tdx.restore_dense(r.shape, r.dl, ds.master_k, ds.master_v, ds)
    ag = torch.arange(cfg.n_agents, dtype=torch.int32, device=DEV)
    ko, vo = tdx.restore_transfer(r.shape, r.dl, ds.master_k, ds.master_v, ds.off, ds.idx, ds.k, ds.v, ag)
    args = (lay.blk_start, lay.src_pos, lay.dst_pos, cfg.theta)
    ref = O.restore_attn(h["q"], lay.priv_off, h["pk"], h["pv"], h["kc"], h["vc"], toff, idx[:cap], dk[:cap],
                         dv[:cap], *args, 1.0 / math.sqrt(cfg.head_dim))
    rkd, rvd = O.restore_dense(h["kc"], h["vc"], toff, idx[:cap], dk[:cap], dv[:cap], *args)
    assert_close(host(fused), ref, "fused restore of a truncated record")
    assert_close(host(kd), rkd, "dense K of a truncated record")
    np.testing.assert_array_equal(host(vd), rvd)
    np.testing.assert_array_equal(host(ko), host(kd))
    np.testing.assert_array_equal(host(vo), rvd)


@pytest.mark.parametrize("name", ["qwen7b_round", "qwen14b_round", "qwen7b_scaleout"])
def test_encode_full_size_planted_rows_and_samples(name):
    # full-size rounds (the 64-agent caches hold over 2^32 elements each),
    # drawn in HBM; every row must equal the planted block set (a property
    # that holds at any size) and sampled rows must be bit-exact against the
    # oracle.
    cfg = CONFIGS[name]
    lay = make_layout(cfg)
    kc, vc = cached_kv(cfg, lay, device=DEV)
    master = 4
    ak, av = agent_caches(cfg, lay, kc, vc, master)
    m = torch.tensor([master], dtype=torch.int32, device=DEV)
    ds = tdx.diff_encode(shape_of(cfg), dlayout(lay), m, ak, av, check=True)
    blocks = mirror_blocks(cfg, lay)
    off = host(ds.off).astype(np.int64)
    idx = host(ds.idx)
    L = cfg.n_layers
    for i in range(cfg.n_agents):
        want = [] if i == master else blocks[i].tolist()
        for l in range(L):
            r = i * L + l
            assert idx[off[r]:off[r + 1]].tolist() == want, (i, l)
    for i, l in ((0, 0), (7, 23), (cfg.n_agents // 2, L // 2), (cfg.n_agents - 1, L - 1)):
        pk = torch.stack([ak[master, l:l + 1], ak[i, l:l + 1]])
        pv = torch.stack([av[master, l:l + 1], av[i, l:l + 1]])
        ref = O.diff_encode(to_numpy_bits(pk), to_numpy_bits(pv), 0)
        r = i * L + l
        a, b = off[r], off[r + 1]
        np.testing.assert_array_equal(idx[a:b], ref[1])
        np.testing.assert_array_equal(to_numpy_bits(ds.k[a:b]), ref[2])
        np.testing.assert_array_equal(to_numpy_bits(ds.v[a:b]), ref[3])
    assert torch.equal(ds.master_k.view(torch.int16), kc.view(torch.int16))
    del ak, av, ds
    torch.cuda.empty_cache()


def test_encode_deterministic():
    cfg = CONFIGS["qwen7b_round"].scaled(n_layers=3)
    lay = make_layout(cfg)
    kc, vc = cached_kv(cfg, lay, device=DEV)
    ak, av = agent_caches(cfg, lay, kc, vc, 0)
    a = _encode(cfg, lay, ak, av, 0)
    b = _encode(cfg, lay, ak, av, 0)
    assert a.nnz() == b.nnz()
    n = a.nnz()
    assert torch.equal(a.idx[:n], b.idx[:n]) and torch.equal(a.k[:n].view(torch.int16), b.k[:n].view(torch.int16))
