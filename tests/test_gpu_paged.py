"""Paged KV layout: the four collective calls over 16-token pages (GPU).

The same round is laid out twice: contiguously and in pools whose pages are
shuffled, padded with junk pages, and whose page-table rows carry unused
entries that point outside the pool.  Each paged call must give exactly the
bits of its contiguous counterpart (which the other GPU tests pin to the
oracle), leave every page it does not own untouched, and match the paged
oracle (gather, then the contiguous definition) within tolerance.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
from collective_kv_cache_amd import tdx
from workload import CONFIGS, make_layout, recomputed_k, to_numpy_bits

from gpu_common import (DEV, Round, assert_close, assert_master, assert_scores, assert_selection, dlayout, host,
                        shape_of)

pytestmark = pytest.mark.gpu

PAGE = 16
UNUSED = 1 << 30  # page-table padding: clamped to the last page if ever read


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def to_pool(seqs, extra, seed, dtype=None):
    """seqs: list of [L][n_r][Hkv][D] device tensors -> (pool, page table)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    L, _, H, D = seqs[0].shape
    dtype = seqs[0].dtype if dtype is None else dtype
    npg = [math.ceil(s.shape[1] / PAGE) for s in seqs]
    n_pages = sum(npg) + extra
    perm = torch.randperm(n_pages, generator=g)
    gd = torch.Generator(device=DEV).manual_seed(seed)
    pool = torch.randn((L, n_pages, PAGE, H, D), generator=gd, device=DEV).to(dtype)
    stride = max(max(npg), 1) + 2
    pages = torch.full((len(seqs), stride), UNUSED, dtype=torch.int32)
    k = 0
    for r, s in enumerate(seqs):
        ids = perm[k:k + npg[r]]
        k += npg[r]
        pages[r, :npg[r]] = ids.to(torch.int32)
        n = s.shape[1]
        if n:
            full = n // PAGE * PAGE
            if full:
                pool[:, ids[:n // PAGE].to(DEV)] = s[:, :full].reshape(L, n // PAGE, PAGE, H, D)
            if n > full:
                pool[:, int(ids[-1]), :n - full] = s[:, full:]
    return pool, pages.to(DEV)


def gather(pool, pages, r, n):
    npg = math.ceil(n / PAGE)
    ids = pages[r, :npg].long()
    L, _, _, H, D = pool.shape
    return pool[:, ids].reshape(L, npg * PAGE, H, D)[:, :n]


CASES = [
    ("tiny", {}),
    ("qwen7b_round", dict(n_layers=2, n_agents=4)),
    ("qwen14b_round", dict(n_layers=1, n_agents=3)),
]


@pytest.mark.parametrize("name,kw", CASES)
def test_rerotate_paged(name, kw):
    cfg = CONFIGS[name].scaled(**kw)
    lay = make_layout(cfg)
    r = Round(cfg, lay, master=0)
    kc = r.dev["kc"]
    N, T = cfg.n_agents, lay.n_tokens
    kr = tdx.rerotate(r.shape, r.dl, kc)
    cpool, cpages = to_pool([kc], 5, 1)
    opool, opages = to_pool([torch.zeros_like(kc)] * N, 7, 2)
    before = opool.clone()
    tdx.rerotate_paged(r.shape, r.dl, tdx.PagedKV(cpool, None, cpages), tdx.PagedKV(opool, None, opages))
    torch.cuda.synchronize()
    owned = torch.zeros(opool.shape[1], dtype=torch.bool, device=DEV)
    for i in range(N):
        assert torch.equal(bits(gather(opool, opages, i, T).contiguous()), bits(kr[i]))
        owned[opages[i, :math.ceil(T / PAGE)].long()] = True
    assert torch.equal(bits(opool[:, ~owned]), bits(before[:, ~owned]))
    ref = O.rerotate(to_numpy_bits(kc.cpu()), lay.blk_start, lay.src_pos, lay.dst_pos, cfg.theta)
    assert_close(host(torch.stack([gather(opool, opages, i, T) for i in range(N)])), ref, f"paged rerotate {name}")


def test_rerotate_paged_partial_last_page():
    # T = 82: the last page holds 2 tokens; rows past T keep their values
    cfg = CONFIGS["tiny"].scaled(n_agents=5, n_layers=2)
    lens = np.array([5, 0, 37, 16, 1, 23], np.int32)
    bs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    src = (bs[:-1] + 100).astype(np.int32)
    dst = np.random.default_rng(0).integers(0, 3000, size=(5, lens.size)).astype(np.int32)
    T = int(bs[-1])
    kc = torch.randn((2, T, cfg.n_kv_heads, cfg.head_dim)).to(DEV)
    shape = shape_of(cfg, 2)
    dl = tdx.RoundLayout(bs, src, dst, DEV)
    kr = tdx.rerotate(shape, dl, kc)
    cpool, cpages = to_pool([kc], 0, 3)
    opool, opages = to_pool([torch.zeros_like(kc)] * 5, 2, 4)
    before = opool.clone()
    tdx.rerotate_paged(shape, dl, tdx.PagedKV(cpool, None, cpages), tdx.PagedKV(opool, None, opages))
    torch.cuda.synchronize()
    for i in range(5):
        assert torch.equal(gather(opool, opages, i, T), kr[i])
        last = int(opages[i, T // PAGE])
        assert torch.equal(opool[:, last, T % PAGE:], before[:, last, T % PAGE:])
    # selection reads the same partial pages: the contiguous call's bits
    kx = kr[:, 1].clone()
    kx[:, ::3] += 0.05
    col = tdx.select_important(shape, dl, kr, kx, 9, check_layer=1)
    got = tdx.select_important_paged(shape, dl, tdx.PagedKV(opool, None, opages), kx, 9, check_layer=1)
    torch.cuda.synchronize()
    for key in ("dev", "score", "agent_dev", "selected", "master"):
        assert torch.equal(got[key], col[key]), key


@pytest.mark.parametrize("name,kw", CASES)
def test_select_paged(name, kw):
    cfg = CONFIGS[name].scaled(**kw)
    lay = make_layout(cfg)
    r = Round(cfg, lay, master=0)
    N, T = cfg.n_agents, lay.n_tokens
    kr = tdx.rerotate(r.shape, r.dl, r.dev["kc"])
    check = cfg.n_layers - 1  # the last layer: the pool's layer offset is exercised
    kx = recomputed_k(cfg, lay, kr[:, check].contiguous())
    k = O.topk_count(cfg.pct, T)
    col = tdx.select_important(r.shape, r.dl, kr, kx, k, check)
    pool, pages = to_pool([kr[i] for i in range(N)], 9, 5)
    got = tdx.select_important_paged(r.shape, r.dl, tdx.PagedKV(pool, None, pages), kx, k, check)
    torch.cuda.synchronize()
    for key in ("dev", "score", "agent_dev", "selected", "master"):
        assert torch.equal(got[key], col[key]), key
    # and the paged oracle (the sequences gathered out of their pages)
    d_ref, s_ref, a_ref = O.paged.deviation_paged(to_numpy_bits(pool), host(pages), check, to_numpy_bits(kx), T)
    assert_scores(host(got["dev"]), d_ref.astype(np.float32), "paged dev")
    assert_scores(host(got["score"]), s_ref.astype(np.float32), "paged score")
    assert_selection(host(got["selected"]), s_ref.astype(np.float32), k)
    assert_master(int(host(got["master"])[0]), a_ref.astype(np.float32))


@pytest.mark.parametrize("name,kw", CASES + [("qwen7b_scaleout", dict(n_layers=1, n_agents=6, n_blocks=8))])
def test_encode_paged(name, kw):
    cfg = CONFIGS[name].scaled(**kw)
    lay = make_layout(cfg)
    r = Round(cfg, lay, master=1)
    d = r.dev
    N, L, T = cfg.n_agents, cfg.n_layers, lay.n_tokens
    ds = r.gpu_encode()
    kpool, pages = to_pool([d["ak"][i] for i in range(N)], 6, 7)
    vpool, _ = to_pool([d["av"][i] for i in range(N)], 6, 7)  # same seed: same page table
    m = torch.tensor([1], dtype=torch.int32, device=DEV)
    pd = tdx.diff_encode_paged(r.shape, r.dl, m, tdx.PagedKV(kpool, vpool, pages), copy_values=True)
    n = pd.nnz()
    assert n == ds.nnz()
    assert torch.equal(pd.off, ds.off) and torch.equal(pd.idx[:n], ds.idx[:n])
    assert torch.equal(bits(pd.k[:n]), bits(ds.k[:n])) and torch.equal(bits(pd.v[:n]), bits(ds.v[:n]))
    off, idx, page = host(pd.off), host(pd.idx), host(pd.page)
    pg = host(pages)
    for row in range(N * L):
        for e in range(off[row], off[row + 1]):
            assert page[e] == pg[row // L, idx[e]]
    # the entry's page holds the entry's values
    if n:
        lay_of = torch.as_tensor(np.repeat(np.arange(N * L) % L, np.diff(off)), device=DEV)
        assert torch.equal(bits(kpool[lay_of, pd.page[:n].long()]), bits(ds.k[:n]))
    # without value copies the record is the same
    pd2 = tdx.diff_encode_paged(r.shape, r.dl, m, tdx.PagedKV(kpool, vpool, pages))
    assert pd2.k is None and torch.equal(pd2.page[:n], pd.page[:n]) and torch.equal(pd2.off, pd.off)


@pytest.mark.parametrize("name,kw", CASES + [("qwen7b_scaleout", dict(n_layers=1, n_agents=6, n_blocks=8))])
def test_restore_attn_paged(name, kw):
    cfg = CONFIGS[name].scaled(**kw)
    lay = make_layout(cfg)
    master = 2
    r = Round(cfg, lay, master=master)
    d = r.dev
    N, L, T = cfg.n_agents, cfg.n_layers, lay.n_tokens
    m = torch.tensor([master], dtype=torch.int32, device=DEV)
    ds_nc = tdx.diff_encode(r.shape, r.dl, m, d["ak"], d["av"], master_copy=False)
    col = tdx.restore_attn(r.shape, r.dl, d["q"], d["po"], d["pk"], d["pv"], r.max_priv, d["ak"], d["av"], ds_nc,
                           master_sel=m)
    kpool, pages = to_pool([d["ak"][i] for i in range(N)], 4, 11)
    vpool, _ = to_pool([d["av"][i] for i in range(N)], 4, 11)
    po = lay.priv_off
    priv_k = [d["pk"][:, po[i]:po[i + 1]] for i in range(N)]
    priv_v = [d["pv"][:, po[i]:po[i + 1]] for i in range(N)]
    pkpool, ppages = to_pool(priv_k, 3, 12)
    pvpool, _ = to_pool(priv_v, 3, 12)
    agents = tdx.PagedKV(kpool, vpool, pages)
    pd = tdx.diff_encode_paged(r.shape, r.dl, m, agents)
    got = tdx.restore_attn_paged(r.shape, r.dl, d["q"], d["po"], tdx.PagedKV(pkpool, pvpool, ppages), r.max_priv,
                                 agents, m, pd)
    torch.cuda.synchronize()
    assert torch.equal(bits(got), bits(col))
    o_fused = r.oracle_full()[0]
    assert_close(host(got), o_fused, f"paged restore {name}")


def test_restore_attn_paged_without_private_history():
    cfg = CONFIGS["tiny"].scaled(n_layers=2)
    lay = make_layout(cfg)
    lay.priv_len[:] = 0
    lay.priv_off[:] = 0
    r = Round(cfg, lay, master=0)
    d = r.dev
    N = cfg.n_agents
    m = torch.tensor([0], dtype=torch.int32, device=DEV)
    kpool, pages = to_pool([d["ak"][i] for i in range(N)], 2, 13)
    vpool, _ = to_pool([d["av"][i] for i in range(N)], 2, 13)
    agents = tdx.PagedKV(kpool, vpool, pages)
    pd = tdx.diff_encode_paged(r.shape, r.dl, m, agents)
    got = tdx.restore_attn_paged(r.shape, r.dl, d["q"], d["po"], None, 0, agents, m, pd)
    torch.cuda.synchronize()
    assert_close(host(got), r.oracle_full()[0], "paged restore, no private history")


def test_full_size_14b_paged_matches_contiguous():
    # the 14B round at full size in the benchmark's launch configuration: every
    # paged call gives the contiguous call's bits; sampled restore outputs are
    # checked one by one against the oracle
    cfg = CONFIGS["qwen14b_round"]
    lay = make_layout(cfg)
    master = 4
    r = Round(cfg, lay, master=master, device_gen=DEV)
    d = r.dev
    shape, dl = r.shape, r.dl
    N, L, T = cfg.n_agents, cfg.n_layers, lay.n_tokens
    m = torch.tensor([master], dtype=torch.int32, device=DEV)
    # a1
    kr = tdx.rerotate(shape, dl, d["kc"])
    cpool, cpages = to_pool([d["kc"]], 3, 21)
    zero = torch.zeros_like(kr[0])
    opool, opages = to_pool([zero] * N, 3, 22)  # zero pages: the call must write every one
    del zero
    tdx.rerotate_paged(shape, dl, tdx.PagedKV(cpool, None, cpages), tdx.PagedKV(opool, None, opages))
    for i in range(N):
        assert torch.equal(bits(gather(opool, opages, i, T).contiguous()), bits(kr[i])), i
    # a2 + a3 at the check layer
    kx = recomputed_k(cfg, lay, kr[:, 0].contiguous())
    k = O.topk_count(cfg.pct, T)
    col = tdx.select_important(shape, dl, kr, kx, k)
    got = tdx.select_important_paged(shape, dl, tdx.PagedKV(opool, None, opages), kx, k)
    for key in ("dev", "score", "agent_dev", "selected", "master"):
        assert torch.equal(got[key], col[key]), key
    del cpool, opool, kr
    torch.cuda.empty_cache()
    # a4 + a5
    ds = tdx.diff_encode(shape, dl, m, d["ak"], d["av"], master_copy=False)
    out = tdx.restore_attn(shape, dl, d["q"], d["po"], d["pk"], d["pv"], r.max_priv, d["ak"], d["av"], ds,
                           master_sel=m)
    kpool, pages = to_pool([d["ak"][i] for i in range(N)], 4, 23)
    vpool, _ = to_pool([d["av"][i] for i in range(N)], 4, 23)
    po = lay.priv_off
    pkpool, ppages = to_pool([d["pk"][:, po[i]:po[i + 1]] for i in range(N)], 2, 24)
    pvpool, _ = to_pool([d["pv"][:, po[i]:po[i + 1]] for i in range(N)], 2, 24)
    agents = tdx.PagedKV(kpool, vpool, pages)
    pd = tdx.diff_encode_paged(shape, dl, m, agents)
    n = pd.nnz()
    assert n == ds.nnz() and torch.equal(pd.off, ds.off) and torch.equal(pd.idx[:n], ds.idx[:n])
    pout = tdx.restore_attn_paged(shape, dl, d["q"], d["po"], tdx.PagedKV(pkpool, pvpool, ppages), r.max_priv,
                                  agents, m, pd)
    torch.cuda.synchronize()
    assert torch.equal(bits(pout), bits(out))
    for i, l in ((0, 0), (master, 17), (N - 1, L - 1)):
        p0, p1 = int(po[i]), int(po[i + 1])
        mk, mv = to_numpy_bits(d["ak"][master, l]), to_numpy_bits(d["av"][master, l])
        _, idx, dk, dv = O.diff_encode(np.stack([mk, to_numpy_bits(d["ak"][i, l])])[:, None],
                                       np.stack([mv, to_numpy_bits(d["av"][i, l])])[:, None], 0)
        ref = O.restore_attn_one(to_numpy_bits(d["q"][i, l]), to_numpy_bits(d["pk"][l, p0:p1]),
                                 to_numpy_bits(d["pv"][l, p0:p1]), mk, mv, idx, dk, dv,
                                 lay.blk_start, lay.src_pos, lay.dst_pos[i], cfg.theta, r.scale)
        assert_close(to_numpy_bits(pout[i, l]), O.narrow(ref, np.uint16), f"paged full i={i} l={l}")
    del kpool, vpool, pkpool, pvpool, r, ds, pd
    torch.cuda.empty_cache()


def test_out_of_range_page_ids_are_clamped():
    # page IDs below 0 or past the pool read (and write) the nearest valid
    # page, as the paged oracle defines; nothing outside the pool is touched
    cfg = CONFIGS["tiny"].scaled(n_layers=2)
    lay = make_layout(cfg)
    r = Round(cfg, lay, master=0)
    d = r.dev
    N, L, T = cfg.n_agents, cfg.n_layers, lay.n_tokens
    npg = T // PAGE
    kc = d["kc"]
    # tile j lives in page j, the last tile in the pool's last page (npg + 1);
    # the table names the first tile's page as -7 and the last one's past the end
    n_pages = npg + 2
    cpool = torch.randn((L, n_pages, PAGE, cfg.n_kv_heads, cfg.head_dim), device=DEV).to(kc.dtype)
    tiles = kc.reshape(L, npg, PAGE, cfg.n_kv_heads, cfg.head_dim)
    cpool[:, :npg - 1] = tiles[:, :npg - 1]
    cpool[:, n_pages - 1] = tiles[:, npg - 1]
    row = list(range(npg))
    row[0], row[npg - 1] = -7, n_pages + 100
    cp = torch.tensor([row], dtype=torch.int32, device=DEV)
    kr = tdx.rerotate(r.shape, r.dl, kc)
    opool, opages = to_pool([torch.zeros_like(kc)] * N, 2, 52)
    tdx.rerotate_paged(r.shape, r.dl, tdx.PagedKV(cpool, None, cp), tdx.PagedKV(opool, None, opages))
    torch.cuda.synchronize()
    ref = O.paged.rerotate_paged(to_numpy_bits(cpool.cpu()), row, to_numpy_bits(torch.zeros_like(opool).cpu()),
                                 host(opages), lay.blk_start, lay.src_pos, lay.dst_pos, cfg.theta)
    for i in range(N):
        got = gather(opool, opages, i, T)
        want = O.paged.gather(ref, host(opages)[i], T)
        assert_close(host(got), want, f"clamped rerotate agent {i}", atol=1e-5, rtol=1e-5)
        assert torch.equal(got, kr[i])  # the clamped IDs point at the right tiles
