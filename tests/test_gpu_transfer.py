"""Transfer-path restore parity (GPU): the requested agents' KV rebuilt from a
Master and diff record kept in pinned host memory equals the oracle's dense
restore of those agents (K within the bf16 tolerance, V bit for bit), only
the requested layers are written, and device-resident sources give the same
bits as pinned host ones."""

import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from collective_kv_cache_amd import tdx
from workload import CONFIGS, make_layout, to_numpy_bits

from gpu_common import DEV, Round, assert_close, host

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1  # a bf16 NaN pattern no restore produces


def pinned(t: torch.Tensor) -> torch.Tensor:
    torch.cuda.synchronize()
    return t.detach().cpu().pin_memory()


def record_on_host(ds):
    return (pinned(ds.master_k), pinned(ds.master_v), pinned(ds.off), pinned(ds.idx), pinned(ds.k),
            pinned(ds.v))


def oracle_restore(r: Round):
    h = {k: to_numpy_bits(v) for k, v in r.host.items()}
    lay = r.lay
    off, idx, dk, dv = O.diff_encode(h["ak"], h["av"], r.master)
    return O.restore_dense(h["kc"], h["vc"], off, idx, dk, dv, lay.blk_start, lay.src_pos, lay.dst_pos,
                           r.cfg.theta)


def sentinel_like(shape, dtype):
    if dtype == torch.bfloat16:
        return torch.full(shape, SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def check_agents(r, k_out, v_out, agents, l0, l1):
    kd, vd = oracle_restore(r)
    ko, vo = host(k_out), host(v_out)
    for j, a in enumerate(agents):
        assert_close(ko[j, l0:l1], kd[a, l0:l1], f"restored K of agent {a}")
        assert np.array_equal(vo[j, l0:l1], vd[a, l0:l1]), f"restored V of agent {a} is not a bit copy"
        outside = np.concatenate([ko[j, :l0].ravel(), ko[j, l1:].ravel(), vo[j, :l0].ravel(),
                                  vo[j, l1:].ravel()])
        if r.cfg.dtype == "bf16":
            assert np.all(outside.view(np.uint16) == SENTINEL), "a layer outside the range was written"
        else:
            assert np.all(np.isnan(outside.view(np.float32))), "a layer outside the range was written"


@pytest.mark.parametrize("name,kw,agents,lr", [
    ("tiny", {}, [0, 1, 2], (0, 1)),
    ("qwen7b_round", dict(n_layers=3, n_agents=4), [1, 3, 0], (1, 3)),
    ("qwen14b_round", dict(n_layers=2, n_agents=3), [2], (0, 2)),
    ("qwen7b_scaleout", dict(n_layers=1, n_agents=6, n_blocks=8), [5, 0, 4, 1, 1], (0, 1)),
])
def test_transfer_restore_from_pinned_host_matches_oracle(name, kw, agents, lr):
    cfg = CONFIGS[name].scaled(**kw)
    lay = make_layout(cfg)
    r = Round(cfg, lay, master=1)
    ds = r.gpu_encode()
    H, D, L, T = cfg.n_kv_heads, cfg.head_dim, cfg.n_layers, lay.n_tokens
    ag = torch.tensor(agents, dtype=torch.int32, device=DEV)
    k_out = sentinel_like((len(agents), L, T, H, D), cfg.torch_dtype)
    v_out = sentinel_like((len(agents), L, T, H, D), cfg.torch_dtype)
    tdx.restore_transfer(r.shape, r.dl, *record_on_host(ds), ag, lr[0], lr[1], k_out, v_out)
    check_agents(r, k_out, v_out, agents, *lr)


def test_device_sources_give_the_same_bits_and_match_dense_restore():
    cfg = CONFIGS["qwen7b_round"].scaled(n_layers=2, n_agents=5)
    lay = make_layout(cfg)
    r = Round(cfg, lay, master=3)
    ds = r.gpu_encode()
    agents = list(range(cfg.n_agents))
    ag = torch.tensor(agents, dtype=torch.int32, device=DEV)
    kh, vh = tdx.restore_transfer(r.shape, r.dl, *record_on_host(ds), ag)
    kdv, vdv = tdx.restore_transfer(r.shape, r.dl, ds.master_k, ds.master_v, ds.off, ds.idx, ds.k, ds.v, ag)
    assert torch.equal(kh.view(torch.int16), kdv.view(torch.int16))
    assert torch.equal(vh.view(torch.int16), vdv.view(torch.int16))
    # the HBM dense restore writes the same caches
    kd, vd = tdx.restore_dense(r.shape, r.dl, ds.master_k, ds.master_v, ds)
    assert torch.equal(vh.view(torch.int16), vd.view(torch.int16))
    assert_close(host(kh), host(kd), "transfer vs dense restore K")


def test_ragged_blocks_and_master_only_agent():
    # shared blocks whose starts are not 16-aligned: a 16-token block of the
    # record then holds rows of two or more shared blocks with different shifts
    cfg = CONFIGS["qwen7b_round"].scaled(n_agents=4, n_layers=2)
    lay = make_layout(cfg)
    lens = np.array([8, 40, 24, 72, 16], np.int32)
    bs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    priv = np.array([0, 5, 300, 17], np.int32)
    perm = np.array([[0, 1, 2, 3, 4], [4, 3, 2, 1, 0], [2, 0, 4, 1, 3], [1, 2, 3, 4, 0]])
    dst = np.zeros((4, 5), np.int32)
    for i in range(4):
        p = priv[i]
        for b in perm[i]:
            dst[i, b] = p
            p += lens[b]
    lay.blk_len, lay.blk_start, lay.src_pos, lay.priv_len, lay.dst_pos = lens, bs, bs[:-1].copy(), priv, dst
    lay.perm = perm
    r = Round(cfg.scaled(n_blocks=5), lay, master=2)
    ds = r.gpu_encode()
    agents = [2, 0, 3, 1]  # the Master's own row is empty: it restores the Master rotated
    ag = torch.tensor(agents, dtype=torch.int32, device=DEV)
    k_out = sentinel_like((4, 2, lay.n_tokens, cfg.n_kv_heads, cfg.head_dim), cfg.torch_dtype)
    v_out = sentinel_like((4, 2, lay.n_tokens, cfg.n_kv_heads, cfg.head_dim), cfg.torch_dtype)
    tdx.restore_transfer(r.shape, r.dl, *record_on_host(ds), ag, 0, 2, k_out, v_out)
    check_agents(r, k_out, v_out, agents, 0, 2)


def test_pageable_host_memory_is_rejected():
    cfg = CONFIGS["tiny"]
    lay = make_layout(cfg)
    r = Round(cfg, lay, master=0)
    ds = r.gpu_encode()
    mk_h, mv_h, off_h, idx_h, dk_h, dv_h = record_on_host(ds)
    ag = torch.tensor([1], dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        tdx.restore_transfer(r.shape, r.dl, ds.master_k.cpu(), mv_h, off_h, idx_h, dk_h, dv_h, ag)
    # the C entry point itself refuses a pointer the GPU cannot read
    pageable = ds.master_k.cpu()
    k_out = torch.empty((1, cfg.n_layers, lay.n_tokens, cfg.n_kv_heads, cfg.head_dim),
                        dtype=cfg.torch_dtype, device=DEV)
    v_out = torch.empty_like(k_out)
    ws = torch.empty(tdx.restore_transfer_workspace(r.shape, r.dl, 1, 0, cfg.n_layers), dtype=torch.uint8,
                     device=DEV)
    s, l = r.shape.c(), r.dl.c()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = tdx.lib().tdx_restore_transfer(ctypes.byref(s), ctypes.byref(l), p(pageable), p(mv_h), p(off_h),
                                        p(idx_h), p(dk_h), p(dv_h), p(ag), 1, 0, cfg.n_layers, p(k_out),
                                        p(v_out), p(ws), ws.numel(), None)
    assert rc == tdx.TDX_EINVAL
    assert b"pinned" in tdx.lib().tdx_last_error()


@pytest.mark.parametrize("name,kw,agents,lr", [
    ("tiny", {}, [2, 0], (0, 1)),
    ("qwen7b_round", dict(n_layers=3, n_agents=4), [3, 1, 1], (1, 3)),
])
def test_transfer_restore_into_pages(name, kw, agents, lr):
    # the requested agents' rebuilt K/V go straight into their pages: the same
    # bits as the dense output, pages of other rows and layers outside the
    # range untouched
    from test_gpu_paged import bits, gather, to_pool
    cfg = CONFIGS[name].scaled(**kw)
    lay = make_layout(cfg)
    r = Round(cfg, lay, master=1)
    ds = r.gpu_encode()
    H, D, L, T = cfg.n_kv_heads, cfg.head_dim, cfg.n_layers, lay.n_tokens
    ag = torch.tensor(agents, dtype=torch.int32, device=DEV)
    rec = record_on_host(ds)
    k_out = sentinel_like((len(agents), L, T, H, D), cfg.torch_dtype)
    v_out = sentinel_like((len(agents), L, T, H, D), cfg.torch_dtype)
    tdx.restore_transfer(r.shape, r.dl, *rec, ag, lr[0], lr[1], k_out, v_out)
    filler = torch.zeros((L, T, H, D), dtype=cfg.torch_dtype, device=DEV)
    kpool, pages = to_pool([filler] * len(agents), 5, 41)
    vpool, _ = to_pool([filler] * len(agents), 5, 41)
    kbefore, vbefore = kpool.clone(), vpool.clone()
    tdx.restore_transfer_paged(r.shape, r.dl, *rec, ag, tdx.PagedKV(kpool, vpool, pages), lr[0], lr[1])
    torch.cuda.synchronize()
    owned = torch.zeros(kpool.shape[1], dtype=torch.bool, device=DEV)
    for j in range(len(agents)):
        gk, gv = gather(kpool, pages, j, T), gather(vpool, pages, j, T)
        assert torch.equal(bits(gk[lr[0]:lr[1]].contiguous()), bits(k_out[j, lr[0]:lr[1]].contiguous())), j
        assert torch.equal(bits(gv[lr[0]:lr[1]].contiguous()), bits(v_out[j, lr[0]:lr[1]].contiguous())), j
        owned[pages[j, :T // 16].long()] = True
    outside = [l for l in range(L) if not lr[0] <= l < lr[1]]
    for pool, before in ((kpool, kbefore), (vpool, vbefore)):
        assert torch.equal(bits(pool[:, ~owned]), bits(before[:, ~owned]))  # other pages untouched
        if outside:
            assert torch.equal(bits(pool[outside]), bits(before[outside]))  # layers outside the range


@pytest.mark.parametrize("name", ["qwen7b_round", "qwen14b_round"])
def test_transfer_full_size_sampled(name):
    # full-size rounds as the benchmark runs them: the Master and the diff
    # record in pinned host memory, every agent and layer restored in one
    # call.  A restored row is the agent's own canonical row (the record is
    # lossless) rotated to its offsets, so sampled rows are checked against
    # the oracle's re-rotation of those rows (K) and bit for bit (V).
    cfg = CONFIGS[name]
    lay = make_layout(cfg)
    master = 3
    r = Round(cfg, lay, master=master, device_gen=DEV)
    d = r.dev
    m = torch.tensor([master], dtype=torch.int32, device=DEV)
    ds = tdx.diff_encode(r.shape, r.dl, m, d["ak"], d["av"], master_copy=False)
    torch.cuda.synchronize()
    n = ds.nnz()
    rec = (pinned(d["ak"][master]), pinned(d["av"][master]), pinned(ds.off), pinned(ds.idx[:max(n, 1)]),
           pinned(ds.k[:max(n, 1)]), pinned(ds.v[:max(n, 1)]))
    ag = torch.arange(cfg.n_agents, dtype=torch.int32, device=DEV)
    ko, vo = tdx.restore_transfer(r.shape, r.dl, *rec, ag)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    toks = np.unique(np.concatenate([rng.choice(lay.n_tokens, 24, replace=False), lay.blk_start[:-1],
                                     [lay.n_tokens - 1]]))
    tt = torch.as_tensor(toks, device=DEV)
    L = cfg.n_layers
    for a, l in ((0, 0), (master, 7), (4, L - 3), (cfg.n_agents - 1, L - 1)):
        own_k = to_numpy_bits(d["ak"][a, l, tt])
        ref = O.rerotate_tokens(own_k, toks, a, lay.blk_start, lay.src_pos, lay.dst_pos, cfg.theta)
        assert_close(to_numpy_bits(ko[a, l, tt]), ref, f"transfer K full a={a} l={l}")
        np.testing.assert_array_equal(to_numpy_bits(vo[a, l, tt]), to_numpy_bits(d["av"][a, l, tt]))
    del ko, vo, r, ds
    torch.cuda.empty_cache()
