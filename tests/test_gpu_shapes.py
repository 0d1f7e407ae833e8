"""Every element type with every head size (GPU).

The workload presets are bf16 with 128-dim heads and fp32 with 64-dim
heads; the calls also accept bf16 with 64-dim heads and fp32 with 128-dim
heads.  Each stage is checked against the oracle for all four combinations:
re-rotation, the key-difference pass and selection, the diff encode, the
fused restore-attention and the dense comparator, and the paged restore.
"""

import numpy as np
import pytest
import torch

import oracle as O
from collective_kv_cache_amd import tdx
from workload import CONFIGS, make_layout, recomputed_k, reuse_stand_in, to_numpy_bits

from gpu_common import (DEV, Round, assert_close, assert_master, assert_scores, assert_selection, dlayout,
                        host, shape_of)

pytestmark = pytest.mark.gpu

SHAPES = [("bf16", 64), ("bf16", 128), ("f32", 64), ("f32", 128)]


def _cfg(dtype, D):
    return CONFIGS["tiny"].scaled(dtype=dtype, head_dim=D, n_layers=2, n_agents=3)


@pytest.mark.parametrize("dtype,D", SHAPES)
def test_rerotate_and_select(dtype, D):
    cfg = _cfg(dtype, D)
    lay = make_layout(cfg)
    r = Round(cfg, lay, master=0)
    kr = host(tdx.rerotate(r.shape, r.dl, r.dev["kc"]))
    ref = O.rerotate(to_numpy_bits(r.host["kc"]), lay.blk_start, lay.src_pos, lay.dst_pos, cfg.theta)
    if dtype == "f32":
        assert_close(kr, ref, f"rerotate {dtype} D={D}", atol=1e-5, rtol=1e-5)
    else:
        assert_close(kr, ref, f"rerotate {dtype} D={D}")
    kin = reuse_stand_in(cfg, lay)
    kx = recomputed_k(cfg, lay, kin)
    k = O.topk_count(cfg.pct, lay.n_tokens)
    out = tdx.select_important(shape_of(cfg, 1), dlayout(lay), kin.unsqueeze(1).contiguous().to(DEV), kx.to(DEV), k)
    torch.cuda.synchronize()
    d, s, a = O.deviation(to_numpy_bits(kin), to_numpy_bits(kx))
    assert_scores(host(out["dev"]), d.astype(np.float32), "dev")
    assert_selection(host(out["selected"]), s.astype(np.float32), k)
    assert_master(int(host(out["master"])[0]), a.astype(np.float32))


@pytest.mark.parametrize("dtype,D", SHAPES)
def test_encode_restore_dense_and_paged(dtype, D):
    cfg = _cfg(dtype, D)
    lay = make_layout(cfg)
    r = Round(cfg, lay, master=1)
    ds = r.gpu_encode()
    fused = host(r.gpu_fused(ds))
    kd, vd, dense = r.gpu_dense(ds)
    o_fused, o_kd, o_vd, o_dense = r.oracle_full()
    h = {key: to_numpy_bits(v) for key, v in r.host.items()}
    off, idx, _, _ = O.diff_encode(h["ak"], h["av"], 1)
    np.testing.assert_array_equal(host(ds.off), off)
    np.testing.assert_array_equal(host(ds.idx)[:len(idx)], idx)
    assert_close(fused, o_fused, f"fused {dtype} D={D}")
    assert_close(host(dense), o_dense, f"dense {dtype} D={D}")
    np.testing.assert_array_equal(host(vd), o_vd)
    # the paged restore of the same round gives the contiguous bits
    from test_gpu_paged import bits, to_pool
    d = r.dev
    N = cfg.n_agents
    m = torch.tensor([1], dtype=torch.int32, device=DEV)
    kpool, pages = to_pool([d["ak"][i] for i in range(N)], 2, 31)
    vpool, _ = to_pool([d["av"][i] for i in range(N)], 2, 31)
    po = lay.priv_off
    pkpool, ppages = to_pool([d["pk"][:, po[i]:po[i + 1]] for i in range(N)], 2, 32)
    pvpool, _ = to_pool([d["pv"][:, po[i]:po[i + 1]] for i in range(N)], 2, 32)
    agents = tdx.PagedKV(kpool, vpool, pages)
    pd = tdx.diff_encode_paged(r.shape, r.dl, m, agents)
    ds_nc = tdx.diff_encode(r.shape, r.dl, m, d["ak"], d["av"], master_copy=False)
    col = tdx.restore_attn(r.shape, r.dl, d["q"], d["po"], d["pk"], d["pv"], r.max_priv, d["ak"], d["av"], ds_nc,
                           master_sel=m)
    got = tdx.restore_attn_paged(r.shape, r.dl, d["q"], d["po"], tdx.PagedKV(pkpool, pvpool, ppages), r.max_priv,
                                 agents, m, pd)
    torch.cuda.synchronize()
    assert torch.equal(bits(got), bits(col))
