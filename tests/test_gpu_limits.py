"""The largest round the calls accept: 1024 agents (GPU).

Every stage of the collective path at N = 1024 (the library's agent limit)
against the oracle: re-rotation, the key-difference pass with selection and
Master, the diff encode (bit-exact indices) and the fused restore-attention.
Small per-agent sizes keep the oracle fast; the agent-indexed paths (the
select kernel's per-agent slices, the encode's per-agent marks, the
restore's agent groups and merge rows) run at their maximum.
"""

import numpy as np
import pytest
import torch

import oracle as O
from collective_kv_cache_amd import tdx
from workload import CONFIGS, make_layout, recomputed_k, reuse_stand_in, to_numpy_bits

from gpu_common import (DEV, Round, assert_close, assert_master, assert_scores, assert_selection,
                        dlayout, host, shape_of)

pytestmark = pytest.mark.gpu

N_MAX = 1024


def _cfg():
    return CONFIGS["tiny"].scaled(n_agents=N_MAX, n_blocks=3, blk_len=(16, 32), priv=("uniform", 0, 40))


def test_max_agents_rerotate_and_select():
    cfg = _cfg()
    lay = make_layout(cfg)
    shape = shape_of(cfg)
    kc = torch.randn((1, lay.n_tokens, cfg.n_kv_heads, cfg.head_dim))
    kr = host(tdx.rerotate(shape, dlayout(lay), kc.to(DEV)))
    ref = O.rerotate(kc.numpy(), lay.blk_start, lay.src_pos, lay.dst_pos, cfg.theta)
    assert_close(kr, ref, "rerotate N=1024", atol=1e-5, rtol=1e-5)
    kr_in = reuse_stand_in(cfg, lay)
    kx = recomputed_k(cfg, lay, kr_in)
    k = O.topk_count(cfg.pct, lay.n_tokens)
    out = tdx.select_important(shape, dlayout(lay), kr_in.unsqueeze(1).contiguous().to(DEV), kx.to(DEV), k)
    torch.cuda.synchronize()
    d, s, a = O.deviation(to_numpy_bits(kr_in), to_numpy_bits(kx))
    assert_scores(host(out["dev"]), d.astype(np.float32), "dev N=1024")
    assert_scores(host(out["agent_dev"]), a.astype(np.float32), "agent_dev N=1024")
    assert_selection(host(out["selected"]), s.astype(np.float32), k)
    assert_master(int(host(out["master"])[0]), a.astype(np.float32))


def test_max_agents_encode_and_restore():
    cfg = _cfg()
    lay = make_layout(cfg)
    master = N_MAX - 3
    r = Round(cfg, lay, master=master)
    ds = r.gpu_encode()
    fused = host(r.gpu_fused(ds))
    h = {key: to_numpy_bits(v) for key, v in r.host.items()}
    off, idx, dk, dv = O.diff_encode(h["ak"], h["av"], master)
    assert ds.nnz() == len(idx)
    np.testing.assert_array_equal(host(ds.off), off)
    np.testing.assert_array_equal(host(ds.idx)[:len(idx)], idx)
    o_fused = O.restore_attn(h["q"], lay.priv_off, h["pk"], h["pv"], h["kc"], h["vc"], off, idx, dk, dv,
                             lay.blk_start, lay.src_pos, lay.dst_pos, cfg.theta, r.scale)
    assert_close(fused, o_fused, "fused N=1024")  # fp32 round: the fp32 bound
