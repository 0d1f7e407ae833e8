"""The collective round captured in a HIP graph (GPU).

Re-rotation, selection, diff encode and fused restore-attention are enqueued
with preallocated outputs and workspaces, so one round can be captured once
and replayed.  Every replay must reproduce the eager round bit for bit; the
replays are separated by eager work of the program and host synchronisation.
"""

import math

import pytest
import torch

from collective_kv_cache_amd import tdx
from workload import CONFIGS, make_layout, recomputed_k

from gpu_common import DEV, Round

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("name,kw", [("qwen7b_round", dict(n_layers=2, n_agents=4)), ("tiny", {})])
def test_round_replays_from_a_graph(name, kw):
    cfg = CONFIGS[name].scaled(**kw)
    lay = make_layout(cfg)
    r = Round(cfg, lay, master=1, device_gen=DEV)
    d = r.dev
    shape, dl = r.shape, r.dl
    N, L, T = cfg.n_agents, cfg.n_layers, lay.n_tokens
    kr = tdx.rerotate(shape, dl, d["kc"])
    kx = recomputed_k(cfg, lay, kr[:, 0].contiguous())
    k = tdx.topk_count(cfg.pct, T)
    sel = tdx.select_important(shape, dl, kr, kx, k)
    cap = (N - 1) * L * (T // 16)
    ds = tdx.diff_encode(shape, dl, sel["master"], d["ak"], d["av"], cap_blocks=cap, master_copy=False)
    out = tdx.restore_attn(shape, dl, d["q"], d["po"], d["pk"], d["pv"], r.max_priv, d["ak"], d["av"], ds,
                           master_sel=sel["master"])
    ws_s = torch.empty(max(tdx.select_workspace(shape, dl), 16), dtype=torch.uint8, device=DEV)
    ws_e = torch.empty(max(tdx.encode_workspace(shape, dl), 16), dtype=torch.uint8, device=DEV)
    ws_a = torch.empty(max(tdx.restore_attn_workspace(shape, dl, r.max_priv), 16), dtype=torch.uint8, device=DEV)

    def step():
        tdx.rerotate(shape, dl, d["kc"], out=kr)
        tdx.select_important(shape, dl, kr, kx, k, out=sel, ws=ws_s)
        tdx.diff_encode(shape, dl, sel["master"], d["ak"], d["av"], out=ds, check=False, ws=ws_e)
        tdx.restore_attn(shape, dl, d["q"], d["po"], d["pk"], d["pv"], r.max_priv, d["ak"], d["av"], ds, out=out,
                         ws=ws_a, master_sel=sel["master"])

    step()
    torch.cuda.synchronize()
    want = {name_: t.clone() for name_, t in (("kr", kr), ("score", sel["score"]), ("selected", sel["selected"]),
                                              ("master", sel["master"]), ("off", ds.off), ("idx", ds.idx),
                                              ("out", out))}
    n_want = ds.nnz()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm the side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        # clobber every output with eager work, then replay
        kr.fill_(0)
        out.fill_(0)
        sel["selected"].fill_(-1)
        ds.idx.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {"kr": kr, "score": sel["score"], "selected": sel["selected"], "master": sel["master"],
               "off": ds.off, "idx": ds.idx, "out": out}
        for key, t in want.items():
            if key == "idx":
                assert torch.equal(got[key][:n_want], t[:n_want]), (rep, key)
            else:
                assert torch.equal(bits(got[key]) if got[key].is_floating_point() else got[key],
                                   bits(t) if t.is_floating_point() else t), (rep, key)
        assert ds.nnz() == n_want
