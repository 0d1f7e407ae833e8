"""tdx_select_important_noalloc (no workspace argument: the library's static
scratch array) against tdx_select_important (caller's workspace), through the
C ABI on the GPU.  Two calls in a row, the second on a smaller round: the
array keeps the first call's contents, which must not leak into the second.
Both calls use the same kernels, so every output must be the same bits; the
oracle pins the selection and the Master on top (O-6 / O-8 band rules)."""

import numpy as np
import pytest
import torch

import oracle as O
from collective_kv_cache_amd import tdx
from workload import CONFIGS, make_layout, recomputed_k, reuse_stand_in, to_numpy_bits

from gpu_common import DEV, assert_master, assert_scores, assert_selection, dlayout, host, shape_of

pytestmark = pytest.mark.gpu

KEYS = ("dev", "score", "agent_dev", "selected", "master")


def _round(name, **kw):
    cfg = CONFIGS[name].scaled(**kw)
    lay = make_layout(cfg)
    kr = reuse_stand_in(cfg, lay)
    kx = recomputed_k(cfg, lay, kr)
    return cfg, lay, kr, kx


def test_noalloc_select_matches_the_workspace_call_twice():
    rounds = [_round("qwen14b_round", n_layers=1),                  # 10 agents, 8 KV heads
              _round("qwen7b_check", n_agents=4, n_blocks=3)]       # smaller: 4 agents
    for cfg, lay, kr, kx in rounds:
        print(f"noalloc select: {cfg.name} N={cfg.n_agents} T={lay.n_tokens}", flush=True)
        shape = shape_of(cfg, 1)
        dl = dlayout(lay)
        k = tdx.topk_count(cfg.pct, lay.n_tokens)
        kr_d = kr.unsqueeze(1).contiguous().to(DEV)
        kx_d = kx.to(DEV)
        assert tdx.select_workspace(shape, dl) <= tdx.SELECT_SCRATCH_BYTES
        ref = tdx.select_important(shape, dl, kr_d, kx_d, k)
        got = tdx.select_important_noalloc(shape, dl, kr_d, kx_d, k)
        torch.cuda.synchronize()
        for key in KEYS:
            assert torch.equal(got[key], ref[key]), key
        d, s, a = O.deviation(to_numpy_bits(kr), to_numpy_bits(kx))
        assert_scores(host(got["dev"]), d.astype(np.float32), "dev")
        assert_scores(host(got["score"]), s.astype(np.float32), "score")
        assert_selection(host(got["selected"]), s.astype(np.float32), k)
        assert_master(int(host(got["master"])[0]), a.astype(np.float32))


def test_noalloc_select_with_preallocated_outputs_allocates_nothing():
    cfg, lay, kr, kx = _round("qwen7b_check", n_agents=6)
    shape = shape_of(cfg, 1)
    dl = dlayout(lay)
    k = tdx.topk_count(cfg.pct, lay.n_tokens)
    kr_d = kr.unsqueeze(1).contiguous().to(DEV)
    kx_d = kx.to(DEV)
    ref = tdx.select_important(shape, dl, kr_d, kx_d, k)
    out = {key: torch.empty_like(v) for key, v in ref.items()}
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    tdx.select_important_noalloc(shape, dl, kr_d, kx_d, k, out=out)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    for key in KEYS:
        assert torch.equal(out[key], ref[key]), key
