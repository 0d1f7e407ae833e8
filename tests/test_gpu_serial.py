"""Serial per-agent path (the per-request fallback) on the GPU.

Per agent, a one-agent re-rotation must write exactly the agent's slice of the
collective re-rotation, and a one-agent selection must be that agent's own
top-k of its own deviations, as the oracle computes them for N = 1.  With a
single agent the serial and collective paths are the same computation.
"""

import numpy as np
import pytest
import torch

import oracle as O
from collective_kv_cache_amd import tdx
from collective_kv_cache_amd.serial import SerialReuse
from workload import CONFIGS, cached_kv, make_layout, recomputed_k, to_numpy_bits

from gpu_common import DEV, assert_scores, assert_selection, dlayout, host, shape_of

pytestmark = pytest.mark.gpu


def _round(name, **kw):
    cfg = CONFIGS[name].scaled(**kw)
    lay = make_layout(cfg)
    kc, _ = cached_kv(cfg, lay, device=DEV)
    shape = shape_of(cfg)
    kr = tdx.rerotate(shape, dlayout(lay), kc)
    kx = recomputed_k(cfg, lay, kr[:, 0].contiguous())
    k = O.topk_count(cfg.pct, lay.n_tokens)
    return cfg, lay, shape, kc, kr, kx, k


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("qwen7b_round", dict(n_layers=2, n_agents=4)),
    ("qwen7b_scaleout", dict(n_layers=1, n_agents=6)),
])
def test_serial_matches_collective_slices_and_oracle(name, kw):
    cfg, lay, shape, kc, kr, kx, k = _round(name, **kw)
    ser = SerialReuse(shape, lay.blk_start, lay.src_pos, lay.dst_pos, k, DEV)
    kr_s, outs = ser.run(kc, kx, check_layer=0)
    torch.cuda.synchronize()
    # a1: bit-identical to the collective output, agent by agent
    assert torch.equal(kr_s.view(torch.int16) if kr_s.dtype == torch.bfloat16 else kr_s.view(torch.int32),
                       kr.view(torch.int16) if kr.dtype == torch.bfloat16 else kr.view(torch.int32))
    # a2 + a3 per agent: the oracle's one-agent deviation, score and top-k
    krh, kxh = to_numpy_bits(kr[:, 0]), to_numpy_bits(kx)
    for i in range(cfg.n_agents):
        d, s, a = O.deviation(krh[i:i + 1], kxh[i:i + 1])
        o = outs[i]
        assert_scores(host(o["dev"]), d.astype(np.float32), f"dev agent {i}")
        assert_scores(host(o["score"]), s.astype(np.float32), f"score agent {i}")
        assert_scores(host(o["agent_dev"]), a.astype(np.float32), f"agent_dev agent {i}")
        assert_selection(host(o["selected"]), s.astype(np.float32), k)
        assert int(host(o["master"])[0]) == 0


def test_single_agent_serial_equals_collective():
    cfg, lay, shape, kc, kr, kx, k = _round("qwen7b_round", n_layers=2, n_agents=1)
    col = tdx.select_important(shape, dlayout(lay), kr, kx, k)
    ser = SerialReuse(shape, lay.blk_start, lay.src_pos, lay.dst_pos, k, DEV)
    kr_s, outs = ser.run(kc, kx)
    torch.cuda.synchronize()
    assert torch.equal(kr_s.view(torch.int16), kr.view(torch.int16))
    for key in ("dev", "score", "agent_dev", "selected", "master"):
        assert torch.equal(outs[0][key], col[key]), key
