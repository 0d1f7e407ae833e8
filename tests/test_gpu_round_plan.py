"""A layout derived from token IDs drives the collective calls (GPU).

The host planner turns one all-gather round's prompts (own history, then the
round's outputs in a per-agent order, separated by a reserved token) into a
group layout; the re-rotation and the select pass on that layout match the
oracle run on the oracle planner's layout.
"""

import numpy as np
import pytest
import torch

import oracle as O
from collective_kv_cache_amd import tdx
from workload import to_numpy_bits

from gpu_common import DEV, assert_close, assert_scores, assert_selection, host

pytestmark = pytest.mark.gpu

SEP = 151643  # a reserved token ID outside every other token drawn here


def _round(rng, n_agents, n_outputs):
    outs = [rng.integers(1, 150000, size=int(rng.integers(40, 200))).tolist() for _ in range(n_outputs)]
    reqs = []
    for _ in range(n_agents):
        toks = rng.integers(150000, 151000, size=int(rng.integers(0, 600))).tolist()
        for b in rng.permutation(n_outputs):
            toks += [SEP] + outs[int(b)]
        reqs.append(toks)
    return reqs


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_token_round_layout_drives_rerotate_and_select(dtype):
    rng = np.random.default_rng(11)
    reqs = _round(rng, 6, 5)
    plan = tdx.round_plan(reqs, SEP)
    ref_plan = O.round_plan(reqs, SEP)
    assert len(plan["groups"]) == 1
    g, rg = plan["groups"][0], ref_plan["groups"][0]
    assert g["blk_start"].tolist() == rg["blk_start"] and g["dst_pos"].tolist() == rg["dst_pos"]
    T = int(g["blk_start"][-1])
    L, H, D, theta = 2, 4, 128, 1e6
    shape = tdx.Shape(L, H, 28, D, dtype, theta)
    dl = tdx.RoundLayout(g["blk_start"], g["src_pos"], g["dst_pos"], DEV)
    gen = torch.Generator(device="cpu").manual_seed(5)
    kc = torch.randn((L, T, H, D), generator=gen).to(dtype)
    kr = tdx.rerotate(shape, dl, kc.to(DEV))
    ref = O.rerotate(to_numpy_bits(kc), rg["blk_start"], rg["src_pos"], np.asarray(rg["dst_pos"]), theta)
    if dtype == torch.bfloat16:
        assert_close(host(kr), ref, "rerotate on a token-derived layout")
    else:
        assert_close(host(kr), ref, "rerotate on a token-derived layout", atol=1e-5, rtol=1e-5)
    # the check layer's recomputed K: a few tokens of each agent perturbed
    kx = kr[:, 0].clone()
    for i in range(kx.shape[0]):
        tok = torch.as_tensor(rng.choice(T, size=T // 8, replace=False), device=DEV)
        kx[i, tok] = (kx[i, tok].float() + 0.05 * torch.randn_like(kx[i, tok].float())).to(dtype)
    k = tdx.topk_count(15, T)
    out = tdx.select_important(shape, dl, kr, kx, k)
    torch.cuda.synchronize()
    d, s, a = O.deviation(to_numpy_bits(kr[:, 0]), to_numpy_bits(kx))
    assert_scores(host(out["score"]), s.astype(np.float32), "score")
    assert_scores(host(out["agent_dev"]), a.astype(np.float32), "agent_dev")
    assert_selection(host(out["selected"]), s.astype(np.float32), k)
