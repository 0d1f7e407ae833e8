"""a2 + a3 parity: tdx_select_important against the oracle (GPU).

Stage-wise on identical inputs: both sides read the same reused K (an
independent N(0,1) draw) and the same synthetic recomputed K.
"""

import numpy as np
import pytest
import torch

import oracle as O
from collective_kv_cache_amd import tdx
from workload import CONFIGS, make_layout, cached_kv, reuse_stand_in, recomputed_k, to_numpy_bits

from gpu_common import (DEV, assert_master, assert_scores, assert_selection, dlayout, host,
                        shape_of)

pytestmark = pytest.mark.gpu


def _check(cfg, lay, kr, kx, k, shape=None, kr5=None, check_layer=0):
    """kr: [N][T][Hkv][D] reused K at the check layer (host); kr5 optionally the
    full [N][L][T][Hkv][D] array the GPU reads from."""
    shape = shape_of(cfg, 1) if shape is None else shape
    kr_dev = (kr.unsqueeze(1) if kr5 is None else kr5).to(DEV).contiguous()
    out = tdx.select_important(shape, dlayout(lay), kr_dev, kx.to(DEV), k, check_layer=check_layer)
    torch.cuda.synchronize()
    d, s, a = O.deviation(to_numpy_bits(kr), to_numpy_bits(kx))
    s32, a32 = s.astype(np.float32), a.astype(np.float32)
    assert_scores(host(out["dev"]), d.astype(np.float32), "dev")
    assert_scores(host(out["score"]), s32, "score")
    assert_scores(host(out["agent_dev"]), a32, "agent_dev")
    sel = host(out["selected"])
    assert_selection(sel, s32, k)
    m = int(host(out["master"])[0])
    assert_master(m, a32)
    return sel, m, O.select_important(s32, k), O.choose_master(a32)


@pytest.mark.parametrize("name", ["tiny", "qwen7b_check", "qwen7b_round", "qwen14b_round", "qwen7b_scaleout"])
def test_select_matches_oracle(name):
    cfg = CONFIGS[name]
    lay = make_layout(cfg)
    kr = reuse_stand_in(cfg, lay)
    kx = recomputed_k(cfg, lay, kr)
    k = O.topk_count(cfg.pct, lay.n_tokens)
    assert k == tdx.topk_count(cfg.pct, lay.n_tokens)
    sel, m, sel_ref, m_ref = _check(cfg, lay, kr, kx, k)
    # no ties inside the band on these inputs: the sets agree exactly
    assert sel.tolist() == sel_ref.tolist()
    assert m == m_ref


def test_select_all_ties_takes_lowest_tokens():
    cfg = CONFIGS["qwen7b_check"]
    lay = make_layout(cfg)
    kr = reuse_stand_in(cfg, lay)
    k = 37
    sel, m, _, _ = _check(cfg, lay, kr, kr.clone(), k)
    assert sel.tolist() == list(range(k))  # every score is 0: ties to the lower t
    assert m == 0


@pytest.mark.parametrize("k_mode", ["one", "all"])
def test_select_extreme_k(k_mode):
    cfg = CONFIGS["tiny"]
    lay = make_layout(cfg)
    kr = reuse_stand_in(cfg, lay)
    kx = recomputed_k(cfg, lay, kr)
    k = 1 if k_mode == "one" else lay.n_tokens
    sel, _, sel_ref, _ = _check(cfg, lay, kr, kx, k)
    assert sel.tolist() == sel_ref.tolist()


def test_select_single_agent_and_planted_master():
    cfg = CONFIGS["qwen7b_check"].scaled(n_agents=1)
    lay = make_layout(cfg)
    kr = reuse_stand_in(cfg, lay)
    kx = recomputed_k(cfg, lay, kr)
    _check(cfg, lay, kr, kx, 100)
    # planted Master: every agent noisy on the same tokens, agent 6 at half sigma
    cfg = CONFIGS["qwen7b_check"]
    lay = make_layout(cfg)
    kr = reuse_stand_in(cfg, lay)
    tok = [np.arange(0, lay.n_tokens, 7)] * cfg.n_agents
    sig = [0.1] * cfg.n_agents
    sig[6] = 0.05
    kx = recomputed_k(cfg, lay, kr, tokens=tok, sigmas=sig)
    _, m, _, m_ref = _check(cfg, lay, kr, kx, 50)
    assert m == 6 and m_ref == 6


def test_select_reads_the_check_layer_of_a_multilayer_reuse_tensor():
    cfg = CONFIGS["tiny"].scaled(n_layers=3)
    lay = make_layout(cfg)
    kr = reuse_stand_in(cfg, lay)
    kx = recomputed_k(cfg, lay, kr)
    kr5 = torch.randn((cfg.n_agents, 3, lay.n_tokens, cfg.n_kv_heads, cfg.head_dim))
    kr5[:, 2] = kr
    _check(cfg, lay, kr, kx, 29, shape=shape_of(cfg, 3), kr5=kr5, check_layer=2)


def test_select_deterministic():
    cfg = CONFIGS["qwen7b_scaleout"]
    lay = make_layout(cfg)
    kr = reuse_stand_in(cfg, lay, device=DEV).unsqueeze(1).contiguous()
    kx = recomputed_k(cfg, lay, kr[:, 0])
    k = tdx.topk_count(15, lay.n_tokens)
    a = tdx.select_important(shape_of(cfg, 1), dlayout(lay), kr, kx, k)
    b = tdx.select_important(shape_of(cfg, 1), dlayout(lay), kr, kx, k)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key].view(torch.int32), b[key].view(torch.int32)), key


# a round longer than the selection's LDS buffer (12288 scores): the scores
# are read from global memory in every pass
LONG = CONFIGS["tiny"].scaled(name="tiny_long", n_blocks=40, blk_len=(512, 512))


def test_select_long_round_reads_scores_from_global_memory():
    lay = make_layout(LONG)
    assert lay.n_tokens > 12288
    kr = reuse_stand_in(LONG, lay)
    kx = recomputed_k(LONG, lay, kr)
    k = O.topk_count(LONG.pct, lay.n_tokens)
    sel, m, sel_ref, m_ref = _check(LONG, lay, kr, kx, k)
    assert sel.tolist() == sel_ref.tolist()
    assert m == m_ref


def _tied_round(cfg, lay):
    """Reused K all zero; recomputed K = 1.0 on every 7th token and 0.5 on
    every 3rd of the others, so scores take three exact values and the 0.5
    band is one long run of ties spread over the whole round."""
    T = lay.n_tokens
    kr = torch.zeros((cfg.n_agents, T, cfg.n_kv_heads, cfg.head_dim), dtype=cfg.torch_dtype)
    kx = kr.clone()
    hi = np.arange(0, T, 7)
    lo = np.setdiff1d(np.arange(0, T, 3), hi)
    kx[:, torch.as_tensor(hi)] = 1.0
    kx[:, torch.as_tensor(lo)] = 0.5
    return kr, kx, hi, lo


@pytest.mark.parametrize("cfg", [CONFIGS["qwen7b_check"], LONG], ids=["qwen7b_check", "tiny_long"])
def test_select_ties_at_the_threshold_take_the_lowest_tokens(cfg):
    lay = make_layout(cfg)
    kr, kx, hi, lo = _tied_round(cfg, lay)
    k = len(hi) + len(lo) // 2 + 1
    sel, _, sel_ref, _ = _check(cfg, lay, kr, kx, k)
    want = np.sort(np.concatenate([hi, lo[:k - len(hi)]]))
    assert sel_ref.tolist() == want.tolist()
    assert sel.tolist() == want.tolist()


@pytest.mark.parametrize("name", ["qwen7b_round", "qwen14b_round", "qwen7b_scaleout"])
def test_select_full_size_last_layer_of_the_rerotated_round(name):
    # the benchmark's inputs at full size: the re-rotated K of every layer
    # (64 agents: over 2^32 elements), with the check layer the last one, so
    # the agents' rows sit at the far end of the tensor
    cfg = CONFIGS[name]
    lay = make_layout(cfg)
    kc, _ = cached_kv(cfg, lay, device=DEV)
    kr = tdx.rerotate(shape_of(cfg), dlayout(lay), kc)
    cl = cfg.n_layers - 1
    kx = recomputed_k(cfg, lay, kr[:, cl].contiguous())
    k = O.topk_count(cfg.pct, lay.n_tokens)
    out = tdx.select_important(shape_of(cfg), dlayout(lay), kr, kx, k, check_layer=cl)
    torch.cuda.synchronize()
    d, s, a = O.deviation(to_numpy_bits(kr[:, cl]), to_numpy_bits(kx))
    s32, a32 = s.astype(np.float32), a.astype(np.float32)
    assert_scores(host(out["dev"]), d.astype(np.float32), "dev")
    assert_scores(host(out["score"]), s32, "score")
    assert_scores(host(out["agent_dev"]), a32, "agent_dev")
    assert_selection(host(out["selected"]), s32, k)
    assert_master(int(host(out["master"])[0]), a32)
    del kr, kx, kc, out
    torch.cuda.empty_cache()


def _planted(cfg, lay, vals):
    """Reused K all zero; recomputed K = vals[t] in every element of token t
    (all agents and heads), so token t's score is N * Hkv * |vals[t]| * sqrt(D)
    and the scores' order is the order of |vals|."""
    N, T = cfg.n_agents, lay.n_tokens
    kr = torch.zeros((N, T, cfg.n_kv_heads, cfg.head_dim), dtype=cfg.torch_dtype)
    kx = torch.as_tensor(np.asarray(vals, dtype=np.float32)).to(cfg.torch_dtype).view(1, T, 1, 1)
    return kr, kx.expand(N, T, cfg.n_kv_heads, cfg.head_dim).contiguous()


def test_select_k_above_the_nonzero_scores_takes_them_all_and_the_lowest_zero_tokens():
    # a third of the tokens score > 0; k exceeds their count, so the set is
    # every scored token plus the lowest-index tokens of score 0
    cfg = CONFIGS["tiny"]
    lay = make_layout(cfg)
    T = lay.n_tokens
    z = np.arange(T) % 3 == 1
    vals = np.where(z, 1.0 + np.arange(T) / T, 0.0)
    kr, kx = _planted(cfg, lay, vals)
    k = int(z.sum()) + 5
    sel, _, sel_ref, _ = _check(cfg, lay, kr, kx, k)
    want = np.sort(np.concatenate([np.flatnonzero(z), np.flatnonzero(~z)[:5]]))
    assert sel_ref.tolist() == want.tolist()
    assert sel.tolist() == want.tolist()


def test_select_equal_nonzero_scores_take_the_lowest_tokens():
    # every scored token has the same score (and the rest score 0): the set
    # is the lowest-index scored tokens
    cfg = CONFIGS["tiny"]
    lay = make_layout(cfg)
    T = lay.n_tokens
    z = np.arange(T) % 4 != 0
    kr, kx = _planted(cfg, lay, np.where(z, 0.75, 0.0))
    k = int(z.sum()) // 2
    sel, _, sel_ref, _ = _check(cfg, lay, kr, kx, k)
    want = np.flatnonzero(z)[:k]
    assert sel_ref.tolist() == want.tolist()
    assert sel.tolist() == want.tolist()


@pytest.mark.parametrize("k_frac", [0.05, 0.5, 0.95])
def test_select_scores_over_many_binades(k_frac):
    # scores from ~1e-14 to ~1e10 (every exponent byte differs) in a shuffled
    # order: the set is the tokens of the k largest planted values
    cfg = CONFIGS["tiny"]
    lay = make_layout(cfg)
    T = lay.n_tokens
    rng = np.random.default_rng(7)
    mags = np.logspace(-15, 8, T)
    vals = rng.permutation(mags)
    kr, kx = _planted(cfg, lay, vals)
    k = max(1, int(k_frac * T))
    sel, _, sel_ref, _ = _check(cfg, lay, kr, kx, k)
    want = np.sort(np.argsort(-vals, kind="stable")[:k])
    assert sel_ref.tolist() == want.tolist()
    assert sel.tolist() == want.tolist()
