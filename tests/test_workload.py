"""Generator checks: determinism, geometry and the stated input recipe (CPU)."""

import numpy as np
import pytest
import torch

from workload import (CONFIGS, make_layout, cached_kv, reuse_stand_in, recomputed_k,
                      noise_tokens, mirror_blocks, agent_caches, to_numpy_bits)


@pytest.mark.parametrize("name", list(CONFIGS))
def test_layout_geometry(name):
    cfg = CONFIGS[name]
    lay = make_layout(cfg)
    lo, hi = cfg.blk_len
    assert lay.blk_len.shape == (cfg.n_blocks,)
    assert np.all(lay.blk_len % 16 == 0) and np.all((lay.blk_len >= lo) & (lay.blk_len <= hi))
    assert lay.blk_start[0] == 0 and np.all(np.diff(lay.blk_start) == lay.blk_len)
    assert np.array_equal(lay.src_pos, lay.blk_start[:-1])
    for i in range(cfg.n_agents):
        assert sorted(lay.perm[i].tolist()) == list(range(cfg.n_blocks))
        # the blocks tile [P_i, P_i + T) in agent i's order without gaps
        pos = int(lay.priv_len[i])
        for b in lay.perm[i]:
            assert lay.dst_pos[i, b] == pos
            pos += int(lay.blk_len[b])
        assert pos == lay.priv_len[i] + lay.n_tokens
    kind = cfg.priv[0]
    if kind == "uniform":
        assert np.all((lay.priv_len >= cfg.priv[1]) & (lay.priv_len <= cfg.priv[2]))
    if kind == "context":
        ctx = lay.priv_len + lay.n_tokens
        assert np.all(ctx <= cfg.priv[2]) and np.all(ctx >= min(cfg.priv[1], lay.n_tokens))
    # deterministic
    lay2 = make_layout(cfg)
    assert np.array_equal(lay.dst_pos, lay2.dst_pos) and np.array_equal(lay.priv_len, lay2.priv_len)


def test_tiny_layout_is_the_stated_one():
    cfg = CONFIGS["tiny"]
    lay = make_layout(cfg)
    assert lay.priv_len.tolist() == [37, 90, 15]
    assert lay.blk_len.tolist() == [64, 64, 64] and lay.n_tokens == 192
    assert all(len(t) == 38 for t in noise_tokens(cfg, lay))  # 20% of 192 tokens


def test_recomputed_k_noise_only_on_drawn_tokens():
    cfg = CONFIGS["qwen7b_check"].scaled(n_blocks=3)
    lay = make_layout(cfg)
    kr = reuse_stand_in(cfg, lay)
    kx = recomputed_k(cfg, lay, kr)
    toks = noise_tokens(cfg, lay)
    a, b = to_numpy_bits(kr), to_numpy_bits(kx)
    for i in range(cfg.n_agents):
        frac = len(toks[i]) / lay.n_tokens
        assert 0.095 <= frac <= 0.205
        rows_diff = np.any(a[i] != b[i], axis=(1, 2))
        mask = np.zeros(lay.n_tokens, bool)
        mask[toks[i]] = True
        assert not rows_diff[~mask].any()      # bit-identical off the noisy tokens
        assert rows_diff[mask].mean() > 0.99   # changed on (almost) all noisy ones
    assert torch.equal(kx, recomputed_k(cfg, lay, kr))


def test_agent_caches_master_exact_and_mirrors_on_drawn_blocks():
    cfg = CONFIGS["tiny"].scaled(n_layers=2)
    lay = make_layout(cfg)
    kc, vc = cached_kv(cfg, lay)
    ak, av = agent_caches(cfg, lay, kc, vc, master=2)
    blocks = mirror_blocks(cfg, lay)
    assert torch.equal(ak[2], kc) and torch.equal(av[2], vc)
    for i in range(cfg.n_agents):
        if i == 2:
            continue
        assert 1 <= len(blocks[i]) <= 3
        for l in range(cfg.n_layers):
            for beta in range(lay.n_tokens // 16):
                sl = slice(16 * beta, 16 * beta + 16)
                differs = not (torch.equal(ak[i, l, sl], kc[l, sl]) and torch.equal(av[i, l, sl], vc[l, sl]))
                assert differs == (beta in set(blocks[i].tolist()))


def test_scaleout_mirror_fraction_exact():
    cfg = CONFIGS["qwen7b_scaleout"]
    lay = make_layout(cfg)
    nblk = lay.n_tokens // 16
    want = max(1, int(np.floor(0.15 * nblk + 0.5)))
    assert all(len(b) == want for b in mirror_blocks(cfg, lay))
