"""a1 parity: tdx_rerotate against the oracle (GPU)."""

import numpy as np
import pytest
import torch

import oracle as O
from collective_kv_cache_amd import tdx
from workload import CONFIGS, make_layout, cached_kv, to_numpy_bits

from gpu_common import DEV, assert_close, dlayout, host, shape_of

pytestmark = pytest.mark.gpu


def _run(cfg, lay, kc_cpu, n_layers):
    shape = shape_of(cfg, n_layers)
    out = tdx.rerotate(shape, dlayout(lay), kc_cpu.to(DEV))
    return host(out)


@pytest.mark.parametrize("name,n_layers", [("tiny", 1), ("qwen7b_check", 1), ("qwen7b_round", 3),
                                           ("qwen14b_round", 2), ("qwen7b_scaleout", 1)])
def test_rerotate_matches_oracle(name, n_layers):
    cfg = CONFIGS[name]
    lay = make_layout(cfg)
    kc, _ = cached_kv(cfg, lay, layers=range(n_layers))
    got = _run(cfg, lay, kc, n_layers)
    ref = O.rerotate(to_numpy_bits(kc), lay.blk_start, lay.src_pos, lay.dst_pos, cfg.theta)
    assert_close(got, ref, f"rerotate {name}")
    if cfg.dtype == "bf16":
        # nearly every bf16 element is bit-identical; the rest sit at rounding ties
        assert np.mean(got == ref) > 0.99


def test_rerotate_ragged_blocks_negative_shifts_and_many_agents():
    # block lengths that are not multiples of 16 (one empty), 70 agents (two
    # LDS agent chunks), negative and zero shifts, fp32 storage
    cfg = CONFIGS["tiny"].scaled(n_agents=70, n_layers=3)
    rng = np.random.default_rng(3)
    lens = np.array([5, 0, 37, 16, 1, 23], np.int32)
    bs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    src = (bs[:-1] + 1000).astype(np.int32)
    dst = rng.integers(0, 5000, size=(70, lens.size)).astype(np.int32)
    dst[0] = src  # agent 0: zero shift everywhere
    kc = torch.randn((3, int(bs[-1]), cfg.n_kv_heads, cfg.head_dim), dtype=torch.float32)
    shape = shape_of(cfg, 3)
    got = host(tdx.rerotate(shape, tdx.RoundLayout(bs, src, dst, DEV), kc.to(DEV)))
    ref = O.rerotate(kc.numpy(), bs, src, dst, cfg.theta)
    assert_close(got, ref, "rerotate ragged", atol=1e-5, rtol=1e-5)
    np.testing.assert_array_equal(got[0].view(np.uint32), kc.numpy().view(np.uint32))


def test_rerotate_zero_shift_is_bitwise_copy_bf16():
    cfg = CONFIGS["qwen7b_check"]
    lay = make_layout(cfg)
    dst = np.tile(lay.src_pos, (cfg.n_agents, 1))
    kc, _ = cached_kv(cfg, lay)
    got = host(tdx.rerotate(shape_of(cfg), tdx.RoundLayout(lay.blk_start, lay.src_pos, dst, DEV), kc.to(DEV)))
    for i in range(cfg.n_agents):
        np.testing.assert_array_equal(got[i], to_numpy_bits(kc))


@pytest.mark.parametrize("name", ["qwen7b_round", "qwen14b_round", "qwen7b_scaleout"])
def test_rerotate_full_size_sampled(name):
    # full-size rounds (7B: 10 agents x 28 layers; 14B: 10 agents x 48 layers x 4912 tokens x 8 heads;
    # 64 agents x 28 layers x ~5.5K tokens x 4 heads, whose output passes 2^32
    # elements): sampled (agent, layer, token) rows against the oracle, in the
    # same launch configuration the benchmark times.
    cfg = CONFIGS[name]
    lay = make_layout(cfg)
    kc, _ = cached_kv(cfg, lay, device=DEV)
    out = tdx.rerotate(shape_of(cfg), dlayout(lay), kc)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    toks = np.unique(np.concatenate([rng.choice(lay.n_tokens, 40, replace=False),
                                     lay.blk_start[:-1], lay.blk_start[1:] - 1, [lay.n_tokens - 1]]))
    tt = torch.as_tensor(toks, device=DEV)
    for i in (0, 3, cfg.n_agents - 1):
        for l in (0, 17, cfg.n_layers - 1):
            rows = to_numpy_bits(kc[l, tt])
            ref = O.rerotate_tokens(rows, toks, i, lay.blk_start, lay.src_pos, lay.dst_pos, cfg.theta)
            assert_close(to_numpy_bits(out[i, l, tt]), ref, f"rerotate full i={i} l={l}")
    del out, kc
    torch.cuda.empty_cache()


def test_rerotate_deterministic():
    cfg = CONFIGS["qwen7b_check"]
    lay = make_layout(cfg)
    kc, _ = cached_kv(cfg, lay, device=DEV)
    a = tdx.rerotate(shape_of(cfg), dlayout(lay), kc)
    b = tdx.rerotate(shape_of(cfg), dlayout(lay), kc)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_shift_keeps_special_values(dtype):
    # R(0) is the identity: re-rotation, the dense restore and the transfer
    # restore store a zero-shift block's bits as they are, also -0 elements
    # with a negative rotate-half partner and infinite elements (x*1 - y*0
    # would give +0 and NaN); agent 0 has zero shifts, the others do not
    cfg = CONFIGS["tiny"].scaled(dtype=dtype, n_layers=2)
    lay = make_layout(cfg)
    N, L, T, H, D = cfg.n_agents, cfg.n_layers, lay.n_tokens, cfg.n_kv_heads, cfg.head_dim
    dst = lay.dst_pos.copy()
    dst[0] = lay.src_pos
    dl = tdx.RoundLayout(lay.blk_start, lay.src_pos, dst, DEV)
    g = torch.Generator().manual_seed(5)
    x = torch.randn((L, T, H, D), generator=g)
    x[..., 0] = -0.0
    x[..., D // 2] = -1.5
    x[0, 3, 1, 5] = float("inf")
    x[1, 20, 0, 6] = float("-inf")
    kc = x.to(cfg.torch_dtype).to(DEV)
    vc = torch.randn((L, T, H, D), generator=g).to(cfg.torch_dtype).to(DEV)
    bits = (lambda t: t.view(torch.int16)) if dtype == "bf16" else (lambda t: t.view(torch.int32))
    shape = shape_of(cfg)
    kr = tdx.rerotate(shape, dl, kc)
    torch.cuda.synchronize()
    assert torch.equal(bits(kr[0]), bits(kc))
    # a round whose agents all hold the Master: an empty record
    ak = kc.unsqueeze(0).repeat(N, 1, 1, 1, 1).contiguous()
    av = vc.unsqueeze(0).repeat(N, 1, 1, 1, 1).contiguous()
    ds = tdx.diff_encode(shape, dl, torch.zeros(1, dtype=torch.int32, device=DEV), ak, av)
    assert ds.nnz() == 0
    kd, vd = tdx.restore_dense(shape, dl, ds.master_k, ds.master_v, ds)
    ko, vo = tdx.restore_transfer(shape, dl, ds.master_k, ds.master_v, ds.off, ds.idx, ds.k, ds.v,
                                  torch.zeros(1, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(bits(kd[0]), bits(kc)) and torch.equal(bits(vd[0]), bits(vc))
    assert torch.equal(bits(ko[0]), bits(kc)) and torch.equal(bits(vo[0]), bits(vc))
