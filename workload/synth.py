"""Seeded synthetic round generator (input recipe only).

A multi-agent round places one set of shared output blocks O_1..O_B after
each agent's private history H_i, in an agent-specific block order Pi_i
(TokenDance deep-dive notes, Summary "Motivation" and Figure 1: the same
content sits at different absolute positions).  This module draws:

* the prompt layout: block lengths (multiples of 16 tokens), private history
  lengths P_i, the orders Pi_i, and from them each block's absolute start in
  each agent's prompt;
* the cached K/V of the shared blocks for every layer, the decode queries and
  the private-history K/V, all N(0, 1) rounded to the storage dtype;
* the stand-in for selective recompute at the check layer: a copy of the
  reused K with N(0, sigma) added on a random subset of each agent's tokens;
* the Mirror caches: the Master cache with N(0, sigma) added on a random
  subset of 16-token blocks (the same subset on every layer).

Small index structure (lengths, orders, token and block subsets) comes from
numpy ``SeedSequence([seed, config id, stream])``; tensors come from a torch
generator seeded from ``SeedSequence([seed, config id, layer/agent, stream])``
on the device the caller names, so large rounds can be drawn directly in HBM.
Values drawn on different devices differ; a caller that needs identical
inputs on both sides draws on the CPU and copies.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

# Stream ids keep every random draw independent of the others.
_S_LAYOUT = 1
_S_KC = 2
_S_VC = 3
_S_Q = 4
_S_PRIV_K = 5
_S_PRIV_V = 6
_S_REUSE = 7
_S_NOISE_TOK = 8
_S_NOISE_VAL = 9
_S_MIRROR_BLK = 10
_S_MIRROR_VAL = 11

DIFF_BLOCK = 16


@dataclass(frozen=True)
class Config:
    """Shapes and structure of one synthetic round."""

    name: str
    cid: int
    n_agents: int
    n_layers: int
    n_kv_heads: int
    n_q_heads: int
    head_dim: int
    dtype: str  # "f32" or "bf16"
    theta: float
    n_blocks: int
    blk_len: Tuple[int, int]  # inclusive token range, multiples of 16
    # private history: ("fixed", (P_0, ...)), ("uniform", lo, hi) or
    # ("context", lo_total, hi_total): P_i ~ U{max(0, lo - T) .. hi - T}
    priv: tuple
    noise_frac: Tuple[float, float]  # fraction of tokens per agent, lo == hi for exact
    noise_sigma: float
    pct: int  # important-position percentage
    mirror_frac: Tuple[float, float]
    mirror_sigma: float
    check_layer: int = 0
    seed: int = 0
    notes: str = field(default="", compare=False)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def scaled(self, **kw) -> "Config":
        d = dict(self.__dict__)
        d.update(kw)
        return Config(**d)


CONFIGS = {
    "tiny": Config(
        name="tiny", cid=0, n_agents=3, n_layers=1, n_kv_heads=2, n_q_heads=4,
        head_dim=64, dtype="f32", theta=1e4, n_blocks=3, blk_len=(64, 64),
        priv=("fixed", (37, 90, 15)), noise_frac=(0.20, 0.20), noise_sigma=0.05,
        pct=15, mirror_frac=(0.10, 0.20), mirror_sigma=0.1,
        notes="3 agents, fp32, 3 shared blocks of 64 tokens"),
    "qwen7b_check": Config(
        name="qwen7b_check", cid=1, n_agents=10, n_layers=1, n_kv_heads=4,
        n_q_heads=28, head_dim=128, dtype="bf16", theta=1e6, n_blocks=10,
        blk_len=(128, 512), priv=("uniform", 256, 2048), noise_frac=(0.10, 0.20),
        noise_sigma=0.05, pct=15, mirror_frac=(0.10, 0.20), mirror_sigma=0.1,
        notes="Qwen2.5-7B-shaped check layer, rerotate + select"),
    "qwen7b_round": Config(
        name="qwen7b_round", cid=2, n_agents=10, n_layers=28, n_kv_heads=4,
        n_q_heads=28, head_dim=128, dtype="bf16", theta=1e6, n_blocks=10,
        blk_len=(128, 512), priv=("context", 4096, 8192), noise_frac=(0.10, 0.20),
        noise_sigma=0.05, pct=15, mirror_frac=(0.10, 0.20), mirror_sigma=0.1,
        notes="Qwen2.5-7B-shaped full round, 4K-8K contexts"),
    "qwen14b_round": Config(
        name="qwen14b_round", cid=3, n_agents=10, n_layers=48, n_kv_heads=8,
        n_q_heads=40, head_dim=128, dtype="bf16", theta=1e6, n_blocks=10,
        blk_len=(256, 768), priv=("context", 4096, 8192), noise_frac=(0.10, 0.20),
        noise_sigma=0.05, pct=15, mirror_frac=(0.10, 0.20), mirror_sigma=0.1,
        notes="Qwen2.5-14B-shaped full round, 4K-8K contexts"),
    "qwen7b_scaleout": Config(
        name="qwen7b_scaleout", cid=4, n_agents=64, n_layers=28, n_kv_heads=4,
        n_q_heads=28, head_dim=128, dtype="bf16", theta=1e6, n_blocks=32,
        blk_len=(64, 256), priv=("uniform", 512, 4096), noise_frac=(0.10, 0.20),
        noise_sigma=0.05, pct=15, mirror_frac=(0.15, 0.15), mirror_sigma=0.1,
        notes="64 agents, 7B shapes, 15% differing blocks per Mirror"),
}


def _ss(cfg: Config, *keys: int) -> np.random.SeedSequence:
    return np.random.SeedSequence([cfg.seed, cfg.cid, *keys])


def _np_rng(cfg: Config, *keys: int) -> np.random.Generator:
    return np.random.default_rng(_ss(cfg, *keys))


def _torch_gen(cfg: Config, device, *keys: int) -> torch.Generator:
    state = _ss(cfg, *keys).generate_state(2, np.uint32)
    g = torch.Generator(device=device)
    g.manual_seed(int(state[0]) | (int(state[1] & 0x7FFFFFFF) << 32))
    return g


def _count(frac: float, n: int) -> int:
    return max(1, int(np.floor(frac * n + 0.5)))


def _frac(rng: np.random.Generator, fr: Tuple[float, float]) -> float:
    lo, hi = fr
    return lo if lo == hi else float(rng.uniform(lo, hi))


@dataclass
class Layout:
    """Prompt geometry of one round (int32 host arrays)."""

    n_agents: int
    blk_len: np.ndarray  # [B]
    blk_start: np.ndarray  # [B+1] canonical starts
    src_pos: np.ndarray  # [B] position the cached K of block b was rotated at
    perm: np.ndarray  # [N, B] block order of each agent
    priv_len: np.ndarray  # [N]
    dst_pos: np.ndarray  # [N, B] first absolute position of block b in agent i

    @property
    def n_blocks(self) -> int:
        return int(self.blk_len.shape[0])

    @property
    def n_tokens(self) -> int:
        return int(self.blk_start[-1])

    @property
    def priv_off(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.priv_len)]).astype(np.int32)


def make_layout(cfg: Config) -> Layout:
    rng = _np_rng(cfg, _S_LAYOUT)
    lo, hi = cfg.blk_len
    assert lo % DIFF_BLOCK == 0 and hi % DIFF_BLOCK == 0
    blk_len = DIFF_BLOCK * rng.integers(lo // DIFF_BLOCK, hi // DIFF_BLOCK + 1,
                                        size=cfg.n_blocks)
    blk_start = np.concatenate([[0], np.cumsum(blk_len)])
    T = int(blk_start[-1])
    perm = np.stack([rng.permutation(cfg.n_blocks) for _ in range(cfg.n_agents)])
    kind = cfg.priv[0]
    if kind == "fixed":
        priv_len = np.asarray(cfg.priv[1], dtype=np.int64)
        assert priv_len.shape == (cfg.n_agents,)
    elif kind == "uniform":
        priv_len = rng.integers(cfg.priv[1], cfg.priv[2] + 1, size=cfg.n_agents)
    elif kind == "context":
        plo = max(0, cfg.priv[1] - T)
        phi = max(plo, cfg.priv[2] - T)
        priv_len = rng.integers(plo, phi + 1, size=cfg.n_agents)
    else:
        raise ValueError(kind)
    # Agent i's prompt is H_i followed by the shared blocks in the order perm[i].
    dst = np.zeros((cfg.n_agents, cfg.n_blocks), dtype=np.int64)
    for i in range(cfg.n_agents):
        pos = int(priv_len[i])
        for b in perm[i]:
            dst[i, b] = pos
            pos += int(blk_len[b])
    return Layout(
        n_agents=cfg.n_agents,
        blk_len=blk_len.astype(np.int32),
        blk_start=blk_start.astype(np.int32),
        src_pos=blk_start[:-1].astype(np.int32),
        perm=perm.astype(np.int32),
        priv_len=priv_len.astype(np.int32),
        dst_pos=dst.astype(np.int32),
    )


def _normal(shape, cfg: Config, device, *keys: int) -> torch.Tensor:
    g = _torch_gen(cfg, device, *keys)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.to(cfg.torch_dtype)


def cached_kv(cfg: Config, lay: Layout, device="cpu",
              layers: Optional[Sequence[int]] = None):
    """Cached K and V of the shared blocks, [L][T][Hkv][D] each.

    K is the cache as stored after its earlier prefill (already rotated at
    ``src_pos``); the values are simply N(0, 1) draws rounded to the dtype.
    """
    layers = range(cfg.n_layers) if layers is None else layers
    shape = (lay.n_tokens, cfg.n_kv_heads, cfg.head_dim)
    k = torch.stack([_normal(shape, cfg, device, l, _S_KC) for l in layers])
    v = torch.stack([_normal(shape, cfg, device, l, _S_VC) for l in layers])
    return k, v


def queries(cfg: Config, device="cpu") -> torch.Tensor:
    """One decode query per agent per layer, [N][L][Hq][D]."""
    return _normal((cfg.n_agents, cfg.n_layers, cfg.n_q_heads, cfg.head_dim),
                   cfg, device, 0, _S_Q)


def private_kv(cfg: Config, lay: Layout, device="cpu", layers: Optional[Sequence[int]] = None):
    """Private-history K/V, [L][sum P_i][Hkv][D] each, agents concatenated
    (``layers``: only those layers, each drawn as in the whole round)."""
    layers = range(cfg.n_layers) if layers is None else layers
    ptot = int(lay.priv_len.sum())
    shape = (ptot, cfg.n_kv_heads, cfg.head_dim)
    k = torch.stack([_normal(shape, cfg, device, l, _S_PRIV_K) for l in layers])
    v = torch.stack([_normal(shape, cfg, device, l, _S_PRIV_V) for l in layers])
    return k, v


def reuse_stand_in(cfg: Config, lay: Layout, device="cpu") -> torch.Tensor:
    """Independent stand-in for the re-rotated check-layer K, [N][T][Hkv][D].

    The deviation pass depends only on the difference between reused and
    recomputed K, so stage-wise tests of selection feed this draw (instead of
    any rotated output) to both sides.
    """
    return _normal((cfg.n_agents, lay.n_tokens, cfg.n_kv_heads, cfg.head_dim),
                   cfg, device, 0, _S_REUSE)


def noise_tokens(cfg: Config, lay: Layout):
    """Per agent: sorted canonical tokens whose recomputed K gets noise."""
    rng = _np_rng(cfg, _S_NOISE_TOK)
    T = lay.n_tokens
    out = []
    for _ in range(cfg.n_agents):
        n = _count(_frac(rng, cfg.noise_frac), T)
        out.append(np.sort(rng.choice(T, size=n, replace=False)).astype(np.int64))
    return out


def recomputed_k(cfg: Config, lay: Layout, k_reuse: torch.Tensor,
                 tokens=None, sigmas=None) -> torch.Tensor:
    """Stand-in for the check layer's recomputed K, [N][T][Hkv][D].

    ``k_reuse`` is [N][T][Hkv][D] (any reused K).  Agent i's copy gets
    N(0, sigma) noise, added in fp32 and rounded to the dtype, on its noisy
    tokens; every other token stays bit-identical to ``k_reuse``.
    ``tokens`` / ``sigmas`` override the drawn token sets and the per-agent
    sigma (used to plant a known answer).
    """
    assert k_reuse.dim() == 4 and k_reuse.shape[0] == cfg.n_agents
    tokens = noise_tokens(cfg, lay) if tokens is None else tokens
    dev = k_reuse.device
    out = k_reuse.clone()
    for i in range(cfg.n_agents):
        tok = torch.as_tensor(np.asarray(tokens[i], dtype=np.int64), device=dev)
        if tok.numel() == 0:
            continue
        sig = cfg.noise_sigma if sigmas is None else float(sigmas[i])
        g = _torch_gen(cfg, dev, i, _S_NOISE_VAL)
        eps = torch.randn((tok.numel(),) + tuple(k_reuse.shape[2:]), generator=g,
                          device=dev, dtype=torch.float32) * sig
        out[i, tok] = (k_reuse[i, tok].float() + eps).to(k_reuse.dtype)
    return out


def mirror_blocks(cfg: Config, lay: Layout):
    """Per agent: sorted 16-token block indices where its cache departs from
    the Master's (drawn for every agent; the Master's own set is unused)."""
    rng = _np_rng(cfg, _S_MIRROR_BLK)
    assert lay.n_tokens % DIFF_BLOCK == 0
    nblk = lay.n_tokens // DIFF_BLOCK
    out = []
    for _ in range(cfg.n_agents):
        n = _count(_frac(rng, cfg.mirror_frac), nblk)
        out.append(np.sort(rng.choice(nblk, size=n, replace=False)).astype(np.int64))
    return out


def agent_caches(cfg: Config, lay: Layout, master_k: torch.Tensor,
                 master_v: torch.Tensor, master: int, blocks=None,
                 out=None, sigma=None):
    """Every agent's canonical-frame cache, K and V as [N][L][T][Hkv][D].

    Agent ``master`` holds ``master_k``/``master_v`` exactly.  Every other
    agent holds the Master plus N(0, sigma) noise (fp32 add, rounded to the
    dtype) on its drawn 16-token blocks, on every layer and for both K and V;
    elsewhere it is bit-identical to the Master.  Each perturbed block is
    checked to differ from the Master in at least one bit.
    ``out`` may pass preallocated (K, V) tensors to fill in place.
    """
    blocks = mirror_blocks(cfg, lay) if blocks is None else blocks
    sig = cfg.mirror_sigma if sigma is None else sigma
    dev = master_k.device
    L, T = master_k.shape[0], master_k.shape[1]
    if out is None:
        ak = master_k.unsqueeze(0).repeat(cfg.n_agents, 1, 1, 1, 1)
        av = master_v.unsqueeze(0).repeat(cfg.n_agents, 1, 1, 1, 1)
    else:
        ak, av = out
        ak.copy_(master_k.unsqueeze(0).expand_as(ak))
        av.copy_(master_v.unsqueeze(0).expand_as(av))
    for i in range(cfg.n_agents):
        if i == master:
            continue
        blk = np.asarray(blocks[i], dtype=np.int64)
        if blk.size == 0:
            continue
        tok = (blk[:, None] * DIFF_BLOCK + np.arange(DIFF_BLOCK)[None, :]).reshape(-1)
        tok_t = torch.as_tensor(tok, device=dev)
        g = _torch_gen(cfg, dev, i, _S_MIRROR_VAL)
        changed = None
        for dst, src in ((ak, master_k), (av, master_v)):
            base = src[:, tok_t]
            eps = torch.randn(base.shape, generator=g, device=dev, dtype=torch.float32) * sig
            new = (base.float() + eps).to(src.dtype)
            ch = (new != base).reshape(L, blk.size, -1).any(dim=2)
            changed = ch if changed is None else (changed | ch)
            dst[i][:, tok_t] = new
        # every (layer, block) of the drawn set must really differ
        if not bool(changed.all()):
            raise RuntimeError("a perturbed diff block is bit-identical to the Master")
    return ak, av


def to_numpy_bits(x: torch.Tensor) -> np.ndarray:
    """Host copy holding exact storage bits: bf16 as uint16, fp32 as float32."""
    x = x.detach().cpu().contiguous()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    if x.dtype == torch.float32:
        return x.numpy()
    raise TypeError(x.dtype)


def from_numpy_bits(a: np.ndarray) -> torch.Tensor:
    """Inverse of ``to_numpy_bits``: uint16 bit patterns -> bf16, float32 as is."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    if a.dtype == np.float32:
        return torch.from_numpy(a)
    raise TypeError(a.dtype)
