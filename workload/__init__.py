"""Seeded synthetic inputs for the collective KV-cache reuse path.

This package draws inputs only: prompt layouts, random K/V/q tensors and the
synthetic perturbations that stand in for selective recompute and for the
per-agent divergence of Mirror caches.  It holds none of the method's
arithmetic (no RoPE, no deviation score, no selection, no diff, no attention),
so both the CPU oracle and the GPU path can be fed from it.
"""

from .synth import (  # noqa: F401
    CONFIGS,
    Config,
    Layout,
    make_layout,
    cached_kv,
    queries,
    private_kv,
    reuse_stand_in,
    recomputed_k,
    noise_tokens,
    mirror_blocks,
    agent_caches,
    to_numpy_bits,
    from_numpy_bits,
)
