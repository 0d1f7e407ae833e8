"""Serial per-agent reuse: the per-request path that a collective round replaces.

TokenDance notes, Figure 7 (path T2, per-request position-independent reuse,
against the collective path T3) and §5 "Scheduling" (a request that cannot
join a compatible group degrades to per-request reuse): each agent re-rotates
the shared blocks to its own offsets and runs its own key-difference pass and
top-k selection, one agent after the other.

Nothing here computes: it issues, per agent, the same two entry points the
collective round issues once (``tdx_rerotate``, ``tdx_select_important``) with
a one-agent layout.  A one-agent re-rotation writes exactly the agent's slice
of the collective output (the shift depends only on the agent's own
offsets); a one-agent selection is that agent's own top-k of its own
deviations, which is what per-request reuse selects.
"""

from __future__ import annotations

from typing import List, Optional

import numpy as np
import torch

from . import tdx


class SerialReuse:
    """One-agent layouts and buffers for the serial path, prepared once.

    blk_start [B+1], src_pos [B], dst_pos [N][B]: the round's geometry (host
    arrays), as for ``tdx.RoundLayout``.
    """

    def __init__(self, shape: tdx.Shape, blk_start, src_pos, dst_pos, k: int, device="cuda"):
        dp = np.asarray(dst_pos, dtype=np.int32)
        self.shape = shape
        self.n_agents = dp.shape[0]
        self.k = int(k)
        self.layouts: List[tdx.RoundLayout] = [
            tdx.RoundLayout(blk_start, src_pos, dp[i:i + 1], device) for i in range(self.n_agents)]
        lay0 = self.layouts[0]
        self.device = lay0.device
        T = lay0.n_tokens
        # every agent's call runs on one stream, so they can share one workspace
        self.ws = torch.empty((max(tdx.select_workspace(shape, lay0), 1),), dtype=torch.uint8,
                              device=self.device)
        self.outs = [dict(
            dev=torch.empty((1, T), dtype=torch.float32, device=self.device),
            score=torch.empty((T,), dtype=torch.float32, device=self.device),
            agent_dev=torch.empty((1,), dtype=torch.float32, device=self.device),
            selected=torch.empty((max(self.k, 1),), dtype=torch.int32, device=self.device),
            master=torch.empty((1,), dtype=torch.int32, device=self.device),
        ) for _ in range(self.n_agents)]

    def run(self, k_cached: torch.Tensor, k_recomp: torch.Tensor, check_layer: int = 0,
            k_out: Optional[torch.Tensor] = None):
        """Per agent i: a1 into ``k_out[i]``, then a2 + a3 on agent i alone.

        k_cached [L][T][Hkv][D]; k_recomp [N][T][Hkv][D] (the check layer);
        k_out [N][L][T][Hkv][D] or None.  Returns (k_out, per-agent result
        dicts as from ``tdx.select_important`` with N = 1).
        """
        N = self.n_agents
        if k_out is None:
            s = self.shape
            k_out = torch.empty((N, s.n_layers, self.layouts[0].n_tokens, s.n_kv_heads, s.head_dim),
                                dtype=s.dtype, device=self.device)
        for i, lay in enumerate(self.layouts):
            ki = k_out[i:i + 1]
            tdx.rerotate(self.shape, lay, k_cached, out=ki)
            tdx.select_important(self.shape, lay, ki, k_recomp[i:i + 1], self.k, check_layer,
                                 out=self.outs[i], ws=self.ws)
        return k_out, self.outs
