"""The collective calls over a paged KV pool: plain definitions.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, never by the product path.

Sources: TokenDance notes §3c A4 and §3d (16/32-token pages; diff indices
aligned to page boundaries; the fused restore relies on the paged KV slot
map) and §5 "Scheduling" (memory management inherits paged attention).

A pool is [L][n_pages][16][Hkv][D]: page p of layer l holds 16 token rows.
A page table row lists one sequence's pages in token order, so token t of
the sequence is row t % 16 of page row[t // 16] (the same page ID in every
layer).  Each paged operation is defined as the contiguous operation applied
to the sequences gathered out of their pages; a paged diff record names, per
entry, the Mirror's own page of the block instead of holding a copy.  Page
IDs outside [0, n_pages) are clamped to the nearest valid page.

Pins (tests/test_oracle_paged.py): an identity page table reduces gather to a
reshape of the pool; scatter/gather round trips leave untouched pages and the
unused rows of a partial page as they were; clamping of out-of-range IDs;
the paged re-rotation on shuffled pages equals the contiguous definition;
the paged deviation on shuffled pages (one clamped ID) equals the contiguous
deviation of the original arrays at the check layer; every diff entry's page
holds the entry's values; the paged
restore-attention on shuffled pages equals the contiguous oracle on the
original arrays.  No function here is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

from . import tdx_oracle as C

PAGE = 16


def clamp_page(p, n_pages: int) -> np.ndarray:
    return np.clip(np.asarray(p, dtype=np.int64), 0, n_pages - 1)


def gather(pool: np.ndarray, row, n_tokens: int) -> np.ndarray:
    """The sequence held by page-table row ``row``: [L][n_tokens][Hkv][D]."""
    L, n_pages = pool.shape[:2]
    out = np.empty((L, n_tokens) + pool.shape[3:], dtype=pool.dtype)
    for t in range(n_tokens):
        out[:, t] = pool[:, clamp_page(row[t // PAGE], n_pages), t % PAGE]
    return out


def scatter(pool: np.ndarray, row, seq: np.ndarray) -> None:
    """Write sequence ``seq`` [L][n][Hkv][D] into the pages of ``row``."""
    n_pages = pool.shape[1]
    for t in range(seq.shape[1]):
        pool[:, clamp_page(row[t // PAGE], n_pages), t % PAGE] = seq[:, t]


def rerotate_paged(kc_pool, kc_row, out_pool, out_pages, blk_start, src_pos, dst_pos, theta):
    """The output pool after agent i's re-rotated K (contiguous definition)
    is written into the pages of out_pages[i]; other pages keep their values."""
    T = int(np.asarray(blk_start)[-1])
    kc = gather(kc_pool, kc_row, T)
    kr = C.rerotate(kc, blk_start, src_pos, dst_pos, theta)
    res = out_pool.copy()
    for i in range(kr.shape[0]):
        scatter(res, out_pages[i], kr[i])
    return res


def deviation_paged(kr_pool, kr_pages, check_layer: int, k_recomp, n_tokens: int):
    """Deviation at the check layer with agent i's reused K gathered from its pages."""
    kr = np.stack([gather(kr_pool, kr_pages[i], n_tokens)[check_layer] for i in range(k_recomp.shape[0])])
    return C.deviation(kr, k_recomp)


def diff_encode_paged(k_pool, v_pool, pages, master: int, n_agents: int, n_tokens: int):
    """(off, idx, page, dk, dv): the contiguous record of the gathered caches
    plus the Mirror's own page of each entry."""
    ak = np.stack([gather(k_pool, pages[i], n_tokens) for i in range(n_agents)])
    av = np.stack([gather(v_pool, pages[i], n_tokens) for i in range(n_agents)])
    off, idx, dk, dv = C.diff_encode(ak, av, master)
    L = k_pool.shape[0]
    page = np.empty(len(idx), dtype=np.int64)
    for r in range(n_agents * L):
        i = r // L
        for e in range(off[r], off[r + 1]):
            page[e] = clamp_page(pages[i][idx[e]], k_pool.shape[1])
    return off, idx, page, dk, dv


def restore_attn_paged(q, priv_off, pk_pool, pv_pool, priv_pages, k_pool, v_pool, pages, master: int,
                       off, idx, page, blk_start, src_pos, dst_pos, theta, scale):
    """Fused restore-attention with every cache read from its pages: agent
    i's private history from priv_pages[i], the Master from pages[master],
    diff entry e's values from page[e] of the agents' pools."""
    N = q.shape[0]
    L = k_pool.shape[0]
    T = int(np.asarray(blk_start)[-1])
    P = np.diff(np.asarray(priv_off))
    pk = np.concatenate([gather(pk_pool, priv_pages[i], int(P[i])) for i in range(N)], axis=1)
    pv = np.concatenate([gather(pv_pool, priv_pages[i], int(P[i])) for i in range(N)], axis=1)
    mk = gather(k_pool, pages[master], T)
    mv = gather(v_pool, pages[master], T)
    n_pages = k_pool.shape[1]
    dk = np.stack([k_pool[r % L, clamp_page(page[e], n_pages)]
                   for r in range(N * L) for e in range(off[r], off[r + 1])]) if len(idx) else \
        np.zeros((0, PAGE) + k_pool.shape[3:], k_pool.dtype)
    dv = np.stack([v_pool[r % L, clamp_page(page[e], n_pages)]
                   for r in range(N * L) for e in range(off[r], off[r + 1])]) if len(idx) else \
        np.zeros((0, PAGE) + v_pool.shape[3:], v_pool.dtype)
    return C.restore_attn(q, priv_off, pk, pv, mk, mv, off, idx, dk, dv, blk_start, src_pos, dst_pos, theta,
                          scale)
