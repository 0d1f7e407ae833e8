"""fp64 NumPy oracle of the TokenDance collective-reuse hot path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the package smoke check
and by the benchmark's CPU-baseline leg, never by the product path.  It
shares no code with the HIP library or its binding.

Sources (cited by page and section; "notes" is the TokenDance deep-dive page
"TokenDance: Scaling Multi-Agent LLM Serving via Collective KV Cache
Sharing", "blog" is the Chinese blog summary of the same paper):

* notes, Summary "Method" and Figure 7: one batched RoPE correction moves the
  cached K of the shared blocks to every agent's own offsets; one
  key-difference analysis at the check layer picks one important-position
  set that all later layers reuse; the least-deviation agent is the Master.
* notes, Deep Analysis §0 ("aha"): position differences are fixed by one
  group-wide RoPE correction; the method leans on RoPE being invertible.
* notes, Figure 8 and §2b: a Mirror is stored as block-sparse
  (indices, values) relative to the Master, one record per Mirror per layer.
* notes, §3d and blog §4.4: the restore merges the diff into Master tiles
  on chip, recovers RoPE and feeds attention without a dense Mirror; the
  dense restore-then-attend path is the comparator.

Every function computes the plain definition of its result in float64.
Storage formats: bf16 values travel as uint16 bit patterns, fp32 as float32.
The readings of points the pages leave open are listed where they are used.

Pins: every function here is checked against something other than itself by
the CPU tests (closed forms, library routines, brute-force loops, planted
answers and the compression table the notes print).  No function is
"parity unpinned".
"""

from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

BLOCK = 16  # diff block, tokens (notes, Deep Analysis §3c A4: 16/32-token pages)

# ---------------------------------------------------------------------------
# Storage formats
# ---------------------------------------------------------------------------


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values (bf16 is the top half of fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return u.view(np.float32).astype(np.float64)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 directly to bf16 (8 significant bits), ties to even.

    With x = f * 2**E (0.5 <= |f| < 1) the bf16 grid spacing near x is
    2**(E - 8); below the smallest normal (2**-126) it is fixed at 2**-133.
    ``np.rint`` rounds the exactly scaled value half-to-even, so there is a
    single rounding from float64 (no detour through fp32).  Values whose
    rounded magnitude reaches 2**128 become infinities.  NaN is not produced
    by any input of this path and is rejected.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN in bf16 rounding")
    _, e = np.frexp(x)
    e = np.maximum(e.astype(np.int64) - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(x, -e)), e)
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, x), r)
    bits32 = r.astype(np.float32).view(np.uint32)  # exact: r is on the bf16 grid
    return (bits32 >> np.uint32(16)).astype(np.uint16)


def widen(a: np.ndarray) -> np.ndarray:
    """Stored values (uint16 bf16 bits or float32) -> float64."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    raise TypeError(a.dtype)


def narrow(x: np.ndarray, like_dtype) -> np.ndarray:
    """float64 -> storage format of ``like_dtype`` (uint16 bf16 or float32), RNE."""
    if np.dtype(like_dtype) == np.uint16:
        return f64_to_bf16(x)
    if np.dtype(like_dtype) == np.float32:
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    raise TypeError(like_dtype)


# ---------------------------------------------------------------------------
# RoPE (notes, Deep Analysis §0: one RoPE correction fixes a position shift)
# ---------------------------------------------------------------------------
# Reading: rotate-half pairing (e, e + D/2) with frequency theta**(-2e/D), the
# convention of the Qwen2.5 models whose shapes the workloads use.  The pages
# give no formula; the invariants tested below hold for any pairing.


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    half = head_dim // 2
    return np.power(float(theta), -2.0 * np.arange(half, dtype=np.float64) / head_dim)


def rope_rotate(x: np.ndarray, pos, theta: float) -> np.ndarray:
    """Rotate float64 vectors x[..., D] by positions ``pos`` (broadcast over
    the leading axes of x): pair (x_e, x_{e+D/2}) at angle pos * inv_freq_e
    becomes (x_e cos - x_{e+D/2} sin, x_{e+D/2} cos + x_e sin).

    R(0) is the identity, so a vector at position 0 is returned exactly as
    given: its signed zeros and non-finite entries included, which the
    products x*1 - y*0 would turn into +0 or NaN."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    p = np.asarray(pos, dtype=np.float64)
    ang = p[..., None] * rope_inv_freq(D, theta)
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :half], x[..., half:]
    with np.errstate(invalid="ignore"):
        out = np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)
    return np.where((p == 0)[..., None], x, out)


# ---------------------------------------------------------------------------
# Layout helpers
# ---------------------------------------------------------------------------


def block_of_token(blk_start: np.ndarray) -> np.ndarray:
    """b(t) for every canonical token t."""
    blk_start = np.asarray(blk_start, dtype=np.int64)
    lens = np.diff(blk_start)
    return np.repeat(np.arange(lens.size), lens)


def shift(src_pos, dst_pos) -> np.ndarray:
    """Delta[i][b] = dst_pos[i][b] - src_pos[b]: the rotation that moves block
    b from the position its cached K was rotated at to agent i's offset."""
    return np.asarray(dst_pos, dtype=np.int64) - np.asarray(src_pos, dtype=np.int64)[None, :]


# ---------------------------------------------------------------------------
# a1: batched RoPE delta re-rotation (notes, Summary "Method"; Figure 7 T3)
# ---------------------------------------------------------------------------


def rerotate(kc: np.ndarray, blk_start, src_pos, dst_pos, theta: float) -> np.ndarray:
    """K_r[i][l][t] = round(R(Delta_{i,b(t)}) K_c[l][t]) for every agent i.

    kc: [L][T][Hkv][D] stored values.  Returns [N][L][T][Hkv][D] in the same
    storage format, tokens in canonical order.  V is not rotated.
    """
    delta = shift(src_pos, dst_pos)  # [N][B]
    bt = block_of_token(blk_start)  # [T]
    x = widen(kc)  # [L][T][H][D]
    out = []
    for i in range(delta.shape[0]):
        p = delta[i][bt]  # [T]
        out.append(narrow(rope_rotate(x, p[None, :, None], theta), kc.dtype))
    return np.stack(out)


def rerotate_tokens(rows: np.ndarray, tokens, agent: int, blk_start, src_pos, dst_pos,
                    theta: float) -> np.ndarray:
    """The same definition evaluated for chosen canonical tokens only.

    rows: [n][Hkv][D] stored cached-K rows of ``tokens`` (any layer); returns
    agent ``agent``'s re-rotated rows in the storage format.
    """
    delta = shift(src_pos, dst_pos)[agent]
    p = delta[block_of_token(blk_start)[np.asarray(tokens, dtype=np.int64)]]
    return narrow(rope_rotate(widen(rows), p[:, None], theta), rows.dtype)


# ---------------------------------------------------------------------------
# a2: check-layer key difference (notes, Summary "Method"; Figure 7)
# ---------------------------------------------------------------------------
# Reading: the deviation of agent i at token t is the sum over KV heads of the
# L2 norm of (recomputed K - reused K); the group score of t sums it over
# agents; an agent's total sums it over tokens.  K only, check layer only.


def deviation(k_reuse: np.ndarray, k_recomp: np.ndarray):
    """k_reuse, k_recomp: [N][T][Hkv][D] stored values at the check layer.

    Returns float64 d[N][T], score[T] = sum_i d, agent_dev[N] = sum_t d.
    """
    diff = widen(k_recomp) - widen(k_reuse)
    d = np.sqrt((diff * diff).sum(axis=3)).sum(axis=2)
    return d, d.sum(axis=0), d.sum(axis=1)


# ---------------------------------------------------------------------------
# a3: one important-position set + Master (notes, Summary "Method";
#     Deep Analysis §3c A2, A3)
# ---------------------------------------------------------------------------


def topk_count(pct: int, n_tokens: int) -> int:
    """k = ceil(pct * T / 100) in integer arithmetic, clamped to [1, T]."""
    k = (int(pct) * int(n_tokens) + 99) // 100
    return min(max(k, 1), int(n_tokens))


def select_important(score32: np.ndarray, k: int) -> np.ndarray:
    """The k largest scores, ties to the lower token index, returned ascending.

    The decision is taken on the emitted fp32 scores.
    """
    s = np.asarray(score32, dtype=np.float32).astype(np.float64)
    order = sorted(range(s.size), key=lambda t: (-s[t], t))
    return np.sort(np.asarray(order[:k], dtype=np.int64)).astype(np.int32)


def choose_master(agent_dev32: np.ndarray) -> int:
    """Index of the least-deviation agent on the emitted fp32 totals,
    ties to the lower index."""
    a = np.asarray(agent_dev32, dtype=np.float32)
    best = 0
    for i in range(1, a.size):
        if a[i] < a[best]:
            best = i
    return best


# ---------------------------------------------------------------------------
# a4: Master-Mirror block-sparse diff encode (notes, Figure 8 and §2b;
#     blog §4.3)
# ---------------------------------------------------------------------------
# Readings: a 16-token block of Mirror i at layer l is recorded when any stored
# bit of its K or its V (all heads, all dims) differs from the Master's; the
# record holds the ascending block indices and the Mirror's own values
# (a replacement, so the round trip is lossless); the Master's record is empty;
# records are ordered (agent, layer) row-major.


def _bits(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    return a if a.dtype == np.uint16 else a.view(np.uint32)


def diff_blocks(k_i: np.ndarray, v_i: np.ndarray, k_m: np.ndarray, v_m: np.ndarray) -> np.ndarray:
    """Ascending 16-token block indices where a Mirror layer [T][Hkv][D]
    differs from the Master layer in any bit of K or V."""
    T = k_i.shape[0]
    nb = T // BLOCK
    out = []
    for beta in range(nb):
        sl = slice(beta * BLOCK, (beta + 1) * BLOCK)
        if (np.any(_bits(k_i[sl]) != _bits(k_m[sl])) or
                np.any(_bits(v_i[sl]) != _bits(v_m[sl]))):
            out.append(beta)
    return np.asarray(out, dtype=np.int32)


def diff_encode(agents_k: np.ndarray, agents_v: np.ndarray, master: int):
    """agents_k/v: [N][L][T][Hkv][D] canonical-frame caches.

    Returns (off[N*L+1] int64, idx[nnz] int32, dk[nnz][16][Hkv][D],
    dv[nnz][16][Hkv][D]) with row r = i*L + l.
    """
    N, L, T = agents_k.shape[:3]
    if T % BLOCK:
        raise ValueError("token count must be a multiple of 16")
    off = [0]
    idx: List[np.ndarray] = []
    dk, dv = [], []
    for i in range(N):
        for l in range(L):
            if i == master:
                row = np.zeros(0, dtype=np.int32)
            else:
                row = diff_blocks(agents_k[i, l], agents_v[i, l],
                                  agents_k[master, l], agents_v[master, l])
            idx.append(row)
            for beta in row:
                sl = slice(int(beta) * BLOCK, (int(beta) + 1) * BLOCK)
                dk.append(agents_k[i, l, sl])
                dv.append(agents_v[i, l, sl])
            off.append(off[-1] + row.size)
    shape = (0, BLOCK) + agents_k.shape[3:]
    dk_a = np.stack(dk) if dk else np.zeros(shape, dtype=agents_k.dtype)
    dv_a = np.stack(dv) if dv else np.zeros(shape, dtype=agents_v.dtype)
    return (np.asarray(off, dtype=np.int64),
            np.concatenate(idx) if idx else np.zeros(0, np.int32), dk_a, dv_a)


def patch_layer(master_k_l, master_v_l, row_idx, row_k, row_v):
    """Mirror layer = Master layer with the recorded blocks replaced."""
    k = np.array(master_k_l, copy=True)
    v = np.array(master_v_l, copy=True)
    for j, beta in enumerate(np.asarray(row_idx)):
        sl = slice(int(beta) * BLOCK, (int(beta) + 1) * BLOCK)
        k[sl] = row_k[j]
        v[sl] = row_v[j]
    return k, v


def decode_mirror(master_k, master_v, off, idx, dk, dv, i: int):
    """Rebuild agent i's full canonical cache [L][T][Hkv][D] (lossless)."""
    L = master_k.shape[0]
    ks, vs = [], []
    for l in range(L):
        r = i * L + l
        a, b = int(off[r]), int(off[r + 1])
        k, v = patch_layer(master_k[l], master_v[l], idx[a:b], dk[a:b], dv[a:b])
        ks.append(k)
        vs.append(v)
    return np.stack(ks), np.stack(vs)


# ---------------------------------------------------------------------------
# a5 / a6: restore + decode attention (notes §3d, Deep Analysis §4 "Fused Diff
#          Restore"; blog §4.4)
# ---------------------------------------------------------------------------
# Readings: scale 1/sqrt(D) unless given; query head hq reads KV head
# floor(hq / (Hq/Hkv)); no mask (every key precedes the decode token); the
# keys of agent i are its private history followed by the shared tokens, the
# latter rotated to agent i's offsets; the output is stored in the K/V dtype.


def attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of q[Hq][D] over keys/vals[n][Hkv][D], float64."""
    Hq, D = q.shape
    Hkv = keys.shape[1]
    g = Hq // Hkv
    out = np.empty((Hq, D), dtype=np.float64)
    for hq in range(Hq):
        h = hq // g
        z = keys[:, h, :] @ q[hq] * scale
        p = np.exp(z - z.max())
        out[hq] = (p @ vals[:, h, :]) / p.sum()
    return out


def shared_keys_rotated(k_l: np.ndarray, blk_start, src_pos, dst_pos_i, theta: float) -> np.ndarray:
    """Canonical shared keys of one agent layer [T][Hkv][D] (stored values)
    rotated to the agent's offsets, unrounded float64."""
    delta = np.asarray(dst_pos_i, dtype=np.int64) - np.asarray(src_pos, dtype=np.int64)
    p = delta[block_of_token(blk_start)]
    return rope_rotate(widen(k_l), p[:, None], theta)


def restore_attn_one(q_il, priv_k_il, priv_v_il, master_k_l, master_v_l,
                     row_idx, row_k, row_v, blk_start, src_pos, dst_pos_i,
                     theta: float, scale: float):
    """Output of agent i at layer l (float64 [Hq][D]).

    K~ = Master layer patched with agent i's recorded blocks; shared keys are
    R(Delta_i) K~ (not rounded); attention runs over private then shared.
    """
    k_t, v_t = patch_layer(master_k_l, master_v_l, row_idx, row_k, row_v)
    ks = shared_keys_rotated(k_t, blk_start, src_pos, dst_pos_i, theta)
    keys = np.concatenate([widen(priv_k_il), ks], axis=0)
    vals = np.concatenate([widen(priv_v_il), widen(v_t)], axis=0)
    return attend(widen(q_il), keys, vals, scale)


def restore_attn(q, priv_off, priv_k, priv_v, master_k, master_v,
                 off, idx, dk, dv, blk_start, src_pos, dst_pos, theta: float,
                 scale: float):
    """Fused-path result, [N][L][Hq][D] in the K/V storage format."""
    N, L = q.shape[:2]
    out = np.empty(q.shape, dtype=np.float64)
    for i in range(N):
        p0, p1 = int(priv_off[i]), int(priv_off[i + 1])
        for l in range(L):
            r = i * L + l
            a, b = int(off[r]), int(off[r + 1])
            out[i, l] = restore_attn_one(q[i, l], priv_k[l, p0:p1], priv_v[l, p0:p1],
                                         master_k[l], master_v[l], idx[a:b], dk[a:b], dv[a:b],
                                         blk_start, src_pos, dst_pos[i], theta, scale)
    return narrow(out, master_k.dtype)


def restore_dense(master_k, master_v, off, idx, dk, dv, blk_start, src_pos, dst_pos,
                  theta: float):
    """Dense comparator, first half: every agent's cache materialised.

    K_d[i][l] = round(R(Delta_i) K~_i[l]), V_d[i][l] = V~_i[l]; [N][L][T][Hkv][D].
    """
    N = np.asarray(dst_pos).shape[0]
    L = master_k.shape[0]
    kd, vd = [], []
    for i in range(N):
        ki, vi = [], []
        for l in range(L):
            r = i * L + l
            a, b = int(off[r]), int(off[r + 1])
            k_t, v_t = patch_layer(master_k[l], master_v[l], idx[a:b], dk[a:b], dv[a:b])
            ki.append(narrow(shared_keys_rotated(k_t, blk_start, src_pos, dst_pos[i], theta),
                             master_k.dtype))
            vi.append(v_t)
        kd.append(np.stack(ki))
        vd.append(np.stack(vi))
    return np.stack(kd), np.stack(vd)


def decode_attn_dense(q, priv_off, priv_k, priv_v, k_dense, v_dense, scale: float):
    """Dense comparator, second half: attention of agent i over its private
    history followed by its materialised shared keys (already rotated)."""
    N, L = q.shape[:2]
    out = np.empty(q.shape, dtype=np.float64)
    for i in range(N):
        p0, p1 = int(priv_off[i]), int(priv_off[i + 1])
        for l in range(L):
            keys = np.concatenate([widen(priv_k[l, p0:p1]), widen(k_dense[i, l])], axis=0)
            vals = np.concatenate([widen(priv_v[l, p0:p1]), widen(v_dense[i, l])], axis=0)
            out[i, l] = attend(widen(q[i, l]), keys, vals, scale)
    return narrow(out, k_dense.dtype)


# ---------------------------------------------------------------------------
# Storage accounting (notes, §7a "Compression ratio" and the Storage
# Compression table)
# ---------------------------------------------------------------------------
# Reading: the table's 11.2x / 17.5x are per Mirror (1/11.2 and 1/17.5 are
# exactly the 8.9% / 5.7% Mirror-to-Master sizes it quotes); the §7a
# definition dense / (Master + diffs) is the group ratio.  Both are reported.


def diff_row_bytes(n_blocks: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes of one (Mirror, layer) record: K and V values of its blocks,
    one int32 index per block and one int32 row offset."""
    return n_blocks * (BLOCK * kv_heads * head_dim * 2 * elem_bytes + 4) + 4


def compression(counts: np.ndarray, master: int, n_tokens: int, kv_heads: int,
                head_dim: int, elem_bytes: int, priv_len=None) -> dict:
    """counts[N][L]: diff blocks per (agent, layer).  Returns the per-Mirror
    ratios, the group ratio and (with ``priv_len``) the footprint including
    private histories, all over the shared region unless stated."""
    counts = np.asarray(counts, dtype=np.int64)
    N, L = counts.shape
    dense_one = L * n_tokens * kv_heads * head_dim * 2 * elem_bytes
    rows = np.vectorize(lambda n: diff_row_bytes(int(n), kv_heads, head_dim, elem_bytes))(counts)
    mirror_bytes = rows.sum(axis=1)
    per_mirror = {i: dense_one / float(mirror_bytes[i]) for i in range(N) if i != master}
    stored = dense_one + sum(int(mirror_bytes[i]) for i in range(N) if i != master)
    res = {
        "dense_shared_bytes": N * dense_one,
        "stored_shared_bytes": stored,
        "group_ratio": N * dense_one / float(stored),
        "per_mirror_ratio": per_mirror,
        "per_mirror_ratio_mean": float(np.mean(list(per_mirror.values()))) if per_mirror else math.inf,
        "caches_equivalent": stored / float(dense_one),
    }
    if priv_len is not None:
        priv = int(np.sum(priv_len)) * L * kv_heads * head_dim * 2 * elem_bytes
        res["dense_total_bytes"] = N * dense_one + priv
        res["stored_total_bytes"] = stored + priv
        res["footprint_ratio"] = (N * dense_one + priv) / float(stored + priv)
    return res


def caches_for_group(n_agents: int, per_mirror_ratio: float) -> float:
    """Dense-cache equivalents held by one Master plus N-1 Mirrors, each
    Mirror 1/ratio of a dense cache."""
    return 1.0 + (n_agents - 1) / float(per_mirror_ratio)
