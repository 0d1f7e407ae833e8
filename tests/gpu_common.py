"""Helpers shared by the GPU parity tests."""

import numpy as np
import torch

import oracle as O
from collective_kv_cache_amd import tdx
from workload import to_numpy_bits

# Tolerances: bf16/fp32 K/V and attention outputs |gpu - ref| <= ATOL + RTOL |ref|;
# fp32 deviation scores: relative 1e-5 (exact zero where the inputs are equal).
ATOL, RTOL = 2e-2, 1e-2
SCORE_RTOL = 1e-5
DEV = "cuda"


def shape_of(cfg, n_layers=None) -> tdx.Shape:
    return tdx.Shape(cfg.n_layers if n_layers is None else n_layers, cfg.n_kv_heads, cfg.n_q_heads,
                     cfg.head_dim, cfg.torch_dtype, cfg.theta)


def dlayout(lay) -> tdx.RoundLayout:
    return tdx.RoundLayout(lay.blk_start, lay.src_pos, lay.dst_pos, DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype in (torch.bfloat16, torch.float32):
        return to_numpy_bits(t)
    return t.detach().cpu().numpy()


def assert_close(gpu_bits: np.ndarray, ref_bits: np.ndarray, what: str, atol=ATOL, rtol=RTOL):
    g = O.widen(gpu_bits)
    r = O.widen(ref_bits)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    err = np.abs(g - r)
    bad = err > atol + rtol * np.abs(r)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance, "
                           f"max abs err {err.max():.3g}")
    return float(err.max())


def assert_scores(gpu: np.ndarray, ref: np.ndarray, what: str, rtol=SCORE_RTOL):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape
    zero = ref == 0
    assert np.all(gpu[zero] == 0), f"{what}: non-zero where the inputs are equal"
    rel = np.abs(gpu - ref) / np.maximum(np.abs(ref), 1e-300)
    assert np.all(rel[~zero] <= rtol), f"{what}: max rel err {rel[~zero].max():.3g}"


def assert_selection(sel_gpu: np.ndarray, score_ref32: np.ndarray, k: int, band=SCORE_RTOL):
    """The GPU set has k distinct ascending indices, holds every position
    scoring clearly above the oracle's k-th score and none clearly below."""
    sel = np.asarray(sel_gpu, np.int64)
    T = score_ref32.size
    assert sel.size == k
    assert np.all(np.diff(sel) > 0) and sel[0] >= 0 and sel[-1] < T
    s = score_ref32.astype(np.float64)
    sk = np.sort(s)[::-1][k - 1]
    must = np.nonzero(s > sk * (1 + band))[0] if sk > 0 else np.nonzero(s > 0)[0]
    never = np.nonzero(s < sk * (1 - band))[0]
    chosen = np.zeros(T, bool)
    chosen[sel] = True
    assert chosen[must].all(), "a position clearly above the k-th score is missing"
    assert not chosen[never].any(), "a position clearly below the k-th score was selected"


def assert_master(m_gpu: int, agent_dev_ref32: np.ndarray, band=SCORE_RTOL):
    a = agent_dev_ref32.astype(np.float64)
    assert a[m_gpu] <= a.min() * (1 + band), (m_gpu, a[m_gpu], a.min())
