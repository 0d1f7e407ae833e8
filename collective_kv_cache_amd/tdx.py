"""Python binding of libtdx (ctypes).

Argument marshalling only: every step of the path runs in the HIP kernels of
libtdx.so.  PyTorch provides device memory and the current stream.  When the
library is missing, loading fails with an error; there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtdx.so")

TDX_OK = 0
TDX_EINVAL = -1
TDX_EUNSUPPORTED = -2
TDX_EHIP = -3
TDX_EINTERNAL = -4
TDX_EWORKSPACE = -5
TDX_F32 = 0
TDX_BF16 = 1
DIFF_BLOCK = 16


class TdxError(RuntimeError):
    def __init__(self, code: int, what: str, detail: str):
        super().__init__(f"{what} failed ({code}: {detail})")
        self.code = code


class CShape(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("rope_theta", ctypes.c_double)]


class CLayout(ctypes.Structure):
    _fields_ = [("n_agents", ctypes.c_int32), ("n_blocks", ctypes.c_int32),
                ("n_tokens", ctypes.c_int32), ("blk_start", ctypes.c_void_p),
                ("src_pos", ctypes.c_void_p), ("dst_pos", ctypes.c_void_p)]


class CPagedKV(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p), ("n_pages", ctypes.c_int64),
                ("pages", ctypes.c_void_p), ("stride", ctypes.c_int64)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float
_PS = ctypes.POINTER(CShape)
_PL = ctypes.POINTER(CLayout)

_SIGS = {
    "tdx_version": (ctypes.c_int, []),
    "tdx_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "tdx_last_error": (ctypes.c_char_p, []),
    "tdx_topk_count": (_I32, [_I32, _I32]),
    "tdx_rerotate": (ctypes.c_int, [_PS, _PL, _P, _P, _P]),
    "tdx_select_workspace": (_SZ, [_PS, _PL]),
    "tdx_select_important": (ctypes.c_int, [_PS, _PL, _I32, _P, _P, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "tdx_select_important_noalloc": (ctypes.c_int, [_PS, _PL, _I32, _P, _P, _I32, _P, _P, _P, _P, _P, _P]),
    "tdx_diff_encode_workspace": (_SZ, [_PS, _PL]),
    "tdx_diff_encode": (ctypes.c_int, [_PS, _PL, _P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "tdx_restore_attn_workspace": (_SZ, [_PS, _PL, _I32]),
    "tdx_restore_attn": (ctypes.c_int, [_PS, _PL, _P, _P, _P, _P, _I32, _P, _P, _P, _I64, _P, _P, _P, _P, _F, _P,
                                        _P, _SZ, _P]),
    "tdx_restore_dense": (ctypes.c_int, [_PS, _PL, _P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "tdx_decode_attn_dense_workspace": (_SZ, [_PS, _PL, _I32]),
    "tdx_decode_attn_dense": (ctypes.c_int, [_PS, _PL, _P, _P, _P, _P, _I32, _P, _P, _F, _P, _P, _SZ, _P]),
    "tdx_restore_transfer_workspace": (_SZ, [_PS, _PL, _I32, _I32, _I32]),
    "tdx_restore_transfer": (ctypes.c_int, [_PS, _PL, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P,
                                            _P, _SZ, _P]),
    "tdx_rerotate_paged": (ctypes.c_int, [_PS, _PL, ctypes.POINTER(CPagedKV), ctypes.POINTER(CPagedKV), _P]),
    "tdx_select_important_paged": (ctypes.c_int, [_PS, _PL, _I32, ctypes.POINTER(CPagedKV), _P, _I32, _P, _P, _P,
                                                  _P, _P, _P, _SZ, _P]),
    "tdx_diff_encode_paged": (ctypes.c_int, [_PS, _PL, _P, ctypes.POINTER(CPagedKV), _I64, _P, _P, _P, _P, _P, _P,
                                             _P, _SZ, _P]),
    "tdx_restore_attn_paged": (ctypes.c_int, [_PS, _PL, _P, _P, ctypes.POINTER(CPagedKV), _I32,
                                              ctypes.POINTER(CPagedKV), _P, _P, _P, _P, _F, _P, _P, _SZ, _P]),
    "tdx_restore_transfer_paged": (ctypes.c_int, [_PS, _PL, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32,
                                                  ctypes.POINTER(CPagedKV), _P, _SZ, _P]),
    "tdx_round_plan_build": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _P, _P, ctypes.POINTER(_P)]),
    "tdx_round_plan_n_groups": (ctypes.c_int, [_P]),
    "tdx_round_plan_group_dims": (ctypes.c_int, [_P, _I32, _P, _P, _P]),
    "tdx_round_plan_group": (ctypes.c_int, [_P, _I32, _P, _P, _P, _P, _P, _P]),
    "tdx_round_plan_request": (ctypes.c_int, [_P, _I32, _P, _P]),
    "tdx_round_plan_free": (None, [_P]),
}

EXPORTED = tuple(_SIGS)

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libtdx.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m collective_kv_cache_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _check(rc: int, what: str):
    if rc != TDX_OK:
        raise TdxError(rc, what, lib().tdx_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if device is not None and _norm(t.device) != _norm(device):
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _norm(d) -> torch.device:
    d = torch.device(d)
    if d.type == "cuda" and d.index is None:
        return torch.device("cuda", torch.cuda.current_device())
    return d


@dataclass(frozen=True)
class Shape:
    n_layers: int
    n_kv_heads: int
    n_q_heads: int
    head_dim: int
    dtype: torch.dtype  # torch.bfloat16 or torch.float32
    rope_theta: float

    def c(self) -> CShape:
        code = {torch.bfloat16: TDX_BF16, torch.float32: TDX_F32}.get(self.dtype, -1)
        return CShape(self.n_layers, self.n_kv_heads, self.n_q_heads, self.head_dim, code,
                      float(self.rope_theta))

    def with_layers(self, n: int) -> "Shape":
        return Shape(n, self.n_kv_heads, self.n_q_heads, self.head_dim, self.dtype, self.rope_theta)


class RoundLayout:
    """Device copy of a round's geometry (int32 tensors) plus host scalars."""

    def __init__(self, blk_start, src_pos, dst_pos, device):
        bs = np.asarray(blk_start, dtype=np.int32)
        sp = np.asarray(src_pos, dtype=np.int32)
        dp = np.asarray(dst_pos, dtype=np.int32)
        self.n_agents, self.n_blocks = dp.shape
        self.n_tokens = int(bs[-1])
        self.device = _norm(device)
        self.blk_start = torch.as_tensor(bs, device=self.device)
        self.src_pos = torch.as_tensor(sp, device=self.device)
        self.dst_pos = torch.as_tensor(dp.reshape(-1), device=self.device)
        self._c = CLayout(self.n_agents, self.n_blocks, self.n_tokens,
                          self.blk_start.data_ptr(), self.src_pos.data_ptr(), self.dst_pos.data_ptr())

    def c(self) -> CLayout:
        return self._c


def version() -> int:
    return lib().tdx_version()


def topk_count(pct: int, n_tokens: int) -> int:
    return int(lib().tdx_topk_count(int(pct), int(n_tokens)))


def strerror(code: int) -> str:
    return lib().tdx_strerror(code).decode()


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def rerotate(shape: Shape, lay: RoundLayout, k_cached: torch.Tensor, out: Optional[torch.Tensor] = None):
    """a1: [L][T][Hkv][D] -> [N][L][T][Hkv][D] re-rotated to every agent's offsets."""
    L, T, H, D = shape.n_layers, lay.n_tokens, shape.n_kv_heads, shape.head_dim
    _need(k_cached, "k_cached", shape.dtype, (L, T, H, D), lay.device)
    if out is None:
        out = torch.empty((lay.n_agents, L, T, H, D), dtype=shape.dtype, device=lay.device)
    _need(out, "out", shape.dtype, (lay.n_agents, L, T, H, D), lay.device)
    s, l = shape.c(), lay.c()
    _check(lib().tdx_rerotate(ctypes.byref(s), ctypes.byref(l), _ptr(k_cached), _ptr(out), _stream()),
           "tdx_rerotate")
    return out


def select_workspace(shape: Shape, lay: RoundLayout) -> int:
    s, l = shape.c(), lay.c()
    return int(lib().tdx_select_workspace(ctypes.byref(s), ctypes.byref(l)))


def select_important(shape: Shape, lay: RoundLayout, k_reuse: torch.Tensor, k_recomp: torch.Tensor,
                     k: int, check_layer: int = 0, out: Optional[dict] = None, ws=None) -> dict:
    """a2 + a3: returns dict(dev, score, agent_dev, selected, master) on the device."""
    N, L, T, H, D = lay.n_agents, shape.n_layers, lay.n_tokens, shape.n_kv_heads, shape.head_dim
    dev_ = lay.device
    _need(k_reuse, "k_reuse", shape.dtype, (N, L, T, H, D), dev_)
    _need(k_recomp, "k_recomp", shape.dtype, (N, T, H, D), dev_)
    if out is None:
        out = dict(
            dev=torch.empty((N, T), dtype=torch.float32, device=dev_),
            score=torch.empty((T,), dtype=torch.float32, device=dev_),
            agent_dev=torch.empty((N,), dtype=torch.float32, device=dev_),
            selected=torch.empty((max(int(k), 1),), dtype=torch.int32, device=dev_),
            master=torch.empty((1,), dtype=torch.int32, device=dev_),
        )
    if ws is None:
        ws = _ws(select_workspace(shape, lay), dev_)
    s, l = shape.c(), lay.c()
    _check(lib().tdx_select_important(
        ctypes.byref(s), ctypes.byref(l), int(check_layer), _ptr(k_reuse), _ptr(k_recomp), int(k),
        _ptr(out["dev"]), _ptr(out["score"]), _ptr(out["agent_dev"]), _ptr(out["selected"]),
        _ptr(out["master"]), _ptr(ws), ws.numel(), _stream()), "tdx_select_important")
    return out


SELECT_SCRATCH_BYTES = 4 << 20  # TDX_SELECT_SCRATCH_BYTES


def select_important_noalloc(shape: Shape, lay: RoundLayout, k_reuse: torch.Tensor, k_recomp: torch.Tensor,
                             k: int, check_layer: int = 0, out: Optional[dict] = None) -> dict:
    """a2 + a3 without a workspace argument: the library's static scratch
    array of the current device serves it (``tdx_select_important_noalloc``).
    Outputs as :func:`select_important`; with ``out`` given, nothing is
    allocated on this call."""
    N, L, T, H, D = lay.n_agents, shape.n_layers, lay.n_tokens, shape.n_kv_heads, shape.head_dim
    dev_ = lay.device
    _need(k_reuse, "k_reuse", shape.dtype, (N, L, T, H, D), dev_)
    _need(k_recomp, "k_recomp", shape.dtype, (N, T, H, D), dev_)
    if out is None:
        out = dict(
            dev=torch.empty((N, T), dtype=torch.float32, device=dev_),
            score=torch.empty((T,), dtype=torch.float32, device=dev_),
            agent_dev=torch.empty((N,), dtype=torch.float32, device=dev_),
            selected=torch.empty((max(int(k), 1),), dtype=torch.int32, device=dev_),
            master=torch.empty((1,), dtype=torch.int32, device=dev_),
        )
    s, l = shape.c(), lay.c()
    _check(lib().tdx_select_important_noalloc(
        ctypes.byref(s), ctypes.byref(l), int(check_layer), _ptr(k_reuse), _ptr(k_recomp), int(k),
        _ptr(out["dev"]), _ptr(out["score"]), _ptr(out["agent_dev"]), _ptr(out["selected"]),
        _ptr(out["master"]), _stream()), "tdx_select_important_noalloc")
    return out


def encode_workspace(shape: Shape, lay: RoundLayout) -> int:
    s, l = shape.c(), lay.c()
    return int(lib().tdx_diff_encode_workspace(ctypes.byref(s), ctypes.byref(l)))


class DiffSet:
    """CSR diff record of every (agent, layer) row plus the dense Master."""

    def __init__(self, off, idx, k, v, nnz, master_k, master_v, cap):
        self.off, self.idx, self.k, self.v = off, idx, k, v
        self.nnz_dev = nnz
        self.master_k, self.master_v = master_k, master_v
        self.cap = cap

    def nnz(self) -> int:
        return int(self.nnz_dev.item())


def diff_encode(shape: Shape, lay: RoundLayout, master: torch.Tensor, agents_k: torch.Tensor,
                agents_v: torch.Tensor, cap_blocks: Optional[int] = None, master_copy: bool = True,
                check: bool = True, out: Optional[DiffSet] = None, ws=None) -> DiffSet:
    """a4: Master-Mirror block-sparse encode.  With ``check`` the stream is
    synchronised and an overflow of ``cap_blocks`` raises."""
    N, L, T, H, D = lay.n_agents, shape.n_layers, lay.n_tokens, shape.n_kv_heads, shape.head_dim
    dev_ = lay.device
    _need(master, "master", torch.int32, (1,), dev_)
    _need(agents_k, "agents_k", shape.dtype, (N, L, T, H, D), dev_)
    _need(agents_v, "agents_v", shape.dtype, (N, L, T, H, D), dev_)
    if out is None:
        nb = T // DIFF_BLOCK
        cap = (N - 1) * L * nb if cap_blocks is None else int(cap_blocks)
        out = DiffSet(
            torch.empty((N * L + 1,), dtype=torch.int32, device=dev_),
            torch.empty((max(cap, 1),), dtype=torch.int32, device=dev_),
            torch.empty((max(cap, 1), DIFF_BLOCK, H, D), dtype=shape.dtype, device=dev_),
            torch.empty((max(cap, 1), DIFF_BLOCK, H, D), dtype=shape.dtype, device=dev_),
            torch.empty((1,), dtype=torch.int64, device=dev_),
            torch.empty((L, T, H, D), dtype=shape.dtype, device=dev_) if master_copy else None,
            torch.empty((L, T, H, D), dtype=shape.dtype, device=dev_) if master_copy else None,
            cap)
    if ws is None:
        ws = _ws(encode_workspace(shape, lay), dev_)
    s, l = shape.c(), lay.c()
    _check(lib().tdx_diff_encode(
        ctypes.byref(s), ctypes.byref(l), _ptr(master), _ptr(agents_k), _ptr(agents_v), int(out.cap),
        _ptr(out.off), _ptr(out.idx), _ptr(out.k), _ptr(out.v), _ptr(out.nnz_dev),
        _ptr(out.master_k), _ptr(out.master_v), _ptr(ws), ws.numel(), _stream()), "tdx_diff_encode")
    if check:
        n = out.nnz()
        if n < 0:
            raise TdxError(TDX_EINVAL, "tdx_diff_encode", "the Master index is outside [0, N)")
        if n > out.cap:
            raise TdxError(TDX_EINVAL, "tdx_diff_encode", f"{n} diff blocks exceed capacity {out.cap}")
    return out


def restore_attn_workspace(shape: Shape, lay: RoundLayout, max_priv: int) -> int:
    s, l = shape.c(), lay.c()
    return int(lib().tdx_restore_attn_workspace(ctypes.byref(s), ctypes.byref(l), int(max_priv)))


def _master_args(shape: Shape, lay: RoundLayout, master_k, master_v, master_sel):
    """(k, v, sel, stride): master_k/v are either the Master's own cache
    [L][T][Hkv][D] (master_sel None) or every agent's cache [N][L][T][Hkv][D]
    with the device int32 [1] ``master_sel`` naming the Master (read in place)."""
    N, L, T, H, D = lay.n_agents, shape.n_layers, lay.n_tokens, shape.n_kv_heads, shape.head_dim
    dev_ = lay.device
    if master_sel is None:
        _need(master_k, "master_k", shape.dtype, (L, T, H, D), dev_)
        _need(master_v, "master_v", shape.dtype, (L, T, H, D), dev_)
        return master_k, master_v, None, 0
    _need(master_sel, "master_sel", torch.int32, (1,), dev_)
    _need(master_k, "master_k", shape.dtype, (N, L, T, H, D), dev_)
    _need(master_v, "master_v", shape.dtype, (N, L, T, H, D), dev_)
    return master_k, master_v, master_sel, L * T * H * D


def restore_attn(shape: Shape, lay: RoundLayout, q: torch.Tensor, priv_off: torch.Tensor,
                 priv_k: torch.Tensor, priv_v: torch.Tensor, max_priv: int,
                 master_k: torch.Tensor, master_v: torch.Tensor, diff: DiffSet,
                 scale: Optional[float] = None, out: Optional[torch.Tensor] = None, ws=None,
                 master_sel: Optional[torch.Tensor] = None):
    """a5: fused restore + decode attention -> [N][L][Hq][D].  The Master is
    ``master_k``/``master_v`` ([L][T][Hkv][D]), or, with ``master_sel``, entry
    ``master_sel[0]`` of the [N][L][T][Hkv][D] agent caches, read in place."""
    N, L, T, H, Hq, D = (lay.n_agents, shape.n_layers, lay.n_tokens, shape.n_kv_heads,
                         shape.n_q_heads, shape.head_dim)
    dev_ = lay.device
    _need(q, "q", shape.dtype, (N, L, Hq, D), dev_)
    _need(priv_off, "priv_off", torch.int32, (N + 1,), dev_)
    _need(priv_k, "priv_k", shape.dtype, None, dev_)
    _need(priv_v, "priv_v", shape.dtype, tuple(priv_k.shape), dev_)
    if priv_k.dim() != 4 or priv_k.shape[0] != L or tuple(priv_k.shape[2:]) != (H, D):
        raise ValueError("priv_k must be [L][P_total][Hkv][D]")
    mk, mv, msel, mstride = _master_args(shape, lay, master_k, master_v, master_sel)
    if out is None:
        out = torch.empty((N, L, Hq, D), dtype=shape.dtype, device=dev_)
    _need(out, "out", shape.dtype, (N, L, Hq, D), dev_)
    if ws is None:
        ws = _ws(restore_attn_workspace(shape, lay, max_priv), dev_)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    s, l = shape.c(), lay.c()
    _check(lib().tdx_restore_attn(
        ctypes.byref(s), ctypes.byref(l), _ptr(q), _ptr(priv_off), _ptr(priv_k), _ptr(priv_v),
        int(max_priv), _ptr(mk), _ptr(mv), _ptr(msel), mstride, _ptr(diff.off), _ptr(diff.idx),
        _ptr(diff.k), _ptr(diff.v), scale, _ptr(out), _ptr(ws), ws.numel(), _stream()),
        "tdx_restore_attn")
    return out


def restore_dense(shape: Shape, lay: RoundLayout, master_k: torch.Tensor, master_v: torch.Tensor,
                  diff: DiffSet, k_dense: Optional[torch.Tensor] = None,
                  v_dense: Optional[torch.Tensor] = None, master_sel: Optional[torch.Tensor] = None):
    """a6 first half: every agent's dense cache, K rotated to its offsets
    (Master given as for :func:`restore_attn`)."""
    N, L, T, H, D = lay.n_agents, shape.n_layers, lay.n_tokens, shape.n_kv_heads, shape.head_dim
    dev_ = lay.device
    mk, mv, msel, mstride = _master_args(shape, lay, master_k, master_v, master_sel)
    if k_dense is None:
        k_dense = torch.empty((N, L, T, H, D), dtype=shape.dtype, device=dev_)
    if v_dense is None:
        v_dense = torch.empty((N, L, T, H, D), dtype=shape.dtype, device=dev_)
    _need(k_dense, "k_dense", shape.dtype, (N, L, T, H, D), dev_)
    _need(v_dense, "v_dense", shape.dtype, (N, L, T, H, D), dev_)
    s, l = shape.c(), lay.c()
    _check(lib().tdx_restore_dense(
        ctypes.byref(s), ctypes.byref(l), _ptr(mk), _ptr(mv), _ptr(msel), mstride, _ptr(diff.off),
        _ptr(diff.idx), _ptr(diff.k), _ptr(diff.v), _ptr(k_dense), _ptr(v_dense), _stream()),
        "tdx_restore_dense")
    return k_dense, v_dense


def restore_transfer_workspace(shape: Shape, lay: RoundLayout, n_req: int, layer_begin: int,
                               layer_end: int) -> int:
    s, l = shape.c(), lay.c()
    return int(lib().tdx_restore_transfer_workspace(ctypes.byref(s), ctypes.byref(l), int(n_req),
                                                    int(layer_begin), int(layer_end)))


def _host_or_device(t: torch.Tensor, name: str, dtype, shape_, dev_):
    """A tensor on the round's device, or a pinned host tensor."""
    if t.device.type == "cpu":
        if not t.is_pinned():
            raise ValueError(f"{name} is in pageable host memory; pin it (pin_memory) or move it to the GPU")
        _need(t, name, dtype, shape_)
    else:
        _need(t, name, dtype, shape_, dev_)


def restore_transfer(shape: Shape, lay: RoundLayout, master_k: torch.Tensor, master_v: torch.Tensor,
                     diff_off: torch.Tensor, diff_idx: torch.Tensor, diff_k: torch.Tensor,
                     diff_v: torch.Tensor, agents: torch.Tensor, layer_begin: int = 0,
                     layer_end: Optional[int] = None, k_out: Optional[torch.Tensor] = None,
                     v_out: Optional[torch.Tensor] = None, ws=None):
    """Transfer-path restore: the requested agents' KV rebuilt layer by layer
    from a Master and diff record that may sit in pinned host memory.  Writes
    layers [layer_begin, layer_end) of k_out / v_out [n_req][L][T][Hkv][D]."""
    N, L, T, H, D = lay.n_agents, shape.n_layers, lay.n_tokens, shape.n_kv_heads, shape.head_dim
    dev_ = lay.device
    layer_end = L if layer_end is None else int(layer_end)
    _need(agents, "agents", torch.int32, None, dev_)
    n_req = agents.numel()
    for t, name in ((master_k, "master_k"), (master_v, "master_v")):
        _host_or_device(t, name, shape.dtype, (L, T, H, D), dev_)
    _host_or_device(diff_off, "diff_off", torch.int32, (N * L + 1,), dev_)
    _host_or_device(diff_idx, "diff_idx", torch.int32, None, dev_)
    for t, name in ((diff_k, "diff_k"), (diff_v, "diff_v")):
        _host_or_device(t, name, shape.dtype, (diff_idx.shape[0], DIFF_BLOCK, H, D), dev_)
    if k_out is None:
        k_out = torch.empty((n_req, L, T, H, D), dtype=shape.dtype, device=dev_)
    if v_out is None:
        v_out = torch.empty((n_req, L, T, H, D), dtype=shape.dtype, device=dev_)
    _need(k_out, "k_out", shape.dtype, (n_req, L, T, H, D), dev_)
    _need(v_out, "v_out", shape.dtype, (n_req, L, T, H, D), dev_)
    if ws is None:
        ws = _ws(restore_transfer_workspace(shape, lay, n_req, layer_begin, layer_end), dev_)
    s, l = shape.c(), lay.c()
    _check(lib().tdx_restore_transfer(
        ctypes.byref(s), ctypes.byref(l), _ptr(master_k), _ptr(master_v), _ptr(diff_off), _ptr(diff_idx),
        _ptr(diff_k), _ptr(diff_v), _ptr(agents), n_req, int(layer_begin), int(layer_end), _ptr(k_out),
        _ptr(v_out), _ptr(ws), ws.numel(), _stream()), "tdx_restore_transfer")
    return k_out, v_out


def decode_attn_dense_workspace(shape: Shape, lay: RoundLayout, max_priv: int) -> int:
    s, l = shape.c(), lay.c()
    return int(lib().tdx_decode_attn_dense_workspace(ctypes.byref(s), ctypes.byref(l), int(max_priv)))


def decode_attn_dense(shape: Shape, lay: RoundLayout, q: torch.Tensor, priv_off: torch.Tensor,
                      priv_k: torch.Tensor, priv_v: torch.Tensor, max_priv: int,
                      k_dense: torch.Tensor, v_dense: torch.Tensor, scale: Optional[float] = None,
                      out: Optional[torch.Tensor] = None, ws=None):
    """a6 second half: plain decode attention over [private; dense shared]."""
    N, L, T, H, Hq, D = (lay.n_agents, shape.n_layers, lay.n_tokens, shape.n_kv_heads,
                         shape.n_q_heads, shape.head_dim)
    dev_ = lay.device
    _need(q, "q", shape.dtype, (N, L, Hq, D), dev_)
    _need(priv_off, "priv_off", torch.int32, (N + 1,), dev_)
    _need(k_dense, "k_dense", shape.dtype, (N, L, T, H, D), dev_)
    _need(v_dense, "v_dense", shape.dtype, (N, L, T, H, D), dev_)
    if out is None:
        out = torch.empty((N, L, Hq, D), dtype=shape.dtype, device=dev_)
    _need(out, "out", shape.dtype, (N, L, Hq, D), dev_)
    if ws is None:
        ws = _ws(decode_attn_dense_workspace(shape, lay, max_priv), dev_)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    s, l = shape.c(), lay.c()
    _check(lib().tdx_decode_attn_dense(
        ctypes.byref(s), ctypes.byref(l), _ptr(q), _ptr(priv_off), _ptr(priv_k), _ptr(priv_v),
        int(max_priv), _ptr(k_dense), _ptr(v_dense), scale, _ptr(out), _ptr(ws), ws.numel(),
        _stream()), "tdx_decode_attn_dense")
    return out


# ---- paged KV layout -------------------------------------------------------------

class PagedKV:
    """A paged view of K (and V) rows: pools [L][n_pages][16][Hkv][D] and a
    device int32 page table [rows][stride] (row r = one sequence's pages in
    token order)."""

    def __init__(self, k_pool: torch.Tensor, v_pool: Optional[torch.Tensor], pages: torch.Tensor):
        if k_pool.dim() != 5 or k_pool.shape[2] != DIFF_BLOCK:
            raise ValueError("a pool is [L][n_pages][16][Hkv][D]")
        _need(k_pool, "k_pool")
        if v_pool is not None:
            _need(v_pool, "v_pool", k_pool.dtype, tuple(k_pool.shape), k_pool.device)
        if pages.dim() != 2:
            raise ValueError("pages is [rows][stride]")
        _need(pages, "pages", torch.int32, None, k_pool.device)
        self.k_pool, self.v_pool, self.pages = k_pool, v_pool, pages
        self._c = CPagedKV(k_pool.data_ptr(), None if v_pool is None else v_pool.data_ptr(), int(k_pool.shape[1]),
                           pages.data_ptr(), int(pages.shape[1]))

    def check(self, shape: Shape, rows: int, per_row: int, device):
        L, H, D = shape.n_layers, shape.n_kv_heads, shape.head_dim
        if self.k_pool.dtype != shape.dtype or self.k_pool.shape[0] != L or tuple(self.k_pool.shape[3:]) != (H, D):
            raise ValueError(f"pool must be [{L}][n_pages][16][{H}][{D}] of {shape.dtype}")
        if self.pages.shape[0] < rows or self.pages.shape[1] < per_row:
            raise ValueError(f"page table must cover {rows} rows of {per_row} pages")
        if _norm(self.k_pool.device) != _norm(device):
            raise ValueError("pool on the wrong device")

    def c(self):
        return ctypes.byref(self._c)


def _pages(n: int) -> int:
    return (int(n) + DIFF_BLOCK - 1) // DIFF_BLOCK


def rerotate_paged(shape: Shape, lay: RoundLayout, cached: PagedKV, out: PagedKV) -> None:
    """a1 over pages: agent i's re-rotated K into the pages of ``out`` row i."""
    cached.check(shape, 1, _pages(lay.n_tokens), lay.device)
    out.check(shape, lay.n_agents, _pages(lay.n_tokens), lay.device)
    s, l = shape.c(), lay.c()
    _check(lib().tdx_rerotate_paged(ctypes.byref(s), ctypes.byref(l), cached.c(), out.c(), _stream()),
           "tdx_rerotate_paged")


def select_important_paged(shape: Shape, lay: RoundLayout, k_reuse: PagedKV, k_recomp: torch.Tensor, k: int,
                           check_layer: int = 0, out: Optional[dict] = None, ws=None) -> dict:
    """a2 + a3 with agent i's re-rotated K in the pages of ``k_reuse`` row i."""
    N, T, H, D = lay.n_agents, lay.n_tokens, shape.n_kv_heads, shape.head_dim
    dev_ = lay.device
    k_reuse.check(shape, N, _pages(T), dev_)
    _need(k_recomp, "k_recomp", shape.dtype, (N, T, H, D), dev_)
    if out is None:
        out = dict(dev=torch.empty((N, T), dtype=torch.float32, device=dev_),
                   score=torch.empty((T,), dtype=torch.float32, device=dev_),
                   agent_dev=torch.empty((N,), dtype=torch.float32, device=dev_),
                   selected=torch.empty((max(int(k), 1),), dtype=torch.int32, device=dev_),
                   master=torch.empty((1,), dtype=torch.int32, device=dev_))
    if ws is None:
        ws = _ws(select_workspace(shape, lay), dev_)
    s, l = shape.c(), lay.c()
    _check(lib().tdx_select_important_paged(
        ctypes.byref(s), ctypes.byref(l), int(check_layer), k_reuse.c(), _ptr(k_recomp), int(k), _ptr(out["dev"]),
        _ptr(out["score"]), _ptr(out["agent_dev"]), _ptr(out["selected"]), _ptr(out["master"]), _ptr(ws),
        ws.numel(), _stream()), "tdx_select_important_paged")
    return out


class PagedDiff:
    """A paged diff record: CSR offsets and block indices, the Mirror's page
    of every entry, and optional value copies."""

    def __init__(self, off, idx, page, k, v, nnz, cap):
        self.off, self.idx, self.page, self.k, self.v = off, idx, page, k, v
        self.nnz_dev = nnz
        self.cap = cap

    def nnz(self) -> int:
        return int(self.nnz_dev.item())


def diff_encode_paged(shape: Shape, lay: RoundLayout, master: torch.Tensor, agents: PagedKV,
                      cap_blocks: Optional[int] = None, copy_values: bool = False, check: bool = True,
                      out: Optional[PagedDiff] = None, ws=None) -> PagedDiff:
    """a4 over pages: each entry names the Mirror's own page of the block."""
    N, L, T, H, D = lay.n_agents, shape.n_layers, lay.n_tokens, shape.n_kv_heads, shape.head_dim
    dev_ = lay.device
    _need(master, "master", torch.int32, (1,), dev_)
    agents.check(shape, N, T // DIFF_BLOCK, dev_)
    if agents.v_pool is None:
        raise ValueError("agents needs a V pool")
    if out is None:
        cap = (N - 1) * L * (T // DIFF_BLOCK) if cap_blocks is None else int(cap_blocks)
        c1 = max(cap, 1)
        out = PagedDiff(torch.empty((N * L + 1,), dtype=torch.int32, device=dev_),
                        torch.empty((c1,), dtype=torch.int32, device=dev_),
                        torch.empty((c1,), dtype=torch.int32, device=dev_),
                        torch.empty((c1, DIFF_BLOCK, H, D), dtype=shape.dtype, device=dev_) if copy_values else None,
                        torch.empty((c1, DIFF_BLOCK, H, D), dtype=shape.dtype, device=dev_) if copy_values else None,
                        torch.empty((1,), dtype=torch.int64, device=dev_), cap)
    if ws is None:
        ws = _ws(encode_workspace(shape, lay), dev_)
    s, l = shape.c(), lay.c()
    _check(lib().tdx_diff_encode_paged(
        ctypes.byref(s), ctypes.byref(l), _ptr(master), agents.c(), int(out.cap), _ptr(out.off), _ptr(out.idx),
        _ptr(out.page), _ptr(out.k), _ptr(out.v), _ptr(out.nnz_dev), _ptr(ws), ws.numel(), _stream()),
        "tdx_diff_encode_paged")
    if check:
        n = out.nnz()
        if n < 0:
            raise TdxError(TDX_EINVAL, "tdx_diff_encode_paged", "the Master index is outside [0, N)")
        if n > out.cap:
            raise TdxError(TDX_EINVAL, "tdx_diff_encode_paged", f"{n} diff blocks exceed capacity {out.cap}")
    return out


def restore_attn_paged(shape: Shape, lay: RoundLayout, q: torch.Tensor, priv_off: torch.Tensor,
                       priv: Optional[PagedKV], max_priv: int, agents: PagedKV, master_sel: Optional[torch.Tensor],
                       diff: PagedDiff, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                       ws=None) -> torch.Tensor:
    """a5 over pages: private history from ``priv`` row i, the Master as row
    ``master_sel[0]`` of ``agents``, diff values from the pages ``diff.page``."""
    N, L, T, Hq, D = lay.n_agents, shape.n_layers, lay.n_tokens, shape.n_q_heads, shape.head_dim
    dev_ = lay.device
    _need(q, "q", shape.dtype, (N, L, Hq, D), dev_)
    _need(priv_off, "priv_off", torch.int32, (N + 1,), dev_)
    if max_priv > 0:
        if priv is None or priv.v_pool is None:
            raise ValueError("priv needs K and V pools")
        priv.check(shape, N, _pages(max_priv), dev_)
    agents.check(shape, N, T // DIFF_BLOCK, dev_)
    if agents.v_pool is None:
        raise ValueError("agents needs a V pool")
    if master_sel is not None:
        _need(master_sel, "master_sel", torch.int32, (1,), dev_)
    if out is None:
        out = torch.empty((N, L, Hq, D), dtype=shape.dtype, device=dev_)
    _need(out, "out", shape.dtype, (N, L, Hq, D), dev_)
    if ws is None:
        ws = _ws(restore_attn_workspace(shape, lay, max_priv), dev_)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    s, l = shape.c(), lay.c()
    _check(lib().tdx_restore_attn_paged(
        ctypes.byref(s), ctypes.byref(l), _ptr(q), _ptr(priv_off), priv.c() if priv is not None else None,
        int(max_priv), agents.c(), _ptr(master_sel), _ptr(diff.off), _ptr(diff.idx), _ptr(diff.page), scale,
        _ptr(out), _ptr(ws), ws.numel(), _stream()), "tdx_restore_attn_paged")
    return out


def _np_ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def round_plan(requests, sep_token: int, min_share: int = 0, slots=None) -> dict:
    """Shared blocks, groups and per-group layouts of one round, from the
    requests' token IDs (host only; ``tdx_round_plan_*``).

    requests: sequence of int token-ID sequences; slots: optional sequence of
    (begin, end) slot ranges, one per request.  Returns dict(groups=[dict(
    agents, seg_ids, blk_start, src_pos, dst_pos [N][B], priv_len)],
    request_group, token_maps) with int32 NumPy arrays.
    """
    reqs = [np.ascontiguousarray(np.asarray(r, dtype=np.int32).reshape(-1)) for r in requests]
    R = len(reqs)
    off = np.zeros(R + 1, dtype=np.int64)
    off[1:] = np.cumsum([r.size for r in reqs])
    tokens = np.ascontiguousarray(np.concatenate(reqs) if R else np.zeros(0, np.int32), dtype=np.int32)
    sb = se = None
    if slots is not None:
        sl = np.asarray(slots, dtype=np.int64).reshape(R, 2)
        sb, se = np.ascontiguousarray(sl[:, 0]), np.ascontiguousarray(sl[:, 1])
    h = ctypes.c_void_p()
    _check(lib().tdx_round_plan_build(_np_ptr(tokens) if tokens.size else None, _np_ptr(off), R, int(sep_token),
                                      int(min_share), _np_ptr(sb), _np_ptr(se), ctypes.byref(h)),
           "tdx_round_plan_build")
    try:
        ng = lib().tdx_round_plan_n_groups(h)
        groups = []
        for g in range(ng):
            n, b, t = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
            _check(lib().tdx_round_plan_group_dims(h, g, ctypes.byref(n), ctypes.byref(b), ctypes.byref(t)),
                   "tdx_round_plan_group_dims")
            N, B = n.value, b.value
            a = dict(agents=np.zeros(N, np.int32), seg_ids=np.zeros(B, np.int32),
                     blk_start=np.zeros(B + 1, np.int32), src_pos=np.zeros(B, np.int32),
                     dst_pos=np.zeros((N, B), np.int32), priv_len=np.zeros(N, np.int32))
            _check(lib().tdx_round_plan_group(h, g, *(_np_ptr(a[k]) for k in (
                "agents", "seg_ids", "blk_start", "src_pos", "dst_pos", "priv_len"))), "tdx_round_plan_group")
            groups.append(a)
        request_group = np.zeros(R, np.int32)
        maps = []
        for r in range(R):
            g = ctypes.c_int32()
            m = np.zeros(reqs[r].size, np.int32)
            _check(lib().tdx_round_plan_request(h, r, ctypes.byref(g), _np_ptr(m)), "tdx_round_plan_request")
            request_group[r] = g.value
            maps.append(m)
    finally:
        lib().tdx_round_plan_free(h)
    return dict(groups=groups, request_group=request_group, token_maps=maps)


def restore_transfer_paged(shape: Shape, lay: RoundLayout, master_k: torch.Tensor, master_v: torch.Tensor,
                           diff_off: torch.Tensor, diff_idx: torch.Tensor, diff_k: torch.Tensor,
                           diff_v: torch.Tensor, agents: torch.Tensor, out: PagedKV, layer_begin: int = 0,
                           layer_end: Optional[int] = None, ws=None) -> None:
    """NEXT-1 into pages: requested agent j's rebuilt K/V (layers
    [layer_begin, layer_end)) into the pages of ``out`` row j.  Sources as for
    ``restore_transfer`` (device memory or pinned host memory)."""
    L, T, H, D = shape.n_layers, lay.n_tokens, shape.n_kv_heads, shape.head_dim
    dev_ = lay.device
    l1 = L if layer_end is None else int(layer_end)
    _need(agents, "agents", torch.int32, None, dev_)
    n_req = agents.numel()
    for name, t, dt, shp in (("master_k", master_k, shape.dtype, (L, T, H, D)),
                             ("master_v", master_v, shape.dtype, (L, T, H, D)),
                             ("diff_off", diff_off, torch.int32, None), ("diff_idx", diff_idx, torch.int32, None),
                             ("diff_k", diff_k, shape.dtype, None), ("diff_v", diff_v, shape.dtype, None)):
        _host_or_device(t, name, dt, shp, dev_)
    out.check(shape, n_req, T // DIFF_BLOCK, dev_)
    if out.v_pool is None:
        raise ValueError("out needs a V pool")
    if ws is None:
        ws = _ws(restore_transfer_workspace(shape, lay, n_req, layer_begin, l1), dev_)
    s, l = shape.c(), lay.c()
    _check(lib().tdx_restore_transfer_paged(
        ctypes.byref(s), ctypes.byref(l), _ptr(master_k), _ptr(master_v), _ptr(diff_off), _ptr(diff_idx),
        _ptr(diff_k), _ptr(diff_v), _ptr(agents), n_req, int(layer_begin), l1, out.c(), _ptr(ws), ws.numel(),
        _stream()), "tdx_restore_transfer_paged")
