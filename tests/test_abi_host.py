"""C-ABI host checks (no GPU): the library loads, exports every declared
symbol, and rejects bad arguments before anything reaches the HIP runtime."""

import ctypes
import math
import os
import re
from fractions import Fraction

import pytest

from collective_kv_cache_amd import tdx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tdx.h")

pytestmark = pytest.mark.skipif(not os.path.exists(tdx.LIB_PATH), reason="libtdx.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tdx_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(tdx.EXPORTED)


def test_every_declared_symbol_is_exported():
    l = ctypes.CDLL(tdx.LIB_PATH)
    for name in declared_functions():
        assert hasattr(l, name), name


def test_version_and_strerror():
    assert tdx.version() == 10000
    assert tdx.strerror(0) == "success"
    assert tdx.strerror(-1) == "invalid argument"
    assert tdx.strerror(-5).startswith("workspace")
    assert tdx.strerror(123) == "unknown error code"


def test_topk_count_is_integer_ceiling():
    for T in (1, 2, 7, 100, 192, 3744, 5536, 20000):
        for pct in (0, 1, 15, 50, 99, 100):
            want = min(max(math.ceil(Fraction(pct * T, 100)), 1), T)
            assert tdx.topk_count(pct, T) == want
    assert tdx.topk_count(15, 0) == 0 and tdx.topk_count(-1, 10) == 0 and tdx.topk_count(101, 10) == 0


FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: calls fail validation first


def _shape(**kw):
    d = dict(n_layers=2, n_kv_heads=4, n_q_heads=28, head_dim=128, dtype=tdx.TDX_BF16, rope_theta=1e6)
    d.update(kw)
    return tdx.CShape(**d)


def _layout(**kw):
    d = dict(n_agents=3, n_blocks=2, n_tokens=64, blk_start=0x20000, src_pos=0x30000, dst_pos=0x40000)
    d.update(kw)
    return tdx.CLayout(**d)


def _rerotate(shape, lay, kc=FAKE, out=FAKE):
    return tdx.lib().tdx_rerotate(ctypes.byref(shape) if shape is not None else None,
                                  ctypes.byref(lay) if lay is not None else None, kc, out, None)


@pytest.mark.parametrize("shape_kw,lay_kw,code", [
    (dict(dtype=7), {}, tdx.TDX_EINVAL),
    (dict(head_dim=96), {}, tdx.TDX_EUNSUPPORTED),
    (dict(n_q_heads=30), {}, tdx.TDX_EINVAL),
    (dict(n_layers=0), {}, tdx.TDX_EINVAL),
    (dict(rope_theta=1.0), {}, tdx.TDX_EINVAL),
    (dict(n_kv_heads=32, n_q_heads=32), {}, tdx.TDX_EUNSUPPORTED),
    ({}, dict(n_agents=0), tdx.TDX_EINVAL),
    ({}, dict(n_tokens=0), tdx.TDX_EINVAL),
    ({}, dict(n_agents=2000), tdx.TDX_EUNSUPPORTED),
    ({}, dict(blk_start=0), tdx.TDX_EINVAL),
    ({}, dict(dst_pos=0x40002), tdx.TDX_EINVAL),
])
def test_rerotate_rejects_bad_arguments(shape_kw, lay_kw, code):
    assert _rerotate(_shape(**shape_kw), _layout(**lay_kw)) == code
    assert tdx.lib().tdx_last_error().decode() != ""


def test_rerotate_rejects_null_and_unaligned_tensors():
    assert _rerotate(None, _layout()) == tdx.TDX_EINVAL
    assert _rerotate(_shape(), None) == tdx.TDX_EINVAL
    assert _rerotate(_shape(), _layout(), kc=None) == tdx.TDX_EINVAL
    assert _rerotate(_shape(), _layout(), out=ctypes.c_void_p(0x10008)) == tdx.TDX_EINVAL
    assert "k_out" in tdx.lib().tdx_last_error().decode()


def _select(k=5, check_layer=0, ws_bytes=1 << 20, ws=FAKE):
    s, l = _shape(), _layout()
    return tdx.lib().tdx_select_important(ctypes.byref(s), ctypes.byref(l), check_layer, FAKE, FAKE, k,
                                          FAKE, FAKE, FAKE, FAKE, FAKE, ws, ws_bytes, None)


def test_select_rejects_bad_arguments():
    assert _select(k=0) == tdx.TDX_EINVAL
    assert _select(k=65) == tdx.TDX_EINVAL
    assert _select(check_layer=2) == tdx.TDX_EINVAL
    assert _select(ws_bytes=0) == tdx.TDX_EWORKSPACE
    assert _select(ws=None) == tdx.TDX_EWORKSPACE


def test_workspace_queries_are_positive_and_grow():
    s, l = _shape(), _layout()
    a = tdx.lib().tdx_select_workspace(ctypes.byref(s), ctypes.byref(l))
    b = tdx.lib().tdx_diff_encode_workspace(ctypes.byref(s), ctypes.byref(l))
    c = tdx.lib().tdx_restore_attn_workspace(ctypes.byref(s), ctypes.byref(l), 100)
    assert a > 0 and b > 0 and c > 0
    l2 = _layout(n_agents=30)
    assert tdx.lib().tdx_diff_encode_workspace(ctypes.byref(s), ctypes.byref(l2)) > b
    bad = _shape(head_dim=96)
    assert tdx.lib().tdx_select_workspace(ctypes.byref(bad), ctypes.byref(l)) == 0


def _encode(T=64, cap=10, nnz=FAKE, mk=FAKE, mv=FAKE, ws_bytes=1 << 30):
    s, l = _shape(), _layout(n_tokens=T)
    return tdx.lib().tdx_diff_encode(ctypes.byref(s), ctypes.byref(l), FAKE, FAKE, FAKE, cap, FAKE, FAKE,
                                     FAKE, FAKE, nnz, mk, mv, FAKE, ws_bytes, None)


def test_encode_rejects_bad_arguments():
    assert _encode(T=60) == tdx.TDX_EINVAL           # not a multiple of 16
    assert _encode(cap=-1) == tdx.TDX_EINVAL
    assert _encode(nnz=ctypes.c_void_p(0x10004)) == tdx.TDX_EINVAL
    assert _encode(mv=None) == tdx.TDX_EINVAL        # one Master output without the other
    assert _encode(ws_bytes=0) == tdx.TDX_EWORKSPACE


def _restore(T=64, scale=0.1, max_priv=10, ws_bytes=1 << 30, hq=28, msel=None, mstride=0, L=2):
    s, l = _shape(n_q_heads=hq, n_layers=L), _layout(n_tokens=T)
    return tdx.lib().tdx_restore_attn(ctypes.byref(s), ctypes.byref(l), FAKE, FAKE, FAKE, FAKE, max_priv,
                                      FAKE, FAKE, msel, mstride, FAKE, FAKE, FAKE, FAKE,
                                      ctypes.c_float(scale), FAKE, FAKE, ws_bytes, None)


def _restore_dense(msel=None, mstride=0):
    s, l = _shape(), _layout(n_tokens=64)
    return tdx.lib().tdx_restore_dense(ctypes.byref(s), ctypes.byref(l), FAKE, FAKE, msel, mstride, FAKE,
                                       FAKE, FAKE, FAKE, FAKE, FAKE, None)


def test_restore_rejects_bad_arguments():
    assert _restore(T=40) == tdx.TDX_EINVAL
    assert _restore(scale=0.0) == tdx.TDX_EINVAL
    assert _restore(max_priv=-1) == tdx.TDX_EINVAL
    assert _restore(ws_bytes=0) == tdx.TDX_EWORKSPACE
    assert _restore(hq=4 * 17) == tdx.TDX_EUNSUPPORTED  # 17 query heads per KV head
    # the tiles the call plans, N * L * (ceil(max_priv / 16) + T / 16), must fit in 31 bits
    # (3 agents x 8 layers x 134217728 tiles here; 2 layers would still fit)
    assert _restore(max_priv=2**31 - 1, L=8) == tdx.TDX_EUNSUPPORTED
    assert "tiles" in tdx.lib().tdx_last_error().decode()
    s, l = _shape(n_layers=8), _layout(n_tokens=64)
    assert tdx.lib().tdx_restore_attn_workspace(ctypes.byref(s), ctypes.byref(l), 2**31 - 1) == 0
    assert tdx.lib().tdx_decode_attn_dense_workspace(ctypes.byref(s), ctypes.byref(l), 2**31 - 1) == 0
    # the Master selector: aligned pointer, stride >= 0 keeping 16-byte alignment (bf16: % 8)
    assert _restore(msel=ctypes.c_void_p(0x10002)) == tdx.TDX_EINVAL
    assert _restore(msel=FAKE, mstride=-8) == tdx.TDX_EINVAL
    assert _restore(msel=FAKE, mstride=12) == tdx.TDX_EINVAL
    assert _restore_dense(msel=FAKE, mstride=12) == tdx.TDX_EINVAL
    assert _restore_dense(msel=ctypes.c_void_p(0x10001)) == tdx.TDX_EINVAL


def _transfer(T=64, n_req=2, l0=0, l1=2, ws_bytes=1 << 30, agents=FAKE, mk=FAKE):
    s, l = _shape(), _layout(n_tokens=T)
    return tdx.lib().tdx_restore_transfer(ctypes.byref(s), ctypes.byref(l), mk, FAKE, FAKE, FAKE, FAKE, FAKE,
                                          agents, n_req, l0, l1, FAKE, FAKE, FAKE, ws_bytes, None)


def test_transfer_rejects_bad_arguments():
    # every check here fails before the pointers are inspected or anything is enqueued
    assert _transfer(T=40) == tdx.TDX_EINVAL          # not a multiple of 16
    assert _transfer(n_req=0) == tdx.TDX_EINVAL
    assert _transfer(l0=1, l1=1) == tdx.TDX_EINVAL    # empty layer range
    assert _transfer(l0=-1) == tdx.TDX_EINVAL
    assert _transfer(l1=3) == tdx.TDX_EINVAL          # past n_layers = 2
    assert _transfer(agents=ctypes.c_void_p(0x10002)) == tdx.TDX_EINVAL
    assert _transfer(mk=None) == tdx.TDX_EINVAL
    assert _transfer(ws_bytes=0) == tdx.TDX_EWORKSPACE
    s, l = _shape(), _layout(n_tokens=64)
    w1 = tdx.lib().tdx_restore_transfer_workspace(ctypes.byref(s), ctypes.byref(l), 1, 0, 1)
    w2 = tdx.lib().tdx_restore_transfer_workspace(ctypes.byref(s), ctypes.byref(l), 3, 0, 2)
    assert 0 < w1 < w2
    assert tdx.lib().tdx_restore_transfer_workspace(ctypes.byref(s), ctypes.byref(l), 1, 0, 3) == 0


def _paged(k_pool=FAKE, v_pool=FAKE, n_pages=8, pages=0x50000, stride=4):
    return tdx.CPagedKV(k_pool, v_pool, n_pages, pages, stride)


def test_paged_calls_reject_bad_arguments():
    s, l = _shape(), _layout(n_tokens=64)  # N = 3 rows of 4 pages
    L = tdx.lib()

    def rer(cached, out):
        return L.tdx_rerotate_paged(ctypes.byref(s), ctypes.byref(l), ctypes.byref(cached) if cached else None,
                                    ctypes.byref(out) if out else None, None)
    assert rer(None, _paged()) == tdx.TDX_EINVAL
    assert rer(_paged(k_pool=None), _paged()) == tdx.TDX_EINVAL
    assert rer(_paged(), _paged(n_pages=0)) == tdx.TDX_EINVAL
    assert rer(_paged(), _paged(stride=3)) == tdx.TDX_EINVAL        # 3 rows need >= 4 pages each
    assert rer(_paged(), _paged(pages=0x50002)) == tdx.TDX_EINVAL   # page table not 4-byte aligned
    assert rer(_paged(), _paged(k_pool=ctypes.c_void_p(0x10008))) == tdx.TDX_EINVAL
    assert "stride" in L.tdx_last_error().decode() or "aligned" in L.tdx_last_error().decode()

    def enc(agents, diff_k=None, diff_v=None, ws_bytes=1 << 30):
        return L.tdx_diff_encode_paged(ctypes.byref(s), ctypes.byref(l), FAKE, ctypes.byref(agents), 10, FAKE,
                                       FAKE, FAKE, diff_k, diff_v, FAKE, FAKE, ws_bytes, None)
    assert enc(_paged(v_pool=None)) == tdx.TDX_EINVAL                # encode compares V too
    assert enc(_paged(), diff_k=FAKE) == tdx.TDX_EINVAL              # value copies: both or neither
    assert enc(_paged(), ws_bytes=0) == tdx.TDX_EWORKSPACE

    def att(priv, max_priv, agents):
        return L.tdx_restore_attn_paged(ctypes.byref(s), ctypes.byref(l), FAKE, FAKE,
                                        ctypes.byref(priv) if priv else None, max_priv, ctypes.byref(agents), None,
                                        FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, FAKE, 1 << 30, None)
    assert att(None, 10, _paged()) == tdx.TDX_EINVAL                 # private history needs its pools
    assert att(_paged(stride=0), 40, _paged()) == tdx.TDX_EINVAL     # 40 tokens = 3 pages per row
    assert att(_paged(), 10, _paged(v_pool=None)) == tdx.TDX_EINVAL


def test_paged_transfer_rejects_bad_arguments():
    s, l = _shape(), _layout(n_tokens=64)
    L = tdx.lib()

    def tr(out, n_req=2):
        return L.tdx_restore_transfer_paged(ctypes.byref(s), ctypes.byref(l), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                            FAKE, n_req, 0, 2, ctypes.byref(out) if out else None, FAKE, 1 << 30,
                                            None)
    assert tr(None) == tdx.TDX_EINVAL
    assert tr(_paged(v_pool=None)) == tdx.TDX_EINVAL   # K and V are both written
    assert tr(_paged(stride=3)) == tdx.TDX_EINVAL      # 2 rows of 4 pages
    assert tr(_paged(), n_req=0) == tdx.TDX_EINVAL


def test_noalloc_select_rejects_rounds_beyond_its_scratch():
    # N * ceil(T/8) * 8 bytes above TDX_SELECT_SCRATCH_BYTES: refused before
    # anything reaches the HIP runtime (aligned fake pointers, never read)
    big = _layout(n_agents=1024, n_blocks=4, n_tokens=8192)
    rc = tdx.lib().tdx_select_important_noalloc(ctypes.byref(_shape(n_layers=1)), ctypes.byref(big), 0, FAKE, FAKE,
                                                10, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert rc == tdx.TDX_EUNSUPPORTED
    assert b"scratch" in tdx.lib().tdx_last_error()
    # and the shared argument checks run first
    rc = tdx.lib().tdx_select_important_noalloc(ctypes.byref(_shape(n_layers=1)), ctypes.byref(big), 1, FAKE, FAKE,
                                                10, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert rc == tdx.TDX_EINVAL
