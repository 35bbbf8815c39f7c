"""CPU checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments on the host before touching the GPU."""
import ctypes
import os
import re
import subprocess

import pytest

import token_level_sparse_hs_amd as hs
from token_level_sparse_hs_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hysparse.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from token_level_sparse_hs_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hs_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_api():
    names = declared_functions()
    assert names == sorted(_lib.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if " T " in l)
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_version_and_status_strings(lib):
    ver = int(re.search(r"#define HS_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lib.hs_version() == ver
    for st in range(6):
        assert lib.hs_status_string(st)
    assert lib.hs_status_string(99) == b"unknown status"


def test_shape_struct_matches_header():
    # 9 int32 + float + 4 int64 + 2 uint32 with natural alignment
    assert ctypes.sizeof(_lib.HsShape) == 80


def base_shape(**kw):
    d = dict(batch=1, n_q=64, n_kv=64, kv_capacity=64, q_heads=8, kv_heads=2, top_k=16, window=8)
    d.update(kw)
    return hs.make_shape(**d)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), _lib.HS_ERR_INVALID_ARG),
    (dict(head_dim=64), _lib.HS_ERR_UNSUPPORTED),
    (dict(q_heads=6, kv_heads=4), _lib.HS_ERR_INVALID_ARG),
    (dict(q_heads=48, kv_heads=3), _lib.HS_ERR_UNSUPPORTED),
    (dict(top_k=-1), _lib.HS_ERR_INVALID_ARG),
    (dict(top_k=9000), _lib.HS_ERR_INVALID_ARG),
    (dict(window=0), _lib.HS_ERR_INVALID_ARG),
    (dict(n_q=65), _lib.HS_ERR_INVALID_ARG),
    (dict(n_kv=65), _lib.HS_ERR_INVALID_ARG),
    (dict(flags=32), _lib.HS_ERR_INVALID_ARG),
    (dict(flags=_lib.HS_FLAG_HEAD_UNION | _lib.HS_FLAG_PROB_SCORE), _lib.HS_ERR_UNSUPPORTED),
    (dict(flags=_lib.HS_FLAG_BLOCK_SELECT), _lib.HS_ERR_INVALID_ARG),  # top_k 16 is not whole blocks
    (dict(flags=_lib.HS_FLAG_BLOCK_SELECT | _lib.HS_FLAG_PROB_SCORE, top_k=64), _lib.HS_ERR_UNSUPPORTED),
    (dict(kv_strides=(0, 0, 12, 0)), _lib.HS_ERR_INVALID_ARG),
])
def test_invalid_shapes_rejected_before_launch(lib, kw, status):
    s = base_shape(**kw)
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    st = lib.hs_full_attn_select(ctypes.byref(s), fake, fake, fake, None, fake, fake, 1 << 30, None)
    assert st == status, lib.hs_last_error()
    assert lib.hs_last_error()


def test_null_pointers_and_workspace(lib):
    s = base_shape()
    fake = ctypes.c_void_p(1 << 20)
    assert lib.hs_full_attn_select(ctypes.byref(s), None, fake, fake, None, fake, fake, 1 << 30, None) == _lib.HS_ERR_INVALID_ARG
    assert lib.hs_full_attn_select(ctypes.byref(s), fake, fake, fake, None, None, fake, 1 << 30, None) == _lib.HS_ERR_INVALID_ARG
    need = _lib.workspace_size(_lib.HS_OP_FULL_ATTN_SELECT, s)
    assert need > 0
    st = lib.hs_full_attn_select(ctypes.byref(s), fake, fake, fake, None, fake, fake, need - 1, None)
    assert st == _lib.HS_ERR_WORKSPACE
    mis = ctypes.c_void_p((1 << 20) + 8)
    assert lib.hs_full_attn_select(ctypes.byref(s), mis, fake, fake, None, fake, fake, need, None) == _lib.HS_ERR_INVALID_ARG
    sd = base_shape(n_q=1)
    assert lib.hs_decode_step(ctypes.byref(sd), fake, fake, fake, None, 64, fake, None, fake, fake, 1 << 30, None) == _lib.HS_ERR_INVALID_ARG
    assert lib.hs_decode_step(ctypes.byref(sd), fake, fake, fake, fake, 65, fake, None, fake, fake, 1 << 30, None) == _lib.HS_ERR_INVALID_ARG
    sp = base_shape(n_q=2)
    assert lib.hs_sparse_attn_reuse(ctypes.byref(sp), fake, fake, fake, fake, fake, fake, 1 << 30, None) == _lib.HS_ERR_INVALID_ARG


def test_head_union_index_rows(lib):
    """Under the per-head union the sparse layers read rows of G * top_k
    entries: their decode workspace follows that row length."""
    s = base_shape(batch=1, n_q=1, n_kv=0, kv_capacity=1 << 17, q_heads=8, kv_heads=1, top_k=512, window=64)
    su = base_shape(batch=1, n_q=1, n_kv=0, kv_capacity=1 << 17, q_heads=8, kv_heads=1, top_k=512, window=64,
                    flags=_lib.HS_FLAG_HEAD_UNION)
    wide = base_shape(batch=1, n_q=1, n_kv=0, kv_capacity=1 << 17, q_heads=8, kv_heads=1, top_k=4096, window=64)
    a = _lib.workspace_size(_lib.HS_OP_SPARSE_ATTN_REUSE, su, 1 << 17)
    assert a == _lib.workspace_size(_lib.HS_OP_SPARSE_ATTN_REUSE, wide, 1 << 17)
    assert a > _lib.workspace_size(_lib.HS_OP_SPARSE_ATTN_REUSE, s, 1 << 17)
    # prefill: the G one-head passes need the heads' lists on top of a pass's workspace
    p = base_shape(n_q=64, n_kv=64, q_heads=8, kv_heads=2, top_k=16, window=8, flags=_lib.HS_FLAG_HEAD_UNION)
    assert _lib.workspace_size(_lib.HS_OP_FULL_ATTN_SELECT, p) >= 4 * 64 * 2 * 16 * 4


def test_workspace_sizes(lib):
    s = base_shape(top_k=0)
    assert _lib.workspace_size(_lib.HS_OP_FULL_ATTN_SELECT, s) == 0
    s = base_shape(n_q=1)
    assert _lib.workspace_size(_lib.HS_OP_SPARSE_ATTN_REUSE, s, 0) == 0
    # decode sparse: one split per row needs no merge buffer; a long row split
    # over many waves does; a batch of 256 (b, g) rows merges inside blocks
    assert _lib.workspace_size(_lib.HS_OP_SPARSE_ATTN_REUSE, s, 64) == 0
    s_long = base_shape(n_q=1, n_kv=0, kv_capacity=1 << 17, top_k=2048, window=512)
    assert _lib.workspace_size(_lib.HS_OP_SPARSE_ATTN_REUSE, s_long, 1 << 17) > 0
    s_batch = base_shape(batch=64, n_q=1, n_kv=0, kv_capacity=1 << 17, q_heads=32, kv_heads=4, top_k=2048,
                         window=512)
    assert _lib.workspace_size(_lib.HS_OP_SPARSE_ATTN_REUSE, s_batch, 1 << 17) == 0
    assert _lib.workspace_size(_lib.HS_OP_DECODE_STEP, s, 64) > 0
    with pytest.raises(_lib.HsError):
        _lib.workspace_size(_lib.HS_OP_DECODE_STEP, s, 0)
    # large workload sizes stay within the memory of one GPU
    big = hs.make_shape(batch=1, n_q=16384, n_kv=1064960, kv_capacity=1064976, q_heads=32, kv_heads=4,
                        top_k=4096, window=1024)
    assert _lib.workspace_size(_lib.HS_OP_FULL_ATTN_SELECT, big) < 16 << 30


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libhysparse.so"))
    with pytest.raises(ImportError):
        _lib.load()


def test_select_diagnostics_offsets(lib):
    """The selection records lie inside the workspace, one int32 per row then
    two uint32 counters; shapes without such records are rejected."""
    s = base_shape(n_q=300, n_kv=900, kv_capacity=900)
    ws = _lib.workspace_size(_lib.HS_OP_FULL_ATTN_SELECT, s)
    a, b, c = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    _lib.check(lib.hs_select_diagnostics(ctypes.byref(s), ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    rows = s.batch * s.n_q * s.kv_heads
    assert b.value == a.value + 4 * rows and c.value == b.value + 4 and c.value + 4 <= ws
    for flags in (hs.HS_FLAG_BLOCK_SELECT, hs.HS_FLAG_HEAD_UNION):
        s2 = base_shape(top_k=64, flags=flags)
        assert lib.hs_select_diagnostics(ctypes.byref(s2), ctypes.byref(a), ctypes.byref(b),
                                         ctypes.byref(c)) == _lib.HS_ERR_UNSUPPORTED
    s3 = base_shape(top_k=0)
    assert lib.hs_select_diagnostics(ctypes.byref(s3), ctypes.byref(a), ctypes.byref(b),
                                     ctypes.byref(c)) == _lib.HS_ERR_UNSUPPORTED
    assert lib.hs_select_diagnostics(ctypes.byref(s), None, ctypes.byref(b),
                                     ctypes.byref(c)) == _lib.HS_ERR_INVALID_ARG


def test_kv_bridge_arguments_rejected_before_launch(lib):
    """hs_kv_bridge validates on the host: d_model a multiple of 64, rows
    inside the cache, non-NULL aligned pointers."""
    fake = ctypes.c_void_p(1 << 20)
    s = base_shape(n_q=32, n_kv=64, kv_capacity=64)
    for d_model, status in ((100, _lib.HS_ERR_UNSUPPORTED), (0, _lib.HS_ERR_UNSUPPORTED),
                            (70000, _lib.HS_ERR_UNSUPPORTED)):
        assert lib.hs_kv_bridge(ctypes.byref(s), fake, d_model, fake, fake, None) == status, lib.hs_last_error()
    assert lib.hs_kv_bridge(ctypes.byref(s), None, 128, fake, fake, None) == _lib.HS_ERR_INVALID_ARG
    mis = ctypes.c_void_p((1 << 20) + 8)
    assert lib.hs_kv_bridge(ctypes.byref(s), fake, 128, mis, fake, None) == _lib.HS_ERR_INVALID_ARG
    s2 = base_shape(n_q=65, n_kv=64, kv_capacity=64)
    assert lib.hs_kv_bridge(ctypes.byref(s2), fake, 128, fake, fake, None) == _lib.HS_ERR_INVALID_ARG
    s3 = base_shape(n_q=1, n_kv=64, kv_capacity=64, flags=_lib.HS_FLAG_FP8_KV)
    assert lib.hs_kv_bridge(ctypes.byref(s3), fake, 128, fake, fake, None) == _lib.HS_ERR_UNSUPPORTED
