"""The C-ABI library loads, exports every entry point include/paged_kv.h declares, and
rejects host-checkable bad arguments before launching anything.  Runs without a GPU:
every call here fails validation on the host (pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

from paged_kv_cache_413_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_kv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libpagedkv.so is not built (run __graft_entry__.build())")
    return B.load()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(B.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def _cache(**kw):
    d = dict(pool=0x1000, num_pages=8, page_size=16, num_kv_heads=2, head_dim=64,
             cache_dtype=B.PKV_BF16)
    d.update(kw)
    return B.PkvCache(d["pool"], d["num_pages"], d["page_size"], d["num_kv_heads"], d["head_dim"],
                      d["cache_dtype"], None, None, None, None)


def _seqs(**kw):
    d = dict(bt=0x2000, ctx=0x3000, num_seqs=2, max_pages=4, max_len=64, window=0)
    d.update(kw)
    return B.PkvSeqs(d["bt"], d["ctx"], d["num_seqs"], d["max_pages"], d["max_len"], d["window"])


def _decode(lib, cache, seqs, q=0x4000, q_dtype=B.PKV_BF16, hq=4, splits=0, out=0x5000, ws=None, wsb=0):
    return lib.paged_attn_decode(ctypes.byref(cache), ctypes.byref(seqs), q, q_dtype, hq, 0.125,
                                 splits, out, None, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(pool=0), B.PKV_EINVAL),
    (dict(pool=0x1004), B.PKV_EINVAL),            # misaligned pool
    (dict(page_size=24), B.PKV_EINVAL),           # not a power of two
    (dict(page_size=1), B.PKV_EINVAL),            # block size must exceed 1
    (dict(num_pages=0), B.PKV_EINVAL),
    (dict(head_dim=96), B.PKV_EUNSUPPORTED),
    (dict(cache_dtype=7), B.PKV_EINVAL),
])
def test_bad_cache_rejected(lib, kw, code):
    assert _decode(lib, _cache(**kw), _seqs()) == code
    assert lib.paged_kv_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(bt=0), B.PKV_EINVAL),
    (dict(ctx=0), B.PKV_EINVAL),
    (dict(max_len=65), B.PKV_EINVAL),             # > max_pages * page_size
    (dict(max_len=0), B.PKV_EINVAL),
    (dict(window=-1), B.PKV_EINVAL),
    (dict(num_seqs=-1), B.PKV_EINVAL),
])
def test_bad_seqs_rejected(lib, kw, code):
    assert _decode(lib, _cache(), _seqs(**kw)) == code


def test_bad_attention_args_rejected(lib):
    c, s = _cache(), _seqs()
    assert _decode(lib, c, s, hq=3) == B.PKV_EINVAL            # not a multiple of Hkv
    assert _decode(lib, c, s, hq=64) == B.PKV_EUNSUPPORTED     # group 32
    assert _decode(lib, c, s, q_dtype=B.PKV_FP8_E4M3) == B.PKV_EINVAL
    assert _decode(lib, c, s, q=0) == B.PKV_EINVAL
    assert _decode(lib, c, s, out=0x5002) == B.PKV_EINVAL      # misaligned
    assert _decode(lib, c, s, splits=-1) == B.PKV_EINVAL
    # a fixed split count needs a workspace
    assert _decode(lib, c, s, splits=4) == B.PKV_EWORKSPACE
    need = lib.paged_attn_decode_workspace_size(ctypes.byref(c), ctypes.byref(s), B.PKV_BF16, 4, 4)
    assert need > 0
    assert _decode(lib, c, s, splits=4, ws=0x100000, wsb=need - 1) == B.PKV_EWORKSPACE
    # FP8 caches need their scales
    c8 = _cache(cache_dtype=B.PKV_FP8_E4M3)
    assert _decode(lib, c8, s) == B.PKV_EINVAL
    assert "scale" in lib.paged_kv_last_error().decode()


def test_empty_batch_is_a_noop(lib):
    c = _cache()
    s = _seqs(num_seqs=0, bt=0, ctx=0)
    assert _decode(lib, c, s) == B.PKV_OK
    assert lib.kv_append(ctypes.byref(c), ctypes.byref(_seqs()), 0x4000, 0x4000, 0x6000, 0, None) == B.PKV_OK


def test_append_rejects_bad_args(lib):
    c, s = _cache(), _seqs()
    assert lib.kv_append(ctypes.byref(c), ctypes.byref(s), 0, 0x4000, 0x6000, 4, None) == B.PKV_EINVAL
    assert lib.kv_append(ctypes.byref(c), ctypes.byref(s), 0x4000, 0x4000, 0x6000, -1, None) == B.PKV_EINVAL
    c8 = _cache(cache_dtype=B.PKV_FP8_E4M3)
    assert lib.kv_append(ctypes.byref(c8), ctypes.byref(s), 0x4000, 0x4000, 0x6000, 4, None) == B.PKV_EINVAL


def test_prefill_rejects_bad_args(lib):
    c, s = _cache(), _seqs()
    f = lambda **k: lib.paged_attn_prefill_chunk(
        ctypes.byref(c), ctypes.byref(s), k.get("q", 0x4000), B.PKV_BF16, k.get("cu", 0x6000),
        k.get("tq", 8), k.get("mq", 4), 4, 0.125, 0x5000, None, None, 0, None)
    assert f(cu=0) == B.PKV_EINVAL
    assert f(mq=0) == B.PKV_EINVAL
    assert f(mq=65) == B.PKV_EINVAL
    assert f(tq=-1) == B.PKV_EINVAL
    assert f(tq=0) == B.PKV_OK


def test_copy_pages_rejects_bad_args(lib):
    c = _cache()
    f = lambda src=0x7000, dst=0x7100, n=2, cache=c: lib.kv_copy_pages(ctypes.byref(cache), src, dst, n, None)
    assert f(n=-1) == B.PKV_EINVAL
    assert f(src=0) == B.PKV_EINVAL
    assert f(dst=0) == B.PKV_EINVAL
    assert f(n=65536) == B.PKV_EINVAL
    assert f(cache=_cache(pool=0)) == B.PKV_EINVAL
    assert f(n=0, src=0, dst=0) == B.PKV_OK          # nothing to copy: no launch


def test_page_bytes(lib):
    f = lambda dt, P, H, D: lib.paged_kv_page_bytes(dt, P, H, D)
    assert f(B.PKV_BF16, 64, 8, 128) == 2 * 8 * 64 * 128 * 2
    assert f(B.PKV_FP8_E4M3, 64, 8, 128) == 2 * 8 * 64 * 128
    assert f(B.PKV_MXFP4, 64, 8, 128) == 2 * 8 * (64 * 128 // 2 + 64 * 128 // 32)   # 17/32 byte each
    assert f(B.PKV_MXFP4, 32, 2, 64) == 2 * 2 * (32 * 64 * 17 // 32)
    assert f(B.PKV_MXFP4, 16, 8, 128) == 0       # MXFP4 needs pages of >= 32 tokens
    assert f(B.PKV_BF16, 24, 8, 128) == 0
    assert f(7, 64, 8, 128) == 0


def test_mxfp4_cache_rules(lib):
    assert _decode(lib, _cache(cache_dtype=B.PKV_MXFP4, page_size=16), _seqs()) == B.PKV_EUNSUPPORTED
    c = _cache(cache_dtype=B.PKV_MXFP4, page_size=32)
    s = _seqs(max_pages=4, max_len=64)
    assert _decode(lib, c, s, q_dtype=B.PKV_F32) == B.PKV_EUNSUPPORTED   # matrix-core path only
    assert _decode(lib, c, s, hq=6) == B.PKV_EUNSUPPORTED                 # group 3
    need = lib.paged_attn_decode_workspace_size(ctypes.byref(c), ctypes.byref(s), B.PKV_BF16, 4, 0)
    assert need > 0
