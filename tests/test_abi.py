"""The C ABI without a GPU: libkivi.so loads, exports every function that
include/kivi.h declares, and rejects invalid arguments on the host before any
HIP call (so these tests never touch a device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kivi.h")
LIB = os.path.join(ROOT, "decode_attention_pack_amd", "libkivi.so")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kivi_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB):
        from decode_attention_pack_amd import build
        build.build()
    from decode_attention_pack_amd import kivi
    return kivi.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert {"kivi_pack_keys", "kivi_pack_values", "kivi_append", "kivi_decode_attn"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    from decode_attention_pack_amd import kivi
    assert set(kivi.EXPORTED) == set(names)


def test_status_strings(L):
    assert L.kivi_status_string(0) == b"ok"
    assert L.kivi_status_string(-3) == b"workspace too small"
    assert L.kivi_status_string(7) == b"unknown status"


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def _cache(**kw):
    from decode_attention_pack_amd.kivi import CCache
    a = dict(batch=1, n_kv_heads=2, head_dim=128, k_bits=2, v_bits=2, group=32, residual=128,
             capacity=1024, n_tokens=0, blocks=0x1000, k_res=0x1000, v_res=0x1000)
    a.update(kw)
    return CCache(a["batch"], a["n_kv_heads"], a["head_dim"], a["k_bits"], a["v_bits"], a["group"],
                  a["residual"], a["capacity"], a["n_tokens"], a["blocks"], a["k_res"], a["v_res"])


def test_record_bytes(L):
    """Record size of the packed store (include/kivi.h): 14336 bytes at 2-bit,
    G 32, head_dim 128 (4096 + 2048 + 1024 + 4096 + 2048 + 1024); 0 for
    shapes outside the layout."""
    assert L.kivi_record_bytes(128, 2, 2, 32) == 14336
    assert L.kivi_record_bytes(128, 4, 4, 32) == 8192 + 2048 + 1024 + 8192 + 2048 + 1024
    assert L.kivi_record_bytes(64, 2, 4, 64) == 2048 + 512 + 256 + 4096 + 512 + 256
    for bad in [(128, 3, 2, 32), (128, 2, 2, 48), (100, 2, 2, 32), (512, 2, 2, 32), (128, 2, 2, 8)]:
        assert L.kivi_record_bytes(*bad) == 0, bad


def _pack(L, fn, cache=None, x=FAKE, T=64, off=0):
    c = _cache() if cache is None else cache
    return getattr(L, fn)(ctypes.byref(c), x, T, off, None)


@pytest.mark.parametrize("kw,status", [
    (dict(cache=_cache(k_bits=3)), -1), (dict(cache=_cache(k_bits=8)), -1),
    (dict(cache=_cache(group=24)), -1), (dict(cache=_cache(group=48)), -1),
    (dict(cache=_cache(head_dim=100)), -1), (dict(cache=_cache(head_dim=512)), -1),
    (dict(T=33), -1), (dict(off=16), -1), (dict(cache=_cache(capacity=1000)), -1),
    (dict(T=-1), -1), (dict(cache=_cache(batch=0)), -1), (dict(T=96, off=960), -2),
    (dict(x=None), -1), (dict(cache=_cache(batch=65536, n_kv_heads=1)), -1),
    (dict(cache=_cache(batch=256, n_kv_heads=256)), -1),
    (dict(cache=_cache(blocks=0x1008)), -1), (dict(cache=_cache(blocks=0)), -1),
])
def test_pack_keys_rejects(L, kw, status):
    assert _pack(L, "kivi_pack_keys", **kw) == status
    assert L.kivi_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(cache=_cache(v_bits=1)), -1), (dict(cache=_cache(group=12, v_bits=4, k_bits=4)), -1),
    (dict(T=1025), -2), (dict(T=65, off=960), -2),
])
def test_pack_values_rejects(L, kw, status):
    assert _pack(L, "kivi_pack_values", **kw) == status


def test_zero_tokens_is_a_no_op(L):
    # valid arguments with T == 0 return before any launch
    assert _pack(L, "kivi_pack_keys", T=0) == 0
    assert _pack(L, "kivi_pack_values", T=0) == 0


@pytest.mark.parametrize("kw", [dict(k_bits=3), dict(v_bits=5), dict(residual=48),
                                dict(capacity=1000), dict(capacity=288, residual=96),
                                dict(n_tokens=-1), dict(n_tokens=2048),
                                dict(batch=0), dict(head_dim=100), dict(group=20),
                                dict(batch=32768, n_kv_heads=2), dict(k_res=0x1004),
                                dict(v_res=0x1002), dict(blocks=0x1001)])
def test_append_rejects_bad_cache(L, kw):
    c = _cache(**kw)
    assert L.kivi_append(ctypes.byref(c), FAKE, FAKE, 1, None) == -1


def test_append_capacity_and_no_op(L):
    c = _cache(n_tokens=1000)
    assert L.kivi_append(ctypes.byref(c), FAKE, FAKE, 25, None) == -2
    assert c.n_tokens == 1000
    assert L.kivi_append(ctypes.byref(c), FAKE, FAKE, 0, None) == 0
    assert L.kivi_append(ctypes.byref(c), FAKE, FAKE, -1, None) == -1
    assert L.kivi_append(ctypes.byref(c), None, FAKE, 1, None) == -1
    assert L.kivi_append(None, FAKE, FAKE, 1, None) == -1


def test_workspace_queries(L):
    c = _cache(n_tokens=300)
    n = L.kivi_decode_attn_workspace_bytes(ctypes.byref(c), 8)
    # partial slots of head_dim + 4 floats for each (batch, query head)
    assert n > 0 and n % (c.batch * 8 * 132 * 4) == 0
    assert L.kivi_decode_attn_workspace_bytes(ctypes.byref(c), 3) == 0      # 3 % 2 != 0
    assert L.kivi_decode_attn_workspace_bytes_ex(ctypes.byref(c), 8, 100, 0) == 0
    assert L.kivi_decode_attn_workspace_bytes_ex(ctypes.byref(c), 8, 64, 9) == 0
    # a smaller split never needs less workspace than the automatic plan's bound
    assert L.kivi_decode_attn_workspace_bytes_ex(ctypes.byref(c), 8, 64, 0) >= n


def test_decode_rejects(L):
    c = _cache(n_tokens=300)
    n = L.kivi_decode_attn_workspace_bytes(ctypes.byref(c), 4)
    ok = dict(q=FAKE, hq=4, out=FAKE, ws=FAKE, nbytes=n, tps=0, path=0)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.kivi_decode_attn_ex(ctypes.byref(c), a["q"], a["hq"], None, a["out"], a["ws"],
                                     a["nbytes"], a["tps"], a["path"], None)

    assert call(hq=3) == -1
    assert call(q=None) == -1
    assert call(out=None) == -1
    assert call(nbytes=n - 1) == -3
    assert call(ws=None) == -3
    assert call(tps=96) == -1
    assert call(path=5) == -1
    assert L.kivi_decode_attn(None, FAKE, 4, None, FAKE, FAKE, n, None) == -1


def test_decode_noalloc_rejects(L):
    """The no-allocation entry point checks its arguments before it plans,
    looks up its scratch array or launches anything."""
    c = _cache(n_tokens=300)
    assert L.kivi_decode_attn_noalloc(ctypes.byref(c), None, 4, None, FAKE, None) == -1
    assert L.kivi_decode_attn_noalloc(ctypes.byref(c), FAKE, 4, None, None, None) == -1
    assert L.kivi_decode_attn_noalloc(ctypes.byref(c), FAKE, 3, None, FAKE, None) == -1
    assert L.kivi_decode_attn_noalloc(None, FAKE, 4, None, FAKE, None) == -1
    assert L.kivi_decode_attn_noalloc(ctypes.byref(_cache(k_bits=3)), FAKE, 4, None, FAKE,
                                      None) == -1


@pytest.mark.parametrize("field", ["blocks", "k_res", "v_res"])
def test_misaligned_cache_rejected_on_every_path(L, field):
    """A cache array that is not 16-byte aligned is rejected before any
    launch, also when the matrix-core path is forced (its global->LDS copies
    move 16 bytes per lane)."""
    c = _cache(n_tokens=300, **{field: 0x1008})
    n = L.kivi_decode_attn_workspace_bytes_ex(ctypes.byref(_cache(n_tokens=300)), 4, 0, 2)
    for path in (0, 1, 2, 3):
        assert L.kivi_decode_attn_ex(ctypes.byref(c), FAKE, 4, None, FAKE, FAKE, n, 0, path,
                                     None) == -1
        assert b"aligned" in L.kivi_last_error()


def test_decode_step_rejects(L):
    """kivi_decode_step checks every argument before anything runs and leaves
    the token count unchanged on failure."""
    c = _cache(n_tokens=300)
    n = L.kivi_decode_attn_workspace_bytes(ctypes.byref(c), 4)
    ok = dict(k=FAKE, v=FAKE, q=FAKE, hq=4, out=FAKE, ws=FAKE, nbytes=n)

    def call(cache=c, **kw):
        a = dict(ok)
        a.update(kw)
        return L.kivi_decode_step(ctypes.byref(cache), a["k"], a["v"], a["q"], a["hq"], None,
                                  a["out"], a["ws"], a["nbytes"], None)

    assert call(k=None) == -1
    assert call(v=None) == -1
    assert call(q=None) == -1
    assert call(out=None) == -1
    assert call(hq=3) == -1
    assert call(nbytes=n - 1) == -3
    assert call(ws=None) == -3
    full = _cache(n_tokens=1024)
    assert call(cache=full) == -2
    assert call(cache=_cache(k_bits=3)) == -1
    assert c.n_tokens == 300 and full.n_tokens == 1024
    assert L.kivi_decode_step(None, FAKE, FAKE, FAKE, 4, None, FAKE, FAKE, n, None) == -1


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without libkivi.so every call raises; nothing falls back to another
    implementation."""
    from decode_attention_pack_amd import kivi
    monkeypatch.setattr(kivi, "_lib", None)
    monkeypatch.setattr(kivi, "LIB_PATH", str(tmp_path / "libkivi.so"))
    with pytest.raises(RuntimeError, match="missing"):
        kivi.lib()


def _ragged(counts, **kw):
    c = _cache(batch=len(counts), **kw)
    arr = (ctypes.c_int64 * len(counts))(*counts)
    c.row_tokens = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64))
    return c, arr


def test_ragged_rejects(L):
    """A ragged batch (row_tokens set): counts outside [0, capacity], more
    than 256 rows, per-row appends on a uniform cache or past a row's
    capacity, and too many workgroups from an explicit split are rejected on
    the host, leaving the counts as they were."""
    big = 1 << 34
    for counts in ([5, 2000], [-1, 3]):
        c, arr = _ragged(counts)
        assert L.kivi_decode_attn(ctypes.byref(c), FAKE, 2, None, FAKE, FAKE, big, None) == -1
        assert b"row_tokens" in L.kivi_last_error()
    c, arr = _ragged([0] * 257, n_kv_heads=1)
    assert L.kivi_decode_attn(ctypes.byref(c), FAKE, 1, None, FAKE, FAKE, big, None) == -1
    assert b"256" in L.kivi_last_error()
    u = _cache()
    assert L.kivi_append_row(ctypes.byref(u), 0, FAKE, FAKE, 1, None) == -1
    c, arr = _ragged([10, 20])
    for b in (2, -1):
        assert L.kivi_append_row(ctypes.byref(c), b, FAKE, FAKE, 1, None) == -1
    assert L.kivi_append_row(ctypes.byref(c), 1, FAKE, FAKE, 1005, None) == -2
    assert L.kivi_append_row(ctypes.byref(c), 1, FAKE, FAKE, 0, None) == 0
    # every row of a ragged append takes the tokens: the longest row decides
    assert L.kivi_append(ctypes.byref(c), FAKE, FAKE, 1005, None) == -2
    assert list(arr) == [10, 20]
    c, arr = _ragged([1024, 3])
    assert L.kivi_decode_step(ctypes.byref(c), FAKE, FAKE, FAKE, 2, None, FAKE, FAKE, big,
                              None) == -2
    assert list(arr) == [1024, 3]
    # 64 rows of 1000 tokens, a workgroup per 64 tokens: 448 workgroups per
    # KV head, more than a ragged launch's table holds
    c, arr = _ragged([1000] * 64, n_kv_heads=1)
    assert L.kivi_decode_attn_ex(ctypes.byref(c), FAKE, 1, None, FAKE, FAKE, big, 64, 2,
                                 None) == -1
    assert b"tokens_per_split" in L.kivi_last_error()


def test_select_rejects(L):
    """kivi_select_attn: tau outside (0, 1], a ragged cache, a NULL q, a small
    or misaligned workspace -- rejected on the host."""
    c = _cache(n_tokens=100)
    ws = L.kivi_select_attn_workspace_bytes(ctypes.byref(c), 2)
    assert ws > 0
    big = 1 << 34
    W = ctypes.c_void_p(0x10000)
    for tau in (0.0, -0.5, 1.5, float("nan")):
        assert L.kivi_select_attn(ctypes.byref(c), FAKE, 2, None, tau, FAKE, None, None, W, big,
                                  None) == -1
    assert L.kivi_select_attn(ctypes.byref(c), None, 2, None, 0.9, FAKE, None, None, W, big,
                              None) == -1
    assert L.kivi_select_attn(ctypes.byref(c), FAKE, 3, None, 0.9, FAKE, None, None, W, big,
                              None) == -1
    assert L.kivi_select_attn(ctypes.byref(c), FAKE, 2, None, 0.9, FAKE, None, None, W, ws - 1,
                              None) == -3
    assert L.kivi_select_attn(ctypes.byref(c), FAKE, 2, None, 0.9, FAKE, None, None,
                              ctypes.c_void_p(0x10010), big, None) == -3
    r, arr = _ragged([10, 20])
    assert L.kivi_select_attn(ctypes.byref(r), FAKE, 2, None, 0.9, FAKE, None, None, W, big,
                              None) == -1
    assert b"ragged" in L.kivi_last_error()


def test_paged_rejects(L):
    """A paged cache: a misaligned page table or a pool of no pages is
    rejected on the host."""
    c = _cache(n_tokens=100)
    c.page_table = 0x1002
    c.n_pages = 10
    big = 1 << 34
    assert L.kivi_decode_attn(ctypes.byref(c), FAKE, 2, None, FAKE, FAKE, big, None) == -1
    assert b"page_table" in L.kivi_last_error()
    c.page_table = 0x1000
    for n in (0, -3, 1 << 45):
        c.n_pages = n
        assert L.kivi_decode_attn(ctypes.byref(c), FAKE, 2, None, FAKE, FAKE, big, None) == -1
        assert b"n_pages" in L.kivi_last_error()


def test_record_bytes_fp16_scales(L):
    """The fp16-scale layout's record: scale sections of 2 bytes per scale
    (4096 + 1024 + 1024 + 4096 + 1024 + 1024 = 12288 at 2-bit, G 32,
    head_dim 128); flag 0 is the fp32 layout; other flags give 0."""
    assert L.kivi_record_bytes_ex(128, 2, 2, 32, 1) == 12288
    assert L.kivi_record_bytes_ex(128, 2, 2, 32, 0) == L.kivi_record_bytes(128, 2, 2, 32)
    assert L.kivi_record_bytes_ex(128, 4, 4, 32, 1) == 8192 + 1024 + 1024 + 8192 + 1024 + 1024
    assert L.kivi_record_bytes_ex(64, 2, 4, 64, 1) == 2048 + 256 + 256 + 4096 + 256 + 256
    assert L.kivi_record_bytes_ex(128, 2, 2, 32, 2) == 0
    assert L.kivi_record_bytes_ex(128, 3, 2, 32, 1) == 0


def test_scale_flag_rejected(L):
    """A cache whose scale_fp16 flag is neither 0 nor 1 is rejected on the
    host by every entry point that takes a cache."""
    c = _cache(n_tokens=100)
    c.scale_fp16 = 3
    big = 1 << 34
    assert L.kivi_decode_attn(ctypes.byref(c), FAKE, 2, None, FAKE, FAKE, big, None) == -1
    assert b"scale_fp16" in L.kivi_last_error()
    assert _pack(L, "kivi_pack_keys", cache=c) == -1
    assert b"scale_fp16" in L.kivi_last_error()
