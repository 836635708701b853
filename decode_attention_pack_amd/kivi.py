"""Thin ctypes binding over libkivi.so (include/kivi.h).

Argument marshalling only: torch tensors are checked for device, dtype, shape
and contiguity, then their device pointers and the current HIP stream are
handed to the C ABI.  Every step of the computation runs in the library's HIP
kernels; there is no fallback.  If libkivi.so is missing the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkivi.so")

KIVI_OK = 0
KIVI_ERR_INVALID_ARG = -1
KIVI_ERR_CAPACITY = -2
KIVI_ERR_WORKSPACE = -3
KIVI_ERR_HIP = -4
KIVI_PATH_AUTO, KIVI_PATH_GENERIC, KIVI_PATH_MATRIX, KIVI_PATH_VECTOR = 0, 1, 2, 3

EXPORTED = ("kivi_record_bytes", "kivi_record_bytes_ex", "kivi_pack_keys", "kivi_pack_values", "kivi_append",
            "kivi_append_row", "kivi_decode_attn", "kivi_decode_attn_ex",
            "kivi_decode_attn_workspace_bytes",
            "kivi_decode_attn_workspace_bytes_ex", "kivi_decode_step", "kivi_decode_attn_noalloc",
            "kivi_select_attn", "kivi_select_attn_workspace_bytes",
            "kivi_status_string", "kivi_last_error")
TOKENS_PER_RECORD = 128
MAX_RAGGED_ROWS = 256


class KiviError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{detail} (status {status})")
        self.status = status


class CCache(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32), ("group", ctypes.c_int32),
        ("residual", ctypes.c_int32),
        ("capacity", ctypes.c_int64), ("n_tokens", ctypes.c_int64),
        ("blocks", ctypes.c_void_p), ("k_res", ctypes.c_void_p), ("v_res", ctypes.c_void_p),
        ("row_tokens", ctypes.POINTER(ctypes.c_int64)),
        ("page_table", ctypes.c_void_p), ("n_pages", ctypes.c_int64),
        ("scale_fp16", ctypes.c_int32),
    ]


_lib = None


def lib():
    """Load libkivi.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m decode_attention_pack_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.kivi_record_bytes.argtypes = [i32, i32, i32, i32]
    L.kivi_record_bytes.restype = sz
    L.kivi_record_bytes_ex.argtypes = [i32, i32, i32, i32, i32]
    L.kivi_record_bytes_ex.restype = sz
    for name in ("kivi_pack_keys", "kivi_pack_values"):
        fn = getattr(L, name)
        fn.argtypes = [ctypes.POINTER(CCache), P, i64, i64, P]
        fn.restype = ctypes.c_int
    L.kivi_append.argtypes = [ctypes.POINTER(CCache), P, P, i64, P]
    L.kivi_append.restype = ctypes.c_int
    L.kivi_append_row.argtypes = [ctypes.POINTER(CCache), i32, P, P, i64, P]
    L.kivi_append_row.restype = ctypes.c_int
    L.kivi_decode_attn.argtypes = [ctypes.POINTER(CCache), P, i32, P, P, P, sz, P]
    L.kivi_decode_attn.restype = ctypes.c_int
    L.kivi_decode_attn_ex.argtypes = [ctypes.POINTER(CCache), P, i32, P, P, P, sz, i32, i32, P]
    L.kivi_decode_attn_ex.restype = ctypes.c_int
    L.kivi_decode_step.argtypes = [ctypes.POINTER(CCache), P, P, P, i32, P, P, P, sz, P]
    L.kivi_decode_step.restype = ctypes.c_int
    L.kivi_decode_attn_noalloc.argtypes = [ctypes.POINTER(CCache), P, i32, P, P, P]
    L.kivi_decode_attn_noalloc.restype = ctypes.c_int
    L.kivi_decode_attn_workspace_bytes.argtypes = [ctypes.POINTER(CCache), i32]
    L.kivi_decode_attn_workspace_bytes.restype = sz
    L.kivi_decode_attn_workspace_bytes_ex.argtypes = [ctypes.POINTER(CCache), i32, i32, i32]
    L.kivi_decode_attn_workspace_bytes_ex.restype = sz
    L.kivi_select_attn.argtypes = [ctypes.POINTER(CCache), P, i32, P, ctypes.c_float, P, P, P, P,
                                   sz, P]
    L.kivi_select_attn.restype = ctypes.c_int
    L.kivi_select_attn_workspace_bytes.argtypes = [ctypes.POINTER(CCache), i32]
    L.kivi_select_attn_workspace_bytes.restype = sz
    L.kivi_status_string.argtypes = [ctypes.c_int]
    L.kivi_status_string.restype = ctypes.c_char_p
    L.kivi_last_error.argtypes = []
    L.kivi_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int):
    if status != KIVI_OK:
        raise KiviError(status, lib().kivi_last_error().decode())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dev(t: torch.Tensor, dtype, shape, name):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def record_bytes(D, kb, vb, G, scale_fp16=False) -> int:
    """Bytes of one 128-token record of the packed store (include/kivi.h),
    with fp32 or (scale_fp16) fp16 scales."""
    n = int(lib().kivi_record_bytes_ex(D, kb, vb, G, int(bool(scale_fp16))))
    if n == 0:
        raise KiviError(KIVI_ERR_INVALID_ARG, f"no record layout for D={D} bits={kb}/{vb} G={G}")
    return n


def layout_shapes(B, H, D, kb, vb, G, R, cap, pages=None, scale_fp16=False):
    """Shapes of the cache arrays (include/kivi.h storage layout); with
    `pages`, a paged cache: a pool of that many pages of H records and a page
    table [B][cap/128]."""
    rb = record_bytes(D, kb, vb, G, scale_fp16)
    shapes = {
        "blocks": (B, H, cap // TOKENS_PER_RECORD, rb) if pages is None else (pages, H, rb),
        "k_res": (B, H, R, D),
        "v_res": (B, H, R, D),
    }
    if pages is not None:
        shapes["page_table"] = (B, cap // TOKENS_PER_RECORD)
    return shapes


_DT = {"blocks": torch.uint8, "k_res": torch.float16, "v_res": torch.float16,
       "page_table": torch.int32}
_ORDER = ("blocks", "k_res", "v_res")


class Cache:
    """A KIVI cache in device memory (torch tensors) plus its C descriptor.

    ``blocks`` is the record array as raw bytes; ``k_res`` / ``v_res`` are the
    fp16 windows.  ``ragged=True`` gives a ragged batch: each row keeps its own
    token count (``row_tokens``), all rows starting empty.  ``pages=N`` gives a
    paged cache: ``blocks`` is a pool of N pages of H records, and
    ``page_table`` (int32 [B][cap/128], zero-filled) names the page of each
    128-token block of each row; the caller fills it.  ``scale_fp16=True``
    stores the scales as binary16 (the fp16-scale layout)."""

    def __init__(self, batch, n_kv_heads, head_dim, k_bits, v_bits, group, residual, capacity,
                 device="cuda", arrays=None, ragged=False, pages=None, scale_fp16=False):
        self.B, self.H, self.D = batch, n_kv_heads, head_dim
        self.kb, self.vb, self.G, self.R, self.cap = k_bits, v_bits, group, residual, capacity
        self.scale_fp16 = bool(scale_fp16)
        if capacity % TOKENS_PER_RECORD:
            raise KiviError(KIVI_ERR_INVALID_ARG,
                            f"capacity {capacity} must be a multiple of {TOKENS_PER_RECORD}")
        shapes = layout_shapes(batch, n_kv_heads, head_dim, k_bits, v_bits, group, residual,
                               capacity, pages, self.scale_fp16)
        if arrays is None:
            arrays = {n: torch.empty(s, dtype=_DT[n], device=device) for n, s in shapes.items()}
            if pages is not None:
                arrays["page_table"].zero_()
        for n in shapes:
            _dev(arrays[n], _DT[n], shapes[n], n)
        self.pages = pages
        self.arrays = arrays
        self._rows = None
        if ragged:
            if not 0 < batch <= MAX_RAGGED_ROWS:
                raise KiviError(KIVI_ERR_INVALID_ARG,
                                f"a ragged batch holds 1 to {MAX_RAGGED_ROWS} rows (got {batch})")
            self._rows = (ctypes.c_int64 * batch)()
        self.c = CCache(batch, n_kv_heads, head_dim, k_bits, v_bits, group, residual, capacity, 0,
                        *[arrays[n].data_ptr() for n in _ORDER],
                        ctypes.cast(self._rows, ctypes.POINTER(ctypes.c_int64))
                        if ragged else None,
                        arrays["page_table"].data_ptr() if pages is not None else None,
                        pages or 0, int(self.scale_fp16))

    def __getattr__(self, name):
        arrays = self.__dict__.get("arrays")
        if arrays is not None and name in arrays:
            return arrays[name]
        raise AttributeError(name)

    @property
    def n_tokens(self) -> int:
        """Token count (the longest row of a ragged batch)."""
        return int(self.c.n_tokens)

    @property
    def ragged(self) -> bool:
        return self._rows is not None

    @property
    def row_tokens(self) -> list:
        """Per-row token counts (every row holds n_tokens unless ragged)."""
        if self._rows is None:
            return [self.n_tokens] * self.B
        return [int(x) for x in self._rows]

    def set_row_tokens(self, counts):
        """Set every row's token count of a ragged batch (host-side fields of
        the descriptor; the storage must hold what the counts say)."""
        if self._rows is None or len(counts) != self.B:
            raise KiviError(KIVI_ERR_INVALID_ARG, "set_row_tokens needs a ragged cache and B counts")
        for b, n in enumerate(counts):
            self._rows[b] = int(n)
        self.c.n_tokens = max(self._rows)

    def reset_row(self, b: int):
        """Empty row b of a ragged batch (host-side count only: later appends
        overwrite what the row's storage held)."""
        if self._rows is None:
            raise KiviError(KIVI_ERR_INVALID_ARG, "reset_row needs a ragged cache")
        if not 0 <= b < self.B:
            raise KiviError(KIVI_ERR_INVALID_ARG, f"row {b} outside [0, {self.B})")
        self._rows[b] = 0
        self.c.n_tokens = max(self._rows)

    def workspace_bytes(self, n_q_heads, tokens_per_split=0, path=KIVI_PATH_AUTO) -> int:
        n = lib().kivi_decode_attn_workspace_bytes_ex(ctypes.byref(self.c), n_q_heads,
                                                      tokens_per_split, path)
        if n == 0:
            raise KiviError(KIVI_ERR_INVALID_ARG, "invalid workspace query")
        return int(n)

    def new_workspace(self, n_q_heads, tokens_per_split=0, path=KIVI_PATH_AUTO):
        n = self.workspace_bytes(n_q_heads, tokens_per_split, path)
        return torch.empty(n, dtype=torch.uint8, device=self.blocks.device)


def kivi_pack_keys(dst: Cache, k, dst_token_offset=0, stream=None):
    """KIVI item 2: quantize k (fp16 [B][H][T][D]) into dst's records at
    tokens [dst_token_offset, dst_token_offset + T)."""
    T = k.shape[2]
    kp = _dev(k, torch.float16, (dst.B, dst.H, T, dst.D), "k")
    _check(lib().kivi_pack_keys(ctypes.byref(dst.c), kp, T, dst_token_offset, _stream(stream)))


def kivi_pack_values(dst: Cache, v, dst_token_offset=0, stream=None):
    """KIVI item 3: quantize v (fp16 [B][H][T][D]) into dst's records."""
    T = v.shape[2]
    vp = _dev(v, torch.float16, (dst.B, dst.H, T, dst.D), "v")
    _check(lib().kivi_pack_values(ctypes.byref(dst.c), vp, T, dst_token_offset, _stream(stream)))


def kivi_append(cache: Cache, k_new, v_new, stream=None):
    n = k_new.shape[2]
    shape = (cache.B, cache.H, n, cache.D)
    kp = _dev(k_new, torch.float16, shape, "k_new")
    vp = _dev(v_new, torch.float16, shape, "v_new")
    _check(lib().kivi_append(ctypes.byref(cache.c), kp, vp, n, _stream(stream)))


def kivi_append_row(cache: Cache, b: int, k_new, v_new, stream=None):
    """Append k_new / v_new (fp16 [H][n][D]) to row b of a ragged cache."""
    n = k_new.shape[1]
    shape = (cache.H, n, cache.D)
    kp = _dev(k_new, torch.float16, shape, "k_new")
    vp = _dev(v_new, torch.float16, shape, "v_new")
    _check(lib().kivi_append_row(ctypes.byref(cache.c), b, kp, vp, n, _stream(stream)))


def kivi_decode_attn(cache: Cache, q, mask=None, out=None, workspace=None, tokens_per_split=0,
                     path=KIVI_PATH_AUTO, stream=None):
    B, Hq, D = q.shape
    qp = _dev(q, torch.float16, (cache.B, Hq, cache.D), "q")
    mp = None
    if mask is not None:
        mp = _dev(mask, torch.float32, (cache.B, cache.n_tokens), "mask")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    op = _dev(out, torch.float32, (cache.B, Hq, cache.D), "out")
    if workspace is None:
        workspace = cache.new_workspace(Hq, tokens_per_split, path)
    wp = _dev(workspace, torch.uint8, None, "workspace")
    _check(lib().kivi_decode_attn_ex(ctypes.byref(cache.c), qp, Hq, mp, op, wp,
                                     workspace.numel(), tokens_per_split, path, _stream(stream)))
    return out


def kivi_decode_attn_noalloc(cache: Cache, q, out, mask=None, stream=None):
    """kivi_decode_attn into a caller-given out ([B][Hq][D] float32), with
    the partial results in the library's own scratch array (no workspace, no
    allocation in the library call); returns out."""
    Hq = q.shape[1]
    qp = _dev(q, torch.float16, (cache.B, Hq, cache.D), "q")
    mp = None
    if mask is not None:
        mp = _dev(mask, torch.float32, (cache.B, cache.n_tokens), "mask")
    op = _dev(out, torch.float32, (cache.B, Hq, cache.D), "out")
    _check(lib().kivi_decode_attn_noalloc(ctypes.byref(cache.c), qp, Hq, mp, op, _stream(stream)))
    return out


def kivi_decode_step(cache: Cache, k_new, v_new, q, mask=None, out=None, workspace=None,
                     stream=None):
    """Append one token ([B][H][1][D] or [B][H][D] fp16) and attend over the
    resulting cache in one library call; returns out."""
    B, Hq, D = q.shape
    shape = (cache.B, cache.H, cache.D)
    kp = _dev(k_new.reshape(shape), torch.float16, shape, "k_new")
    vp = _dev(v_new.reshape(shape), torch.float16, shape, "v_new")
    qp = _dev(q, torch.float16, (cache.B, Hq, cache.D), "q")
    mp = None
    if mask is not None:
        mp = _dev(mask, torch.float32, (cache.B, cache.n_tokens + 1), "mask")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    op = _dev(out, torch.float32, (cache.B, Hq, cache.D), "out")
    if workspace is None:
        workspace = cache.new_workspace(Hq)
    wp = _dev(workspace, torch.uint8, None, "workspace")
    _check(lib().kivi_decode_step(ctypes.byref(cache.c), kp, vp, qp, Hq, mp, op, wp,
                                  workspace.numel(), _stream(stream)))
    return out


def kivi_select_attn(cache: Cache, q, tau: float, mask=None, out=None, n_selected=None,
                     sel_mask=None, workspace=None, stream=None):
    """Token selection by attention mass (smallest top-score set reaching tau)
    and attention over the selected tokens; returns out.  n_selected (int32
    [B][Hq]) and sel_mask (int32 [B][Hq][ceil(t/32)], the bits as uint32)
    are optional outputs."""
    B, Hq, D = q.shape
    qp = _dev(q, torch.float16, (cache.B, Hq, cache.D), "q")
    mp = None
    if mask is not None:
        mp = _dev(mask, torch.float32, (cache.B, cache.n_tokens), "mask")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    op = _dev(out, torch.float32, (cache.B, Hq, cache.D), "out")
    np_ = None if n_selected is None else _dev(n_selected, torch.int32, (cache.B, Hq), "n_selected")
    words = (cache.n_tokens + 31) // 32
    sp = None if sel_mask is None else _dev(sel_mask, torch.int32, (cache.B, Hq, words), "sel_mask")
    if workspace is None:
        workspace = select_workspace(cache, Hq)
    wp = _dev(workspace, torch.uint8, None, "workspace")
    _check(lib().kivi_select_attn(ctypes.byref(cache.c), qp, Hq, mp, ctypes.c_float(tau), op, np_,
                                  sp, wp, workspace.numel(), _stream(stream)))
    return out


class BoundCall:
    """A library call whose arguments were checked and marshalled once.

    Calling it re-issues the same call on the same tensors (their contents may
    change between calls; the cache descriptor is passed by reference, so the
    token count the library keeps in it stays current).  For loops that issue
    the same call many times, where per-call argument checks would cost more
    host time than the kernels take.
    """

    def __init__(self, fn, args, keep):
        self._fn, self._args, self._keep = fn, tuple(args), keep

    def __call__(self):
        _check(self._fn(*self._args))


def bind_append(cache: Cache, k_new, v_new, stream=None) -> BoundCall:
    n = k_new.shape[2]
    shape = (cache.B, cache.H, n, cache.D)
    kp = _dev(k_new, torch.float16, shape, "k_new")
    vp = _dev(v_new, torch.float16, shape, "v_new")
    return BoundCall(lib().kivi_append, [ctypes.byref(cache.c), kp, vp, n, _stream(stream)],
                     (cache, k_new, v_new))


def bind_decode_attn(cache: Cache, q, out, workspace, tokens_per_split=0, path=KIVI_PATH_AUTO,
                     stream=None) -> BoundCall:
    """Bound kivi_decode_attn without a mask (a mask row's length follows the
    token count, which changes between calls; masked calls go through
    kivi_decode_attn)."""
    Hq = q.shape[1]
    qp = _dev(q, torch.float16, (cache.B, Hq, cache.D), "q")
    op = _dev(out, torch.float32, (cache.B, Hq, cache.D), "out")
    wp = _dev(workspace, torch.uint8, None, "workspace")
    return BoundCall(lib().kivi_decode_attn_ex,
                     [ctypes.byref(cache.c), qp, Hq, None, op, wp, workspace.numel(),
                      tokens_per_split, path, _stream(stream)], (cache, q, out, workspace))


def bind_select_attn(cache: Cache, q, tau: float, out, workspace, n_selected=None,
                     stream=None) -> BoundCall:
    """Bound kivi_select_attn (no mask, no selection bits)."""
    Hq = q.shape[1]
    qp = _dev(q, torch.float16, (cache.B, Hq, cache.D), "q")
    op = _dev(out, torch.float32, (cache.B, Hq, cache.D), "out")
    np_ = None if n_selected is None else _dev(n_selected, torch.int32, (cache.B, Hq), "n_selected")
    wp = _dev(workspace, torch.uint8, None, "workspace")
    return BoundCall(lib().kivi_select_attn,
                     [ctypes.byref(cache.c), qp, Hq, None, ctypes.c_float(tau), op, np_, None, wp,
                      workspace.numel(), _stream(stream)], (cache, q, out, workspace, n_selected))


def select_workspace(cache: Cache, n_q_heads: int):
    n = int(lib().kivi_select_attn_workspace_bytes(ctypes.byref(cache.c), n_q_heads))
    if n == 0:
        raise KiviError(KIVI_ERR_INVALID_ARG, "invalid workspace query")
    return torch.empty(n, dtype=torch.uint8, device=cache.blocks.device)


def bind_decode_step(cache: Cache, k_new, v_new, q, out, workspace, stream=None) -> BoundCall:
    """Bound kivi_decode_step (no mask)."""
    Hq = q.shape[1]
    shape = (cache.B, cache.H, cache.D)
    kp = _dev(k_new.reshape(shape), torch.float16, shape, "k_new")
    vp = _dev(v_new.reshape(shape), torch.float16, shape, "v_new")
    qp = _dev(q, torch.float16, (cache.B, Hq, cache.D), "q")
    op = _dev(out, torch.float32, (cache.B, Hq, cache.D), "out")
    wp = _dev(workspace, torch.uint8, None, "workspace")
    return BoundCall(lib().kivi_decode_step,
                     [ctypes.byref(cache.c), kp, vp, qp, Hq, None, op, wp, workspace.numel(),
                      _stream(stream)], (cache, k_new, v_new, q, out, workspace))
