"""CPU oracle for KIVI packed-KV decode attention (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never does, and the two share no code.

The arithmetic lives in ``kivi_oracle.c`` (plain C, built with gcc, no
fast-math, no FP contraction).  This module only marshals numpy arrays.

Method source: web page "Literature audit -- Group 2 (KV-cache compression
primary sources)", section "1. KIVI -- kivi2024", list "Core algorithm
(implementation-grade)", items 1-5.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kivi_oracle.c")
_LIB = os.path.join(_HERE, "libkivi_oracle.so")
_lib = None


def build() -> str:
    """Compile the oracle with gcc (every call recompiles)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", "-o", _LIB, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.kivi_oracle_half_to_float.argtypes = [ctypes.c_uint16]
    lib.kivi_oracle_half_to_float.restype = ctypes.c_float
    lib.kivi_oracle_float_to_half.argtypes = [ctypes.c_float, P]
    lib.kivi_oracle_float_to_half.restype = ctypes.c_int
    lib.kivi_oracle_record_bytes.argtypes = [i32, i32, i32, i32]
    lib.kivi_oracle_record_bytes.restype = i64
    lib.kivi_oracle_record_bytes_s.argtypes = [i32, i32, i32, i32, i32]
    lib.kivi_oracle_record_bytes_s.restype = i64
    lib.kivi_oracle_half_rne.argtypes = [ctypes.c_float]
    lib.kivi_oracle_half_rne.restype = ctypes.c_uint16
    lib.kivi_oracle_quantize_group_s16.argtypes = [P, i32, i32, P, P, P]
    lib.kivi_oracle_quantize_group_s16.restype = None
    lib.kivi_oracle_quantize_group.argtypes = [P, i32, i32, P, P, P]
    lib.kivi_oracle_quantize_group.restype = None
    lib.kivi_oracle_dequant.argtypes = [ctypes.c_uint32, ctypes.c_float, ctypes.c_float]
    lib.kivi_oracle_dequant.restype = ctypes.c_float
    lib.kivi_oracle_pack_codes.argtypes = [P, i32, i32, P]
    lib.kivi_oracle_pack_codes.restype = None
    lib.kivi_oracle_unpack_codes.argtypes = [P, i32, i32, P]
    lib.kivi_oracle_unpack_codes.restype = None
    for name in ("kivi_oracle_pack_keys", "kivi_oracle_pack_values"):
        fn = getattr(lib, name)
        fn.argtypes = [P, P, i64, i64]
        fn.restype = ctypes.c_int
    lib.kivi_oracle_append.argtypes = [P, P, P, i64]
    lib.kivi_oracle_append.restype = ctypes.c_int
    lib.kivi_oracle_materialize.argtypes = [P, P, P]
    lib.kivi_oracle_materialize.restype = ctypes.c_int
    lib.kivi_oracle_decode_attn.argtypes = [P, P, i32, P, P]
    lib.kivi_oracle_decode_attn.restype = ctypes.c_int
    lib.kivi_oracle_decode_attn_heads.argtypes = [P, P, i32, P, i32, i32, i32, P]
    lib.kivi_oracle_decode_attn_heads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _req(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


class _CCache(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32), ("group", ctypes.c_int32),
        ("residual", ctypes.c_int32),
        ("capacity", ctypes.c_int64), ("n_tokens", ctypes.c_int64),
        ("blocks", ctypes.c_void_p), ("k_res", ctypes.c_void_p), ("v_res", ctypes.c_void_p),
        ("scale_fp16", ctypes.c_int32),
    ]


TOKENS_PER_RECORD = 128


def record_bytes(D: int, kb: int, vb: int, G: int, scale_fp16: bool = False) -> int:
    """Bytes of one 128-token record (0 for a shape the layout does not take)."""
    return int(_load().kivi_oracle_record_bytes_s(D, kb, vb, G, int(bool(scale_fp16))))


def record_sections(D: int, kb: int, vb: int, G: int, scale_fp16: bool = False):
    """(name, byte offset, byte size) of the sections of a record, in order."""
    n, g = TOKENS_PER_RECORD, TOKENS_PER_RECORD // G
    sb = 2 if scale_fp16 else 4
    sizes = [("k_codes", n * D * kb // 8), ("k_scale", g * D * sb), ("k_zero", g * D * 2),
             ("v_codes", n * D * vb // 8), ("v_scale", (D // G) * n * sb),
             ("v_zero", (D // G) * n * 2)]
    out, off = [], 0
    for name, size in sizes:
        out.append((name, off, size))
        off += size
    return out


def unpack_records(blocks, B, H, cap, D, kb, vb, G, scale_fp16: bool = False):
    """Re-index a record array ([B][H][cap/128][record] bytes) into the
    logical arrays: k_codes [B][H][cap/G][D][G*kb/32] u32, k_scale, k_zero
    [B][H][cap/G][D] (f32 or f16, f16), v_codes [B][H][cap][D*vb/32] u32,
    v_scale, v_zero [B][H][D/G][cap] (f32 or f16, f16).  Copies; no
    arithmetic."""
    n = TOKENS_PER_RECORD
    nb = cap // n
    secs = record_sections(D, kb, vb, G, scale_fp16)
    rb = sum(size for _, _, size in secs)
    raw = np.ascontiguousarray(blocks).view(np.uint8).reshape(B, H, nb, rb)
    sec = {name: raw[..., off:off + size] for name, off, size in secs}
    g = n // G
    st = np.float16 if scale_fp16 else np.float32

    def cast(x, dtype):
        return np.ascontiguousarray(x).view(dtype)

    out = {}
    out["k_codes"] = cast(sec["k_codes"], np.uint32).reshape(B, H, nb * g, D, G * kb // 32)
    out["k_scale"] = cast(sec["k_scale"], st).reshape(B, H, nb * g, D)
    out["k_zero"] = cast(sec["k_zero"], np.float16).reshape(B, H, nb * g, D)
    out["v_codes"] = cast(sec["v_codes"], np.uint32).reshape(B, H, nb * n, D * vb // 32)
    vs = cast(sec["v_scale"], st).reshape(B, H, nb, D // G, n)
    out["v_scale"] = np.ascontiguousarray(vs.transpose(0, 1, 3, 2, 4)).reshape(B, H, D // G, cap)
    vz = cast(sec["v_zero"], np.float16).reshape(B, H, nb, D // G, n)
    out["v_zero"] = np.ascontiguousarray(vz.transpose(0, 1, 3, 2, 4)).reshape(B, H, D // G, cap)
    return out


LOGICAL = ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero")


def half_to_float(bits: int) -> float:
    return float(_load().kivi_oracle_half_to_float(int(bits) & 0xFFFF))


def quantize_group(x, bits: int):
    """KIVI item 1 on one group: returns (codes uint8[n], scale f32, zero f32)."""
    x = _req(x, np.float32)
    codes = np.zeros(x.size, np.uint8)
    s = np.zeros(1, np.float32)
    z = np.zeros(1, np.float32)
    _load().kivi_oracle_quantize_group(_ptr(x), x.size, bits, _ptr(codes), _ptr(s), _ptr(z))
    return codes, np.float32(s[0]), np.float32(z[0])


def quantize_group_s16(x, bits: int):
    """KIVI item 1 with an fp16 scale: (codes uint8[n], scale f16, zero f32)."""
    x = _req(x, np.float32)
    codes = np.zeros(x.size, np.uint8)
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.float32)
    _load().kivi_oracle_quantize_group_s16(_ptr(x), x.size, bits, _ptr(codes), _ptr(s), _ptr(z))
    return codes, s.view(np.float16)[0], np.float32(z[0])


def half_rne(value) -> int:
    """Bit pattern of the binary16 value nearest to an fp32 value (ties to
    even)."""
    return int(_load().kivi_oracle_half_rne(float(np.float32(value))))


def dequant(code: int, scale, zero) -> np.float32:
    return np.float32(_load().kivi_oracle_dequant(int(code), float(scale), float(zero)))


def pack_codes(codes, bits: int):
    codes = _req(codes, np.uint8)
    per = 32 // bits
    words = np.zeros((codes.size + per - 1) // per, np.uint32)
    _load().kivi_oracle_pack_codes(_ptr(codes), codes.size, bits, _ptr(words))
    return words


def unpack_codes(words, n: int, bits: int):
    words = _req(words, np.uint32)
    codes = np.zeros(n, np.uint8)
    _load().kivi_oracle_unpack_codes(_ptr(words), n, bits, _ptr(codes))
    return codes


def float_to_half(value) -> int:
    """Bit pattern of an fp32 value that is exactly an fp16 value."""
    out = np.zeros(1, np.uint16)
    if _load().kivi_oracle_float_to_half(float(value), _ptr(out)):
        raise ValueError(f"{value!r} has no exact fp16 form")
    return int(out[0])


def _round_cap(t: int) -> int:
    return max(TOKENS_PER_RECORD, -(-t // TOKENS_PER_RECORD) * TOKENS_PER_RECORD)


def pack_keys(k_fp16, bits: int, G: int, cap: int | None = None, offset: int = 0,
              scale_fp16: bool = False):
    """KIVI item 2 into a fresh zero-filled record array.  k_fp16: uint16
    [B][H][T][D] -> logical (codes, scale, zero) over the capacity (a multiple
    of 128, by default the smallest that holds offset + T)."""
    k = _req(k_fp16, np.uint16)
    B, H, T, D = k.shape
    cap = _round_cap(T + offset) if cap is None else cap
    c = Cache(B, H, D, bits, bits, G, G, cap, scale_fp16=scale_fp16)
    if _load().kivi_oracle_pack_keys(ctypes.byref(c._c), _ptr(k), T, offset):
        raise ValueError("oracle pack_keys rejected its arguments")
    return c.k_codes, c.k_scale, c.k_zero


def pack_values(v_fp16, bits: int, G: int, cap: int | None = None, offset: int = 0,
                scale_fp16: bool = False):
    """KIVI item 3 into a fresh zero-filled record array.  v_fp16: uint16
    [B][H][T][D] -> logical (codes, scale, zero)."""
    v = _req(v_fp16, np.uint16)
    B, H, T, D = v.shape
    cap = _round_cap(T + offset) if cap is None else cap
    c = Cache(B, H, D, bits, bits, G, G, cap, scale_fp16=scale_fp16)
    if _load().kivi_oracle_pack_values(ctypes.byref(c._c), _ptr(v), T, offset):
        raise ValueError("oracle pack_values rejected its arguments")
    return c.v_codes, c.v_scale, c.v_zero


class Cache:
    """Host-memory KIVI cache driven by the oracle (numpy arrays, zero-filled).

    ``arrays`` holds the storage itself: ``blocks`` (the record array, bytes),
    ``k_res`` and ``v_res``.  The logical arrays ``k_codes`` ... ``v_zero``
    are re-indexed copies of the records (see unpack_records)."""

    def __init__(self, batch, n_kv_heads, head_dim, k_bits, v_bits, group, residual, capacity,
                 scale_fp16: bool = False):
        self.B, self.H, self.D = batch, n_kv_heads, head_dim
        self.kb, self.vb, self.G, self.R, self.cap = k_bits, v_bits, group, residual, capacity
        self.scale_fp16 = bool(scale_fp16)
        rb = record_bytes(head_dim, k_bits, v_bits, group, self.scale_fp16)
        if rb == 0 or capacity % TOKENS_PER_RECORD:
            raise ValueError("shape or capacity outside the record layout")
        self.arrays = {
            "blocks": np.zeros((batch, n_kv_heads, capacity // TOKENS_PER_RECORD, rb), np.uint8),
            "k_res": np.zeros((batch, n_kv_heads, residual, head_dim), np.uint16),
            "v_res": np.zeros((batch, n_kv_heads, residual, head_dim), np.uint16),
        }
        self._c = _CCache(batch, n_kv_heads, head_dim, k_bits, v_bits, group, residual,
                          capacity, 0, _ptr(self.arrays["blocks"]), _ptr(self.arrays["k_res"]),
                          _ptr(self.arrays["v_res"]), int(self.scale_fp16))

    def __getattr__(self, name):
        arrays = self.__dict__.get("arrays")
        if arrays is None:
            raise AttributeError(name)
        if name in arrays:
            return arrays[name]
        if name in LOGICAL:
            return unpack_records(arrays["blocks"], self.B, self.H, self.cap, self.D, self.kb,
                                  self.vb, self.G, self.scale_fp16)[name]
        raise AttributeError(name)

    def logical(self):
        """All six logical arrays at once."""
        return unpack_records(self.arrays["blocks"], self.B, self.H, self.cap, self.D, self.kb,
                              self.vb, self.G, self.scale_fp16)

    @property
    def n_tokens(self) -> int:
        return int(self._c.n_tokens)

    def append(self, k_new, v_new):
        """KIVI item 4: append fp16 (uint16) [B][H][n][D] keys/values."""
        k = _req(k_new, np.uint16)
        v = _req(v_new, np.uint16)
        n = k.shape[2]
        assert k.shape == (self.B, self.H, n, self.D) and v.shape == k.shape
        rc = _load().kivi_oracle_append(ctypes.byref(self._c), _ptr(k), _ptr(v), n)
        if rc:
            raise ValueError("oracle append rejected its arguments")

    def materialize(self):
        """(k_hat, v_hat) f32 [B][H][t][D] as the attention sees them."""
        t = self.n_tokens
        kh = np.zeros((self.B, self.H, t, self.D), np.float32)
        vh = np.zeros((self.B, self.H, t, self.D), np.float32)
        rc = _load().kivi_oracle_materialize(ctypes.byref(self._c), _ptr(kh), _ptr(vh))
        if rc:
            raise ValueError("oracle materialize rejected its arguments")
        return kh, vh

    def decode_attn(self, q_fp16, mask=None):
        """KIVI item 5.  q: uint16 [B][Hq][D]; mask: f32 [B][t] or None."""
        q = _req(q_fp16, np.uint16)
        Hq = q.shape[1]
        m = None if mask is None else _req(mask, np.float32)
        out = np.zeros((self.B, Hq, self.D), np.float32)
        rc = _load().kivi_oracle_decode_attn(ctypes.byref(self._c), _ptr(q), Hq, _ptr(m),
                                             _ptr(out))
        if rc:
            raise ValueError("oracle decode_attn rejected its arguments")
        return out

    def decode_attn_heads(self, q_fp16, b, h0, h1, mask=None):
        """Attention for batch row b and query heads [h0, h1): f32 [h1-h0][D]."""
        q = _req(q_fp16, np.uint16)
        Hq = q.shape[1]
        m = None if mask is None else _req(mask, np.float32)
        out = np.zeros((h1 - h0, self.D), np.float32)
        rc = _load().kivi_oracle_decode_attn_heads(ctypes.byref(self._c), _ptr(q), Hq, _ptr(m),
                                                   b, h0, h1, _ptr(out))
        if rc:
            raise ValueError("oracle decode_attn_heads rejected its arguments")
        return out
