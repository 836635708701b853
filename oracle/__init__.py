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
        fn.argtypes = [P, i32, i32, i64, i32, i32, i32, P, P, P, i64, i64]
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
        ("k_codes", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("k_zero", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p), ("v_scale", ctypes.c_void_p), ("v_zero", ctypes.c_void_p),
        ("k_res", ctypes.c_void_p), ("v_res", ctypes.c_void_p),
    ]


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


def layout_shapes(B, H, D, kb, vb, G, R, cap):
    """Array shapes of the cache storage contract."""
    return {
        "k_codes": (B, H, cap // G, D, G * kb // 32),
        "k_scale": (B, H, cap // G, D),
        "k_zero": (B, H, cap // G, D),
        "v_codes": (B, H, cap, D * vb // 32),
        "v_scale": (B, H, D // G, cap),
        "v_zero": (B, H, D // G, cap),
        "k_res": (B, H, R, D),
        "v_res": (B, H, R, D),
    }


_DTYPES = {"k_codes": np.uint32, "k_scale": np.float32, "k_zero": np.float32,
           "v_codes": np.uint32, "v_scale": np.float32, "v_zero": np.float32,
           "k_res": np.uint16, "v_res": np.uint16}


def pack_keys(k_fp16, bits: int, G: int, cap: int | None = None, offset: int = 0, out=None):
    """KIVI item 2.  k_fp16: uint16 [B][H][T][D] -> (codes, scale, zero)."""
    k = _req(k_fp16, np.uint16)
    B, H, T, D = k.shape
    cap = T + offset if cap is None else cap
    if out is None:
        codes = np.zeros((B, H, cap // G, D, G * bits // 32), np.uint32)
        scale = np.zeros((B, H, cap // G, D), np.float32)
        zero = np.zeros((B, H, cap // G, D), np.float32)
    else:
        codes, scale, zero = out
    rc = _load().kivi_oracle_pack_keys(_ptr(k), B, H, T, D, bits, G, _ptr(codes), _ptr(scale),
                                       _ptr(zero), cap, offset)
    if rc:
        raise ValueError("oracle pack_keys rejected its arguments")
    return codes, scale, zero


def pack_values(v_fp16, bits: int, G: int, cap: int | None = None, offset: int = 0, out=None):
    """KIVI item 3.  v_fp16: uint16 [B][H][T][D] -> (codes, scale, zero)."""
    v = _req(v_fp16, np.uint16)
    B, H, T, D = v.shape
    cap = T + offset if cap is None else cap
    if out is None:
        codes = np.zeros((B, H, cap, D * bits // 32), np.uint32)
        scale = np.zeros((B, H, D // G, cap), np.float32)
        zero = np.zeros((B, H, D // G, cap), np.float32)
    else:
        codes, scale, zero = out
    rc = _load().kivi_oracle_pack_values(_ptr(v), B, H, T, D, bits, G, _ptr(codes), _ptr(scale),
                                         _ptr(zero), cap, offset)
    if rc:
        raise ValueError("oracle pack_values rejected its arguments")
    return codes, scale, zero


class Cache:
    """Host-memory KIVI cache driven by the oracle (numpy arrays, zero-filled)."""

    def __init__(self, batch, n_kv_heads, head_dim, k_bits, v_bits, group, residual, capacity):
        self.B, self.H, self.D = batch, n_kv_heads, head_dim
        self.kb, self.vb, self.G, self.R, self.cap = k_bits, v_bits, group, residual, capacity
        shapes = layout_shapes(batch, n_kv_heads, head_dim, k_bits, v_bits, group, residual,
                               capacity)
        self.arrays = {n: np.zeros(s, _DTYPES[n]) for n, s in shapes.items()}
        self._c = _CCache(batch, n_kv_heads, head_dim, k_bits, v_bits, group, residual,
                          capacity, 0, *[_ptr(self.arrays[n]) for n in
                                         ("k_codes", "k_scale", "k_zero", "v_codes",
                                          "v_scale", "v_zero", "k_res", "v_res")])

    def __getattr__(self, name):
        arrays = self.__dict__.get("arrays")
        if arrays is not None and name in arrays:
            return arrays[name]
        raise AttributeError(name)

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
