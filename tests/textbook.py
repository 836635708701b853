"""Textbook references used to pin the oracle (numpy, float64).

These are written from the mathematics alone -- dense softmax attention and the
definition of bit packing -- and do not call the oracle.
"""
from __future__ import annotations

import numpy as np


def dense_attention(q, k, v, mask=None):
    """softmax(q k^T / sqrt(d) + mask) v for every (batch, query head).

    q: [B][Hq][D]; k, v: [B][Hkv][t][D]; mask: [B][t] additive or None.
    Query head h reads KV head h // (Hq // Hkv).  Float64 throughout.
    A row whose scores are all -inf gives zeros.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Hq, D = q.shape
    Hkv, t = k.shape[1], k.shape[2]
    rep = Hq // Hkv
    out = np.zeros((B, Hq, D), np.float64)
    for b in range(B):
        for h in range(Hq):
            kk = k[b, h // rep]
            vv = v[b, h // rep]
            s = kk @ q[b, h] / np.sqrt(D)
            if mask is not None:
                s = s + np.asarray(mask[b], np.float64)
            if t == 0 or not np.isfinite(s.max()):
                continue
            p = np.exp(s - s.max())
            out[b, h] = (p / p.sum()) @ vv
    return out


def pack_bits(codes, bits):
    """Pack a flat sequence of codes into u32 words, first code in the lowest bits."""
    per = 32 // bits
    codes = [int(c) for c in codes]
    words = []
    for i in range(0, len(codes), per):
        w = 0
        for j, c in enumerate(codes[i:i + per]):
            w |= c << (bits * j)
        words.append(w)
    return np.array(words, np.uint32)
