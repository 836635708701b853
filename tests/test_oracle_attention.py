"""Pins for the oracle's decode attention (CPU only).

Method: KIVI item 5 of the page "Literature audit -- Group 2", section 1
(KIVI), "Core algorithm": scores over the quantized keys and the fp16 keys,
divided by sqrt(d), mask, softmax, then the probability-weighted sum over the
quantized values plus the fp16 values; GQA per the same page's README note.
"""
import numpy as np
import pytest

import oracle
from tests.textbook import dense_attention

TOL = dict(rtol=1e-6, atol=1e-6)


def _rand(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float16)


def _filled(B, H, D, G, R, t, kb=2, vb=2, seed=0, kscale=1.0):
    rng = np.random.default_rng(seed)
    K = _rand(rng, (B, H, t, D), kscale)
    V = _rand(rng, (B, H, t, D))
    m = int(np.lcm(R, oracle.TOKENS_PER_RECORD))
    cap = (t // m + 1) * m
    c = oracle.Cache(B, H, D, kb, vb, G, R, cap)
    c.append(K.view(np.uint16), V.view(np.uint16))
    return c, K, V


@pytest.mark.parametrize("t", [1, 5, 31])
def test_all_fp16_window_is_dense_attention(t):
    """P8: t < R keeps everything in fp16, so the result is textbook dense
    attention on the fp16 inputs."""
    rng = np.random.default_rng(t)
    c, K, V = _filled(2, 2, 64, 32, 32, t, seed=t)
    q = _rand(rng, (2, 4, 64))
    got = c.decode_attn(q.view(np.uint16))
    ref = dense_attention(q.astype(np.float32), K.astype(np.float32), V.astype(np.float32))
    np.testing.assert_allclose(got, ref, **TOL)


def _grid_tensor(rng, B, H, t, D, G, bits, along_tokens):
    """Every quantization group is {z + k*s : k in 0..2^B-1} with both ends
    present, s a power of two and z an integer multiple of s -- so quantization is
    lossless and the packed cache dequantizes back to the input exactly."""
    qmax = (1 << bits) - 1
    x = np.zeros((B, H, t, D), np.float32)
    if along_tokens:   # key groups: G tokens of one channel
        for b in range(B):
            for h in range(H):
                for g in range(t // G):
                    for ch in range(D):
                        s = 2.0 ** int(rng.integers(-4, 1))
                        z = s * int(rng.integers(-40, 40))
                        k = rng.integers(0, qmax + 1, G)
                        k[rng.choice(G, 2, replace=False)] = [0, qmax]
                        x[b, h, g * G:(g + 1) * G, ch] = z + k * s
    else:              # value groups: G channels of one token
        for b in range(B):
            for h in range(H):
                for tau in range(t):
                    for g in range(D // G):
                        s = 2.0 ** int(rng.integers(-4, 1))
                        z = s * int(rng.integers(-40, 40))
                        k = rng.integers(0, qmax + 1, G)
                        k[rng.choice(G, 2, replace=False)] = [0, qmax]
                        x[b, h, tau, g * G:(g + 1) * G] = z + k * s
    x16 = x.astype(np.float16)
    assert np.array_equal(x16.astype(np.float32), x)   # fp16-exact by construction
    return x16


@pytest.mark.parametrize("kb,vb", [(2, 2), (4, 4), (2, 4)])
def test_grid_exact_end_to_end(kb, vb):
    """P9: on grid-exact inputs the packed cache reproduces K and V exactly, so
    attention over it equals dense attention over the original fp16 K/V."""
    rng = np.random.default_rng(kb * 7 + vb)
    B, H, D, G, R, t = 1, 2, 64, 32, 32, 3 * 32 + 5
    K = _grid_tensor(rng, B, H, t - t % G, D, G, kb, True)
    K = np.concatenate([K, _rand(rng, (B, H, t % G, D))], axis=2)
    V = _grid_tensor(rng, B, H, t, D, G, vb, False)
    c = oracle.Cache(B, H, D, kb, vb, G, R, 4 * R)
    c.append(K.view(np.uint16), V.view(np.uint16))
    kh, vh = c.materialize()
    assert np.array_equal(kh, K.astype(np.float32))
    assert np.array_equal(vh, V.astype(np.float32))
    q = _rand(rng, (B, 4, D))
    got = c.decode_attn(q.view(np.uint16))
    ref = dense_attention(q.astype(np.float32), K.astype(np.float32), V.astype(np.float32))
    np.testing.assert_allclose(got, ref, **TOL)


@pytest.mark.parametrize("t", [32, 64, 65, 97, 101])
@pytest.mark.parametrize("Hq", [2, 4])
def test_brute_force_over_dequantized_cache(t, Hq):
    """P10: oracle attention equals numpy dense softmax attention over the
    oracle's own dequantized K and V (quantized and fp16 parts together)."""
    rng = np.random.default_rng(t * 3 + Hq)
    c, K, V = _filled(2, 2, 128, 32, 32, t, seed=t, kscale=3.0)
    kh, vh = c.materialize()
    q = _rand(rng, (2, Hq, 128))
    mask = np.where(rng.random((2, t)) < 0.2, -np.inf, rng.standard_normal((2, t))).astype(np.float32)
    mask[:, -1] = 0.0
    for m in (None, mask):
        got = c.decode_attn(q.view(np.uint16), m)
        ref = dense_attention(q.astype(np.float32), kh, vh, m)
        np.testing.assert_allclose(got, ref, **TOL)
    # quantization changed the keys: the test is not vacuous
    assert not np.array_equal(kh, K.astype(np.float32))


def test_gqa_equals_repeated_kv_mha():
    """P11: GQA with n_rep = 2 equals MHA with each KV head repeated."""
    rng = np.random.default_rng(9)
    B, Hkv, D, G, R, t = 2, 2, 64, 32, 32, 77
    K = _rand(rng, (B, Hkv, t, D)).view(np.uint16)
    V = _rand(rng, (B, Hkv, t, D)).view(np.uint16)
    q = _rand(rng, (B, 4, D)).view(np.uint16)
    g = oracle.Cache(B, Hkv, D, 2, 2, G, R, 128)
    g.append(K, V)
    m = oracle.Cache(B, 4, D, 2, 2, G, R, 128)
    m.append(np.repeat(K, 2, axis=1), np.repeat(V, 2, axis=1))
    assert np.array_equal(g.decode_attn(q), m.decode_attn(q))


def test_mask_semantics():
    rng = np.random.default_rng(4)
    c, K, V = _filled(1, 1, 64, 32, 32, 70, seed=4)
    q = _rand(rng, (1, 2, 64)).view(np.uint16)
    t = c.n_tokens
    # all-zero mask == no mask
    assert np.array_equal(c.decode_attn(q, np.zeros((1, t), np.float32)), c.decode_attn(q))
    # a fully masked row gives zeros, no NaN
    out = c.decode_attn(q, np.full((1, t), -np.inf, np.float32))
    assert not np.isnan(out).any() and not out.any()
    # masking tokens == dropping them
    kh, vh = c.materialize()
    keep = np.arange(t) % 3 != 1
    m = np.where(keep, 0.0, -np.inf).astype(np.float32)[None]
    ref = dense_attention(q.view(np.float16).astype(np.float32), kh[:, :, keep], vh[:, :, keep])
    np.testing.assert_allclose(c.decode_attn(q, m), ref, **TOL)


def test_heads_entry_matches_full():
    c, K, V = _filled(2, 2, 64, 32, 32, 50, seed=2)
    q = _rand(np.random.default_rng(2), (2, 4, 64)).view(np.uint16)
    full = c.decode_attn(q)
    assert np.array_equal(c.decode_attn_heads(q, 1, 1, 3), full[1, 1:3])


def test_empty_cache_gives_zeros():
    c = oracle.Cache(1, 1, 32, 2, 2, 32, 32, 128)
    out = c.decode_attn(np.zeros((1, 1, 32), np.uint16))
    assert not out.any()


@pytest.mark.parametrize("lengths", [(1, 31, 32, 33), (77, 128, 129, 96)])
def test_ragged_rows_are_independent_sequences(lengths):
    """A ragged batch is a set of independent sequences (the serving setting
    of the KIVI section's "Original evaluation setting"): the reference for
    row b is the oracle on that row alone.  Pinned two ways: each row's own
    window split (keys [0, t - t%R) and values [0, t - R) quantized, the rest
    the exact fp16 inputs) and its attention against dense attention over
    its dequantized tokens; and row b of a batched oracle cache equals the
    same sequence in a cache of batch 1."""
    D, G, R = 64, 32, 32
    rng = np.random.default_rng(sum(lengths))
    for t in lengths:
        c, K, V = _filled(1, 2, D, G, R, t, seed=t, kscale=3.0)
        kh, vh = c.materialize()
        n_kq, n_vq = t - t % R, max(0, t - R)
        assert np.array_equal(kh[:, :, n_kq:], K[:, :, n_kq:].astype(np.float32))
        assert np.array_equal(vh[:, :, n_vq:], V[:, :, n_vq:].astype(np.float32))
        if n_kq:
            assert not np.array_equal(kh[:, :, :n_kq], K[:, :, :n_kq].astype(np.float32))
        if n_vq:
            assert not np.array_equal(vh[:, :, :n_vq], V[:, :, :n_vq].astype(np.float32))
        q = _rand(rng, (1, 4, D))
        got = c.decode_attn(q.view(np.uint16))
        np.testing.assert_allclose(got, dense_attention(q.astype(np.float32), kh, vh), **TOL)
    t = max(lengths)
    both, K, V = _filled(3, 2, D, G, R, t, seed=5)
    q = _rand(rng, (3, 4, D)).view(np.uint16)
    full = both.decode_attn(q)
    for b in range(3):
        one = oracle.Cache(1, 2, D, 2, 2, G, R, both.cap)
        one.append(np.ascontiguousarray(K[b:b + 1]).view(np.uint16),
                   np.ascontiguousarray(V[b:b + 1]).view(np.uint16))
        assert np.array_equal(one.decode_attn(q[b:b + 1]), full[b:b + 1])
