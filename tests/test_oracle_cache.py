"""Pins for the oracle's residual-window bookkeeping (CPU only).

Method: KIVI item 4 of the page "Literature audit -- Group 2", section 1
(KIVI), "Core algorithm": keys keep the last t mod R tokens in fp16 and are
quantized in whole R-blocks; values keep the last R tokens in fp16 and pop the
oldest into the quantized store when the window would hold R+1.
"""
import numpy as np
import pytest

import oracle


def _cap(t, R):
    """Smallest capacity >= t that is a multiple of R and of the 128-token record."""
    m = np.lcm(R, oracle.TOKENS_PER_RECORD)
    return int(max(m, -(-t // m) * m))


def _rand(rng, shape):
    return rng.standard_normal(shape).astype(np.float16)


def _check_invariants(cache, K, V):
    """P6: after t tokens, keys [0, t - t%R) are quantized and the rest are in
    the window; values [0, max(0, t-R)) are quantized and the rest are in the
    window; window slots hold tokens bit for bit; quantized groups equal the
    quantizer applied to the source tokens."""
    t = cache.n_tokens
    R, G = cache.R, cache.G
    n_kq = t - t % R
    n_vq = max(0, t - R)
    Kb, Vb = K.view(np.uint16), V.view(np.uint16)
    for tau in range(n_kq, t):
        assert np.array_equal(cache.k_res[:, :, tau % R], Kb[:, :, tau])
    for tau in range(n_vq, t):
        assert np.array_equal(cache.v_res[:, :, tau % R], Vb[:, :, tau])
    if n_kq:
        kc, ks, kz = oracle.pack_keys(Kb[:, :, :n_kq], cache.kb, G)
        ng = n_kq // G
        assert np.array_equal(cache.k_codes[:, :, :ng], kc[:, :, :ng])
        assert np.array_equal(cache.k_scale[:, :, :ng], ks[:, :, :ng])
        assert np.array_equal(cache.k_zero[:, :, :ng].view(np.uint16), kz[:, :, :ng].view(np.uint16))
    # nothing beyond the quantized prefix has been written
    assert not cache.k_codes[:, :, n_kq // G:].any()
    assert not cache.k_scale[:, :, n_kq // G:].any()
    if n_vq:
        vc, vs, vz = oracle.pack_values(Vb[:, :, :n_vq], cache.vb, G)
        assert np.array_equal(cache.v_codes[:, :, :n_vq], vc[:, :, :n_vq])
        assert np.array_equal(cache.v_scale[:, :, :, :n_vq], vs[:, :, :, :n_vq])
        assert np.array_equal(cache.v_zero[:, :, :, :n_vq].view(np.uint16),
                              vz[:, :, :, :n_vq].view(np.uint16))
    assert not cache.v_codes[:, :, n_vq:].any()
    assert not cache.v_scale[:, :, :, n_vq:].any()


@pytest.mark.parametrize("kb,vb,R", [(2, 2, 32), (4, 2, 64), (2, 4, 32)])
def test_window_invariants_random_chunks(kb, vb, R):
    rng = np.random.default_rng(R + kb * 10 + vb)
    B, H, D, G = 2, 2, 64, 32
    t_end = 3 * R + 5
    cap = _cap(t_end, R)
    K = _rand(rng, (B, H, t_end, D))
    V = _rand(rng, (B, H, t_end, D))
    cache = oracle.Cache(B, H, D, kb, vb, G, R, cap)
    _check_invariants(cache, K, V)
    t = 0
    while t < t_end:
        n = int(min(t_end - t, rng.integers(1, R + 7)))
        cache.append(K[:, :, t:t + n].view(np.uint16), V[:, :, t:t + n].view(np.uint16))
        t += n
        assert cache.n_tokens == t
        _check_invariants(cache, K, V)


def test_every_length_up_to_3R_plus_5():
    rng = np.random.default_rng(7)
    B, H, D, G, R = 1, 1, 32, 32, 32
    t_end = 3 * R + 5
    K = _rand(rng, (B, H, t_end, D))
    V = _rand(rng, (B, H, t_end, D))
    cache = oracle.Cache(B, H, D, 2, 2, G, R, 4 * R)
    for t in range(t_end):
        cache.append(K[:, :, t:t + 1].view(np.uint16), V[:, :, t:t + 1].view(np.uint16))
        _check_invariants(cache, K, V)


@pytest.mark.parametrize("T", [1, 31, 32, 33, 64, 100, 128, 129])
def test_prefill_equals_single_appends_equals_slicing(T):
    """P7: append(T) == T x append(1) == the prefill slicing rule, bit for bit."""
    rng = np.random.default_rng(T)
    B, H, D, G, R = 2, 2, 64, 32, 32
    cap = 256
    K = _rand(rng, (B, H, T, D)).view(np.uint16)
    V = _rand(rng, (B, H, T, D)).view(np.uint16)
    a = oracle.Cache(B, H, D, 2, 2, G, R, cap)
    a.append(K, V)
    b = oracle.Cache(B, H, D, 2, 2, G, R, cap)
    for t in range(T):
        b.append(K[:, :, t:t + 1], V[:, :, t:t + 1])
    for name in a.arrays:
        assert np.array_equal(a.arrays[name], b.arrays[name]), name
    # slicing rule: keys [:T - T%R] quantized, values [:T - R] quantized
    n_kq, n_vq = T - T % R, max(0, T - R)
    kc, ks, kz = oracle.pack_keys(K[:, :, :n_kq], 2, G, cap=cap)
    vc, vs, vz = oracle.pack_values(V[:, :, :n_vq], 2, G, cap=cap)
    assert np.array_equal(a.k_codes, kc) and np.array_equal(a.k_scale, ks)
    assert np.array_equal(a.k_zero, kz)
    assert np.array_equal(a.v_codes, vc) and np.array_equal(a.v_scale, vs)
    assert np.array_equal(a.v_zero, vz)


def test_prefill_multiple_of_R_leaves_key_window_empty():
    """Reading of the page's slice for t % R == 0: every key is quantized."""
    rng = np.random.default_rng(1)
    K = _rand(rng, (1, 1, 64, 32)).view(np.uint16)
    V = _rand(rng, (1, 1, 64, 32)).view(np.uint16)
    c = oracle.Cache(1, 1, 32, 2, 2, 32, 32, 128)
    c.append(K, V)
    kh, vh = c.materialize()
    assert c.k_scale[0, 0, :2].all()          # both key groups quantized
    assert c.v_scale[0, 0, 0, :32].all() and not c.v_scale[0, 0, 0, 32:].any()
    # values 32..63 come back exactly (fp16 window); keys do not in general
    assert np.array_equal(vh[0, 0, 32:], V[0, 0, 32:].view(np.float16).astype(np.float32))


def test_capacity_and_argument_errors():
    c = oracle.Cache(1, 1, 32, 2, 2, 32, 32, 128)
    x = np.zeros((1, 1, 129, 32), np.uint16)
    with pytest.raises(ValueError):
        c.append(x, x)
    with pytest.raises(ValueError):
        oracle.pack_keys(np.zeros((1, 1, 33, 32), np.uint16), 2, 32)   # T % G != 0
    with pytest.raises(ValueError):
        oracle.pack_keys(np.zeros((1, 1, 32, 32), np.uint16), 3, 32)   # bits
