"""GPU parity of ragged batches: every batch row its own sequence with its
own token count (the serving setting of the KIVI section's "Original
evaluation setting" on the page "Literature audit -- Group 2").  Each
(row, KV head) slab is rebuilt alone by the CPU oracle from that row's
tokens; packed stores and windows compare bit for bit, attention within
2e-3 + 1e-3*|ref| elementwise."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_pack_amd import kivi, synth
from tests.gpu_util import (assert_close, b16, cap_for, check_every_slab, dev, host, pool, say)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

P = kivi


def _inputs(B, H, Hq, D, T_max, n_steps, seed):
    rng = np.random.default_rng(seed)

    def f16(shape, scale=1.0):
        return (rng.standard_normal(shape, dtype=np.float32) * scale).astype(np.float16)

    gain = np.ones((B, H, 1, D), np.float32)
    gain[:, :, :, :4] = 12.0                  # outlier key channels
    k0 = (rng.standard_normal((B, H, T_max, D), dtype=np.float32) * gain).astype(np.float16)
    return {"k0": k0, "v0": f16((B, H, T_max, D)),
            "k_steps": [(rng.standard_normal((B, H, 1, D), dtype=np.float32) * gain)
                        .astype(np.float16) for _ in range(n_steps)],
            "v_steps": [f16((B, H, 1, D)) for _ in range(n_steps)],
            "q_steps": [f16((B, Hq, D)) for _ in range(n_steps + 1)]}


def _prefill(g, inp, lengths):
    for b, T in enumerate(lengths):
        if T:
            kivi.kivi_append_row(g, b, dev(inp["k0"][b, :, :T]), dev(inp["v0"][b, :, :T]))
    assert g.row_tokens == [int(x) for x in lengths]


def _oracle_rows(g, inp, lengths):
    """Oracle caches of every slab: row b's prefill alone."""
    def one(bh):
        b, h = bh
        o = oracle.Cache(1, 1, g.D, g.kb, g.vb, g.G, g.R, g.cap, scale_fp16=g.scale_fp16)
        T = int(lengths[b])
        if T:
            o.append(b16(inp["k0"][b:b + 1, h:h + 1, :T]), b16(inp["v0"][b:b + 1, h:h + 1, :T]))
        return o
    slabs = [(b, h) for b in range(g.B) for h in range(g.H)]
    return dict(zip(slabs, pool().map(one, slabs)))


def _oracle_step(orc, inp, s):
    def one(bh):
        b, h = bh
        orc[bh].append(b16(inp["k_steps"][s][b:b + 1, h:h + 1]),
                       b16(inp["v_steps"][s][b:b + 1, h:h + 1]))
    list(pool().map(one, sorted(orc)))


class _W:
    """Shape record for check_every_slab."""

    def __init__(self, name, g, Hq):
        self.name, self.B, self.Hkv, self.Hq, self.D = name, g.B, g.H, Hq, g.D


def _paths(g, Hq):
    rep = Hq // g.H
    paths = [P.KIVI_PATH_AUTO, P.KIVI_PATH_GENERIC]
    if g.D == 128 and g.G == 32 and (rep == 1 or (rep % 2 == 0 and rep <= 64)) and g.R % 32 == 0:
        paths.append(P.KIVI_PATH_VECTOR)
    # the matrix kernel forced where it takes the cache: 2-bit, or 4-bit keys
    # and values (any batch, contiguous or paged), on the shape it serves
    if (g.D == 128 and g.G == 32 and rep in (1, 2, 4) and (g.kb, g.vb) in ((2, 2), (4, 4))
            and g.n_tokens > 0):
        paths.append(P.KIVI_PATH_MATRIX)
    return paths


def test_ragged_b8_1k_32k():
    """Eight rows with prefills spread over 1k..32k tokens on the Llama-3-8B
    GQA shape (32 query / 8 KV heads, 2-bit, G 32, R 128), each prefilled
    into its row alone, then one fused decode step; the step's output, every
    attention path and the no-allocation call against the oracle on all 64
    slabs, with the stores after the step bit for bit."""
    w = synth.RAGGED
    lengths = synth.ragged_lengths(w.B, 1024, w.T0)
    say(f"{w.name}: lengths {lengths.tolist()}")
    inp = synth.make_inputs(w)
    g = kivi.Cache(w.B, w.Hkv, w.D, w.k_bits, w.v_bits, w.G, w.R, w.capacity, ragged=True)
    _prefill(g, inp, lengths)
    q = inp["q_steps"][0]
    out_step = host(kivi.kivi_decode_step(g, dev(inp["k_steps"][0]), dev(inp["v_steps"][0]),
                                          dev(q)))
    assert g.row_tokens == [int(x) + 1 for x in lengths]
    assert g.n_tokens == int(lengths.max()) + 1
    outs = {"step": out_step}
    for p in _paths(g, w.Hq):
        outs[f"path {p}"] = host(kivi.kivi_decode_attn(g, dev(q), path=p))
    noalloc = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    outs["noalloc"] = host(kivi.kivi_decode_attn_noalloc(g, dev(q), noalloc))
    say(f"{w.name}: oracle over {w.B * w.Hkv} slabs")
    orc = _oracle_rows(g, inp, lengths)
    _oracle_step(orc, inp, 0)
    check_every_slab(w, g, orc, outs, q)


@pytest.mark.parametrize("rep,R,bits", [(4, 128, 2), (1, 128, 2), (2, 32, 2), (4, 64, 4),
                                        (1, 128, 4)])
def test_ragged_steps_cross_boundaries(rep, R, bits):
    """Fused (2-bit) and unfused (4-bit) decode steps on rows whose lengths
    make different rows pop a value, complete a key block or start from an
    empty row at different steps; every slab against the oracle after each
    of four steps."""
    H, D, G = 2, 128, 32
    lengths = [0, 1, R - 2, 2 * R - 1, 3 * R + 5, 900, 129, R]
    B, Hq, n_steps = len(lengths), 2 * rep, 4
    cap = cap_for(max(lengths) + n_steps, R)
    inp = _inputs(B, H, Hq, D, max(lengths), n_steps, seed=rep * 100 + R + bits)
    g = kivi.Cache(B, H, D, bits, bits, G, R, cap, ragged=True)
    _prefill(g, inp, lengths)
    orc = _oracle_rows(g, inp, lengths)
    w = _W(f"ragged rep{rep} R{R} {bits}-bit", g, Hq)
    for s in range(n_steps):
        q = inp["q_steps"][s]
        out = host(kivi.kivi_decode_step(g, dev(inp["k_steps"][s]), dev(inp["v_steps"][s]),
                                         dev(q)))
        _oracle_step(orc, inp, s)
        outs = {f"step {s}": out}
        if s == n_steps - 1:
            for p in _paths(g, Hq):
                outs[f"path {p}"] = host(kivi.kivi_decode_attn(g, dev(q), path=p))
        check_every_slab(w, g, orc, outs, q)


@pytest.mark.parametrize("D,G,bits", [(64, 32, 2), (128, 128, 2), (128, 64, 4)])
def test_ragged_other_shapes(D, G, bits):
    """Shapes outside the matrix and vector kernels (scalar kernel; per-row
    appends where the one-launch step kernel does not take G): a ragged
    prefill, two decode steps and attention against the oracle."""
    H, Hq, R = 2, 4, 128
    lengths = [300, 0, 129, 1000]
    B, n_steps = len(lengths), 2
    cap = cap_for(max(lengths) + n_steps, R)
    inp = _inputs(B, H, Hq, D, max(lengths), n_steps, seed=D + G + bits)
    g = kivi.Cache(B, H, D, bits, bits, G, R, cap, ragged=True)
    _prefill(g, inp, lengths)
    orc = _oracle_rows(g, inp, lengths)
    w = _W(f"ragged D{D} G{G} {bits}-bit", g, Hq)
    for s in range(n_steps):
        q = inp["q_steps"][s]
        out = host(kivi.kivi_decode_step(g, dev(inp["k_steps"][s]), dev(inp["v_steps"][s]),
                                         dev(q)))
        _oracle_step(orc, inp, s)
        check_every_slab(w, g, orc, {f"step {s}": out}, q)


@pytest.mark.parametrize("rep", [1, 4])
def test_ragged_mask(rep):
    """A mask [B][longest row]: entries past a row's count are NaN, so any
    read of them would show in the output; a fully masked row gives zeros."""
    H, D, G, R = 2, 128, 32, 128
    lengths = [2000, 37, 640, 1281]
    B, Hq = len(lengths), 2 * rep
    cap = cap_for(max(lengths), R)
    inp = _inputs(B, H, Hq, D, max(lengths), 0, seed=rep)
    g = kivi.Cache(B, H, D, 2, 2, G, R, cap, ragged=True)
    _prefill(g, inp, lengths)
    rng = np.random.default_rng(rep)
    t = max(lengths)
    m = np.where(rng.random((B, t)) < 0.2, -np.inf, rng.standard_normal((B, t))).astype(np.float32)
    for b, T in enumerate(lengths):
        m[b, T:] = np.nan
    m[1, :lengths[1]] = -np.inf
    q = inp["q_steps"][0]
    outs = {f"path {p}": host(kivi.kivi_decode_attn(g, dev(q), mask=dev(m), path=p))
            for p in _paths(g, Hq)}
    for label, o in outs.items():
        assert not o[1].any(), f"{label}: a fully masked row"
    check_every_slab(_W(f"ragged mask rep{rep}", g, Hq), g, _oracle_rows(g, inp, lengths),
                     outs, q, mask=m, stores=False)


def test_ragged_equal_rows_match_uniform():
    """Rows of equal length: the ragged launch (its own plan and tables)
    gives the uniform cache's output up to the rounding order of merges."""
    B, H, Hq, D, G, R, T = 4, 8, 32, 128, 32, 128, 5000
    inp = _inputs(B, H, Hq, D, T, 0, seed=11)
    cap = cap_for(T, R)
    u = kivi.Cache(B, H, D, 2, 2, G, R, cap)
    kivi.kivi_append(u, dev(inp["k0"]), dev(inp["v0"]))
    r = kivi.Cache(B, H, D, 2, 2, G, R, cap, ragged=True)
    _prefill(r, inp, [T] * B)
    q = dev(inp["q_steps"][0])
    for p in _paths(u, Hq):
        a = host(kivi.kivi_decode_attn(u, q, path=p))
        b = host(kivi.kivi_decode_attn(r, q, path=p))
        np.testing.assert_allclose(b, a, rtol=1e-5, atol=1e-6, err_msg=f"path {p}")


def test_ragged_reset_row_and_refill():
    """The serving cycle: a row is emptied and a new, shorter request is
    prefilled into it; its slabs then match the oracle on the new sequence
    while the other rows keep theirs."""
    H, Hq, D, G, R = 2, 8, 128, 32, 128
    lengths = [700, 1500, 260]
    B = len(lengths)
    cap = cap_for(2000, R)
    inp = _inputs(B, H, Hq, D, max(lengths), 1, seed=5)
    new = _inputs(1, H, Hq, D, 333, 0, seed=6)
    g = kivi.Cache(B, H, D, 2, 2, G, R, cap, ragged=True)
    _prefill(g, inp, lengths)
    g.reset_row(1)
    assert g.row_tokens == [700, 0, 260] and g.n_tokens == 700
    kivi.kivi_append_row(g, 1, dev(new["k0"][0]), dev(new["v0"][0]))
    lengths2 = [700, 333, 260]
    inp2 = dict(inp)
    k0 = inp["k0"].copy()
    v0 = inp["v0"].copy()
    k0[1, :, :333] = new["k0"][0]
    v0[1, :, :333] = new["v0"][0]
    inp2["k0"], inp2["v0"] = k0, v0
    q = inp["q_steps"][0]
    out = host(kivi.kivi_decode_step(g, dev(inp["k_steps"][0]), dev(inp["v_steps"][0]), dev(q)))
    orc = _oracle_rows(g, inp2, lengths2)
    _oracle_step(orc, inp2, 0)
    check_every_slab(_W("ragged refill", g, Hq), g, orc, {"step": out}, q)
