"""GPU parity of the second workload, kivi_select_attn: token selection by
attention mass on the packed keys (Eq. 4 of the paper reviewed on the page
"HCAttention: Extreme KV Cache Compression via Heterogeneous Attention
Computing for LLMs", section "What carries the argument", with the KIVI
scores of the page "Literature audit -- Group 2", section 1, item 5) and the
renormalized attention over the selected tokens (the same review, major
comment 2 on Eq. 5), against oracle/select.py.

The GPU takes the selection from fp32 scores, the oracle from fp64 ones, so a
token at the boundary can differ; what is unique is checked exactly and the
rest for validity: the GPU's set, scored by the oracle, must reach tau, fall
below it without its lowest-scored token, and hold every token scoring
clearly above its lowest member; its size must equal the number of set bits;
and its output must match the oracle's output over that same set."""
import numpy as np
import pytest
import torch

import oracle
from oracle import select as oselect
from decode_attention_pack_amd import kivi, synth
from tests.gpu_util import (assert_close, b16, cap_for, dev, gpu_cache, host, oracle_all_slabs,
                            pool, say)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

MASS_TOL = 1e-4     # oracle mass of the GPU's set vs tau
SCORE_TOL = 2e-3    # fp32 vs fp64 score (scores are O(10))


def _bits(sel_mask, t):
    m = host(sel_mask).view(np.uint32)
    bits = np.unpackbits(m.view(np.uint8), axis=-1, bitorder="little")
    return bits[..., :t].astype(bool)


def _run(g, q, tau, mask=None):
    B, Hq = q.shape[0], q.shape[1]
    t = g.n_tokens
    n_sel = torch.full((B, Hq), -1, dtype=torch.int32, device="cuda")
    smask = torch.zeros((B, Hq, (t + 31) // 32), dtype=torch.int32, device="cuda")
    out = kivi.kivi_select_attn(g, dev(q), tau, mask=None if mask is None else dev(mask),
                                n_selected=n_sel, sel_mask=smask)
    return host(out), host(n_sel), _bits(smask, t)


def _check_row(s, a, vh, sel, out, n, tau, what):
    """One (b, hq) row: s, a the oracle's scores and probabilities, vh its
    dequantized values of the row's KV head, sel / out / n the GPU's."""
    assert n == sel.sum(), f"{what}: count {n} vs {sel.sum()} set bits"
    pos = a > 0
    if not pos.any():
        assert n == 0 and not out.any(), what
        return
    assert not (sel & ~pos).any() or (a[sel & ~pos] < 1e-9).all(), f"{what}: a masked token"
    mass = a[sel].sum()
    assert mass >= tau - MASS_TOL or (sel | ~(a > 1e-10)).all(), f"{what}: mass {mass} < {tau}"
    low = np.nonzero(sel)[0][np.argmin(s[sel])]
    assert mass - a[low] < tau + MASS_TOL, f"{what}: not the smallest set ({mass}, {a[low]})"
    if (~sel & pos).any():
        assert s[~sel & pos].max() <= s[sel].min() + SCORE_TOL, f"{what}: not a top-score set"
    e = np.exp(s[sel] - s[sel].max())
    ref = e @ vh[sel].astype(np.float64) / e.sum()
    assert_close(out, ref, what)


def _check(o, q, tau, out, n_sel, sel, mask=None, label=""):
    ref_out, ref_sel, a, s = oselect.select_attn(o, q, tau, mask)
    _, vh = o.materialize()
    rep = q.shape[1] // o.H
    for b in range(q.shape[0]):
        for hq in range(q.shape[1]):
            _check_row(s[b, hq], a[b, hq], vh[b, hq // rep], sel[b, hq], out[b, hq],
                       int(n_sel[b, hq]), tau, f"{label} b{b} hq{hq}")
    # the oracle's own count is within a few boundary tokens of the GPU's,
    # apart from tokens the GPU counts as mass zero (below 2^-37 of the
    # largest e^(s - max); the oracle keeps every positive mass)
    with np.errstate(invalid="ignore"):   # fully masked rows: -inf - -inf
        rel = np.exp(s - s.max(axis=-1, keepdims=True))
    tiny = (ref_sel & (rel < 2.0 ** -35)).sum(-1)
    diff = np.abs(ref_sel.sum(-1) - n_sel) - tiny
    assert diff.max() <= 2, f"{label}: counts differ by up to {diff.max()}"


def _pair(B, H, Hq, D, kb, vb, G, R, t, seed, kscale=3.0):
    rng = np.random.default_rng(seed)
    K = (rng.standard_normal((B, H, t, D)) * kscale).astype(np.float16)
    V = rng.standard_normal((B, H, t, D)).astype(np.float16)
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    cap = cap_for(t, R)
    g = kivi.Cache(B, H, D, kb, vb, G, R, cap)
    if t:
        kivi.kivi_append(g, dev(K), dev(V))
    o = oracle.Cache(B, H, D, kb, vb, G, R, cap)
    if t:
        o.append(b16(K), b16(V))
    return g, o, q, rng


@pytest.mark.parametrize("t", [1, 31, 300, 2049])
@pytest.mark.parametrize("rep", [1, 2, 4, 8])
@pytest.mark.parametrize("tau", [0.5, 0.9, 1.0])
def test_select_small(t, rep, tau):
    """2-bit D128 G32 (the vector kernel's scores) over windows, boundaries
    and several key groups, 1 to 8 query heads per KV head."""
    g, o, q, _ = _pair(2, 2, 2 * rep, 128, 2, 2, 32, 128, t, seed=t * 7 + rep)
    out, n_sel, sel = _run(g, q, tau)
    _check(o, q.view(np.uint16), tau, out, n_sel, sel, label=f"t{t} rep{rep} tau{tau}")
    if tau == 1.0:
        full = host(kivi.kivi_decode_attn(g, dev(q)))
        assert_close(out, full, "tau 1 vs kivi_decode_attn")


@pytest.mark.parametrize("D,kb,vb,G,R", [(64, 2, 2, 32, 64), (128, 4, 4, 32, 128),
                                          (128, 2, 4, 64, 128), (256, 4, 2, 32, 32)])
def test_select_other_shapes(D, kb, vb, G, R):
    """Other bit widths, groups and head sizes (scalar kernel's scores where
    the vector kernel does not take the shape)."""
    g, o, q, _ = _pair(2, 2, 4, D, kb, vb, G, R, 777, seed=D + kb * 10 + G)
    for tau in (0.3, 0.9):
        out, n_sel, sel = _run(g, q, tau)
        _check(o, q.view(np.uint16), tau, out, n_sel, sel, label=f"D{D} {kb}/{vb} G{G} tau{tau}")


def test_select_mask_and_empty_rows():
    """An additive mask (-inf tokens are never selected; a fully masked row
    selects nothing and gives zeros), and an empty cache."""
    g, o, q, rng = _pair(2, 2, 4, 128, 2, 2, 32, 128, 1000, seed=5)
    t = g.n_tokens
    mask = np.where(rng.random((2, t)) < 0.3, -np.inf, rng.standard_normal((2, t))).astype(np.float32)
    mask[1] = -np.inf
    out, n_sel, sel = _run(g, q, 0.9, mask)
    assert (n_sel[1] == 0).all() and not out[1].any() and not sel[1].any()
    assert not (sel[0] & np.isinf(mask[0])[None]).any()
    _check(o, q.view(np.uint16), 0.9, out, n_sel, sel, mask, "masked")
    e = kivi.Cache(1, 1, 128, 2, 2, 32, 128, 128)
    out, n_sel, _ = _run(e, q[:1, :1].copy(), 0.9)
    assert not out.any() and n_sel[0, 0] == 0


def test_select_ties_by_index():
    """Equal scores are taken by increasing token index: every key row the
    same (all tokens in the fp16 window, so every score is the same float),
    tau = 0.5 of 64 tokens keeps exactly tokens 0..31."""
    rng = np.random.default_rng(8)
    D, t = 128, 64
    K = np.repeat(rng.standard_normal((1, 1, 1, D)).astype(np.float16), t, axis=2)
    V = rng.standard_normal((1, 1, t, D)).astype(np.float16)
    g = kivi.Cache(1, 1, D, 2, 2, 32, 128, 128)
    kivi.kivi_append(g, dev(K), dev(V))
    q = rng.standard_normal((1, 1, D)).astype(np.float16)
    out, n_sel, sel = _run(g, q, 0.5)
    assert n_sel[0, 0] == 32
    assert sel[0, 0, :32].all() and not sel[0, 0, 32:].any()
    assert_close(out[0, 0], V[0, 0, :32].astype(np.float64).mean(0), "ties")


def test_select_llama3_gqa_32k():
    """The 32k GQA workload (4 x 8 KV heads, 32 query heads, 2-bit, G 32,
    R 128) after its prefill and one step, tau = 0.9: every row against the
    oracle, slab by slab."""
    w = synth.WORKLOADS[4]
    inp = synth.make_inputs(w)
    g = gpu_cache(w)
    kivi.kivi_append(g, dev(inp["k0"]), dev(inp["v0"]))
    kivi.kivi_append(g, dev(inp["k_steps"][0]), dev(inp["v_steps"][0]))
    q = inp["q_steps"][0]
    tau = 0.9
    out, n_sel, sel = _run(g, q, tau)
    say(f"{w.name}: selected {n_sel.min()}..{n_sel.max()} of {g.n_tokens} tokens per row")
    orc = oracle_all_slabs(w, inp, n_steps=1)
    rep = w.Hq // w.Hkv

    def one(bh):
        b, h = bh
        o = orc[bh]
        qs = b16(q[b:b + 1, h * rep:(h + 1) * rep])
        _check(o, qs, tau, out[b:b + 1, h * rep:(h + 1) * rep], n_sel[b:b + 1, h * rep:(h + 1) * rep],
               sel[b:b + 1, h * rep:(h + 1) * rep], label=f"slab ({b}, {h})")
        return bh
    list(pool().map(one, sorted(orc)))
