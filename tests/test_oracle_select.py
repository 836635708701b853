"""Pins for the oracle of the second workload (CPU only): cumulative-mass
token selection, Eq. (4) of the paper reviewed on the page "HCAttention:
Extreme KV Cache Compression via Heterogeneous Attention Computing for LLMs"
(section "What carries the argument"), on the KIVI scores (page "Literature
audit -- Group 2", section 1, item 5), and the renormalized output over the
selected tokens (the same review, major comment 2 on Eq. (5))."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from oracle import select

HERE = os.path.dirname(os.path.abspath(__file__))


def _cases():
    with open(os.path.join(HERE, "golden", "select_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["note"][:40])
def test_hand_worked_selections(case):
    s = np.array([float(x) for x in case["scores"]])
    sel, a = select.select_prefix(s, case["tau"])
    assert sorted(np.nonzero(sel)[0].tolist()) == case["selected"]
    if np.isfinite(s).any():
        assert abs(a.sum() - 1.0) < 1e-12


def test_brute_force_smallest_set():
    """For small rows, the selection has the smallest size of any token set
    whose mass reaches tau (enumerating every subset), and among sets of that
    size the largest mass -- the defining property of the sorted prefix."""
    rng = np.random.default_rng(3)
    for trial in range(300):
        n = int(rng.integers(1, 9))
        s = rng.standard_normal(n) * rng.choice([0.5, 2.0, 6.0])
        if trial % 5 == 0:
            s[rng.integers(0, n)] = -np.inf
        tau = float(rng.choice([0.3, 0.5, 0.8, 0.9, 0.99, 1.0]))
        sel, a = select.select_prefix(s, tau)
        pos = np.nonzero(a > 0)[0]
        best = None
        for k in range(1, len(pos) + 1):
            masses = [a[list(c)].sum() for c in itertools.combinations(pos, k)]
            if max(masses) >= tau:
                best = (k, max(masses))
                break
        if best is None:                   # rounding: the whole positive mass < tau
            assert sel.sum() == len(pos) and sel[pos].all()
            continue
        assert sel.sum() == best[0], (s, tau)
        assert abs(a[sel].sum() - best[1]) < 1e-12


def _cache(seed, t=300, B=2, H=2, D=64, G=32, R=64):
    rng = np.random.default_rng(seed)
    K = (rng.standard_normal((B, H, t, D)) * 3).astype(np.float16)
    V = rng.standard_normal((B, H, t, D)).astype(np.float16)
    c = oracle.Cache(B, H, D, 2, 2, G, R, 384)
    c.append(K.view(np.uint16), V.view(np.uint16))
    q = rng.standard_normal((B, 2 * H, D)).astype(np.float16).view(np.uint16)
    return c, q, rng


def test_tau_one_is_full_attention():
    """tau = 1 keeps every token with positive mass: the output is KIVI
    item 5's attention as the C oracle computes it."""
    c, q, rng = _cache(1)
    mask = np.where(rng.random((2, c.n_tokens)) < 0.1, -np.inf, 0.0).astype(np.float32)
    for m in (None, mask):
        out, sel, a, s = select.select_attn(c, q, 1.0, m)
        np.testing.assert_allclose(out, c.decode_attn(q, m), rtol=1e-5, atol=1e-6)
        assert (sel == (a > 0)).all()


def test_tiny_tau_is_the_top_token():
    """A tau below every single mass keeps only the highest-scoring token:
    the output is that token's dequantized value."""
    c, q, _ = _cache(2)
    out, sel, a, s = select.select_attn(c, q, 1e-9)
    _, vh = c.materialize()
    assert (sel.sum(axis=2) == 1).all()
    for b in range(2):
        for hq in range(4):
            j = int(np.argmax(s[b, hq]))
            assert sel[b, hq, j]
            np.testing.assert_array_equal(out[b, hq], vh[b, hq // 2, j].astype(np.float64))


def test_selected_mass_and_size():
    """On a real cache: the selected mass reaches tau, dropping the selection's
    lowest-scored token falls below it, and every selected score is at least
    every unselected one."""
    c, q, _ = _cache(3, t=333)
    for tau in (0.5, 0.9, 0.99):
        _, sel, a, s = select.select_attn(c, q, tau)
        for b in range(2):
            for hq in range(4):
                m = sel[b, hq]
                assert a[b, hq, m].sum() >= tau
                low = np.nonzero(m)[0][np.argmin(s[b, hq, m])]
                assert a[b, hq, m].sum() - a[b, hq, low] < tau
                if (~m).any():
                    assert s[b, hq, m].min() >= s[b, hq, ~m].max()
