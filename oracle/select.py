"""CPU oracle for the second workload on the packed cache: token selection by
approximate attention mass, then attention over the selected tokens.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this module; the HIP library
and its binding never do.

Method source: web page "HCAttention: Extreme KV Cache Compression via
Heterogeneous Attention Computing for LLMs" (a review of that paper), section
"What carries the argument": Eq. (3) (an approximate attention score per
token from quantized keys) and Eq. (4) (sort the tokens by approximate score
and keep the smallest prefix whose scores sum to at least tau); its major
comment 2 on Eq. (5) (the output over the selected set).  The approximate
score of token j is the KIVI score of the page "Literature audit -- Group 2",
section "1. KIVI -- kivi2024", "Core algorithm" item 5: q . K_j / sqrt(D)
(+ mask), with K_j the dequantized key where quantized and the fp16 key in the
window -- the KIVI codes stand in for the product-quantization codebook of
Eq. (3).

Readings where the pages leave the step open:
  - Selection is per query: recomputed at every decode step from that step's
    q; nothing is removed from the cache (the review's major comment 1 names
    both readings; this is the reversible one).
  - The scores summed in Eq. (4) are the softmax probabilities a = softmax(s)
    over all t tokens, so that tau is a fraction of the attention mass.
  - Order: decreasing score; equal scores by increasing token index.
  - Tokens with a == 0 (masked with -inf, or underflowed) are never selected;
    when the positive masses do not reach tau, every token with a > 0 is.
  - The output is renormalized over the selected set (the review's major
    comment 2): out = sum_S a_j V_j / sum_S a_j.
Arithmetic in fp64 on the oracle's own dequantized keys and values.
"""
from __future__ import annotations

import numpy as np


def select_prefix(scores, tau: float):
    """Eq. (4) on one row of scores.  Returns (selected: bool [t], a: f64 [t])."""
    s = np.asarray(scores, np.float64)
    t = s.shape[0]
    sel = np.zeros(t, bool)
    finite = s > -np.inf
    if not finite.any():
        return sel, np.zeros(t)
    e = np.where(finite, np.exp(s - s[finite].max()), 0.0)
    a = e / e.sum()
    order = np.lexsort((np.arange(t), -s))        # score descending, then index ascending
    cum = np.cumsum(a[order])
    n_pos = int((a > 0).sum())
    hit = np.nonzero(cum >= tau)[0]
    k = min(int(hit[0]) + 1, n_pos) if hit.size else n_pos
    sel[order[:k]] = True
    return sel, a


def scores(cache, q_fp16, mask=None):
    """KIVI item 5 scores of every (batch row, query head) over the oracle
    cache's tokens: f64 [B][Hq][t]."""
    kh, _ = cache.materialize()
    q = np.ascontiguousarray(q_fp16, np.uint16).view(np.float16).astype(np.float64)
    B, Hq, D = q.shape
    rep = Hq // cache.H
    s = np.empty((B, Hq, cache.n_tokens))
    for b in range(B):
        for hq in range(Hq):
            s[b, hq] = kh[b, hq // rep].astype(np.float64) @ q[b, hq] / np.sqrt(D)
            if mask is not None:
                s[b, hq] += np.asarray(mask, np.float64)[b]
    return s


def attend_selected(cache, q_fp16, sel, mask=None):
    """Eq. (5), renormalized: the output of every row over the tokens sel
    marks (bool [B][Hq][t]).  f64 [B][Hq][D]."""
    _, vh = cache.materialize()
    s = scores(cache, q_fp16, mask)
    B, Hq, t = s.shape
    rep = Hq // cache.H
    out = np.zeros((B, Hq, cache.D))
    for b in range(B):
        for hq in range(Hq):
            m = sel[b, hq] & (s[b, hq] > -np.inf)
            if not m.any():
                continue
            e = np.exp(s[b, hq, m] - s[b, hq, m].max())
            out[b, hq] = e @ vh[b, hq // rep][m].astype(np.float64) / e.sum()
    return out


def select_attn(cache, q_fp16, tau: float, mask=None):
    """The whole workload: (out f64 [B][Hq][D], selected bool [B][Hq][t],
    a f64 [B][Hq][t], s f64 [B][Hq][t])."""
    s = scores(cache, q_fp16, mask)
    sel = np.zeros(s.shape, bool)
    a = np.zeros(s.shape)
    for b in range(s.shape[0]):
        for hq in range(s.shape[1]):
            sel[b, hq], a[b, hq] = select_prefix(s[b, hq], tau)
    return attend_selected(cache, q_fp16, sel, mask), sel, a, s
