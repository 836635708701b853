"""GPU parity of paged caches: the records of each row's 128-token blocks
live in pages of a shared pool, in any order, named by a device page table
(include/kivi.h).  Every slab is compared with the CPU oracle (which keeps
the contiguous layout) after gathering the pages back into token order:
packed stores and windows bit for bit, attention within 2e-3 + 1e-3*|ref|
(KIVI items 1-5 of the page "Literature audit -- Group 2", section 1; paging
serves the section's serving setting, "Original evaluation setting")."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_pack_amd import kivi
from tests.gpu_util import (assert_close, b16, cap_for, check_every_slab, dev, host, logical,
                            pool, say)
from tests.test_gpu_ragged import _W, _inputs, _oracle_rows, _oracle_step, _paths

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _map_pages(g, lengths, rng, spare=5):
    """Give each row's first blocks (enough for `lengths` tokens) distinct
    pages of the pool, in a random order; other entries -1."""
    nrec = g.cap // kivi.TOKENS_PER_RECORD
    need = [min(nrec, -(-int(t) // kivi.TOKENS_PER_RECORD)) for t in lengths]
    perm = rng.permutation(g.pages)
    assert sum(need) <= g.pages
    pt = np.full((g.B, nrec), -1, np.int32)
    k = 0
    for b, n in enumerate(need):
        pt[b, :n] = perm[k:k + n]
        k += n
    g.page_table.copy_(torch.from_numpy(pt))
    return pt


@pytest.mark.parametrize("D,bits,rep,G,R", [(128, 2, 4, 32, 128), (128, 4, 4, 32, 128),
                                            (128, 2, 1, 32, 32), (64, 2, 2, 32, 64)])
def test_paged_uniform_batch(D, bits, rep, G, R):
    """A uniform batch in a shuffled pool: prefill, three decode steps across
    a key block, every attention path."""
    rng = np.random.default_rng(D + bits * 10 + rep + R)
    B, H, T0, n_steps = 3, 2, 2 * R * 5 + R - 2, 3
    Hq = H * rep
    cap = cap_for(T0 + n_steps, R)
    nrec = cap // kivi.TOKENS_PER_RECORD
    inp = _inputs(B, H, Hq, D, T0, n_steps, seed=int(rng.integers(1 << 30)))
    g = kivi.Cache(B, H, D, bits, bits, G, R, cap, pages=B * nrec + 7)
    _map_pages(g, [cap] * B, rng)
    kivi.kivi_append(g, dev(inp["k0"]), dev(inp["v0"]))
    orc = _oracle_rows(g, inp, [T0] * B)
    w = _W(f"paged D{D} {bits}-bit rep{rep} R{R}", g, Hq)
    for s in range(n_steps):
        q = inp["q_steps"][s]
        out = host(kivi.kivi_decode_step(g, dev(inp["k_steps"][s]), dev(inp["v_steps"][s]),
                                         dev(q)))
        _oracle_step(orc, inp, s)
        outs = {f"step {s}": out}
        if s == n_steps - 1:
            for p in _paths(g, Hq):
                outs[f"path {p}"] = host(kivi.kivi_decode_attn(g, dev(q), path=p))
            o = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
            outs["noalloc"] = host(kivi.kivi_decode_attn_noalloc(g, dev(q), o))
        check_every_slab(w, g, orc, outs, q)


def test_paged_ragged_rows_hold_only_their_pages():
    """A ragged batch whose pool holds just the pages its rows use (plus the
    blocks two decode steps open): per-row prefill, steps, attention; rows of
    1 to 20 blocks in one pool, every slab against the oracle."""
    rng = np.random.default_rng(17)
    H, Hq, D, G, R = 2, 8, 128, 32, 128
    lengths = [2500, 130, 0, 1023, 700, 127]
    B, n_steps = len(lengths), 2
    cap = cap_for(max(lengths) + n_steps, R)
    need = sum(-(-(t + n_steps) // 128) for t in lengths)
    inp = _inputs(B, H, Hq, D, max(lengths), n_steps, seed=3)
    g = kivi.Cache(B, H, D, 2, 2, G, R, cap, ragged=True, pages=need)
    _map_pages(g, [t + n_steps for t in lengths], rng)
    nrec = cap // 128
    say(f"pool of {need} pages against {B * nrec} for a contiguous cache")
    for b, T in enumerate(lengths):
        if T:
            kivi.kivi_append_row(g, b, dev(inp["k0"][b, :, :T]), dev(inp["v0"][b, :, :T]))
    orc = _oracle_rows(g, inp, lengths)
    w = _W("paged ragged", g, Hq)
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


@pytest.mark.parametrize("kb,vb,G", [(2, 2, 32), (4, 2, 64)])
def test_paged_pack_entry_points(kb, vb, G):
    """kivi_pack_keys / kivi_pack_values into a paged destination at a token
    offset: the records, gathered back into token order, equal the oracle's
    pack bit for bit."""
    rng = np.random.default_rng(kb * 7 + G)
    B, H, D, T, off = 2, 3, 128, 384, 128
    cap = 640
    k = (rng.standard_normal((B, H, T, D)) * 4).astype(np.float16)
    v = rng.standard_normal((B, H, T, D)).astype(np.float16)
    g = kivi.Cache(B, H, D, kb, vb, G, G, cap, pages=B * cap // 128 + 3)
    _map_pages(g, [cap] * B, rng)
    kivi.kivi_pack_keys(g, dev(k), off)
    kivi.kivi_pack_values(g, dev(v), off)
    gl = logical(g)
    kc, ks, kz = oracle.pack_keys(b16(k), kb, G, cap=cap, offset=off)
    vc, vs, vz = oracle.pack_values(b16(v), vb, G, cap=cap, offset=off)
    g0, g1 = off // G, (off + T) // G
    for name, ref in (("k_codes", kc), ("k_scale", ks), ("k_zero", kz)):
        assert np.array_equal(np.ascontiguousarray(gl[name][:, :, g0:g1]).view(np.uint8),
                              np.ascontiguousarray(ref[:, :, g0:g1]).view(np.uint8)), name
    for name, ref in (("v_codes", vc),):
        assert np.array_equal(gl[name][:, :, off:off + T], ref[:, :, off:off + T]), name
    for name, ref in (("v_scale", vs), ("v_zero", vz)):
        assert np.array_equal(np.ascontiguousarray(gl[name][..., off:off + T]).view(np.uint8),
                              np.ascontiguousarray(ref[..., off:off + T]).view(np.uint8)), name


def test_paged_equals_contiguous_for_selection():
    """The selection workload on a paged cache gives the contiguous cache's
    selection and output (same data, same kernels, other addresses)."""
    rng = np.random.default_rng(5)
    B, H, Hq, D, G, R, T = 2, 2, 8, 128, 32, 128, 3000
    inp = _inputs(B, H, Hq, D, T, 0, seed=9)
    cap = cap_for(T, R)
    a = kivi.Cache(B, H, D, 2, 2, G, R, cap)
    p = kivi.Cache(B, H, D, 2, 2, G, R, cap, pages=B * cap // 128 + 11)
    _map_pages(p, [cap] * B, rng)
    for c in (a, p):
        kivi.kivi_append(c, dev(inp["k0"]), dev(inp["v0"]))
    q = dev(inp["q_steps"][0])
    res = []
    for c in (a, p):
        n = torch.empty((B, Hq), dtype=torch.int32, device="cuda")
        out = kivi.kivi_select_attn(c, q, 0.9, n_selected=n)
        res.append((host(out), host(n)))
    assert np.array_equal(res[0][1], res[1][1])
    np.testing.assert_allclose(res[1][0], res[0][0], rtol=1e-5, atol=1e-6)
