"""GPU parity of the fp16-scale layout: scales stored as binary16 (s rounded
to the nearest binary16 value, codes chosen for it -- KIVI item 1 of the page
"Literature audit -- Group 2", section 1, with the storage precision the page
leaves open; its item 6 puts storage on the hyperparameter axis).  Packed
codes, scales and zeros against the CPU oracle bit for bit; attention within
2e-3 + 1e-3*|ref| elementwise, through every kernel that takes the shape:
the matrix kernel (2-bit, G 32, D 128), the vector kernel, the scalar one."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_pack_amd import kivi, synth
from tests.gpu_util import (assert_close, b16, cap_for, check_every_slab, compare_slab, dev,
                            gpu_cache, host, logical, oracle_all_slabs, say)
from tests.test_gpu_decode import paths_for as _decode_paths
from tests.test_gpu_pack import _edge_tensor, _same
from tests.test_gpu_ragged import _W, _inputs, _oracle_rows, _oracle_step, _paths
from tests.test_gpu_select import _check, _run

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def paths_for(D, kb, vb, G, R, rep, cap):
    """Every path that takes the shape, the matrix kernel forced where it
    does (2-bit, G 32, D 128, 1, 2 or 4 query heads per KV head)."""
    paths = _decode_paths(D, kb, vb, G, R, rep, cap)
    if (kb, vb, G, D) == (2, 2, 32, 128) and rep in (1, 2, 4):
        paths.append(kivi.KIVI_PATH_MATRIX)
    return paths


def _fp16_scale_edges(x):
    """Groups whose scale is subnormal in fp16 or rounds to zero, and whose
    largest code clamps after the rounding (worked out in the oracle's
    hand-worked cases): key channel 8 along tokens, value token 14 along
    channels."""
    u = np.float16(2.0 ** -24)
    pat = np.array([0, u, 2 * u, 4 * u], np.float16)           # s16 = 2^-24: top code clamps
    zero = np.array([0, u, 0, u], np.float16)                   # s rounds to 0
    T, D = x.shape[2], x.shape[3]
    x[0, 0, :, 8] = np.tile(pat, T // 4)
    x[0, 0, :, 9] = np.tile(zero, T // 4)
    x[0, 0, 14, :] = np.tile(pat, D // 4)
    x[0, 0, 15, :] = np.tile(zero, D // 4)
    return x


def _pack(x16, bits, G, cap, off, keys):
    B, H, T, D = x16.shape
    dst = kivi.Cache(B, H, D, bits, bits, G, G, cap, scale_fp16=True)
    dst.blocks.zero_()
    (kivi.kivi_pack_keys if keys else kivi.kivi_pack_values)(dst, dev(x16), off)
    torch.cuda.synchronize()
    lg = logical(dst)
    n = "k" if keys else "v"
    return lg[f"{n}_codes"], lg[f"{n}_scale"], lg[f"{n}_zero"]


@pytest.mark.parametrize("bits,G,D", [(2, 32, 128), (4, 32, 128), (2, 16, 256), (4, 64, 64),
                                      (2, 128, 256), (4, 8, 64), (2, 16, 96)])
def test_pack_fp16_scales(bits, G, D):
    """Both pack entry points (tile kernels and the general ones), random
    inputs with the edge rows of the fp32 layout's test and fp16-scale edge
    groups, at offset 0 and at an offset off the tile grid."""
    rng = np.random.default_rng(bits * 1000 + G + D)
    B, H, T = 2, 3, max(64, G)
    x = rng.standard_normal((B, H, T, D)).astype(np.float32) * rng.uniform(0.01, 30, (1, H, 1, D))
    x = x.astype(np.float16)
    if D >= 64:
        x[:1, :1] = _fp16_scale_edges(_edge_tensor(rng, T, D)[:, :, :, :D])
    for keys in (True, False):
        for off in (0, 32 if keys else 5):
            if keys and off % G:
                continue
            cap = cap_for(off + T, 128)
            got = _pack(x, bits, G, cap, off, keys)
            fn = oracle.pack_keys if keys else oracle.pack_values
            ref = fn(b16(x), bits, G, cap=cap, offset=off, scale_fp16=True)
            if keys:
                sls = [np.s_[:, :, off // G:(off + T) // G]] * 3
            else:
                sls = [np.s_[:, :, off:off + T], np.s_[..., off:off + T], np.s_[..., off:off + T]]
            for name, g_, r_, sl in zip(("codes", "scale", "zero"), got, ref, sls):
                assert g_.dtype == r_.dtype
                assert _same(g_[sl], r_[sl]), (keys, off, name)


def _sequence(rep, R, T0, n_steps, kb=2, vb=2, B=2, H=2, D=128, G=32, masked=False, seed=0):
    """Prefill, then fused decode steps through pops and key blocks: every
    step's output and, at key-block boundaries and the end, every store."""
    rng = np.random.default_rng(seed + 7 * rep + R + T0)
    t_end = T0 + n_steps
    cap = cap_for(t_end, R)
    K = (rng.standard_normal((B, H, t_end, D)) * rng.uniform(0.5, 15, (1, H, 1, D))).astype(np.float16)
    V = rng.standard_normal((B, H, t_end, D)).astype(np.float16)
    g = kivi.Cache(B, H, D, kb, vb, G, R, cap, scale_fp16=True)
    o = oracle.Cache(B, H, D, kb, vb, G, R, cap, scale_fp16=True)
    kivi.kivi_append(g, dev(K[:, :, :T0]), dev(V[:, :, :T0]))
    o.append(b16(K[:, :, :T0]), b16(V[:, :, :T0]))
    say(f"fp16 scales: rep={rep} R={R} T0={T0} steps={n_steps} bits={kb}/{vb} masked={masked}")
    for i in range(n_steps):
        t = T0 + i
        q = rng.standard_normal((B, H * rep, D)).astype(np.float16)
        k1, v1 = np.ascontiguousarray(K[:, :, t:t + 1]), np.ascontiguousarray(V[:, :, t:t + 1])
        mask = None
        if masked:
            mask = np.where(rng.random((B, t + 1)) < 0.2, -np.inf,
                            rng.standard_normal((B, t + 1))).astype(np.float32)
        out = host(kivi.kivi_decode_step(g, dev(k1), dev(v1), dev(q),
                                         None if mask is None else dev(mask)))
        o.append(b16(k1), b16(v1))
        assert_close(out, o.decode_attn(b16(q), mask), f"step t={t + 1}")
        if (t + 1) % R in (0, 1) or i == n_steps - 1:
            torch.cuda.synchronize()
            for b in range(B):
                for h in range(H):
                    compare_slab(g, b, h, o, b, h)
    q = rng.standard_normal((B, H * rep, D)).astype(np.float16)
    ref = o.decode_attn(b16(q))
    for p in paths_for(D, kb, vb, G, R, rep, cap):
        assert_close(host(kivi.kivi_decode_attn(g, dev(q), path=p)), ref, f"path {p}")


@pytest.mark.parametrize("rep,R,T0,n_steps", [(4, 128, 250, 12), (1, 32, 90, 40), (2, 64, 1000, 30),
                                              (4, 128, 5, 130)])
def test_decode_steps_fp16_scales(rep, R, T0, n_steps):
    """2-bit, G 32, D 128: the fused step and the matrix kernel (pops,
    key blocks quantized inside the launch), then every attention path."""
    _sequence(rep, R, T0, n_steps)


@pytest.mark.parametrize("kb,vb,rep,D,G", [(4, 4, 1, 128, 32), (2, 4, 2, 128, 32),
                                           (4, 2, 8, 128, 32), (2, 2, 2, 64, 32),
                                           (4, 4, 2, 128, 64)])
def test_decode_steps_fp16_scales_other_shapes(kb, vb, rep, D, G):
    """The vector kernel's and the scalar kernel's shapes (unfused appends)."""
    _sequence(rep, 128, 300, 10, kb=kb, vb=vb, D=D, G=G)


def test_decode_masked_fp16_scales():
    """The masked variant of the matrix kernel."""
    _sequence(4, 128, 700, 6, masked=True)


@pytest.mark.parametrize("index", [3, 4])
def test_full_workload_fp16_scales(index):
    """The kivi4-b64 (vector kernel) and 32k GQA (matrix kernel) workloads in
    the fp16-scale layout: prefill, one fused step, every path; every slab's
    store and output against the oracle."""
    w = synth.WORKLOADS[index].replace(scale_fp16=True)
    inp = synth.make_inputs(w)
    g = gpu_cache(w)
    assert g.blocks.shape[-1] == kivi.record_bytes(w.D, w.k_bits, w.v_bits, w.G, True)
    say(f"{w.name} fp16 scales: prefill {w.T0} + 1 fused step")
    kivi.kivi_append(g, dev(inp["k0"]), dev(inp["v0"]))
    q = inp["q_steps"][0]
    outs = {"step": host(kivi.kivi_decode_step(g, dev(inp["k_steps"][0]),
                                               dev(inp["v_steps"][0]), dev(q)))}
    rep = w.Hq // w.Hkv
    for p in paths_for(w.D, w.k_bits, w.v_bits, w.G, w.R, rep, w.capacity):
        outs[f"path {p}"] = host(kivi.kivi_decode_attn(g, dev(q), path=p))
    say(f"{w.name}: oracle over {w.B * w.Hkv} slabs")
    orc = oracle_all_slabs(w, inp, n_steps=1)
    check_every_slab(w, g, orc, outs, q)


def test_ragged_paged_fp16_scales():
    """Ragged rows in a shuffled page pool with fp16 scales: per-row
    prefill, two fused steps, every path, every slab against the oracle."""
    rng = np.random.default_rng(31)
    H, Hq, D, G, R = 2, 8, 128, 32, 128
    lengths = [1500, 130, 0, 700]
    B, n_steps = len(lengths), 2
    cap = cap_for(max(lengths) + n_steps, R)
    nrec = cap // 128
    need = [-(-(t + n_steps) // 128) for t in lengths]
    inp = _inputs(B, H, Hq, D, max(lengths), n_steps, seed=12)
    g = kivi.Cache(B, H, D, 2, 2, G, R, cap, ragged=True, pages=sum(need) + 3, scale_fp16=True)
    perm = rng.permutation(g.pages)
    pt = np.full((B, nrec), -1, np.int32)
    k = 0
    for b, n in enumerate(need):
        pt[b, :n] = perm[k:k + n]
        k += n
    g.page_table.copy_(torch.from_numpy(pt))
    for b, T in enumerate(lengths):
        if T:
            kivi.kivi_append_row(g, b, dev(inp["k0"][b, :, :T]), dev(inp["v0"][b, :, :T]))
    orc = _oracle_rows(g, inp, lengths)
    w = _W("ragged paged fp16 scales", g, Hq)
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


@pytest.mark.parametrize("kb,vb,rep", [(2, 2, 4), (4, 4, 1), (2, 2, 1)])
def test_select_fp16_scales(kb, vb, rep):
    """The selection workload on an fp16-scale cache against the oracle's
    selection over the same stored grid."""
    rng = np.random.default_rng(kb * 10 + rep)
    B, H, D, G, R, t = 2, 2, 128, 32, 128, 1500
    K = (rng.standard_normal((B, H, t, D)) * 3).astype(np.float16)
    V = rng.standard_normal((B, H, t, D)).astype(np.float16)
    q = rng.standard_normal((B, H * rep, D)).astype(np.float16)
    cap = cap_for(t, R)
    g = kivi.Cache(B, H, D, kb, vb, G, R, cap, scale_fp16=True)
    kivi.kivi_append(g, dev(K), dev(V))
    o = oracle.Cache(B, H, D, kb, vb, G, R, cap, scale_fp16=True)
    o.append(b16(K), b16(V))
    for tau in (0.5, 0.9):
        out, n_sel, sel = _run(g, q, tau)
        _check(o, q.view(np.uint16), tau, out, n_sel, sel, label=f"fp16 scales tau{tau}")


def test_fp16_scales_differ_from_fp32_scales():
    """The two layouts are different stores of the same input: their records
    differ in size, and codes differ where the rounding of s moves a ratio
    across a half-integer.  4-bit key groups of -2, -1, 0, 1.5, 3 repeated
    along tokens: 1.5 is code 10 with the fp32 scale (3.5 / 0.33333334
    rounds to 10.5, then to even) and 11 with the fp16 one (3.5 / 0.33325 =
    10.5025), as in the oracle's hand-worked case."""
    D, G = 128, 32
    assert kivi.record_bytes(D, 2, 2, G) == 14336
    assert kivi.record_bytes(D, 2, 2, G, True) == 12288
    x = np.zeros((1, 1, 32, D), np.float16)
    x[0, 0] = np.tile(np.array([-2.0, -1.0, 0.0, 1.5, 3.0], np.float16), 7)[:32, None]
    a = kivi.Cache(1, 1, D, 4, 4, G, G, 128)
    b = kivi.Cache(1, 1, D, 4, 4, G, G, 128, scale_fp16=True)
    for c in (a, b):
        c.blocks.zero_()
        kivi.kivi_pack_keys(c, dev(x), 0)
    torch.cuda.synchronize()
    ka, kb_ = logical(a)["k_codes"][0, 0, 0], logical(b)["k_codes"][0, 0, 0]
    # token 3 of every channel: bits 12..15 of the group's first word
    assert ((ka[:, 0] >> 12) & 15 == 10).all() and ((kb_[:, 0] >> 12) & 15 == 11).all()
