"""Pins of the oracle's fp16-scale layout (KIVI item 1 of the page
"Literature audit -- Group 2", section 1, with the scale stored as binary16;
the storage precision of s is a reading, the page fixes none).

- the fp32 -> binary16 rounding against hand-worked patterns
  (tests/golden/scale_fp16_cases.json) and against numpy's own conversion,
  an independent implementation, over every binade's ties and neighbours;
- the quantizer against hand-worked groups, against a brute-force nearest
  grid point search, and against the fp32-scale quantizer wherever the
  scale is exactly a binary16 value (there the two layouts must agree);
- the record layout against hand-worked offsets and bytes;
- the cache: dequantized keys and values are code * s16 + z read from the
  records, and a cache whose scales are binary16-exact reproduces the
  fp32-scale cache's attention."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "scale_fp16_cases.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("e", _golden()["half_rne"], ids=lambda e: e["what"][:24])
def test_half_rne_hand_worked(e):
    x = np.array([int(e["x"], 16)], np.uint32).view(np.float32)[0]
    assert oracle.half_rne(x) == int(e["bits"], 16)


def _rne_sample():
    """Every finite binary16 value, the fp32 midpoints between neighbours
    (the ties), the fp32 values one ulp either side of each midpoint, and
    random fp32 values across the whole range."""
    pats = np.arange(0, 0x7c00, dtype=np.uint16)
    h = pats.view(np.float16).astype(np.float64)
    mids = ((h[:-1] + h[1:]) / 2).astype(np.float32)      # exact in fp32
    m_bits = mids.view(np.uint32)
    near = np.concatenate([m_bits - 1, m_bits + 1]).view(np.float32)
    rng = np.random.default_rng(3)
    rnd = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 18, 20000))).astype(np.float32)
    top = np.array([65504, 65519.99, 65520, 65536, 1e30, 3.4e38], np.float32)
    x = np.concatenate([h.astype(np.float32), mids, near, rnd, top])
    return np.concatenate([x, -x])


def test_half_rne_against_numpy():
    x = _rne_sample()
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle.half_rne(v) for v in x], np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


@pytest.mark.parametrize("c", _golden()["quantizer"], ids=lambda c: c["name"])
def test_quantizer_hand_worked(c):
    codes, s16, z = oracle.quantize_group_s16(np.array(c["x"], np.float32), c["bits"])
    assert codes.tolist() == c["codes"]
    assert int(np.array([s16]).view(np.uint16)[0]) == int(c["scale_bits"], 16)
    assert z == np.float32(c["zero"])
    deq = [float(oracle.dequant(q, np.float32(s16), z)) for q in codes]
    assert deq == c["dequant"]


def _groups(rng, n, count):
    """fp16 groups with spreads from subnormal to large, as fp32."""
    out = []
    for i in range(count):
        spread = float(np.exp2(rng.uniform(-26, 15)))
        x = (rng.uniform(-1, 1, n) * spread + rng.normal() * spread * rng.integers(0, 2))
        out.append(np.clip(x, -65504, 65504).astype(np.float16).astype(np.float32))
    return out


@pytest.mark.parametrize("bits", [2, 4])
def test_codes_are_nearest_grid_points(bits):
    """Every code is a nearest point of the stored grid {c s16 + z : 0 <= c
    <= 2^B - 1} to its input (fp64 distances; a tie may go either way), and
    s16 is the binary16 value nearest to (max - min) / (2^B - 1)."""
    rng = np.random.default_rng(bits)
    qmax = (1 << bits) - 1
    for x in _groups(rng, 32, 400):
        codes, s16, z = oracle.quantize_group_s16(x, bits)
        s = np.float32(np.float32(x.max()) - np.float32(x.min())) / np.float32(qmax)
        assert np.float16(s).view(np.uint16) == np.array([s16]).view(np.uint16)[0]
        assert z == x.min()
        s16 = float(s16)
        if s16 == 0.0:
            assert not codes.any()
            continue
        grid = np.arange(qmax + 1) * s16 + float(z)
        dist = np.abs(x.astype(np.float64)[:, None] - grid[None, :])
        best = dist.min(axis=1)
        mine = dist[np.arange(x.size), codes]
        assert np.all(mine <= best + 1e-6 * s16), (x, codes, s16)


@pytest.mark.parametrize("bits", [2, 4])
def test_equals_fp32_quantizer_when_scale_is_half_exact(bits):
    """Where (max - min) / (2^B - 1) is itself a binary16 value the rounding
    is the identity, so codes, scale and zero equal the fp32-scale
    quantizer's (pinned by hand-worked cases of its own)."""
    rng = np.random.default_rng(10 + bits)
    qmax = (1 << bits) - 1
    n_checked = 0
    for _ in range(300):
        s = np.float16(rng.integers(1, 64) * 2.0 ** int(rng.integers(-12, 6)))
        z = np.float16(rng.integers(-50, 50) * 2.0 ** int(rng.integers(-6, 2)))
        hi = np.float16(np.float32(z) + np.float32(s) * qmax)
        if not np.isfinite(hi) or np.float32(hi) - np.float32(z) != np.float32(s) * qmax:
            continue
        x = rng.uniform(float(z), float(hi), 30).astype(np.float16).astype(np.float32)
        x = np.concatenate([x, [np.float32(z), np.float32(hi)]]).astype(np.float32)
        c16, s16, z16 = oracle.quantize_group_s16(x, bits)
        c32, s32, z32 = oracle.quantize_group(x, bits)
        assert np.float32(s16) == s32 and z16 == z32
        assert np.array_equal(c16, c32)
        n_checked += 1
    assert n_checked > 100


def test_record_case():
    """Section offsets and raw bytes of an fp16-scale record, by hand."""
    case = _golden()["record_case"]
    shp = case["shape"]
    D, G, cap = shp["D"], shp["G"], shp["capacity"]
    off = case["section_offsets"]
    assert oracle.record_bytes(D, 2, 2, G, scale_fp16=True) == off["record_bytes"]
    assert [(n, o) for n, o, _ in oracle.record_sections(D, 2, 2, G, scale_fp16=True)] == \
        [(n, off[n]) for n in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero")]
    tau = np.arange(32)[:, None]
    ch = np.arange(32)[None, :]
    x = (((tau + ch) % 4) - 1.5).astype(np.float16)[None, None]
    c = oracle.Cache(1, 1, D, 2, 2, G, 32, cap, scale_fp16=True)
    c.append(x.view(np.uint16), x.view(np.uint16))          # t = 32: keys quantized
    d = oracle.Cache(1, 1, D, 2, 2, G, 32, cap, scale_fp16=True)
    xx = np.concatenate([x, x], axis=2).view(np.uint16)
    d.append(xx, xx)                                        # t = 64: values 0..31 popped
    for e in case["bytes"]:
        rec = (d if "value" in e["what"] else c).blocks[0, 0, 0]
        got = bytes(rec[e["offset"]:e["offset"] + len(e["hex"]) // 2]).hex()
        assert got == e["hex"], e["what"]


def _seq(rng, B, H, T, D, outliers=True):
    k = rng.standard_normal((B, H, T, D)).astype(np.float32)
    if outliers:
        k[..., :4] *= 12.0
    v = rng.standard_normal((B, H, T, D)).astype(np.float32)
    return k.astype(np.float16), v.astype(np.float16)


@pytest.mark.parametrize("kb,vb,G,R", [(2, 2, 32, 32), (4, 2, 64, 64), (2, 4, 32, 128)])
def test_materialize_reads_the_stored_grid(kb, vb, G, R):
    """Every dequantized key and value of an fp16-scale cache is code * s16
    + z (fp32 product, then sum) with code, s16 and z as the records hold
    them (numpy's binary16 widening); window tokens are the fp16 inputs."""
    rng = np.random.default_rng(kb * 10 + vb + G)
    B, H, D, T = 1, 2, 128, 3 * R + 17
    cap = -(-T // 128) * 128              # R divides 128
    k, v = _seq(rng, B, H, T, D)
    c = oracle.Cache(B, H, D, kb, vb, G, R, cap, scale_fp16=True)
    c.append(k.view(np.uint16), v.view(np.uint16))
    kh, vh = c.materialize()
    L = c.logical()
    t = c.n_tokens
    n_kq, n_vq = t - t % R, max(0, t - R)
    assert L["k_scale"].dtype == np.float16 and L["v_scale"].dtype == np.float16
    for tau in range(t):
        if tau < n_kq:
            g = tau // G
            e = tau % G
            w = L["k_codes"][0, :, g, :, e // (32 // kb)]
            code = (w >> np.uint32(kb * (e % (32 // kb)))) & np.uint32((1 << kb) - 1)
            ref = (code.astype(np.float32) * L["k_scale"][0, :, g].astype(np.float32)) \
                + L["k_zero"][0, :, g].astype(np.float32)
        else:
            ref = k[0, :, tau].astype(np.float32)
        assert np.array_equal(kh[0, :, tau], ref), ("key", tau)
        if tau < n_vq:
            ch = np.arange(D)
            w = L["v_codes"][0, :, tau][:, ch // (32 // vb)]
            code = (w >> (np.uint32(vb) * (ch % (32 // vb)).astype(np.uint32))) & \
                np.uint32((1 << vb) - 1)
            ref = (code.astype(np.float32) * L["v_scale"][0][:, ch // G, tau].astype(np.float32)) \
                + L["v_zero"][0][:, ch // G, tau].astype(np.float32)
        else:
            ref = v[0, :, tau].astype(np.float32)
        assert np.array_equal(vh[0, :, tau], ref), ("value", tau)


def test_half_exact_scales_give_the_fp32_layout_attention():
    """Inputs built so that every key and value group spans [0, 3 f] with f
    = m 2^j (m odd, at most 7) on a grid of f / 8: every scale (3 f) / 3 = f
    is binary16-exact, so the fp16-scale cache holds the fp32-scale cache's
    codes, scales and zeros, and attention is identical (the fp32 layout is
    pinned against textbook attention)."""
    rng = np.random.default_rng(8)
    B, H, Hq, D, G, R, T = 1, 2, 4, 64, 32, 32, 200

    def factors(shape):
        return rng.choice([1, 3, 5, 7], shape) * np.exp2(rng.integers(-4, 3, shape))

    k = rng.integers(0, 25, (B, H, T, D)) / 8.0
    v = rng.integers(0, 25, (B, H, T, D)) / 8.0
    for g0 in range(0, T, G):                      # every key group spans [0, 3]
        k[:, :, g0, :] = 0.0
        k[:, :, g0 + 1, :] = 3.0
    for c0 in range(0, D, G):                      # every value group spans [0, 3]
        v[..., c0] = 0.0
        v[..., c0 + 1] = 3.0
    n_g = -(-T // G)
    fk = np.repeat(factors((B, H, n_g, 1, D)), G, axis=3).reshape(B, H, n_g * G, D)[:, :, :T]
    fv = np.repeat(factors((B, H, T, D // G, 1)), G, axis=4).reshape(B, H, T, D)
    k = (k * fk).astype(np.float16)
    v = (v * fv).astype(np.float16)
    cap = 256
    a = oracle.Cache(B, H, D, 2, 2, G, R, cap)
    b = oracle.Cache(B, H, D, 2, 2, G, R, cap, scale_fp16=True)
    for c in (a, b):
        c.append(k.view(np.uint16), v.view(np.uint16))
    la, lb = a.logical(), b.logical()
    t = a.n_tokens
    n_kq, n_vq = t - t % R, t - R
    assert np.array_equal(la["k_scale"][..., :n_kq // G, :],
                          lb["k_scale"][..., :n_kq // G, :].astype(np.float32))
    assert np.array_equal(la["v_scale"][..., :n_vq], lb["v_scale"][..., :n_vq].astype(np.float32))
    assert np.array_equal(la["k_codes"], lb["k_codes"]) and np.array_equal(la["v_codes"], lb["v_codes"])
    assert len(np.unique(la["k_scale"][..., :n_kq // G, :])) > 10
    q = rng.standard_normal((B, Hq, D)).astype(np.float16).view(np.uint16)
    assert np.array_equal(a.decode_attn(q), b.decode_attn(q))
