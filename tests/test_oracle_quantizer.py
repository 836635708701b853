"""Pins for the oracle's quantizer and bit packing (CPU only).

Method: KIVI item 1 (asymmetric round-to-nearest group quantizer) and items
2-3 (packing along tokens for keys, along channels for values) of the page
"Literature audit -- Group 2", section 1 (KIVI), "Core algorithm".
"""
import json
import os

import numpy as np
import pytest

import oracle
from tests.textbook import pack_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden("quantizer_cases.json")["cases"], ids=lambda c: c["name"])
def test_hand_worked_cases(case):
    codes, s, z = oracle.quantize_group(np.array(case["x"], np.float32), case["bits"])
    assert codes.tolist() == case["codes"]
    assert s == np.float32(case["scale"]) and z == np.float32(case["zero"])
    deq = [oracle.dequant(c, s, z) for c in codes]
    assert deq == [np.float32(v) for v in case["dequant"]]
    assert not np.isnan(deq).any()


def _fp16_groups(rng, n_groups, G, scale=1.0):
    x = (rng.standard_normal((n_groups, G)) * scale).astype(np.float16)
    return x.astype(np.float32)


@pytest.mark.parametrize("bits", [2, 4])
def test_endpoints_round_trip(bits):
    """P1: the min element gets code 0 and dequantizes to exactly min; the max
    element gets code 2^B-1 and dequantizes to max within fp32 rounding."""
    rng = np.random.default_rng(11 + bits)
    qmax = (1 << bits) - 1
    for scale in (1e-3, 1.0, 20.0, 300.0):
        for x in _fp16_groups(rng, 200, 32, scale):
            codes, s, z = oracle.quantize_group(x, bits)
            i_min, i_max = int(np.argmin(x)), int(np.argmax(x))
            assert z == x[i_min]
            assert codes[i_min] == 0 and oracle.dequant(0, s, z) == x[i_min]
            assert codes[i_max] == qmax
            d = oracle.dequant(qmax, s, z)
            assert abs(float(d) - float(x[i_max])) <= 4 * np.spacing(np.float32(abs(x[i_max]) + abs(z)))
            # s is the fp32 quotient of the fp32 range
            assert s == np.float32(np.float32(x[i_max] - x[i_min]) / np.float32(qmax))


@pytest.mark.parametrize("bits", [2, 4])
def test_error_bound(bits):
    """P2: |deq - x| <= s/2 plus fp32 slack, for every element."""
    rng = np.random.default_rng(23 + bits)
    qmax = (1 << bits) - 1
    for scale in (1e-2, 1.0, 15.0):
        for x in _fp16_groups(rng, 300, 32, scale):
            codes, s, z = oracle.quantize_group(x, bits)
            assert codes.max() <= qmax
            deq = np.array([oracle.dequant(c, s, z) for c in codes], np.float64)
            slack = 2.0 ** -21 * (np.abs(x) + abs(z) + qmax * s)
            assert np.all(np.abs(deq - x) <= s / 2 + slack)


def test_error_bound_catches_wrong_rounding():
    """The bound is tight enough that truncation (floor) would violate it."""
    x = np.array([0.0, 0.9, 3.0, 1.0], np.float32)
    codes, s, z = oracle.quantize_group(x, 2)
    assert codes.tolist() == [0, 1, 3, 1]
    assert abs(float(np.floor(0.9)) * s + z - 0.9) > s / 2  # floor would fail P2


def test_constant_group():
    """P3: s = 0, every code 0, dequantized value equals x, no NaN."""
    for v in (0.0, -0.0, 1.5, -7.25, 65504.0, 6e-8):
        x = np.full(32, np.float16(v), np.float32)
        for bits in (2, 4):
            codes, s, z = oracle.quantize_group(x, bits)
            assert s == 0.0 and z == x[0] and not codes.any()
            assert oracle.dequant(0, s, z) == x[0]


def test_signed_zero_minimum_keeps_the_first_zero():
    """Reading of the group minimum for +0.0 / -0.0 ties (the pages leave it
    open): a scan in element order keeps the first of equal values, so the
    stored zero point -- and a constant group's scale -- carry the sign of
    the first zero.  Values are unaffected (+0.0 == -0.0)."""
    bits_of = lambda v: np.float32(v).view(np.uint32)
    for first, second in ((0.0, -0.0), (-0.0, 0.0)):
        x = np.array([first, second] + [1.0, 2.0] * 15, np.float32)
        codes, s, z = oracle.quantize_group(x, 2)
        assert bits_of(z) == bits_of(first) and z == 0.0
        assert codes[:2].tolist() == [0, 0]
        y = np.array([first, second] * 16, np.float32)      # all zeros, mixed signs
        codes, s, z = oracle.quantize_group(y, 4)
        assert bits_of(z) == bits_of(first) and s == 0.0 and not codes.any()


def test_tie_breaks_to_even_in_a_full_group():
    """P4: a 32-element group whose ratios hit k + 1/2 exactly."""
    x = np.array([0.0, 3.0] + [0.5, 1.5, 2.5] * 10, np.float32)
    codes, s, z = oracle.quantize_group(x, 2)
    assert s == 1.0 and z == 0.0
    assert codes[:2].tolist() == [0, 3]
    assert codes[2:].tolist() == [0, 2, 2] * 10


def test_smallest_fp16_range_is_normal_fp32():
    """The smallest nonzero fp16 difference gives a normal fp32 scale."""
    x = np.array([0.0, np.float16(2 ** -24)] + [0.0] * 30, np.float32)
    codes, s, z = oracle.quantize_group(x, 4)
    assert s > 0 and np.isfinite(s) and s >= np.finfo(np.float32).tiny
    assert codes[1] == 15


@pytest.mark.parametrize("entry", _golden("pack_layout.json")["words"], ids=lambda e: e["word"])
def test_hand_written_words(entry):
    words = oracle.pack_codes(np.array(entry["codes"], np.uint8), entry["bits"])
    assert words.tolist() == [int(entry["word"], 16)]
    assert oracle.unpack_codes(words, len(entry["codes"]), entry["bits"]).tolist() == entry["codes"]


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_round_trip(bits):
    """P5: unpack(pack(Q)) == Q, and the words match a textbook packer."""
    rng = np.random.default_rng(5)
    for n in (16, 32, 128, 40):
        codes = rng.integers(0, 1 << bits, n).astype(np.uint8)
        words = oracle.pack_codes(codes, bits)
        assert np.array_equal(words, pack_bits(codes, bits))
        assert np.array_equal(oracle.unpack_codes(words, n, bits), codes)


def test_half_to_float_exhaustive():
    """Every finite binary16 pattern widens to the value numpy assigns it."""
    pats = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float32)
    finite = np.isfinite(ref)
    got = np.array([oracle.half_to_float(int(p)) for p in pats[finite][::7]], np.float32)
    assert np.array_equal(got.view(np.uint32), ref[finite][::7].view(np.uint32))


def test_layout_case():
    """Key codes sit at [b][h][g][c][w] packed along tokens; value codes at
    [b][h][tau][w] packed along channels (hand-worked words)."""
    case = _golden("pack_layout.json")["layout_case"]
    tau = np.arange(32)[:, None]
    c = np.arange(32)[None, :]
    x = ((tau + c) % 4).astype(np.float16)[None, None]          # [1][1][32][32]
    kc, ks, kz = oracle.pack_keys(x.view(np.uint16), 2, 32)
    vc, vs, vz = oracle.pack_values(x.view(np.uint16), 2, 32)
    kwords = [int(w, 16) for w in case["key_words_by_channel_mod4"]]
    vwords = [int(w, 16) for w in case["value_words_by_token_mod4"]]
    assert kc.shape == (1, 1, 4, 32, 2) and vc.shape == (1, 1, 128, 2)
    for ch in range(32):
        assert kc[0, 0, 0, ch].tolist() == [kwords[ch % 4]] * 2
        assert ks[0, 0, 0, ch] == 1.0 and kz[0, 0, 0, ch] == 0.0
    assert not kc[0, 0, 1:].any() and not ks[0, 0, 1:].any()
    for t in range(32):
        assert vc[0, 0, t].tolist() == [vwords[t % 4]] * 2
        assert vs[0, 0, 0, t] == 1.0 and vz[0, 0, 0, t] == 0.0
    assert not vc[0, 0, 32:].any() and not vs[0, 0, 0, 32:].any()


def test_record_case():
    """The record layout: section offsets and raw record bytes worked out by
    hand (tests/golden/pack_layout.json, record_case)."""
    case = _golden("pack_layout.json")["record_case"]
    shp = case["shape"]
    D, G, cap = shp["D"], shp["G"], shp["capacity"]
    off = case["section_offsets"]
    assert oracle.record_bytes(D, shp["k_bits"], shp["v_bits"], G) == off["record_bytes"]
    assert [(n, o) for n, o, _ in oracle.record_sections(D, 2, 2, G)] == \
        [(n, off[n]) for n in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero")]
    tau = np.arange(32)[:, None]
    ch = np.arange(32)[None, :]
    x = (((tau + ch) % 4) - 1.5).astype(np.float16)[None, None]   # [1][1][32][32]
    c = oracle.Cache(1, 1, D, 2, 2, G, 32, cap)
    c.append(x.view(np.uint16), x.view(np.uint16))      # t = 32 = R: keys quantized, values not
    rec = c.blocks[0, 0, 0]
    for e in case["bytes"]:
        if "value" in e["what"]:
            continue
        got = bytes(rec[e["offset"]:e["offset"] + len(e["hex"]) // 2]).hex()
        assert got == e["hex"], e["what"]
    d = oracle.Cache(1, 1, D, 2, 2, G, 32, cap)
    d.append(np.concatenate([x, x], axis=2).view(np.uint16),
             np.concatenate([x, x], axis=2).view(np.uint16))  # t = 64: values 0..31 popped
    rec = d.blocks[0, 0, 0]
    for e in case["bytes"]:
        if "value" not in e["what"]:
            continue
        got = bytes(rec[e["offset"]:e["offset"] + len(e["hex"]) // 2]).hex()
        assert got == e["hex"], e["what"]


def test_float_to_half_round_trips_every_finite_pattern():
    """Zero points are stored as fp16: the oracle's exact float -> fp16
    conversion inverts the fp16 widening for every finite pattern, and
    refuses a value with no fp16 form."""
    pats = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = pats.view(np.float16)
    for p, v in zip(pats[::97], vals[::97]):
        if np.isfinite(v):
            assert oracle.float_to_half(np.float32(v)) == int(p)
    assert oracle.float_to_half(np.float32(-0.0)) == 0x8000
    assert oracle.float_to_half(np.float32(2 ** -24)) == 0x0001
    with pytest.raises(ValueError):
        oracle.float_to_half(np.float32(1.0 + 2 ** -20))


def test_pack_keys_groups_along_tokens():
    """Each key group is the quantizer applied to G consecutive tokens of one
    channel; each value group to G consecutive channels of one token."""
    rng = np.random.default_rng(3)
    B, H, T, D, G = 2, 3, 64, 64, 32
    x = rng.standard_normal((B, H, T, D)).astype(np.float16)
    for bits in (2, 4):
        kc, ks, kz = oracle.pack_keys(x.view(np.uint16), bits, G)
        vc, vs, vz = oracle.pack_values(x.view(np.uint16), bits, G)
        for b, h, g, ch in [(0, 0, 0, 0), (1, 2, 1, 63), (0, 1, 1, 17)]:
            codes, s, z = oracle.quantize_group(x[b, h, g * G:(g + 1) * G, ch].astype(np.float32), bits)
            assert np.array_equal(kc[b, h, g, ch], pack_bits(codes, bits))
            assert ks[b, h, g, ch] == s and kz[b, h, g, ch] == z
        for b, h, t, g in [(0, 0, 0, 0), (1, 2, 63, 1), (1, 0, 40, 0)]:
            codes, s, z = oracle.quantize_group(x[b, h, t, g * G:(g + 1) * G].astype(np.float32), bits)
            per = 32 // bits
            assert np.array_equal(vc[b, h, t, g * G // per:(g + 1) * G // per], pack_bits(codes, bits))
            assert vs[b, h, g, t] == s and vz[b, h, g, t] == z
