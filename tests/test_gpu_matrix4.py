"""GPU parity of the 4-bit matrix-core path of kivi_decode_attn: 4-bit keys
and values (KIVI item 1 with B = 4, the KIVI-4 setting of the page
"Literature audit -- Group 2", section 1), and 2-bit keys with 4-bit values
or the reverse (item 6 puts the widths on the hyperparameter axis),
attention as item 5.  The matrix
kernel's block role takes the whole 128-token blocks and its window role the
tokens past them; outputs within 2e-3 + 1e-3*|ref| of the CPU oracle
elementwise, on shapes that span several blocks, workgroups and a ragged
tail."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_pack_amd import kivi
from tests.gpu_util import assert_close, b16, cap_for, dev, host, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

M = kivi.KIVI_PATH_MATRIX


WIDTHS = [(4, 4), (2, 4), (4, 2)]


def _case(seed, B, H, rep, t, R=128, scale_fp16=False, kscale=15.0, extra=0, kb=4, vb=4):
    """Gaussian keys with per-channel magnitudes up to `kscale` (outlier
    channels), Gaussian values and queries; the same cache on the GPU and in
    the oracle."""
    rng = np.random.default_rng(seed)
    D = 128
    K = (rng.standard_normal((B, H, t, D)) * rng.uniform(0.5, kscale, (1, H, 1, D))).astype(np.float16)
    V = rng.standard_normal((B, H, t, D)).astype(np.float16)
    q = rng.standard_normal((B, H * rep, D)).astype(np.float16)
    cap = cap_for(t + extra, R)
    g = kivi.Cache(B, H, D, kb, vb, 32, R, cap, scale_fp16=scale_fp16)
    o = oracle.Cache(B, H, D, kb, vb, 32, R, cap, scale_fp16=scale_fp16)
    if t:
        kivi.kivi_append(g, dev(K), dev(V))
        o.append(b16(K), b16(V))
    return g, o, q, rng


@pytest.mark.parametrize("t", [1, 31, 32, 33, 100, 128, 129, 255, 256, 257, 300, 383, 384, 385,
                               511, 512, 513, 1000, 2049, 4097])
@pytest.mark.parametrize("rep", [1, 2, 4])
def test_lengths(t, rep):
    """Rows with no whole block (the window role alone), then tails of
    0..R + 127 tokens past the blocks (quantized keys, quantized and fp16
    values)."""
    g, o, q, _ = _case(t * 10 + rep, 2, 2, rep, t)
    ref = o.decode_attn(b16(q))
    for p in (M, kivi.KIVI_PATH_AUTO):
        assert_close(host(kivi.kivi_decode_attn(g, dev(q), path=p)), ref, f"t={t} rep={rep} path={p}")


@pytest.mark.parametrize("R", [32, 96])
@pytest.mark.parametrize("t", [160, 161, 223, 224, 255, 256, 257, 1000, 1377])
@pytest.mark.parametrize("rep", [1, 4])
def test_windows_of_the_ablation(R, t, rep):
    """Window lengths the pages' ablation uses besides 128: the quantized-key
    and quantized-value limits fall inside a 128-token block."""
    g, o, q, _ = _case(t * 3 + R + rep, 2, 2, rep, t, R=R)
    ref = o.decode_attn(b16(q))
    assert_close(host(kivi.kivi_decode_attn(g, dev(q), path=M)), ref, f"R={R} t={t} rep={rep}")


@pytest.mark.parametrize("rep", [4, 2, 1])
def test_mask(rep):
    g, o, q, rng = _case(80 + rep, 2, 2, rep, 1500)
    t = g.n_tokens
    m = np.where(rng.random((2, t)) < 0.3, -np.inf, rng.standard_normal((2, t))).astype(np.float32)
    m[1, :] = -np.inf                      # a fully masked batch row
    ref = o.decode_attn(b16(q), m)
    out = host(kivi.kivi_decode_attn(g, dev(q), mask=dev(m), path=M))
    assert not np.isnan(out).any() and not out[1].any()
    assert_close(out, ref, f"mask rep={rep}")


@pytest.mark.parametrize("rep", [4, 1])
@pytest.mark.parametrize("t", [700, 2049])
def test_fp16_scales(rep, t):
    """The fp16-scale layout (scales stored as binary16) at 4 bits."""
    g, o, q, _ = _case(t + rep, 2, 2, rep, t, scale_fp16=True)
    assert_close(host(kivi.kivi_decode_attn(g, dev(q), path=M)), o.decode_attn(b16(q)),
                 f"fp16 scales t={t} rep={rep}")


@pytest.mark.parametrize("rep", [4, 2])
def test_workgroup_splits(rep):
    """One to many workgroups per slab: every split matches the oracle, and
    the splits agree with each other to within the matrix cores' rounding."""
    g, o, q, _ = _case(40 + rep, 1, 2, rep, 5000)
    ref = o.decode_attn(b16(q))
    base = host(kivi.kivi_decode_attn(g, dev(q), path=M))
    assert_close(base, ref, "default split")
    for tps in (128, 384, 1024, 4096, 8192):
        out = host(kivi.kivi_decode_attn(g, dev(q), tokens_per_split=tps, path=M))
        assert_close(out, ref, f"tps={tps}")
        np.testing.assert_allclose(out, base, atol=2e-4, rtol=1e-3)


@pytest.mark.parametrize("kscale,vscale", [(1e-3, 1.0), (200.0, 1.0), (1.0, 1e-3), (1.0, 300.0)])
def test_value_ranges(kscale, vscale):
    """Magnitudes far from N(0, 1): the per-workgroup rescaling of the key
    operand and the unscaled value operand stay within the tolerance."""
    rng = np.random.default_rng(int(kscale * 7 + vscale * 3))
    B, H, rep, D, t = 1, 2, 4, 128, 3000
    K = (rng.standard_normal((B, H, t, D)) * kscale).astype(np.float16)
    V = (rng.standard_normal((B, H, t, D)) * vscale).astype(np.float16)
    q = rng.standard_normal((B, H * rep, D)).astype(np.float16)
    g = kivi.Cache(B, H, D, 4, 4, 32, 128, 3072)
    o = oracle.Cache(B, H, D, 4, 4, 32, 128, 3072)
    kivi.kivi_append(g, dev(K), dev(V))
    o.append(b16(K), b16(V))
    assert_close(host(kivi.kivi_decode_attn(g, dev(q), path=M)), o.decode_attn(b16(q)),
                 f"kscale={kscale} vscale={vscale}", value_scale=max(1.0, vscale))


def test_decode_steps_across_a_block():
    """Fused decode steps (kivi_decode_step: the append inside the 4-bit
    matrix launch) across the point where a value block completes."""
    g, o, q, rng = _case(77, 1, 2, 4, 380, extra=8)
    for step in range(6):
        k = rng.standard_normal((1, 2, 1, 128)).astype(np.float16)
        v = rng.standard_normal((1, 2, 1, 128)).astype(np.float16)
        qs = rng.standard_normal((1, 8, 128)).astype(np.float16)
        out = host(kivi.kivi_decode_step(g, dev(k), dev(v), dev(qs)))
        o.append(b16(k), b16(v))
        say(f"step {step}: t={g.n_tokens}")
        assert_close(out, o.decode_attn(b16(qs)), f"step {step}")


@pytest.mark.parametrize("kb,vb", WIDTHS[1:])
@pytest.mark.parametrize("t", [33, 255, 256, 385, 1000, 2049])
@pytest.mark.parametrize("rep", [1, 2, 4])
def test_mixed_widths(kb, vb, t, rep):
    """2-bit keys with 4-bit values and the reverse: each half of the block
    role and of the window role takes its own width."""
    g, o, q, _ = _case(t * 10 + rep + kb, 2, 2, rep, t, kb=kb, vb=vb)
    ref = o.decode_attn(b16(q))
    for p in (M, kivi.KIVI_PATH_AUTO):
        assert_close(host(kivi.kivi_decode_attn(g, dev(q), path=p)), ref,
                     f"kb={kb} vb={vb} t={t} rep={rep} path={p}")


@pytest.mark.parametrize("kb,vb", WIDTHS[1:])
def test_mixed_widths_masked_fp16_scales_and_splits(kb, vb):
    g, o, q, rng = _case(90 + kb, 2, 2, 4, 3000, kb=kb, vb=vb)
    t = g.n_tokens
    m = np.where(rng.random((2, t)) < 0.3, -np.inf, rng.standard_normal((2, t))).astype(np.float32)
    assert_close(host(kivi.kivi_decode_attn(g, dev(q), mask=dev(m), path=M)),
                 o.decode_attn(b16(q), m), f"mask kb={kb} vb={vb}")
    ref = o.decode_attn(b16(q))
    for tps in (256, 1024):
        assert_close(host(kivi.kivi_decode_attn(g, dev(q), tokens_per_split=tps, path=M)), ref,
                     f"tps={tps} kb={kb} vb={vb}")
    g, o, q, _ = _case(95 + kb, 2, 2, 2, 1500, kb=kb, vb=vb, scale_fp16=True)
    assert_close(host(kivi.kivi_decode_attn(g, dev(q), path=M)), o.decode_attn(b16(q)),
                 f"fp16 scales kb={kb} vb={vb}")
