"""GPU parity of kivi_decode_attn against the CPU oracle (KIVI item 5 of the
page "Literature audit -- Group 2", section 1, "Core algorithm"): outputs
within 2e-3 + 1e-3*|ref| elementwise; packed stores bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_pack_amd import kivi, synth
from tests.gpu_util import (assert_close, b16, cap_for, check_every_slab, compare_rows, dev,
                            gpu_cache, host, host_windows, logical, oracle_all_slabs, pool, say)
from tests.textbook import dense_attention

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

PATHS = [kivi.KIVI_PATH_AUTO, kivi.KIVI_PATH_GENERIC]


def vector_ok(D, kb, vb, G, R, rep, cap):
    """Shapes the vector kernel takes (the ABI rejects it elsewhere)."""
    return (D == 128 and G == 32 and kb in (2, 4) and vb in (2, 4)
            and (rep == 1 or (rep % 2 == 0 and rep <= 64)) and R % 32 == 0 and cap % 32 == 0)


def paths_for(D, kb, vb, G, R, rep, cap):
    return PATHS + ([kivi.KIVI_PATH_VECTOR] if vector_ok(D, kb, vb, G, R, rep, cap) else [])


def _run_workload(w, paths=None):
    """Prefill + one decode step of workload w on the GPU, in the launch
    configuration the benchmark times; the oracle rebuilds every (batch, kv
    head) slab alone and checks its packed store, windows and attention."""
    inp = synth.make_inputs(w)
    g = gpu_cache(w)
    say(f"{w.name}: prefill {w.T0} + 1 step")
    kivi.kivi_append(g, dev(inp["k0"]), dev(inp["v0"]))
    kivi.kivi_append(g, dev(inp["k_steps"][0]), dev(inp["v_steps"][0]))
    q = inp["q_steps"][0]
    rep = w.Hq // w.Hkv
    if paths is None:
        paths = paths_for(w.D, w.k_bits, w.v_bits, w.G, w.R, rep, w.capacity)
    outs = {f"path {p}": host(kivi.kivi_decode_attn(g, dev(q), path=p)) for p in paths}
    say(f"{w.name}: oracle over {w.B * w.Hkv} slabs")
    orc = oracle_all_slabs(w, inp, n_steps=1)
    check_every_slab(w, g, orc, outs, q)
    return g, outs


def test_tiny():
    _run_workload(synth.WORKLOADS[1])


def test_kivi4_b64():
    _run_workload(synth.WORKLOADS[3])


def test_llama3_gqa_32k():
    _run_workload(synth.WORKLOADS[4])


def test_llama3_gqa_32k_4bit():
    """The 32k GQA shape (4 query heads per KV head) with 4-bit keys and
    values: the vector kernel in workgroups of two query heads."""
    _run_workload(synth.WORKLOADS[4].replace(name="llama3-8b-gqa-32k-kivi4", k_bits=4, v_bits=4))


def test_long_128k():
    _run_workload(synth.WORKLOADS[5])


def _small_case(rng, B, H, rep, D, kb, vb, G, R, t):
    K = (rng.standard_normal((B, H, t, D)) * rng.uniform(0.5, 15, (1, H, 1, D))).astype(np.float16)
    V = rng.standard_normal((B, H, t, D)).astype(np.float16)
    q = rng.standard_normal((B, H * rep, D)).astype(np.float16)
    cap = cap_for(t, R)
    g = kivi.Cache(B, H, D, kb, vb, G, R, cap)
    o = oracle.Cache(B, H, D, kb, vb, G, R, cap)
    if t:
        kivi.kivi_append(g, dev(K), dev(V))
        o.append(b16(K), b16(V))
    return g, o, q


@pytest.mark.parametrize("t", [0, 1, 31, 32, 33, 64, 95, 96, 97, 127, 128, 129, 200, 255, 256,
                               257, 511, 640, 1000])
@pytest.mark.parametrize("rep", [1, 4])
def test_lengths_around_boundaries(t, rep):
    rng = np.random.default_rng(t * 10 + rep)
    g, o, q = _small_case(rng, 2, 2, rep, 128, 2, 2, 32, 64, t)
    ref = o.decode_attn(b16(q))
    for p in paths_for(128, 2, 2, 32, 64, rep, g.cap):
        out = host(kivi.kivi_decode_attn(g, dev(q), path=p))
        assert_close(out, ref, f"t={t} rep={rep} path={p}")


@pytest.mark.parametrize("R", [32, 96])
@pytest.mark.parametrize("t", [31, 95, 96, 97, 191, 192, 255, 256, 383, 384, 385, 1000, 2977])
@pytest.mark.parametrize("rep", [1, 4])
def test_window_lengths_of_the_ablation(R, t, rep):
    """Window lengths the pages' ablation uses besides 128: R = 96 is not a
    multiple of the matrix kernel's 128-token block, so the quantized-key and
    quantized-value limits fall inside a block."""
    rng = np.random.default_rng(t * 3 + R + rep)
    g, o, q = _small_case(rng, 2, 2, rep, 128, 2, 2, 32, R, t)
    ref = o.decode_attn(b16(q))
    for p in paths_for(128, 2, 2, 32, R, rep, g.cap):
        assert_close(host(kivi.kivi_decode_attn(g, dev(q), path=p)), ref, f"R={R} t={t} rep={rep} path={p}")
    assert_close(host(kivi.kivi_decode_attn(g, dev(q), path=kivi.KIVI_PATH_MATRIX)), ref,
                 f"R={R} t={t} rep={rep} matrix")


@pytest.mark.parametrize("rep", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("kb,vb", [(2, 2), (4, 4), (2, 4), (4, 2)])
def test_head_groups_and_bits(rep, kb, vb):
    rng = np.random.default_rng(rep * 7 + kb + 3 * vb)
    g, o, q = _small_case(rng, 2, 2, rep, 128, kb, vb, 32, 128, 777)
    ref = o.decode_attn(b16(q))
    for p in paths_for(128, kb, vb, 32, 128, rep, g.cap):
        assert_close(host(kivi.kivi_decode_attn(g, dev(q), path=p)), ref, f"rep={rep} kb={kb} vb={vb}")


@pytest.mark.parametrize("D,G", [(64, 32), (256, 32), (128, 64), (128, 128)])
def test_head_dims_and_groups(D, G):
    rng = np.random.default_rng(D + G)
    g, o, q = _small_case(rng, 1, 2, 2, D, 2, 2, G, 128, 600)
    ref = o.decode_attn(b16(q))
    assert_close(host(kivi.kivi_decode_attn(g, dev(q))), ref, f"D={D} G={G}")


@pytest.mark.parametrize("rep,kb,vb", [(4, 2, 2), (2, 4, 4), (1, 4, 2)])
def test_mask(rep, kb, vb):
    rng = np.random.default_rng(8 + rep)
    g, o, q = _small_case(rng, 2, 2, rep, 128, kb, vb, 32, 128, 900)
    t = g.n_tokens
    m = np.where(rng.random((2, t)) < 0.3, -np.inf, rng.standard_normal((2, t))).astype(np.float32)
    m[1, :] = -np.inf                      # a fully masked batch row
    ref = o.decode_attn(b16(q), m)
    for p in paths_for(128, kb, vb, 32, 128, rep, g.cap):
        out = host(kivi.kivi_decode_attn(g, dev(q), mask=dev(m), path=p))
        assert not np.isnan(out).any() and not out[1].any()
        assert_close(out, ref, f"mask path={p}")
    zero = host(kivi.kivi_decode_attn(g, dev(q), mask=dev(np.zeros((2, t), np.float32))))
    # an all-zero mask changes nothing but the rounding order of the merges
    np.testing.assert_allclose(zero, host(kivi.kivi_decode_attn(g, dev(q))), atol=1e-5, rtol=1e-5)


# The matrix cores sum the fp16 products of one MFMA after aligning them to the
# largest, keeping about 16 bits below it (measured on gfx950), so a different
# split of the tokens changes the rounding of the matrix kernel at ~1e-4.
SPLIT_TOL = {kivi.KIVI_PATH_GENERIC: dict(atol=2e-5, rtol=1e-5),
             kivi.KIVI_PATH_VECTOR: dict(atol=2e-5, rtol=1e-5),
             kivi.KIVI_PATH_AUTO: dict(atol=2e-4, rtol=1e-3)}


@pytest.mark.parametrize("rep,kb,vb", [(4, 2, 2), (1, 4, 4), (2, 2, 4)])
def test_split_invariance(rep, kb, vb):
    """Different split counts agree to within rounding (P12)."""
    rng = np.random.default_rng(12 + rep)
    g, o, q = _small_case(rng, 1, 2, rep, 128, kb, vb, 32, 128, 5000)
    for p in paths_for(128, kb, vb, 32, 128, rep, g.cap):
        base = host(kivi.kivi_decode_attn(g, dev(q), path=p))
        for tps in (64, 256, 1024, 4096):
            out = host(kivi.kivi_decode_attn(g, dev(q), tokens_per_split=tps, path=p))
            np.testing.assert_allclose(out, base, **SPLIT_TOL[p])


def test_gqa_equals_repeated_kv_mha():
    rng = np.random.default_rng(13)
    B, H, rep, D, t = 1, 2, 4, 128, 1500
    K = rng.standard_normal((B, H, t, D)).astype(np.float16)
    V = rng.standard_normal((B, H, t, D)).astype(np.float16)
    q = dev(rng.standard_normal((B, H * rep, D)).astype(np.float16))
    g = kivi.Cache(B, H, D, 2, 2, 32, 128, 1536)
    kivi.kivi_append(g, dev(K), dev(V))
    m = kivi.Cache(B, H * rep, D, 2, 2, 32, 128, 1536)
    kivi.kivi_append(m, dev(np.repeat(K, rep, axis=1)), dev(np.repeat(V, rep, axis=1)))
    np.testing.assert_allclose(host(kivi.kivi_decode_attn(g, q)), host(kivi.kivi_decode_attn(m, q)),
                               atol=1e-5, rtol=1e-5)


def test_grid_exact_inputs_match_dense_attention():
    """Keys/values that quantize losslessly: GPU attention over the packed
    cache equals dense attention over the original fp16 tensors."""
    rng = np.random.default_rng(21)
    B, H, rep, D, G, R, t = 1, 2, 2, 128, 32, 128, 640
    n_kq = t - t % R
    s = 2.0 ** rng.integers(-3, 1, (B, H, n_kq // G, 1, D))
    z = s * rng.integers(-20, 20, (B, H, n_kq // G, 1, D))
    k = rng.integers(0, 4, (B, H, n_kq // G, G, D))
    k[:, :, :, 0, :], k[:, :, :, 1, :] = 0, 3
    K = (z + k * s).reshape(B, H, n_kq, D).astype(np.float16)
    sv = 2.0 ** rng.integers(-3, 1, (B, H, t, D // G, 1))
    zv = sv * rng.integers(-20, 20, (B, H, t, D // G, 1))
    kv = rng.integers(0, 4, (B, H, t, D // G, G))
    kv[..., 0], kv[..., 1] = 0, 3
    V = (zv + kv * sv).reshape(B, H, t, D).astype(np.float16)
    q = rng.standard_normal((B, H * rep, D)).astype(np.float16)
    g = kivi.Cache(B, H, D, 2, 2, G, R, t + R)
    kivi.kivi_append(g, dev(K), dev(V[:, :, :n_kq]))
    ref = dense_attention(q.astype(np.float32), K.astype(np.float32), V[:, :, :n_kq].astype(np.float32))
    for p in paths_for(D, 2, 2, G, R, rep, t + R):
        assert_close(host(kivi.kivi_decode_attn(g, dev(q), path=p)), ref, f"grid path={p}")


@pytest.mark.parametrize("kscale,vscale", [(1e-3, 1.0), (40.0, 1.0), (1.0, 1e-3), (1.0, 300.0),
                                           (200.0, 50.0)])
@pytest.mark.parametrize("rep", [4, 2])
def test_value_ranges(kscale, vscale, rep):
    """Key/value magnitudes far from N(0, 1): every kernel stays within the
    tolerance (the matrix kernel rescales its fp16 operands per block)."""
    rng = np.random.default_rng(int(kscale * 7 + vscale * 3) + rep)
    B, H, D, t = 1, 2, 128, 3000
    K = (rng.standard_normal((B, H, t, D)) * kscale).astype(np.float16)
    V = (rng.standard_normal((B, H, t, D)) * vscale).astype(np.float16)
    q = rng.standard_normal((B, H * rep, D)).astype(np.float16)
    g = kivi.Cache(B, H, D, 2, 2, 32, 128, 3072)
    o = oracle.Cache(B, H, D, 2, 2, 32, 128, 3072)
    kivi.kivi_append(g, dev(K), dev(V))
    o.append(b16(K), b16(V))
    ref = o.decode_attn(b16(q))
    for p in paths_for(D, 2, 2, 32, 128, rep, 3072):
        out = host(kivi.kivi_decode_attn(g, dev(q), path=p))
        assert_close(out, ref, f"kscale={kscale} vscale={vscale} path={p}",
                     value_scale=max(1.0, vscale))


def test_matrix_and_scalar_paths_agree_closely():
    """Where the matrix kernel runs, it matches the scalar kernel to ~1e-5."""
    rng = np.random.default_rng(31)
    for rep in (1, 2, 4):
        g, o, q = _small_case(rng, 2, 3, rep, 128, 2, 2, 32, 128, 4000)
        a = host(kivi.kivi_decode_attn(g, dev(q), path=kivi.KIVI_PATH_MATRIX))
        s = host(kivi.kivi_decode_attn(g, dev(q), path=kivi.KIVI_PATH_GENERIC))
        np.testing.assert_allclose(a, s, atol=5e-4, rtol=1e-3)


@pytest.mark.parametrize("kb,vb", [(2, 2), (4, 4), (2, 4), (4, 2)])
def test_vector_and_scalar_paths_agree_closely(kb, vb):
    """The vector kernel (fp32 throughout; scores as sum (q s) code + q z, a
    different rounding order) stays within 2e-4 of the scalar kernel, ten
    times inside the oracle tolerance, over many splits and a ragged window."""
    rng = np.random.default_rng(41 + kb + 3 * vb)
    for rep, t in ((1, 4001), (2, 2500), (4, 1800)):
        g, o, q = _small_case(rng, 2, 3, rep, 128, kb, vb, 32, 128, t)
        for tps in (0, 64, 192, 8192):   # 8192: one split, output written directly
            v = host(kivi.kivi_decode_attn(g, dev(q), tokens_per_split=tps,
                                           path=kivi.KIVI_PATH_VECTOR))
            s = host(kivi.kivi_decode_attn(g, dev(q), tokens_per_split=tps,
                                           path=kivi.KIVI_PATH_GENERIC))
            np.testing.assert_allclose(v, s, atol=2e-4, rtol=1e-3, err_msg=f"rep={rep} tps={tps}")


def test_vector_path_rejects_other_shapes():
    rng = np.random.default_rng(5)
    g, _, q = _small_case(rng, 1, 2, 3, 128, 2, 2, 32, 128, 300)   # an odd head count above 1
    with pytest.raises(kivi.KiviError):
        kivi.kivi_decode_attn(g, dev(q), path=kivi.KIVI_PATH_VECTOR)


def test_most_slabs_append_and_decode():
    """65535 slabs (batch x KV heads), the most a cache may hold: prefill,
    one appended token, and attention through every path the shape allows.
    The oracle rebuilds every slab (in chunks of batch rows, in parallel) and
    checks the packed stores bit for bit and every output."""
    rng = np.random.default_rng(4242)
    B, H, D, G, R, t0 = 65535, 1, 128, 32, 32, 40
    cap = 128
    K = rng.standard_normal((B, H, t0 + 1, D), dtype=np.float32).astype(np.float16)
    V = rng.standard_normal((B, H, t0 + 1, D), dtype=np.float32).astype(np.float16)
    q = rng.standard_normal((B, H, D), dtype=np.float32).astype(np.float16)
    say(f"{B} slabs: prefill {t0} + 1 token")
    g = kivi.Cache(B, H, D, 2, 2, G, R, cap)
    kivi.kivi_append(g, dev(K[:, :, :t0]), dev(V[:, :, :t0]))
    kivi.kivi_append(g, dev(K[:, :, t0:]), dev(V[:, :, t0:]))
    outs = {p: host(kivi.kivi_decode_attn(g, dev(q), path=p))
            for p in paths_for(D, 2, 2, G, R, 1, cap) + [kivi.KIVI_PATH_MATRIX]}
    gl, gres = logical(g), host_windows(g)
    chunk = 4096

    def rows(b0):
        b1 = min(B, b0 + chunk)
        o = oracle.Cache(b1 - b0, H, D, 2, 2, G, R, cap)
        o.append(b16(K[b0:b1, :, :t0]), b16(V[b0:b1, :, :t0]))
        o.append(b16(K[b0:b1, :, t0:]), b16(V[b0:b1, :, t0:]))
        compare_rows(g, b0, o, gl, gres)
        return b0, o.decode_attn(b16(q[b0:b1]))

    ref = np.zeros((B, H, D), np.float32)
    for b0, r in pool().map(rows, range(0, B, chunk)):
        ref[b0:b0 + r.shape[0]] = r
    for p, out in outs.items():
        assert_close(out, ref, f"all {B} slabs, path {p}")


def test_llama3_gqa_32k_masked():
    """The full 32k GQA workload with an additive mask (a fifth of the tokens
    at -inf, the rest N(0, 1)): the masked instantiation of the matrix kernel,
    whose workgroups stage each block's mask row by DMA, against the oracle on
    every slab."""
    w = synth.WORKLOADS[4]
    inp = synth.make_inputs(w)
    g = gpu_cache(w)
    say(f"{w.name}: prefill {w.T0} + 1 step, masked")
    kivi.kivi_append(g, dev(inp["k0"]), dev(inp["v0"]))
    kivi.kivi_append(g, dev(inp["k_steps"][0]), dev(inp["v_steps"][0]))
    t = g.n_tokens
    rng = np.random.default_rng(77)
    mask = np.where(rng.random((w.B, t)) < 0.2, -np.inf,
                    rng.standard_normal((w.B, t))).astype(np.float32)
    q = inp["q_steps"][0]
    out = host(kivi.kivi_decode_attn(g, dev(q), mask=dev(mask)))
    orc = oracle_all_slabs(w, inp, n_steps=1)
    check_every_slab(w, g, orc, {"masked": out}, q, mask=mask, stores=False)
