"""GPU parity of kivi_pack_keys / kivi_pack_values against the CPU oracle:
codes, scales and zeros must match bit for bit (KIVI items 1-3 of the page
"Literature audit -- Group 2", section 1, "Core algorithm")."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_pack_amd import kivi, synth
from tests.gpu_util import b16, cap_for, dev, host, logical, pool, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _gpu_pack(x16, bits, G, cap, off, keys):
    """Pack on the GPU into the records of a fresh destination cache; returns
    the logical (codes, scale, zero) of that destination."""
    B, H, T, D = x16.shape
    dst = kivi.Cache(B, H, D, bits, bits, G, G, cap)
    dst.blocks.zero_()
    fn = kivi.kivi_pack_keys if keys else kivi.kivi_pack_values
    fn(dst, dev(x16), off)
    torch.cuda.synchronize()
    lg = logical(dst)
    n = "k" if keys else "v"
    return lg[f"{n}_codes"], lg[f"{n}_scale"], lg[f"{n}_zero"]


def _same(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("G", [32, 64])
@pytest.mark.parametrize("D", [64, 128])
def test_pack_small(bits, G, D):
    rng = np.random.default_rng(bits * 100 + G + D)
    B, H = 2, 3
    T = 5 * G
    x = (rng.standard_normal((B, H, T, D)) * rng.uniform(0.01, 30, (1, 1, 1, D))).astype(np.float16)
    cap, off = cap_for(T + 2 * G, G), G
    for keys in (True, False):
        got = _gpu_pack(x, bits, G, cap, off, keys)
        fn = oracle.pack_keys if keys else oracle.pack_values
        ref = fn(b16(x), bits, G, cap=cap, offset=off)
        if keys:
            sls = [np.s_[:, :, off // G:(off + T) // G]] * 3
        else:
            sls = [np.s_[:, :, off:off + T], np.s_[..., off:off + T], np.s_[..., off:off + T]]
        for g_, r_, sl in zip(got, ref, sls):
            assert _same(g_[sl], r_[sl])


@pytest.mark.parametrize("bits,G,D", [(2, 16, 256), (4, 16, 64), (2, 16, 96), (4, 8, 64),
                                      (2, 128, 256), (4, 64, 256), (2, 32, 256), (4, 32, 256),
                                      (4, 16, 256)])
def test_pack_other_shapes(bits, G, D):
    """Shapes on both sides of the fast-path limits (power-of-two G <= 64, at
    most 16 KB per key tile, D in {64, 128, 256}); the rest take the general
    kernels."""
    test_pack_small(bits, G, D)


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_values_off_the_tile_grid(bits):
    """Values packed from a token that is not a multiple of 64 take the
    per-row kernel (the tile kernel needs its 64 tokens in one record); the
    result is the same bit for bit, across a record boundary."""
    rng = np.random.default_rng(9 + bits)
    x = rng.standard_normal((2, 3, 170, 128)).astype(np.float16)
    got = _gpu_pack(x, bits, 32, 256, 5, False)
    ref = oracle.pack_values(b16(x), bits, 32, cap=256, offset=5)
    assert _same(got[0][:, :, 5:175], ref[0][:, :, 5:175])
    assert _same(got[1][..., 5:175], ref[1][..., 5:175])
    assert _same(got[2][..., 5:175], ref[2][..., 5:175])


def test_pack_values_ragged_rows():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 2, 77, 128)).astype(np.float16)
    got = _gpu_pack(x, 2, 32, 128, 13, False)
    ref = oracle.pack_values(b16(x), 2, 32, cap=128, offset=13)
    assert _same(got[0][:, :, 13:90], ref[0][:, :, 13:90])
    assert _same(got[1][..., 13:90], ref[1][..., 13:90])
    assert _same(got[2][..., 13:90], ref[2][..., 13:90])


def _edge_tensor(rng, T, D):
    x = rng.standard_normal((1, 1, T, D)).astype(np.float32)
    x[0, 0, :, 0] = 1.25                                  # constant key groups
    x[0, 0, 3, :] = -0.0                                  # constant value row
    x[0, 0, :, 1] = np.tile([0.0, 3.0, 0.5, 1.5, 2.5, 1.0, 2.0, 0.25], T // 8)   # ties
    x[0, 0, :, 2] = rng.choice([-65504.0, 65504.0, 6e-8, -6e-8], T)  # extremes
    x[0, 0, 5, :] = np.linspace(-2, 2, D)
    x[0, 0, :, 3] = rng.standard_normal(T) * 1e-6        # subnormal-scale group
    # exact ties for 4-bit codes ((x - min) / s = k + 1/2 with s = 1): along
    # tokens for a key group, along channels for value groups
    x[0, 0, :, 4] = np.tile([0.0, 15.0, 0.5, 7.5, 14.5, 3.5, 1.0, 2.5], T // 8)
    x[0, 0, 7, :] = np.tile([0.0, 15.0, 0.5, 7.5, 14.5, 3.5, 1.0, 2.5], D // 8)
    x[0, 0, 9, :] = np.tile([0.0, 3.0, 0.5, 1.5, 2.5, 1.0, 2.0, 0.25], D // 8)
    # signed zeros at the group minimum, in both orders, and all-zero groups
    # of mixed sign: the stored zero point (and scale) keep the first zero
    x = x.astype(np.float16)
    pz, nz = np.float16(0.0), np.float16(-0.0)
    x[0, 0, :, 6] = np.tile(np.array([pz, nz, 1, 2], np.float16), T // 4)
    x[0, 0, 32:, 6] = np.tile(np.array([nz, pz, 1, 2], np.float16), (T - 32) // 4)
    x[0, 0, :, 7] = np.tile(np.array([nz, pz], np.float16), T // 2)
    x[0, 0, 11, :] = np.tile(np.array([pz, nz, 3, 1], np.float16), D // 4)
    x[0, 0, 12, :] = np.tile(np.array([nz, pz, 2, 1], np.float16), D // 4)
    x[0, 0, 13, :] = np.tile(np.array([pz, nz], np.float16), D // 2)
    return x


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_edge_values(bits):
    x = _edge_tensor(np.random.default_rng(1), 64, 128)
    for keys in (True, False):
        got = _gpu_pack(x, bits, 32, 128, 0, keys)
        ref = (oracle.pack_keys if keys else oracle.pack_values)(b16(x), bits, 32, cap=128)
        sls = [np.s_[:, :, :2]] * 3 if keys else [np.s_[:, :, :64], np.s_[..., :64], np.s_[..., :64]]
        for g_, r_, sl in zip(got, ref, sls):
            assert _same(g_[sl], r_[sl])
            if g_.dtype == np.float32:
                assert not np.isnan(g_[sl]).any()


@pytest.mark.parametrize("index", [4, 5])
def test_pack_full_prefill(index):
    """The full prefill of the 32k and 128k workloads on the GPU; the oracle
    packs every (batch, head) slab (in parallel) and checks every byte."""
    w = synth.WORKLOADS[index]
    inp = synth.make_inputs(w)
    cap = w.T0
    for keys in (True, False):
        x = inp["k0"] if keys else inp["v0"]
        say(f"pack {'keys' if keys else 'values'} {w.name} T={w.T0}, all {w.B * w.Hkv} slabs")
        got = _gpu_pack(x, w.k_bits, w.G, cap, 0, keys)
        fn = oracle.pack_keys if keys else oracle.pack_values

        def one(bh):
            b, h = bh
            ref = fn(b16(x[b:b + 1, h:h + 1]), w.k_bits, w.G, cap=cap)
            for g_, r_ in zip(got, ref):
                assert _same(g_[b:b + 1, h:h + 1], r_), (keys, b, h)

        list(pool().map(one, [(b, h) for b in range(w.B) for h in range(w.Hkv)]))


def test_pack_most_slabs():
    """65535 slabs (batch x heads), the most a pack call accepts: every slab
    is one workgroup row of the launch grid.  The oracle packs every slab (in
    chunks of batch rows, in parallel) and checks every byte (one slab more
    is rejected on the host, which the ABI tests check)."""
    rng = np.random.default_rng(65535)
    B, H, T, D, G, bits = 65535, 1, 32, 64, 32, 2
    x = rng.standard_normal((B, H, T, D)).astype(np.float16)
    say(f"pack {B} slabs of {T} tokens")
    for keys in (True, False):
        got = _gpu_pack(x, bits, G, 128, 0, keys)
        fn = oracle.pack_keys if keys else oracle.pack_values
        sls = [np.s_[:, :, :1]] * 3 if keys else [np.s_[:, :, :T], np.s_[..., :T], np.s_[..., :T]]

        def rows(b0, keys=keys, got=got, fn=fn, sls=sls):
            b1 = min(B, b0 + 4096)
            ref = fn(b16(x[b0:b1]), bits, G, cap=128)
            for g_, r_, sl in zip(got, ref, sls):
                assert _same(g_[b0:b1][sl], r_[sl]), (keys, b0)

        list(pool().map(rows, range(0, B, 4096)))
