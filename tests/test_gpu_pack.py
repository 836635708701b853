"""GPU parity of kivi_pack_keys / kivi_pack_values against the CPU oracle:
codes, scales and zeros must match bit for bit (KIVI items 1-3 of the page
"Literature audit -- Group 2", section 1, "Core algorithm")."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_pack_amd import kivi, synth
from tests.gpu_util import b16, dev, host, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _gpu_pack(x16, bits, G, cap, off, keys, codes_offset=0):
    """Pack on the GPU; codes_offset > 0 places the code array that many
    words into a larger buffer (a destination that is not 16-byte aligned)."""
    B, H, T, D = x16.shape
    shp = kivi.layout_shapes(B, H, D, bits, bits, G, 1, cap)
    n = "k" if keys else "v"
    n_codes = int(np.prod(shp[f"{n}_codes"]))
    buf = torch.zeros(n_codes + codes_offset, dtype=torch.int32, device="cuda")
    codes = buf[codes_offset:].view(shp[f"{n}_codes"])
    scale = torch.zeros(shp[f"{n}_scale"], dtype=torch.float32, device="cuda")
    zero = torch.zeros(shp[f"{n}_zero"], dtype=torch.float32, device="cuda")
    fn = kivi.kivi_pack_keys if keys else kivi.kivi_pack_values
    fn(dev(x16), bits, G, codes, scale, zero, cap, off)
    torch.cuda.synchronize()
    return host(codes).view(np.uint32), host(scale), host(zero)


def _same(a, b):
    return np.array_equal(np.ascontiguousarray(a).view(np.uint32),
                          np.ascontiguousarray(b).view(np.uint32))


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("G", [32, 64])
@pytest.mark.parametrize("D", [64, 128])
def test_pack_small(bits, G, D):
    rng = np.random.default_rng(bits * 100 + G + D)
    B, H = 2, 3
    T = 5 * G
    x = (rng.standard_normal((B, H, T, D)) * rng.uniform(0.01, 30, (1, 1, 1, D))).astype(np.float16)
    cap, off = T + 2 * G, G
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


@pytest.mark.parametrize("bits,G,D", [(2, 16, 256), (4, 16, 64), (2, 48, 96), (4, 8, 64),
                                      (2, 128, 256), (4, 64, 256), (2, 32, 256), (4, 32, 256),
                                      (4, 16, 256)])
def test_pack_other_shapes(bits, G, D):
    """Shapes on both sides of the fast-path limits (power-of-two G <= 64, at
    most 16 KB per key tile, D in {64, 128, 256}); the rest take the general
    kernels."""
    test_pack_small(bits, G, D)


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_values_unaligned_destination(bits):
    """A code array 4 bytes past a 16-byte boundary takes the per-row kernel;
    the result is the same bit for bit."""
    rng = np.random.default_rng(9 + bits)
    x = rng.standard_normal((2, 3, 70, 128)).astype(np.float16)
    got = _gpu_pack(x, bits, 32, 128, 5, False, codes_offset=1)
    ref = oracle.pack_values(b16(x), bits, 32, cap=128, offset=5)
    assert _same(got[0][:, :, 5:75], ref[0][:, :, 5:75])
    assert _same(got[1][..., 5:75], ref[1][..., 5:75])
    assert _same(got[2][..., 5:75], ref[2][..., 5:75])


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
        got = _gpu_pack(x, bits, 32, 64, 0, keys)
        ref = (oracle.pack_keys if keys else oracle.pack_values)(b16(x), bits, 32)
        for g_, r_ in zip(got, ref):
            assert _same(g_, r_)
            assert not np.isnan(g_.view(np.float32)).any() if g_.dtype == np.float32 else True


@pytest.mark.parametrize("index", [4, 5])
def test_pack_full_prefill(index):
    """The full prefill of the 32k and 128k workloads on the GPU; the oracle
    checks every byte of three sampled (batch, head) slabs."""
    w = synth.WORKLOADS[index]
    inp = synth.make_inputs(w)
    cap = w.T0
    for keys in (True, False):
        x = inp["k0"] if keys else inp["v0"]
        say(f"pack {'keys' if keys else 'values'} {w.name} T={w.T0}")
        got = _gpu_pack(x, w.k_bits, w.G, cap, 0, keys)
        for b, h in {(0, 0), (w.B - 1, w.Hkv - 1), (w.B // 2, w.Hkv // 2)}:
            fn = oracle.pack_keys if keys else oracle.pack_values
            ref = fn(b16(x[b:b + 1, h:h + 1]), w.k_bits, w.G, cap=cap)
            for g_, r_ in zip(got, ref):
                assert _same(g_[b:b + 1, h:h + 1], r_), (keys, b, h)


def test_pack_most_slabs():
    """65535 slabs (batch x heads), the most a pack call accepts: every slab
    is one workgroup row of the launch grid.  Three sampled slabs against the
    oracle, bit for bit (one slab more is rejected on the host, which the
    ABI tests check)."""
    rng = np.random.default_rng(65535)
    B, H, T, D, G, bits = 65535, 1, 32, 64, 32, 2
    x = rng.standard_normal((B, H, T, D)).astype(np.float16)
    say(f"pack {B} slabs of {T} tokens")
    for keys in (True, False):
        got = _gpu_pack(x, bits, G, T, 0, keys)
        fn = oracle.pack_keys if keys else oracle.pack_values
        for b in (0, B // 2 + 7, B - 1):
            ref = fn(b16(x[b:b + 1]), bits, G, cap=T, offset=0)
            for g_, r_ in zip(got, ref):
                assert _same(g_[b:b + 1], r_), (keys, b)
