"""kivi_decode_attn_noalloc, the entry point that allocates nothing, against
kivi_decode_attn with a workspace: the same outputs (up to the rounding order
of the merges, far inside the 2e-3 + 1e-3 |ref| attention tolerance) on two
calls in a row, the second on a smaller cache, and the size check of its
scratch array."""
import numpy as np
import pytest
import torch

from decode_attention_pack_amd import kivi
from tests.gpu_util import dev, host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _cache(rng, B, H, rep, T, kb=2, vb=2, R=128):
    cap = -(-(T + 1) // 384) * 384
    c = kivi.Cache(B, H, 128, kb, vb, 32, R, cap)
    k = rng.standard_normal((B, H, T, 128)).astype(np.float16)
    k[:, :, :, :4] *= 15                      # outlier key channels
    v = rng.standard_normal((B, H, T, 128)).astype(np.float16)
    kivi.kivi_append(c, dev(k), dev(v))
    q = dev(rng.standard_normal((B, H * rep, 128)).astype(np.float16))
    return c, q


def test_noalloc_matches_workspace_call_twice():
    rng = np.random.default_rng(2024)
    # the second call has a smaller cache: fewer slabs, tokens and slots
    # (4-bit GQA and mixed widths on the matrix kernel, 4-bit MHA on the vector one)
    for B, H, rep, T, kb, vb in [(2, 4, 4, 5000, 2, 2), (2, 2, 4, 3000, 4, 4),
                                 (1, 2, 2, 2000, 2, 4), (1, 2, 2, 700, 2, 2),
                                 (2, 2, 1, 1500, 4, 4)]:
        c, q = _cache(rng, B, H, rep, T, kb, vb)
        ref = host(kivi.kivi_decode_attn(c, q))
        out = torch.full((B, H * rep, 128), float("nan"), dtype=torch.float32, device="cuda")
        kivi.kivi_decode_attn_noalloc(c, q, out)
        got = host(out)
        assert np.isfinite(got).all()
        np.testing.assert_allclose(got, ref, atol=1e-5, rtol=1e-5, err_msg=f"B={B} T={T}")


def test_noalloc_with_mask():
    rng = np.random.default_rng(7)
    c, q = _cache(rng, 2, 2, 4, 900)
    m = np.where(rng.random((2, c.n_tokens)) < 0.3, -np.inf, 0.0).astype(np.float32)
    ref = host(kivi.kivi_decode_attn(c, q, mask=dev(m)))
    out = torch.empty((2, 8, 128), dtype=torch.float32, device="cuda")
    got = host(kivi.kivi_decode_attn_noalloc(c, q, out, mask=dev(m)))
    np.testing.assert_allclose(got, ref, atol=1e-5, rtol=1e-5)


def test_noalloc_rejects_partials_past_the_scratch():
    """256 batch rows x 32 query heads x 7 partial slots (one workgroup and
    six window chunks per slab) pass 16 MiB: rejected on the host before any
    launch, the output left untouched."""
    c = kivi.Cache(256, 8, 128, 2, 2, 32, 128, 384)
    for a in c.arrays.values():
        a.zero_()
    c.c.n_tokens = 300
    q = torch.zeros((256, 32, 128), dtype=torch.float16, device="cuda")
    out = torch.full((256, 32, 128), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(kivi.KiviError) as e:
        kivi.kivi_decode_attn_noalloc(c, q, out)
    assert e.value.status == -3
    assert "scratch" in str(e.value)
    assert bool((out == 7.0).all())
