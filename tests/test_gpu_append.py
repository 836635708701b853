"""GPU parity of kivi_append against the CPU oracle: the quantized stores and
the fp16 window must match bit for bit after every call (KIVI item 4 of the
page "Literature audit -- Group 2", section 1, "Core algorithm")."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_pack_amd import kivi, synth
from tests.gpu_util import assert_close, b16, compare_slab, dev, host, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("kb,vb,R,D", [(2, 2, 32, 128), (4, 4, 64, 128), (2, 4, 32, 64),
                                       (4, 2, 128, 128)])
def test_append_random_chunks(kb, vb, R, D):
    rng = np.random.default_rng(kb * 1000 + vb * 100 + R)
    B, H, G = 2, 3, 32
    t_end = 3 * R + 5
    cap = ((t_end + R - 1) // R) * R
    K = rng.standard_normal((B, H, t_end, D)).astype(np.float16)
    V = rng.standard_normal((B, H, t_end, D)).astype(np.float16)
    g = kivi.Cache(B, H, D, kb, vb, G, R, cap)
    o = oracle.Cache(B, H, D, kb, vb, G, R, cap)
    t = 0
    while t < t_end:
        n = int(min(t_end - t, rng.choice([1, 1, 2, 7, R - 1, R, R + 3])))
        kivi.kivi_append(g, dev(K[:, :, t:t + n]), dev(V[:, :, t:t + n]))
        o.append(b16(K[:, :, t:t + n]), b16(V[:, :, t:t + n]))
        t += n
        torch.cuda.synchronize()
        assert g.n_tokens == t
        for b in range(B):
            for h in range(H):
                compare_slab(g, b, h, o, b, h)


@pytest.mark.parametrize("kb,vb,G,D,R", [(2, 2, 16, 64, 32), (4, 4, 64, 128, 64), (2, 4, 32, 96, 64),
                                         (4, 2, 48, 96, 48), (2, 2, 128, 256, 128)])
def test_single_token_appends(kb, vb, G, D, R):
    """Decode-step appends (one token per call) through both the fused
    single-token kernel (G a power of two <= 64) and the general path (other
    G), across the key-block and window-wrap boundaries."""
    rng = np.random.default_rng(G * 7 + D + kb)
    B, H = 2, 2
    t_end = 2 * R + 3
    cap = ((t_end + R - 1) // R) * R
    K = rng.standard_normal((B, H, t_end, D)).astype(np.float16)
    V = (rng.standard_normal((B, H, t_end, D)) * 3).astype(np.float16)
    g = kivi.Cache(B, H, D, kb, vb, G, R, cap)
    o = oracle.Cache(B, H, D, kb, vb, G, R, cap)
    for t in range(t_end):
        kivi.kivi_append(g, dev(K[:, :, t:t + 1]), dev(V[:, :, t:t + 1]))
        o.append(b16(K[:, :, t:t + 1]), b16(V[:, :, t:t + 1]))
        if t % 5 == 4 or t >= t_end - 3 or (t + 1) % R <= 1:
            torch.cuda.synchronize()
            for b in range(B):
                for h in range(H):
                    compare_slab(g, b, h, o, b, h)


def test_prefill_equals_single_appends_on_gpu():
    rng = np.random.default_rng(3)
    B, H, D, G, R, T = 1, 2, 128, 32, 128, 300
    K = dev(rng.standard_normal((B, H, T, D)).astype(np.float16))
    V = dev(rng.standard_normal((B, H, T, D)).astype(np.float16))
    a = kivi.Cache(B, H, D, 2, 2, G, R, 384)
    kivi.kivi_append(a, K, V)
    s = kivi.Cache(B, H, D, 2, 2, G, R, 384)
    for t in range(T):
        kivi.kivi_append(s, K[:, :, t:t + 1].contiguous(), V[:, :, t:t + 1].contiguous())
    torch.cuda.synchronize()
    n_kq, n_vq = T - T % R, T - R
    assert torch.equal(a.k_codes[:, :, :n_kq // G], s.k_codes[:, :, :n_kq // G])
    assert torch.equal(a.k_scale[:, :, :n_kq // G], s.k_scale[:, :, :n_kq // G])
    assert torch.equal(a.v_codes[:, :, :n_vq], s.v_codes[:, :, :n_vq])
    assert torch.equal(a.v_zero[..., :n_vq], s.v_zero[..., :n_vq])
    assert torch.equal(a.k_res[:, :, :T % R], s.k_res[:, :, :T % R])
    assert torch.equal(a.v_res, s.v_res)


def test_llama2_decode_steps():
    """The Llama-2-7B-shaped workload: 4064-token prefill then 64 decode steps
    (append one token, attend).  Step 32 reaches t = 4096 and quantizes a key
    block.  Three sampled (batch, head) slabs are checked bit for bit after
    every step, and their attention against the oracle."""
    w = synth.WORKLOADS[2]
    inp = synth.make_inputs(w)
    g = kivi.Cache(w.B, w.Hkv, w.D, w.k_bits, w.v_bits, w.G, w.R, w.capacity)
    say(f"{w.name}: prefill {w.T0}")
    kivi.kivi_append(g, dev(inp["k0"]), dev(inp["v0"]))
    slabs = [(0, 0), (w.B - 1, w.Hkv - 1), (3, 17)]
    orc = {}
    for b, h in slabs:
        o = oracle.Cache(1, 1, w.D, w.k_bits, w.v_bits, w.G, w.R, w.capacity)
        o.append(b16(inp["k0"][b:b + 1, h:h + 1]), b16(inp["v0"][b:b + 1, h:h + 1]))
        orc[(b, h)] = o
    ws = g.new_workspace(w.Hq)
    for step in range(w.steps):
        kivi.kivi_append(g, dev(inp["k_steps"][step]), dev(inp["v_steps"][step]))
        q = inp["q_steps"][step]
        out = host(kivi.kivi_decode_attn(g, dev(q), workspace=ws))
        for (b, h), o in orc.items():
            o.append(b16(inp["k_steps"][step][b:b + 1, h:h + 1]),
                     b16(inp["v_steps"][step][b:b + 1, h:h + 1]))
            compare_slab(g, b, h, o)
            ref = o.decode_attn(b16(q[b:b + 1, h:h + 1]))
            if step % 16 == 0 or step == 31 or step == w.steps - 1:
                assert_close(out[b, h], ref[0, 0], f"step {step} t={g.n_tokens} b{b} h{h}")
            else:
                np.testing.assert_allclose(out[b, h], ref[0, 0], atol=2e-3, rtol=1e-3)
