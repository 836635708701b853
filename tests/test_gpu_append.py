"""GPU parity of kivi_append against the CPU oracle: the quantized stores and
the fp16 window must match bit for bit after every call (KIVI item 4 of the
page "Literature audit -- Group 2", section 1, "Core algorithm")."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_pack_amd import kivi, synth
from tests.gpu_util import (assert_close, b16, cap_for, check_every_slab, compare_slab, dev,
                            gpu_cache, host, logical, oracle_all_slabs, pool, say)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("kb,vb,R,D", [(2, 2, 32, 128), (4, 4, 64, 128), (2, 4, 32, 64),
                                       (4, 2, 128, 128)])
def test_append_random_chunks(kb, vb, R, D):
    rng = np.random.default_rng(kb * 1000 + vb * 100 + R)
    B, H, G = 2, 3, 32
    t_end = 3 * R + 5
    cap = cap_for(t_end, R)
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
                                         (4, 2, 16, 96, 48), (2, 2, 128, 256, 128),
                                         (4, 4, 8, 64, 96)])
def test_single_token_appends(kb, vb, G, D, R):
    """Decode-step appends (one token per call) through both the fused
    single-token kernel (G a power of two <= 64) and the general path (other
    G), across the key-block and window-wrap boundaries."""
    rng = np.random.default_rng(G * 7 + D + kb)
    B, H = 2, 2
    t_end = 2 * R + 3
    cap = cap_for(t_end, R)
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
    la, ls = logical(a), logical(s)
    for name, sl in (("k_codes", np.s_[:, :, :n_kq // G]), ("k_scale", np.s_[:, :, :n_kq // G]),
                     ("k_zero", np.s_[:, :, :n_kq // G]), ("v_codes", np.s_[:, :, :n_vq]),
                     ("v_scale", np.s_[..., :n_vq]), ("v_zero", np.s_[..., :n_vq])):
        assert np.array_equal(np.ascontiguousarray(la[name][sl]).view(np.uint8),
                              np.ascontiguousarray(ls[name][sl]).view(np.uint8)), name
    assert torch.equal(a.k_res[:, :, :T % R], s.k_res[:, :, :T % R])
    assert torch.equal(a.v_res, s.v_res)


def test_llama2_decode_steps():
    """The Llama-2-7B-shaped workload: 4064-token prefill then 64 decode steps
    (kivi_append of one token, then kivi_decode_attn).  Step 32 reaches
    t = 4096 and quantizes a key block.  Every slab's attention after every
    step, and every packed store and window at steps 0, 31, 32, 33, every 8th
    and the last, against the oracle."""
    w = synth.WORKLOADS[2]
    inp = synth.make_inputs(w)
    g = gpu_cache(w)
    say(f"{w.name}: prefill {w.T0}")
    kivi.kivi_append(g, dev(inp["k0"]), dev(inp["v0"]))
    orc = oracle_all_slabs(w, inp, n_steps=0)
    ws = g.new_workspace(w.Hq)
    store_steps = {0, 31, 32, 33, w.steps - 1} | set(range(7, w.steps, 8))
    for step in range(w.steps):
        kivi.kivi_append(g, dev(inp["k_steps"][step]), dev(inp["v_steps"][step]))
        q = inp["q_steps"][step]
        out = host(kivi.kivi_decode_attn(g, dev(q), workspace=ws))

        def one(bh, step=step):
            b, h = bh
            orc[bh].append(b16(inp["k_steps"][step][b:b + 1, h:h + 1]),
                           b16(inp["v_steps"][step][b:b + 1, h:h + 1]))
        list(pool().map(one, sorted(orc)))
        check_every_slab(w, g, orc, {f"step {step} t={g.n_tokens}": out}, q,
                         stores=step in store_steps)
