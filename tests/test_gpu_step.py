"""GPU parity of kivi_decode_step -- one decode step that appends a token and
attends over the resulting cache (KIVI items 4 and 5 of the page "Literature
audit -- Group 2", section 1, "Core algorithm") -- against the CPU oracle's
append followed by its attention: outputs within 2e-3 + 1e-3*|ref|
elementwise, packed stores and window rows bit for bit.

The sequences cross every case of the fused path: steps before any value
leaves the window, the first value to leave it, a popped token at a block
boundary of the attention kernel (n_vq a multiple of 128), and the steps that
complete a key block (quantized inside the launch)."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_pack_amd import kivi, synth
from tests.gpu_util import (assert_close, b16, cap_for, check_every_slab, compare_slab, dev,
                            gpu_cache, host, logical, oracle_all_slabs, pool, say)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _signed_zeros(X, rng):
    """Put +0.0 / -0.0 ties at the minimum of some value groups (along
    channels) and key groups (along tokens), in both orders."""
    B, H, T, D = X.shape
    pz, nz = np.float16(0.0), np.float16(-0.0)
    for tau in rng.choice(T, size=max(1, T // 8), replace=False):
        c0 = 32 * int(rng.integers(D // 32))
        X[:, :, tau, c0:c0 + 32] = np.abs(X[:, :, tau, c0:c0 + 32])
        X[:, :, tau, c0] = pz if tau % 2 else nz
        X[:, :, tau, c0 + 1] = nz if tau % 2 else pz
    for c in rng.choice(D, size=4, replace=False):
        X[:, :, :, c] = np.abs(X[:, :, :, c])
        X[:, :, 0::32, c] = pz if c % 2 else nz
        X[:, :, 1::32, c] = nz if c % 2 else pz
    return X


def _steps(rep, R, T0, n_steps, masked, kb=2, vb=2, B=2, H=2, D=128, G=32, seed=0,
           zeros=False):
    rng = np.random.default_rng(seed + 7 * rep + R + T0)
    t_end = T0 + n_steps
    cap = cap_for(t_end, R)
    scale = rng.uniform(0.5, 15, (1, H, 1, D))
    K = (rng.standard_normal((B, H, t_end, D)) * scale).astype(np.float16)
    V = rng.standard_normal((B, H, t_end, D)).astype(np.float16)
    if zeros:
        K, V = _signed_zeros(K, rng), _signed_zeros(V, rng)
    g = kivi.Cache(B, H, D, kb, vb, G, R, cap)
    o = oracle.Cache(B, H, D, kb, vb, G, R, cap)
    if T0:
        kivi.kivi_append(g, dev(K[:, :, :T0]), dev(V[:, :, :T0]))
        o.append(b16(K[:, :, :T0]), b16(V[:, :, :T0]))
    ws = g.new_workspace(H * rep)
    say(f"decode_step rep={rep} R={R} T0={T0} steps={n_steps} masked={masked} kb={kb} vb={vb}")
    for i in range(n_steps):
        t = T0 + i
        q = rng.standard_normal((B, H * rep, D)).astype(np.float16)
        k1 = np.ascontiguousarray(K[:, :, t:t + 1])
        v1 = np.ascontiguousarray(V[:, :, t:t + 1])
        mask = None
        if masked:
            mask = np.where(rng.random((B, t + 1)) < 0.2, -np.inf,
                            rng.standard_normal((B, t + 1))).astype(np.float32)
            mask[:, -1] = 0.0
        out = host(kivi.kivi_decode_step(g, dev(k1), dev(v1), dev(q),
                                         None if mask is None else dev(mask), workspace=ws))
        o.append(b16(k1), b16(v1))
        ref = o.decode_attn(b16(q), mask)
        assert g.n_tokens == t + 1
        assert_close(out, ref, f"step t={t + 1}")
        if i % 16 == 15 or i == n_steps - 1 or (t + 1) % R in (0, 1):
            torch.cuda.synchronize()
            for b in range(B):
                for h in range(H):
                    compare_slab(g, b, h, o, b, h)


@pytest.mark.parametrize("rep,R,T0,n_steps", [
    (4, 128, 120, 150),     # first pops, key blocks at 128 and 256, n_vq = 128 at t = 256
    (1, 32, 3, 80),         # short window: many pops and key blocks
    (2, 64, 500, 70),       # blocks in the block role from the start
    (4, 128, 1, 20),        # nearly empty cache: nothing in the block role
    (2, 64, 0, 70),         # the first token of an empty cache, then the first pop
    (4, 96, 300, 200),      # R = 96: key blocks and pops off the 128-token block grid
    (1, 96, 0, 200),
])
def test_decode_step_matches_oracle(rep, R, T0, n_steps):
    _steps(rep, R, T0, n_steps, masked=False)


@pytest.mark.parametrize("rep,R,bits", [(4, 32, 2), (1, 64, 2), (1, 64, 4), (4, 64, 4)])
def test_decode_step_signed_zeros(rep, R, bits):
    """Groups whose minimum is a +0.0 / -0.0 tie, quantized by the prefill and
    by the steps -- inside the fused launch at 2 bits and at 4 bits with
    several query heads per KV head (popped values, completed key blocks), by
    kivi_append at 4 bits with one on short rows: bit for bit."""
    _steps(rep, R, 40, 3 * R, masked=False, zeros=True, kb=bits, vb=bits)


def test_decode_step_masked():
    _steps(4, 128, 250, 12, masked=True)


@pytest.mark.parametrize("rep,R,T0,n_steps", [
    (4, 128, 120, 150),     # first pops, key blocks at 128 and 256
    (2, 64, 500, 70),
    (4, 96, 300, 200),      # key blocks and pops off the 128-token block grid
    (4, 32, 3, 80),         # short window: many pops and key blocks
    (1, 128, 2600, 40),     # one query head per KV head, long enough rows
])
def test_decode_step_4bit_matches_oracle(rep, R, T0, n_steps):
    """4-bit keys and values: the step fused into the matrix launch, whose
    window role quantizes the popped values and the completed key blocks to
    4-bit codes; outputs within tolerance, packed stores bit for bit."""
    _steps(rep, R, T0, n_steps, masked=False, kb=4, vb=4)


def test_decode_step_4bit_masked():
    _steps(4, 128, 250, 12, masked=True, kb=4, vb=4)


@pytest.mark.parametrize("kb,vb,rep,R,T0,n_steps", [
    (2, 4, 4, 128, 120, 150), (4, 2, 4, 128, 120, 150), (2, 4, 2, 64, 500, 70),
    (4, 2, 4, 32, 3, 80)])
def test_decode_step_mixed_widths(kb, vb, rep, R, T0, n_steps):
    """2-bit keys with 4-bit values and the reverse, fused: the popped value
    quantized at the value width, a completed key block at the key width."""
    _steps(rep, R, T0, n_steps, masked=False, kb=kb, vb=vb)


@pytest.mark.parametrize("kb,vb,rep", [(4, 4, 1), (2, 2, 8)])
def test_decode_step_other_shapes(kb, vb, rep):
    """Shapes the matrix kernel does not take run as append + attention."""
    _steps(rep, 64, 100, 20, masked=False, kb=kb, vb=vb)


@pytest.mark.parametrize("bits", [2, 4])
def test_decode_step_equals_append_then_attend(bits):
    """Fused and unfused steps leave bit-identical caches and outputs within
    rounding-order differences."""
    rng = np.random.default_rng(11 + bits)
    B, H, D, R, rep, T0, n = 2, 4, 128, 128, 4, 1000, 140
    cap = cap_for(T0 + n, R)
    K = rng.standard_normal((B, H, T0 + n, D)).astype(np.float16)
    V = rng.standard_normal((B, H, T0 + n, D)).astype(np.float16)
    a = kivi.Cache(B, H, D, bits, bits, 32, R, cap)
    u = kivi.Cache(B, H, D, bits, bits, 32, R, cap)
    for c in (a, u):
        kivi.kivi_append(c, dev(K[:, :, :T0]), dev(V[:, :, :T0]))
    for i in range(n):
        t = T0 + i
        q = dev(rng.standard_normal((B, H * rep, D)).astype(np.float16))
        k1, v1 = dev(K[:, :, t:t + 1]), dev(V[:, :, t:t + 1])
        fa = host(kivi.kivi_decode_step(a, k1, v1, q))
        kivi.kivi_append(u, k1, v1)
        fu = host(kivi.kivi_decode_attn(u, q))
        np.testing.assert_allclose(fa, fu, atol=1e-4, rtol=1e-4, err_msg=f"t={t + 1}")
    torch.cuda.synchronize()
    assert a.n_tokens == u.n_tokens == T0 + n
    la, lu = logical(a), logical(u)
    for name in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero"):
        ga, gu = la[name], lu[name]
        if name.startswith("k"):
            n_kq = a.n_tokens - a.n_tokens % R
            sl = (slice(None), slice(None), slice(0, n_kq // 32))
        elif name == "v_codes":
            sl = (slice(None), slice(None), slice(0, a.n_tokens - R))
        else:
            sl = (slice(None), slice(None), slice(None), slice(0, a.n_tokens - R))
        assert np.array_equal(np.ascontiguousarray(ga[sl]).view(np.uint8),
                              np.ascontiguousarray(gu[sl]).view(np.uint8)), name


def test_decode_step_rejects_full_cache_and_small_workspace():
    rng = np.random.default_rng(3)
    B, H, D, R = 1, 1, 128, 32
    g = kivi.Cache(B, H, D, 2, 2, 32, R, 128)
    full = rng.standard_normal((B, H, 128, D)).astype(np.float16)
    kivi.kivi_append(g, dev(full), dev(full))
    x = full[:, :, :R]
    k1 = dev(x[:, :, :1])
    q = dev(rng.standard_normal((B, H, D)).astype(np.float16))
    with pytest.raises(kivi.KiviError):
        kivi.kivi_decode_step(g, k1, k1, q)
    g2 = kivi.Cache(B, H, D, 2, 2, 32, R, 4 * R)
    kivi.kivi_append(g2, dev(x), dev(x))
    with pytest.raises(kivi.KiviError):
        kivi.kivi_decode_step(g2, k1, k1, q, workspace=torch.empty(16, dtype=torch.uint8,
                                                                    device="cuda"))
    assert g2.n_tokens == R


@pytest.mark.parametrize("index", [1, 4, 5])
def test_decode_step_full_workload(index):
    """Two fused steps on the full tiny, 32k GQA and 128k single-stream
    workloads, in the configuration the benchmark times; the oracle rebuilds
    every slab and checks every output and, after the second step, every
    packed store."""
    w = synth.WORKLOADS[index].replace(steps=2)
    inp = synth.make_inputs(w)
    g = gpu_cache(w)
    say(f"{w.name}: prefill {w.T0} + 2 fused steps")
    kivi.kivi_append(g, dev(inp["k0"]), dev(inp["v0"]))
    outs = []
    for s in range(2):
        outs.append(host(kivi.kivi_decode_step(g, dev(inp["k_steps"][s]), dev(inp["v_steps"][s]),
                                               dev(inp["q_steps"][s]))))
    orc = oracle_all_slabs(w, inp, n_steps=0)
    _append_step(orc, inp, 0)
    check_every_slab(w, g, orc, {"step 0": outs[0]}, inp["q_steps"][0], stores=False)
    _append_step(orc, inp, 1)
    check_every_slab(w, g, orc, {"step 1": outs[1]}, inp["q_steps"][1])


def _append_step(orc, inp, step):
    """Append token `step` of the workload to every slab's oracle cache."""
    def one(bh):
        b, h = bh
        orc[bh].append(b16(inp["k_steps"][step][b:b + 1, h:h + 1]),
                       b16(inp["v_steps"][step][b:b + 1, h:h + 1]))
    list(pool().map(one, sorted(orc)))


def _fused_sequence(w, store_steps):
    """Prefill, then w.steps calls of kivi_decode_step; after every step the
    oracle advances every slab and checks every output, and at the steps in
    store_steps every packed store and window bit for bit."""
    inp = synth.make_inputs(w)
    g = gpu_cache(w)
    say(f"{w.name}: prefill {w.T0} + {w.steps} fused steps")
    kivi.kivi_append(g, dev(inp["k0"]), dev(inp["v0"]))
    orc = oracle_all_slabs(w, inp, n_steps=0)
    ws = g.new_workspace(w.Hq)
    for step in range(w.steps):
        q = inp["q_steps"][step]
        out = host(kivi.kivi_decode_step(g, dev(inp["k_steps"][step]), dev(inp["v_steps"][step]),
                                         dev(q), workspace=ws))
        _append_step(orc, inp, step)
        check_every_slab(w, g, orc, {f"step {step} t={g.n_tokens}": out}, q,
                         stores=step in store_steps)


def test_decode_step_llama2_sequence():
    """The Llama-2-7B-shaped workload as fused steps: 4064-token prefill, then
    64 calls of kivi_decode_step.  Step 32 reaches t = 4096, so its launch
    quantizes a key block and every step pops a value.  Every slab's output
    after every step; every packed store and window at steps 0, 31, 32, 33,
    every 8th and the last."""
    w = synth.WORKLOADS[2]
    _fused_sequence(w, {0, 31, 32, 33, w.steps - 1} | set(range(7, w.steps, 8)))


def test_decode_step_32k_key_block():
    """The 32k GQA workload's shape from 8 tokens before a key-block boundary:
    ten fused steps, the eighth of which completes the block (t = 33024) and
    quantizes it inside the launch.  Every slab's output and packed store
    after every step."""
    w = synth.WORKLOADS[4].replace(T0=33024 - 8, steps=10)
    assert (w.T0 + 8) % w.R == 0
    _fused_sequence(w, set(range(w.steps)))
