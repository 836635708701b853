"""The pre-marshalled calls of the binding (kivi.bind_append,
kivi.bind_decode_attn) issue exactly the library calls they stand for: the
same cache contents and token count as the per-call binding, and the same
attention output up to the rounding order of its merges."""
import numpy as np
import pytest
import torch

from decode_attention_pack_amd import kivi
from tests.gpu_util import dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def test_bound_calls_match_unbound():
    rng = np.random.default_rng(11)
    B, H, Hq, D, G, R = 2, 2, 8, 128, 32, 32
    T0, steps = 700, 40
    cap = 768
    K0 = dev(rng.standard_normal((B, H, T0, D)).astype(np.float16))
    V0 = dev(rng.standard_normal((B, H, T0, D)).astype(np.float16))
    caches = [kivi.Cache(B, H, D, 2, 2, G, R, cap) for _ in range(2)]
    for c in caches:
        for arr in c.arrays.values():   # slots past the written tokens compare too
            arr.zero_()
        kivi.kivi_append(c, K0, V0)
    k1 = dev(rng.standard_normal((B, H, 1, D)).astype(np.float16))
    v1 = dev(rng.standard_normal((B, H, 1, D)).astype(np.float16))
    q = dev(rng.standard_normal((B, Hq, D)).astype(np.float16))
    out_b = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    ws = caches[1].new_workspace(Hq)
    app = kivi.bind_append(caches[1], k1, v1)
    dec = kivi.bind_decode_attn(caches[1], q, out_b, ws)
    for s in range(steps):
        kivi.kivi_append(caches[0], k1, v1)
        out_a = kivi.kivi_decode_attn(caches[0], q)
        app()
        dec()
        torch.cuda.synchronize()
        assert caches[1].n_tokens == caches[0].n_tokens == T0 + s + 1
        # the matrix kernel's waves take blocks in run-time order, so two
        # calls may merge the same terms in different orders
        torch.testing.assert_close(out_a, out_b, atol=1e-5, rtol=1e-5, msg=f"step {s}")
    for n, a in caches[0].arrays.items():
        assert torch.equal(a, caches[1].arrays[n]), n
