"""Seeded synthetic inputs for the KIVI decode-attention workloads.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic, so both the HIP path's tests and the CPU oracle can take
their inputs from it.  All tensors are fp16 (numpy ``float16``, rounded to
nearest even from fp32 draws).

Workloads (the shapes of the models the KIVI evaluation uses; no weights or
datasets are involved -- seeded Gaussian activations stand in for them):

  1 tiny            B1, 1 q / 1 kv head, D128, 2-bit K/V, G32, R32,  512-token prefill, 1 step
  2 llama2-7b-mha   B8, 32 / 32,         D128, 2-bit,     G32, R128, 4064-token prefill, 64 steps
  3 kivi4-b64       B64, 32 / 32,        D128, 4-bit,     G32, R128, 2048-token prefill, 1 step
  4 llama3-8b-gqa   B4, 32 / 8,          D128, 2-bit,     G32, R128, 32768-token prefill, 1 step
  5 long-128k       B1, 32 / 8,          D128, 2-bit,     G32, R128, 131072-token prefill, 1 step
  ragged            B8, 32 / 8,          D128, 2-bit,     G32, R128, prefills of 1024..32768
                    tokens per row (ragged_lengths), 1 step

q and V are N(0, 1).  K is N(0, 1) except 4 distinct "outlier" channels per
KV head, drawn without replacement, which are multiplied by 15 (tiny) or by a
per-channel factor drawn from U[10, 20] (the others) -- for prefill and
appended keys alike.  The llama2-7b-mha prefill is 4064 tokens so that its
64 decode steps (contexts 4065..4128) cross a multiple of R=128 and exercise
the key-block quantization.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    k_bits: int
    v_bits: int
    G: int
    R: int
    T0: int
    steps: int
    outlier_fixed: float | None  # fixed factor, or None for U[10, 20]
    scale_fp16: bool = False     # the cache stores its scales as binary16

    @property
    def capacity(self) -> int:
        """Token capacity: prefill + steps rounded up to a multiple of R and
        of the 128-token record."""
        t = self.T0 + self.steps
        m = self.R * 128 // math.gcd(self.R, 128)
        return ((t + m - 1) // m) * m

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "tiny", 1, 1, 1, 128, 2, 2, 32, 32, 512, 1, 15.0),
    2: Workload(2, "llama2-7b-mha", 8, 32, 32, 128, 2, 2, 32, 128, 4064, 64, None),
    3: Workload(3, "kivi4-b64", 64, 32, 32, 128, 4, 4, 32, 128, 2048, 1, None),
    4: Workload(4, "llama3-8b-gqa-32k", 4, 32, 8, 128, 2, 2, 32, 128, 32768, 1, None),
    5: Workload(5, "long-128k", 1, 32, 8, 128, 2, 2, 32, 128, 131072, 1, None),
}


# A ragged batch on the llama3-8b-gqa shape: 8 rows whose prefill lengths
# spread over [1024, 32768] (ragged_lengths).  T0 is the longest row.
RAGGED = Workload(6, "llama3-8b-gqa-ragged-b8", 8, 32, 8, 128, 2, 2, 32, 128, 32768, 1, None)


def ragged_lengths(n: int, lo: int, hi: int, seed: int = 7) -> np.ndarray:
    """n sequence lengths for a ragged batch, log-uniform over [lo, hi] (a
    long-tailed mix like the request lengths of a serving trace), with the
    first row at hi so that the batch spans the whole range.  int64 [n]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = np.exp(rng.uniform(np.log(lo), np.log(hi), size=n))
    out = np.clip(np.rint(x), lo, hi).astype(np.int64)
    out[0] = hi
    return out


def _normal_f16(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16)


def make_inputs(w: Workload, seed: int | None = None) -> dict:
    """Draw every tensor the workload needs.

    Returns a dict of fp16 arrays:
      k0, v0   [B][Hkv][T0][D]          prefill keys / values
      k_steps  [steps][B][Hkv][1][D]    appended keys
      v_steps  [steps][B][Hkv][1][D]    appended values
      q_steps  [steps][B][Hq][D]        decode queries
    plus ``outlier_channels`` [B][Hkv][4] and ``outlier_factor`` [B][Hkv][4].
    """
    seed = 1000 + w.index if seed is None else seed
    ss = np.random.SeedSequence(seed)
    r_idx, r_scale, r_k0, r_v0, r_q, r_k, r_v = [np.random.Generator(np.random.PCG64(s))
                                                  for s in ss.spawn(7)]
    B, H, D = w.B, w.Hkv, w.D
    chans = np.stack([np.stack([r_idx.choice(D, size=4, replace=False) for _ in range(H)])
                      for _ in range(B)]).astype(np.int64)
    if w.outlier_fixed is not None:
        factor = np.full((B, H, 4), w.outlier_fixed, np.float32)
    else:
        factor = r_scale.uniform(10.0, 20.0, size=(B, H, 4)).astype(np.float32)
    gain = np.ones((B, H, D), np.float32)
    for b in range(B):
        for h in range(H):
            gain[b, h, chans[b, h]] = factor[b, h]

    def keys(rng, shape):  # shape [..., B, H, T, D]
        x = rng.standard_normal(shape, dtype=np.float32)
        x *= gain[:, :, None, :]
        return x.astype(np.float16)

    k0 = keys(r_k0, (B, H, w.T0, D))
    v0 = _normal_f16(r_v0, (B, H, w.T0, D))
    k_steps = keys(r_k, (w.steps, B, H, 1, D))
    v_steps = _normal_f16(r_v, (w.steps, B, H, 1, D))
    q_steps = _normal_f16(r_q, (w.steps, B, w.Hq, D))
    return {"k0": k0, "v0": v0, "k_steps": k_steps, "v_steps": v_steps, "q_steps": q_steps,
            "outlier_channels": chans, "outlier_factor": factor}


def bits(a: np.ndarray) -> np.ndarray:
    """fp16 array -> its raw uint16 bit patterns (no copy)."""
    return np.ascontiguousarray(a).view(np.uint16)
