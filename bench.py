"""Benchmark: one KIVI decode step (append one token, then attention over the
packed cache) on one MI355X, reported as achieved HBM GB/s and us/step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4]

A step appends one token to the cache of one layer and attends over it with
kivi_decode_step, which runs the append inside the attention launch where the
shape allows (--unfused: kivi_append, then kivi_decode_attn).  Steps rotate
over L layer replicas (L x footprint >= 1 GiB) so the 256 MB Infinity Cache
cannot serve the working set; inputs are resident in HBM before the timed
region starts.  `value` is the algorithmic bytes a step must move (packed
codes + fp32 scale/zero + fp16 window + q + out, plus the append's bytes)
divided by the measured step time (HIP events at the two ends of the K timed
steps).  `roofline` covers the attention launch alone (its split kernel and
combine): a second timed loop issues K kivi_decode_attn calls back to back
over the same replicas, with HIP events on the stream the library launches on
around rounds of calls, and divides by the call count.  `cpu_baseline` times
the CPU oracle on a bounded sample of (batch, KV head) slabs of the same
workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["decode_attention_pack_amd/csrc/" + f for f in
                  ("api.cpp", "decode_matrix.hip", "decode_generic.hip", "kivi_internal.hpp",
                   "kivi_device.hpp")] + ["decode_attention_pack_amd/build.py"]


def kernel_source_hash() -> str:
    """sha256 over the sources and build flags of the attention kernels."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload_name: str):
    """HBM bytes per attention launch from the committed counter record of this
    workload, or None when there is none or the kernels changed since."""
    path = os.path.join(PROFILES, f"traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def attn_bytes(w, t: int) -> int:
    """Algorithmic bytes of one kivi_decode_attn call at context t."""
    R, G, D = w.R, w.G, w.D
    n_kq = t - t % R
    n_vq = max(0, t - R)
    rep = w.Hq // w.Hkv
    per = (n_kq * D * w.k_bits // 8 + (n_kq // G) * D * 8
           + n_vq * D * w.v_bits // 8 + n_vq * (D // G) * 8
           + ((t % R) + min(t, R)) * D * 2
           + rep * D * 2 + rep * D * 4)
    return per * w.B * w.Hkv


def append_bytes(w, t_before: int) -> int:
    """Algorithmic bytes of appending one token to a cache holding t_before."""
    R, G, D = w.R, w.G, w.D
    per = 2 * D * 2 + 2 * D * 2                       # read k, v; write window slots
    if t_before >= R:                                 # value leaves the window
        per += D * 2 + D * w.v_bits // 8 + (D // G) * 8
    if (t_before + 1) % R == 0:                       # key block quantized
        per += R * D * 2 + R * D * w.k_bits // 8 + (R // G) * D * 8
    return per * w.B * w.Hkv


def pack_bytes(w, T: int, bits: int) -> int:
    """Algorithmic bytes of packing T tokens of keys (or values): fp16 in,
    codes + fp32 scale/zero out."""
    return w.B * w.Hkv * (T * w.D * 2 + T * w.D * bits // 8 + (T // w.G) * w.D * 8)


def time_pack(w, inp, dev, stream, reps: int = 5):
    """Full-prefill pack pass (kivi_pack_keys, kivi_pack_values) in us and GB/s."""
    import torch

    from decode_attention_pack_amd import kivi
    T = w.T0 - w.T0 % w.G
    k = torch.from_numpy(inp["k0"][:, :, :T]).to(dev).contiguous()
    v = torch.from_numpy(inp["v0"][:, :, :T]).to(dev).contiguous()
    out = {}
    for name, x, bits in (("keys", k, w.k_bits), ("values", v, w.v_bits)):
        shp = kivi.layout_shapes(w.B, w.Hkv, w.D, bits, bits, w.G, 1, T)
        pre = "k_" if name == "keys" else "v_"
        codes = torch.empty(shp[pre + "codes"], dtype=torch.int32, device=dev)
        scale = torch.empty(shp[pre + "scale"], dtype=torch.float32, device=dev)
        zero = torch.empty(shp[pre + "zero"], dtype=torch.float32, device=dev)
        fn = kivi.kivi_pack_keys if name == "keys" else kivi.kivi_pack_values
        fn(x, bits, w.G, codes, scale, zero, T, 0, stream=stream)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn(x, bits, w.G, codes, scale, zero, T, 0, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        out[name] = {"tokens": T, "us": round(us, 2),
                     "GBps": round(pack_bytes(w, T, bits) / us / 1e3, 1)}
    return out


def cpu_baseline(w, inp, budget_s: float = 12.0):
    """Time the CPU oracle on (batch, KV head) slabs until ~budget_s of work."""
    import oracle
    rep = w.Hq // w.Hkv
    slabs = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    t = w.T0 + 1
    done, spent = 0, 0.0
    q = inp["q_steps"][0]
    for b, h in slabs:
        o = oracle.Cache(1, 1, w.D, w.k_bits, w.v_bits, w.G, w.R, w.capacity)
        o.append(inp["k0"][b:b + 1, h:h + 1].view(np.uint16), inp["v0"][b:b + 1, h:h + 1].view(np.uint16))
        o.append(inp["k_steps"][0][b:b + 1, h:h + 1].view(np.uint16),
                 inp["v_steps"][0][b:b + 1, h:h + 1].view(np.uint16))
        qs = np.ascontiguousarray(q[b:b + 1, h * rep:(h + 1) * rep]).view(np.uint16)
        t0 = time.perf_counter()
        o.decode_attn(qs)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= budget_s:
            break
    slab_bytes = attn_bytes(w, t) / (w.B * w.Hkv)
    return {"value": round(slab_bytes * done / spent / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{done} of {w.B * w.Hkv} (batch, kv-head) slabs of {w.name}, one decode "
                      f"step at context {t} ({rep} query heads each), single-threaded C oracle, "
                      f"{spent:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--layers", type=int, default=0, help="layer replicas (0 = auto, >= 1 GiB)")
    ap.add_argument("--path", type=int, default=0, help="0 auto, 1 scalar kernel, 2 matrix kernel")
    ap.add_argument("--tokens-per-split", type=int, default=0,
                    help="split size of the attention call (0 = the library's automatic plan)")
    ap.add_argument("--unfused", action="store_true",
                    help="time a step as kivi_append + kivi_decode_attn instead of kivi_decode_step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-pack", action="store_true", help="skip the full-prefill pack pass")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="after the timed steps, run one plain device-to-device copy of this "
                         "many MiB (a known-size reference for hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: each GPU of a "
                                   "multi-GPU deployment holds whole (batch row, KV head) slabs "
                                   "and decodes them with no collectives",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    from decode_attention_pack_amd import kivi, synth

    w = synth.WORKLOADS[args.workload]
    inp = synth.make_inputs(w.replace(steps=1))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    total = args.warmup + args.steps
    # one replica's footprint at the prefill length
    probe = kivi.Cache(w.B, w.Hkv, w.D, w.k_bits, w.v_bits, w.G, w.R,
                       ((w.T0 + 2 * w.R) // w.R) * w.R)
    footprint = sum(a.numel() * a.element_size() for a in probe.arrays.values())
    del probe
    L = args.layers or max(2, math.ceil((1 << 30) / footprint))
    per_layer = math.ceil(total / L) + 1
    cap = ((w.T0 + per_layer + w.R - 1) // w.R) * w.R
    print(f"# {w.name}: footprint {footprint / 1e6:.1f} MB/layer, {L} layers, capacity {cap}",
          file=sys.stderr, flush=True)

    base = kivi.Cache(w.B, w.Hkv, w.D, w.k_bits, w.v_bits, w.G, w.R, cap)
    kivi.kivi_append(base, torch.from_numpy(inp["k0"]).to(dev), torch.from_numpy(inp["v0"]).to(dev))
    torch.cuda.synchronize()
    caches = [base]
    for _ in range(L - 1):
        arrays = {n: a.clone() for n, a in base.arrays.items()}
        c = kivi.Cache(w.B, w.Hkv, w.D, w.k_bits, w.v_bits, w.G, w.R, cap, arrays=arrays)
        c.c.n_tokens = base.n_tokens
        caches.append(c)
    k1 = torch.from_numpy(inp["k_steps"][0]).to(dev)
    v1 = torch.from_numpy(inp["v_steps"][0]).to(dev)
    q = torch.from_numpy(inp["q_steps"][0]).to(dev)
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=dev)
    ws = caches[0].new_workspace(w.Hq, args.tokens_per_split, args.path)
    torch.cuda.synchronize()

    # calls marshalled once per layer replica, so that the host enqueues a step
    # faster than the GPU runs it and the timed region measures the GPU
    appends = [kivi.bind_append(c, k1, v1, stream=stream) for c in caches]
    decodes = [kivi.bind_decode_attn(c, q, out, ws, tokens_per_split=args.tokens_per_split,
                                     path=args.path, stream=stream) for c in caches]

    # the fused step (kivi_decode_step) takes the automatic plan
    fused = not args.unfused and args.path == 0 and args.tokens_per_split == 0
    fused_steps = [kivi.bind_decode_step(c, k1, v1, q, out, ws, stream=stream) for c in caches]

    def step(i):
        c = caches[i % L]
        t_before = c.n_tokens
        if fused:
            fused_steps[i % L]()
        else:
            appends[i % L]()
            decodes[i % L]()
        return attn_bytes(w, t_before + 1), append_bytes(w, t_before)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region 1: K whole steps (append + attention), events at its ends only
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    a_bytes = p_bytes = 0
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        ab, pb = step(args.warmup + i)
        a_bytes += ab
        p_bytes += pb
    stop.record(stream)
    torch.cuda.synchronize()
    # timed region 2: the attention launch alone, K calls back to back over the
    # same replicas (no append in between), in rounds of 25 calls so that the
    # spread across rounds can be reported
    n_rounds = max(1, args.steps // 25)
    per_round = max(1, args.steps // n_rounds)
    a2_bytes = 0
    rounds_ms = []
    for r in range(n_rounds):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(per_round):
            c = caches[(r * per_round + i) % L]
            decodes[(r * per_round + i) % L]()
            a2_bytes += attn_bytes(w, c.n_tokens)
        e1.record(stream)
        rounds_ms.append((e0, e1))
    torch.cuda.synchronize()
    attn_ms = [e0.elapsed_time(e1) / per_round for e0, e1 in rounds_ms]
    if args.calibration_copy_mib > 0:
        src = torch.empty(args.calibration_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps
    attn_avg_ms = float(np.mean(attn_ms))
    attn_gbps = a2_bytes / (n_rounds * per_round) / (attn_avg_ms * 1e-3) / 1e9
    value = (a_bytes + p_bytes) / (total_ms * 1e-3) / 1e9

    line = {
        "metric": "quantized-KV decode attn: achieved HBM GB/s (% of peak) and us/step",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.D, "context": w.T0 + 1, "k_bits": w.k_bits, "v_bits": w.v_bits,
                   "group": w.G, "residual": w.R, "layers_rotated": L,
                   "storage": "packed codes, fp32 scale/zero, fp16 window; fp16 q"},
        "step_call": "kivi_decode_step" if fused else "kivi_append + kivi_decode_attn",
        "us_per_step": round(ms_step * 1e3, 2),
        "attn_us": round(attn_avg_ms * 1e3, 2),
        "attn_us_rounds_min_p50_max": [round(float(np.percentile(attn_ms, p)) * 1e3, 2)
                                       for p in (0, 50, 100)],
        "attn_pct_of_peak": round(100 * attn_gbps / HBM_PEAK_GBPS, 1),
        "roofline": {"bound": "hbm", "achieved": round(attn_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(attn_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(w.name),
                     "kernel": "kivi_decode_attn launch (split kernel + combine)",
                     "bytes_per_launch": a2_bytes // (n_rounds * per_round)},
    }
    if not args.no_pack:
        del caches, base
        torch.cuda.empty_cache()
        line["pack_full_prefill"] = time_pack(w, inp, dev, stream)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
