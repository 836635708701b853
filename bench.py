"""Benchmark: one KIVI decode step (append one token, then attention over the
packed cache) on one MI355X, reported as achieved HBM GB/s and us/step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4]

A step appends one token to the cache of one layer and attends over it with
kivi_decode_step, which runs the append inside the attention launch where the
shape allows (--unfused: kivi_append, then kivi_decode_attn).  Steps rotate
over L layer replicas (L x footprint >= 1 GiB) so the 256 MB Infinity Cache
cannot serve the working set; inputs are resident in HBM before the timed
region starts.  Every replica runs at the context the workload states: its
token count (a host-side field of the cache descriptor) is set back to the
prefill length once it has taken the workload's decode steps, so the timed
steps attend over the stated context, not a growing one.

`value` is the algorithmic bytes a step must move (packed codes + fp32
scales -- fp16 with --scale-fp16 -- + fp16 zero points + fp16 window + q +
out, plus the append's bytes)
divided by the measured step time (HIP events at the two ends of the K timed
steps).  `roofline` covers the attention launch alone: a second timed loop
issues kivi_decode_attn calls back to back over the same replicas, in at
least three rounds, with HIP events on the stream the library launches on
around each round.  `cpu_baseline` times the CPU oracle on a bounded sample
of (batch, KV head) slabs of the same workload, on one host thread and on
every host core (one slab per thread).
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
KERNEL_SOURCES = sorted(
    "decode_attention_pack_amd/csrc/" + f
    for f in os.listdir(os.path.join(ROOT, "decode_attention_pack_amd", "csrc"))
    if f.endswith((".hip", ".cpp", ".hpp"))) + ["decode_attention_pack_amd/build.py"]


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


def group_bytes(w) -> int:
    """Bytes of one group's scale and zero point: an fp32 (or, in the
    fp16-scale layout, fp16) scale and an fp16 zero point."""
    return (2 if w.scale_fp16 else 4) + 2


def attn_bytes(w, t) -> int:
    """Algorithmic bytes of one kivi_decode_attn call at context t (an int,
    or one count per batch row of a ragged batch)."""
    R, G, D = w.R, w.G, w.D
    rep = w.Hq // w.Hkv
    total = 0
    for tb in ([t] * w.B if isinstance(t, int) else t):
        n_kq = tb - tb % R
        n_vq = max(0, tb - R)
        # scale + fp16 zero per group
        gb = group_bytes(w)
        total += (n_kq * D * w.k_bits // 8 + (n_kq // G) * D * gb
                  + n_vq * D * w.v_bits // 8 + n_vq * (D // G) * gb
                  + ((tb % R) + min(tb, R)) * D * 2
                  + rep * D * 2 + rep * D * 4)
    return total * w.Hkv


def append_bytes(w, t_before) -> int:
    """Algorithmic bytes of appending one token to every row of a cache
    holding t_before tokens (an int, or one count per row)."""
    R, G, D = w.R, w.G, w.D
    total = 0
    for tb in ([t_before] * w.B if isinstance(t_before, int) else t_before):
        per = 2 * D * 2 + 2 * D * 2                       # read k, v; write window slots
        if tb >= R:                                       # value leaves the window
            per += D * 2 + D * w.v_bits // 8 + (D // G) * group_bytes(w)
        if (tb + 1) % R == 0:                             # key block quantized
            per += R * D * 2 + R * D * w.k_bits // 8 + (R // G) * D * group_bytes(w)
        total += per
    return total * w.Hkv


def pack_bytes(w, T: int, bits: int) -> int:
    """Algorithmic bytes of packing T tokens of keys (or values): fp16 in,
    codes + scales + fp16 zeros out."""
    return w.B * w.Hkv * (T * w.D * 2 + T * w.D * bits // 8 + (T // w.G) * w.D * group_bytes(w))


def time_pack(w, inp, dev, stream, reps: int = 5):
    """Full-prefill pack pass (kivi_pack_keys, kivi_pack_values) in us and GB/s."""
    import torch

    from decode_attention_pack_amd import kivi
    T = w.T0 - w.T0 % w.G
    cap = -(-T // 128) * 128
    k = torch.from_numpy(inp["k0"][:, :, :T]).to(dev).contiguous()
    v = torch.from_numpy(inp["v0"][:, :, :T]).to(dev).contiguous()
    dst = kivi.Cache(w.B, w.Hkv, w.D, w.k_bits, w.v_bits, w.G, w.G, cap, scale_fp16=w.scale_fp16)
    out = {}
    for name, x, bits in (("keys", k, w.k_bits), ("values", v, w.v_bits)):
        fn = kivi.kivi_pack_keys if name == "keys" else kivi.kivi_pack_values
        fn(dst, x, 0, stream=stream)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn(dst, x, 0, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        out[name] = {"tokens": T, "us": round(us, 2),
                     "GBps": round(pack_bytes(w, T, bits) / us / 1e3, 1)}
    return out


def select_bytes(w, t: int, sel_union) -> int:
    """Algorithmic bytes of one kivi_select_attn call at context t: every key
    (codes, fp32 scales, fp16 zeros; fp16 window rows), the values of the
    tokens any query head of a KV head selects (sel_union: bool [B][Hkv][t]),
    q and out."""
    R, G, D = w.R, w.G, w.D
    n_kq, n_vq = t - t % R, max(0, t - R)
    rep = w.Hq // w.Hkv
    keys = n_kq * D * w.k_bits // 8 + (n_kq // G) * D * group_bytes(w) + (t - n_kq) * D * 2
    sel = sel_union.reshape(-1, t)
    n_q = int(sel[:, :n_vq].sum())          # selected quantized values
    n_f = int(sel[:, n_vq:].sum())          # selected fp16 values
    vals = n_q * (D * w.v_bits // 8 + (D // G) * group_bytes(w)) + n_f * D * 2
    return (keys + rep * D * 6) * w.B * w.Hkv + vals


def time_select(w, caches, q, tau: float, stream, n_rounds: int = 5, per_round: int = 40):
    """kivi_select_attn back to back over the layer replicas: us per call,
    GB/s on the algorithmic bytes and the selected fraction."""
    import torch

    from decode_attention_pack_amd import kivi
    L = len(caches)
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=q.device)
    ws = kivi.select_workspace(caches[0], w.Hq)
    nsel = torch.empty((w.B, w.Hq), dtype=torch.int32, device=q.device)
    t = caches[0].n_tokens
    words = (t + 31) // 32
    smask = torch.zeros((w.B, w.Hq, words), dtype=torch.int32, device=q.device)
    kivi.kivi_select_attn(caches[0], q, tau, out=out, n_selected=nsel, sel_mask=smask,
                          workspace=ws, stream=stream)
    torch.cuda.synchronize()
    bits = np.unpackbits(smask.cpu().numpy().view(np.uint32).view(np.uint8), axis=-1,
                         bitorder="little")[..., :t].astype(bool)
    union = bits.reshape(w.B, w.Hkv, w.Hq // w.Hkv, t).any(axis=2)
    n_bytes = select_bytes(w, t, union)
    calls = [kivi.bind_select_attn(c, q, tau, out, ws, stream=stream) for c in caches]
    for i in range(2 * L):
        calls[i % L]()
    torch.cuda.synchronize()
    ms = []
    for r in range(n_rounds):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for j in range(per_round):
            calls[(r * per_round + j) % L]()
        e1.record(stream)
        ms.append((e0, e1))
    torch.cuda.synchronize()
    us = [e0.elapsed_time(e1) * 1e3 / per_round for e0, e1 in ms]
    mean = float(np.mean(us))
    return {"call": "kivi_select_attn", "tau": tau, "context": t,
            "us": round(mean, 2),
            "us_rounds_min_p50_max": [round(float(np.percentile(us, p)), 2) for p in (0, 50, 100)],
            "GBps": round(n_bytes / mean / 1e3, 1),
            "bytes_per_call": n_bytes,
            "selected_fraction_mean": round(float(bits.sum()) / bits.size, 4),
            "values_read_fraction": round(float(union.sum()) / union.size, 4)}


def host_cpu():
    """CPU model and the cores this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return model, cores


def cpu_baseline(w, inp, lengths, budget_s: float = 10.0):
    """Time the CPU oracle on (batch, KV head) slabs of the workload (row b
    prefilled with lengths[b] tokens): first on one thread until ~budget_s of
    work, then the same slabs on every host core (one slab per thread; the
    oracle's C code runs outside the GIL)."""
    import concurrent.futures

    import oracle
    rep = w.Hq // w.Hkv
    t = max(lengths) + 1
    q = inp["q_steps"][0]
    model, n_cores = host_cpu()

    def build(bh):
        b, h = bh
        o = oracle.Cache(1, 1, w.D, w.k_bits, w.v_bits, w.G, w.R, w.capacity,
                         scale_fp16=w.scale_fp16)
        T = lengths[b]
        o.append(np.ascontiguousarray(inp["k0"][b:b + 1, h:h + 1, :T]).view(np.uint16),
                 np.ascontiguousarray(inp["v0"][b:b + 1, h:h + 1, :T]).view(np.uint16))
        o.append(inp["k_steps"][0][b:b + 1, h:h + 1].view(np.uint16),
                 inp["v_steps"][0][b:b + 1, h:h + 1].view(np.uint16))
        return o

    def attend(bh, o):
        b, h = bh
        o.decode_attn(np.ascontiguousarray(q[b:b + 1, h * rep:(h + 1) * rep]).view(np.uint16))

    def slab_bytes(bh):
        return attn_bytes(w, [lengths[bh[0]] + 1]) / w.Hkv

    slabs = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    done, spent, n_bytes = [], 0.0, 0.0
    for bh in slabs:
        o = build(bh)
        t0 = time.perf_counter()
        attend(bh, o)
        spent += time.perf_counter() - t0
        done.append((bh, o))
        n_bytes += slab_bytes(bh)
        if spent >= budget_s:
            break
    ctx = (f"context {t}" if min(lengths) == max(lengths) else
           f"contexts {min(lengths) + 1}..{t} by row")
    res = {"value": round(n_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": 1,
           "kind": "oracle",
           "sample": f"{len(done)} of {w.B * w.Hkv} (batch, kv-head) slabs of {w.name}, one decode "
                     f"step at {ctx} ({rep} query heads each), single-threaded C oracle, "
                     f"{spent:.1f} s",
           "host_cpu": model, "host_cores": n_cores}
    # the same sample on every core: each thread runs whole slabs
    reps = max(1, n_cores // max(1, len(done)))
    work = [bh_o for bh_o in done for _ in range(reps)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=n_cores) as ex:
        t0 = time.perf_counter()
        list(ex.map(lambda x: attend(*x), work))
        wall = time.perf_counter() - t0
    res["all_cores"] = {"value": round(n_bytes * reps / wall / 1e9, 4), "unit": "GB/s",
                        "cores": n_cores,
                        "sample": f"{len(work)} slab attention calls ({len(done)} slabs x {reps}) "
                                  f"on {n_cores} threads, {wall:.1f} s wall"}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", type=int, default=4,
                    help="1-5: the workloads of synth.WORKLOADS; 6: the ragged batch")
    ap.add_argument("--layers", type=int, default=0, help="layer replicas (0 = auto, >= 1 GiB)")
    ap.add_argument("--path", type=int, default=0, help="0 auto, 1 scalar kernel, 2 matrix kernel")
    ap.add_argument("--tokens-per-split", type=int, default=0,
                    help="split size of the attention call (0 = the library's automatic plan)")
    ap.add_argument("--unfused", action="store_true",
                    help="time a step as kivi_append + kivi_decode_attn instead of kivi_decode_step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-pack", action="store_true", help="skip the full-prefill pack pass")
    ap.add_argument("--select", type=float, default=0.0,
                    help="also time kivi_select_attn (token selection by attention mass tau, "
                         "then attention over the selected tokens) on the same replicas")
    ap.add_argument("--scale-fp16", action="store_true",
                    help="the fp16-scale layout: scales stored as binary16")
    ap.add_argument("--kv-bits", type=int, default=0, choices=(0, 2, 4),
                    help="code width of keys and values (0 = the workload's own); 4 on a 2-bit "
                         "workload is its KIVI-4 variant, named with a -kivi4 suffix")
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

    ragged = args.workload == synth.RAGGED.index
    w = synth.RAGGED if ragged else synth.WORKLOADS[args.workload]
    w = w.replace(scale_fp16=args.scale_fp16)
    if args.kv_bits and (args.kv_bits, args.kv_bits) != (w.k_bits, w.v_bits):
        w = w.replace(k_bits=args.kv_bits, v_bits=args.kv_bits,
                      name=w.name + f"-kivi{args.kv_bits}")
    inp = synth.make_inputs(w.replace(steps=1))
    # prefill length of each batch row (a ragged batch: its own per row)
    lengths = ([int(x) for x in synth.ragged_lengths(w.B, 1024, w.T0)] if ragged
               else [w.T0] * w.B)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    # Each replica takes the workload's decode steps (contexts T0 + 1 ..
    # T0 + steps), then its token count is set back to T0: the cache then
    # holds T0 tokens again as far as every kernel is concerned (the data the
    # steps wrote stays, and the next steps overwrite it).
    n_cyc = w.steps
    m = w.R * 128 // math.gcd(w.R, 128)
    cap = -(-(w.T0 + n_cyc) // m) * m
    probe = kivi.Cache(w.B, w.Hkv, w.D, w.k_bits, w.v_bits, w.G, w.R, cap,
                       scale_fp16=w.scale_fp16)
    footprint = sum(a.numel() * a.element_size() for a in probe.arrays.values())
    del probe
    L = args.layers or max(2, math.ceil((1 << 30) / footprint))
    print(f"# {w.name}: footprint {footprint / 1e6:.1f} MB/layer, {L} layers, capacity {cap}",
          file=sys.stderr, flush=True)

    base = kivi.Cache(w.B, w.Hkv, w.D, w.k_bits, w.v_bits, w.G, w.R, cap, ragged=ragged,
                      scale_fp16=w.scale_fp16)
    if ragged:
        # each row prefilled alone, as a request entering a serving batch
        for b, T in enumerate(lengths):
            kivi.kivi_append_row(base, b, torch.from_numpy(inp["k0"][b, :, :T]).to(dev),
                                 torch.from_numpy(inp["v0"][b, :, :T]).to(dev))
    else:
        kivi.kivi_append(base, torch.from_numpy(inp["k0"]).to(dev),
                         torch.from_numpy(inp["v0"]).to(dev))
    torch.cuda.synchronize()
    caches = [base]
    for _ in range(L - 1):
        arrays = {n: a.clone() for n, a in base.arrays.items()}
        c = kivi.Cache(w.B, w.Hkv, w.D, w.k_bits, w.v_bits, w.G, w.R, cap, arrays=arrays,
                       ragged=ragged, scale_fp16=w.scale_fp16)
        if ragged:
            c.set_row_tokens(lengths)
        else:
            c.c.n_tokens = base.n_tokens
        caches.append(c)

    def rewind(c):
        if ragged:
            c.set_row_tokens(lengths)
        else:
            c.c.n_tokens = w.T0

    def offset(c):
        """Decode steps the replica has taken since its prefill."""
        return (c.row_tokens[0] if ragged else c.n_tokens) - lengths[0]

    # algorithmic bytes by steps taken: attention over prefill + k tokens,
    # and the append of token prefill + k
    attn_by_off = [attn_bytes(w, [T + k for T in lengths]) for k in range(n_cyc + 1)]
    app_by_off = [append_bytes(w, [T + k for T in lengths]) for k in range(n_cyc + 1)]
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
    contexts = set()

    def step(i):
        c = caches[i % L]
        if offset(c) >= n_cyc:
            rewind(c)
        k = offset(c)
        contexts.add(lengths[0] + k + 1)
        if fused:
            fused_steps[i % L]()
        else:
            appends[i % L]()
            decodes[i % L]()
        return attn_by_off[k + 1], app_by_off[k]

    # warm-up: the requested steps, and at least ~1 s of back-to-back steps
    # (with fewer, the clocks have not settled and the first timed calls run
    # slower)
    t_w = time.perf_counter()
    i = 0
    while i < args.warmup or time.perf_counter() - t_w < 1.0:
        for _ in range(50):
            step(i)
            i += 1
        torch.cuda.synchronize()
    i0 = i
    contexts.clear()

    # timed region 1: K whole steps (append + attention), events at its ends only
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    a_bytes = p_bytes = 0
    torch.cuda.synchronize()
    start.record(stream)
    for j in range(args.steps):
        ab, pb = step(i0 + j)
        a_bytes += ab
        p_bytes += pb
    stop.record(stream)
    torch.cuda.synchronize()
    step_contexts = sorted(contexts)
    # timed region 2: the attention launch alone, back to back over the same
    # replicas (no append in between), in 5 rounds of 50 calls whatever K is,
    # so that the spread across rounds is reported
    n_rounds, per_round = 5, 50
    a2_bytes = 0
    rounds_ms = []
    attn_contexts = set()
    for r in range(n_rounds):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for j in range(per_round):
            c = caches[(r * per_round + j) % L]
            decodes[(r * per_round + j) % L]()
            a2_bytes += attn_by_off[offset(c)]
            attn_contexts.add(lengths[0] + offset(c))
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
        "dtype": "fp16",
        "dtype_detail": ("2/4-bit integer codes; fp16 x fp16 matrix products whose fp32 "
                         "scale-folded operands are split into fp16 high and low parts; fp32 "
                         "accumulation, softmax and output"),
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.D, "context": max(lengths) + 1, "decode_steps": n_cyc,
                   **({"row_contexts": [T + 1 for T in lengths]} if ragged else {}),
                   "k_bits": w.k_bits, "v_bits": w.v_bits,
                   "group": w.G, "residual": w.R, "layers_rotated": L,
                   "storage": "128-token records: packed codes, "
                              + ("fp16" if w.scale_fp16 else "fp32")
                              + " scales, fp16 zero points; fp16 window; fp16 q"},
        "step_call": "kivi_decode_step" if fused else "kivi_append + kivi_decode_attn",
        "step_contexts_min_max": [step_contexts[0], step_contexts[-1]],
        "us_per_step": round(ms_step * 1e3, 2),
        "attn_us": round(attn_avg_ms * 1e3, 2),
        "attn_us_rounds_min_p50_max": [round(float(np.percentile(attn_ms, p)) * 1e3, 2)
                                       for p in (0, 50, 100)],
        "attn_contexts_min_max": [min(attn_contexts), max(attn_contexts)],
        "attn_pct_of_peak": round(100 * attn_gbps / HBM_PEAK_GBPS, 1),
        "roofline": {"bound": "hbm", "achieved": round(attn_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(attn_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(w.name + ("-fp16-scales" if w.scale_fp16
                                                           else "")),
                     "kernel": "kivi_decode_attn launch (split kernel + combine)",
                     "bytes_per_launch": a2_bytes // (n_rounds * per_round)},
    }
    if args.select > 0.0 and not ragged:
        line["select"] = time_select(w, caches, q, args.select, stream)
    if not args.no_pack and not ragged:
        del caches, base, appends, decodes, fused_steps
        torch.cuda.empty_cache()
        line["pack_full_prefill"] = time_pack(w, inp, dev, stream)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp, lengths)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
