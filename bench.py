"""Throughput of the routed-expert MXFP4 layer on one MI355X.

A step is one pass of the whole layer (route top-k -> group rows -> fused
MXFP4 dequant + SwiGLU expert FFN -> weighted combine) over one batch of
synthetic input already resident in HBM.  The default workload is batch-1
decode on one layer of 896 resident experts (hidden 7168, intermediate
1536, top-16): every step reads the 16 routed experts' MXFP4 weights,
16 x 17,547,264 bytes.  Steps rotate over 64 seeded (x, logits) variants so
the routed experts differ from step to step and the 256 MB last-level cache
cannot serve them.

Every timed region is queued behind a short spin kernel, so the host's
latency to its first launch stays out of the figure.

Prints one JSON line: value = routed-expert weight GB/s of the whole layer
(its own fraction of the HBM peak in layer_roofline), the roofline of the
expert-FFN call (HIP events on the launch stream), and the CPU oracle's rate
on the host cores as a reported baseline (threads used, the host's core
count and a single-thread rate beside it).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
FP4_PEAK_TFLOPS = 10100.0  # MI355X dense MXFP4 MFMA
FP32_PEAK_TFLOPS = 157.3  # MI355X fp32 (vector and MFMA)
METRIC = "MoE MXFP4 expert layer: decode weight GB/s + prefill TFLOP/s, % of roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--variants", type=int, default=64)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--clock-warmup-ms", type=float, default=60.0,
                   help="untimed sustained load before the warm-up steps (the GPU's clocks rise over the first "
                        "~20 ms of continuous work; 0 = none)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="bounded oracle sample (0 = skip)")
    p.add_argument("--cpu-threads", type=int, default=16)
    p.add_argument("--prefill-reps", type=int, default=20, help="prefill512 / dense side measures (0 = skip)")
    p.add_argument("--side-reps", type=int, default=100, help="verify8 side measure (0 = skip)")
    p.add_argument("--stack-reps", type=int, default=20, help="92-layer stack side measure (0 = skip)")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="only run a plain device copy of this many MiB 5 times (calibrates HBM byte counters)")
    return p.parse_args()


def profiled_traffic(what="ffn_call"):
    """HBM bytes per expert-FFN call (what="ffn_call") or per decode layer
    (what="layer") from the committed counter summary, or None when the
    kernel sources changed since those counters were taken."""
    import re

    path = os.path.join(ROOT, "profiles", "decode896_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"sources_sha256: ([0-9a-f]{64})", text)
    pattern = r"ffn_call_traffic_bytes: (\d+)" if what == "ffn_call" else r"Per decode layer: (\d+) bytes"
    m_bytes = re.search(pattern, text)
    if not (m_sha and m_bytes):
        return None
    return int(m_bytes.group(1)) if ffn_sources_sha256() == m_sha.group(1) else None


def ffn_sources_sha256():
    """Fingerprint of the sources of the decode expert-FFN kernels (the
    register GEMVs and the device helpers they include)."""
    import hashlib

    h = hashlib.sha256()
    for name in ("ffn_gemv.hip", "moe_internal.h"):
        f = os.path.join(ROOT, "mxfp4_routed_expert_02_amd", "csrc", name)
        h.update(name.encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()


def copy_probe(mib):
    """A plain copy kernel of known size: FETCH_SIZE / WRITE_SIZE read for it
    give the counters' scale against true bytes."""
    import torch

    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy probe: 5 copies of {mib} MiB ({n * 4} bytes read and written each)")


def stream_read_gbs(dev, gib=4, reps=5):
    """The box's achievable read bandwidth: a plain streaming-read kernel
    (non-temporal loads, 512 blocks) over a `gib` GiB buffer (synth library),
    median of `reps` event-timed runs."""
    import numpy as np
    import torch

    from mxfp4_routed_expert_02_amd import synth

    L = synth.gpu_lib()
    nbytes = gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    blocks = 512
    out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def run(i):
        rc = L.synth_stream_read(buf.data_ptr(), nbytes, out.data_ptr(), blocks, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"synth_stream_read failed ({rc})")

    run(0)
    each = per_call_us(run, reps, stream)
    del buf
    gbs = nbytes / (float(np.median(each)) * 1e-6) / 1e9
    log(f"streaming-read probe: {gbs:.0f} GB/s over {gib} GiB")
    return gbs


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world})", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib)
        return

    import numpy as np
    import torch

    from mxfp4_routed_expert_02_amd import ExpertPool, synth, expert_ffn_mxfp4
    from mxfp4_routed_expert_02_amd.layer import RoutedExpertLayer

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    wl = synth.WORKLOADS["decode896"]
    V = args.variants
    t0 = time.time()
    slabs = synth.device_pool_slabs(args.seed, wl.pool, 0, wl.E, wl.H, wl.I, dev)
    torch.cuda.synchronize()
    pool = ExpertPool(slabs, wl.H, wl.I)
    log(f"pool: {wl.E} experts, {slabs.numel() / 1e9:.2f} GB resident ({time.time() - t0:.1f} s)")
    xs = torch.stack([torch.from_numpy(synth.activations_bf16(args.seed, wl, variant=v).view(np.int16))
                      for v in range(V)]).to(dev).view(torch.bfloat16)  # [V, 1, H]
    ls = torch.stack([torch.from_numpy(synth.router_logits(args.seed, wl, variant=v)) for v in range(V)]).to(dev)
    layer = RoutedExpertLayer(wl.E, wl.H, wl.I, wl.k, wl.T, dev)
    out = torch.empty((wl.T, wl.H), dtype=torch.float32, device=dev)
    slab_b = synth.slab_bytes(wl.H, wl.I)
    weight_bytes = wl.T * wl.k * slab_b  # top-16 distinct experts per token, each read once
    ffn_bytes = weight_bytes + wl.T * wl.H * 2 + wl.R * wl.H * 4  # + x read + y_rows written

    def step(i):
        layer(xs[i % V], ls[i % V], pool, out)

    # sustained-load warm-up (untimed): the same layer steps until clock_warmup_ms
    # of GPU time have passed, so the timed steps see the clocks a continuously
    # busy GPU runs at (from cold, a layer takes about 10% longer for the first
    # ~20 ms of work); then the W warm-up steps of the contract
    warm_ms, warm_steps = 0.0, 0
    while warm_ms < args.clock_warmup_ms:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(50):
            step(warm_steps)
            warm_steps += 1
        b.record()
        torch.cuda.synchronize()
        warm_ms += a.elapsed_time(b)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    sleep_cycles = sleep_calibration(stream)
    # timed region: K whole-layer steps
    ms_step = timed_eager(lambda: [step(i) for i in range(args.steps)], stream, sleep_cycles) / args.steps
    value = weight_bytes / (ms_step * 1e-3) / 1e9
    log(f"layer: {ms_step * 1e3:.1f} us/step, {value:.0f} GB/s")

    # expert-FFN call alone, events on its launch stream around every call
    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    groupings = []
    for v in range(V):
        _, _, g = layer.route(ls[v])
        groupings.append(tuple(t.clone() for t in (g.expert_offsets, g.sorted_rows, g.row_pos, g.active)))
    from mxfp4_routed_expert_02_amd import Grouping

    gobjs = [Grouping(*g) for g in groupings]
    y_rows = torch.empty((wl.R, wl.H), dtype=torch.float32, device=dev)
    for i in range(args.warmup):
        expert_ffn_mxfp4(xs[i % V], wl.k, pool, gobjs[i % V], layer.workspace, y_rows)
    torch.cuda.synchronize()
    # average launch duration: K back-to-back calls between one event pair,
    # queued behind a spin kernel so the host's launch latency stays outside
    ffn_us = timed_eager(lambda: [expert_ffn_mxfp4(xs[i % V], wl.k, pool, gobjs[i % V], layer.workspace, y_rows)
                                  for i in range(K)], stream, sleep_cycles) * 1e3 / K
    # spread of single calls (each bracketed by its own events, whose records add some time)
    for i in range(K):
        a, b = evs[i]
        a.record(stream)
        expert_ffn_mxfp4(xs[i % V], wl.k, pool, gobjs[i % V], layer.workspace, y_rows)
        b.record(stream)
    torch.cuda.synchronize()
    ffn_each = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
    achieved = ffn_bytes / (ffn_us * 1e-6) / 1e9
    stream_gbs = stream_read_gbs(dev)  # outside the timed regions
    log(f"expert FFN call: {ffn_us:.1f} us, {achieved:.0f} GB/s of {ffn_bytes} algorithmic bytes")
    layer_each = per_call_us(lambda i: step(i), K, stream)

    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp4", "data": "synthetic",
        "config": {"workload": "decode896", "experts": wl.E, "hidden": wl.H, "inter": wl.I, "topk": wl.k,
                   "tokens": wl.T, "variants": V, "weight_bytes_per_step": weight_bytes},
        "clock_warmup": {"ms": round(warm_ms, 1), "steps": warm_steps,
                         "what": "untimed layer steps before the warm-up steps, until the GPU runs at its sustained clock"},
        "layer_roofline": {"bound": "hbm", "what": "whole decode layer (value / peak)", "achieved": round(value, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(value / HBM_PEAK_GBS, 4),
                           "algorithmic_bytes": weight_bytes, "us_per_step": round(ms_step * 1e3, 2),
                           "traffic": profiled_traffic("layer")},
        "roofline": {"bound": "hbm", "kernel": "moe_expert_ffn_mxfp4 call", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": profiled_traffic(), "launch_us": round(ffn_us, 2),
                     "algorithmic_bytes": ffn_bytes, "achievable_read_gbs": round(stream_gbs, 1),
                     "frac_achievable": round(achieved / stream_gbs, 4)},
        "decode896_us": {"ffn_call": pct(ffn_each), "layer": pct(layer_each),
                         "ffn_call_gbs_at_median": round(ffn_bytes / (np.median(ffn_each) * 1e-6) / 1e9, 1)},
    }

    if args.side_reps > 0:
        res["verify8"] = verify_side(dev, pool, args.seed, args.side_reps)
    if args.prefill_reps > 0:
        res["prefill512"] = prefill_side(dev, pool, args.seed, args.prefill_reps, "prefill512")
        res["prefill_dense"] = prefill_side(dev, pool, args.seed, args.prefill_reps, "prefill_dense")
        res["prefill4096"] = prefill_side(dev, pool, args.seed, max(2, args.prefill_reps // 4), "prefill4096")
    if args.side_reps > 0:
        res["router"] = router_side(dev, args.seed, args.side_reps)
        res["decode896_tp8_share"] = tp8_side(dev, args.seed, args.side_reps)
    if args.stack_reps > 0:
        res["stack92"] = stack_side(dev, args.seed, args.stack_reps)

    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(args, wl)
    print(json.dumps(res), flush=True)


def sleep_calibration(stream):
    """Device-clock cycles of torch's spin kernel that keep the GPU busy for
    about 2 ms (0 if the build has no spin kernel)."""
    import torch

    if not hasattr(torch.cuda, "_sleep"):
        return 0
    torch.cuda._sleep(1000)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    torch.cuda._sleep(200000)
    b.record(stream)
    torch.cuda.synchronize()
    ms = max(a.elapsed_time(b), 1e-3)
    return int(min(2.0 / ms, 100.0) * 200000)


def prime(stream, cycles):
    """Queue a spin kernel, so the launches that follow are queued before
    the GPU reaches them."""
    import torch

    if cycles > 0:
        torch.cuda._sleep(cycles)


def timed_eager(fn, stream, cycles):
    """ms between two events around fn()'s launches, queued behind a spin
    kernel so the first launch's host latency is not in the figure."""
    import torch

    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    prime(stream, cycles)
    a.record(stream)
    fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def per_call_us(fn, reps, stream):
    """Durations (us) of reps calls of fn(i), one event pair around each."""
    import numpy as np
    import torch

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        evs[i][0].record(stream)
        fn(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in evs]) * 1e3


def pct(v):
    import numpy as np

    return {"p10": round(float(np.percentile(v, 10)), 2), "median": round(float(np.median(v)), 2),
            "p90": round(float(np.percentile(v, 90)), 2)}


def verify_side(dev, pool, seed, reps):
    """8-token speculative-verify batch on the same pool: weight GB/s over
    the unique experts the batch reads."""
    import numpy as np
    import torch

    from mxfp4_routed_expert_02_amd import synth
    from mxfp4_routed_expert_02_amd.layer import RoutedExpertLayer

    wl = synth.WORKLOADS["verify8"]
    V = 16  # rotate over variants like decode, against the last-level cache
    xs = [torch.from_numpy(synth.activations_bf16(seed, wl, variant=v).view(np.int16)).to(dev).view(torch.bfloat16)
          for v in range(V)]
    ls = [torch.from_numpy(synth.router_logits(seed, wl, variant=v)).to(dev) for v in range(V)]
    layer = RoutedExpertLayer(wl.E, wl.H, wl.I, wl.k, wl.T, dev)
    uniq = []
    for v in range(V):
        layer(xs[v], ls[v], pool)
        uniq.append(int(layer.grp.active[0].item()))
    stream = torch.cuda.current_stream(dev)
    each = per_call_us(lambda i: layer(xs[i % V], ls[i % V], pool), reps, stream)
    per_call_bytes = np.array([uniq[i % V] for i in range(reps)]) * synth.slab_bytes(wl.H, wl.I)
    gbs = float(per_call_bytes.sum() / (each.sum() * 1e-6) / 1e9)
    log(f"verify8: {np.median(each):.1f} us/layer (median), {gbs:.0f} GB/s over {np.mean(uniq):.1f} unique experts")
    return {"us_per_layer": pct(each), "weight_gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "unique_experts_mean": round(float(np.mean(uniq)), 2), "variants": V}


def tp8_side(dev, seed, reps):
    """One GPU's share of decode896 under an 8-way split of every expert's I
    (the layer at I = 192): layer time and weight GB/s of that share."""
    import numpy as np
    import torch

    from mxfp4_routed_expert_02_amd import ExpertPool, synth
    from mxfp4_routed_expert_02_amd.layer import RoutedExpertLayer

    wl = synth.WORKLOADS["decode896_tp8"]
    pool = ExpertPool(synth.device_pool_slabs(seed, wl.pool, 0, wl.E, wl.H, wl.I, dev), wl.H, wl.I)
    V = 64
    xs = [torch.from_numpy(synth.activations_bf16(seed, wl, variant=v).view(np.int16)).to(dev).view(torch.bfloat16)
          for v in range(V)]
    ls = [torch.from_numpy(synth.router_logits(seed, wl, variant=v)).to(dev) for v in range(V)]
    layer = RoutedExpertLayer(wl.E, wl.H, wl.I, wl.k, wl.T, dev)
    for v in range(V):
        layer(xs[v], ls[v], pool)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(reps):
        layer(xs[i % V], ls[i % V], pool)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    share_bytes = wl.k * synth.slab_bytes(wl.H, wl.I)
    gbs = share_bytes / (us * 1e-6) / 1e9
    log(f"decode896 tp8 share (I {wl.I}): {us:.1f} us/layer, {gbs:.0f} GB/s of its {share_bytes} weight bytes")
    del pool
    torch.cuda.empty_cache()
    return {"us_per_layer": round(us, 2), "weight_bytes": share_bytes, "weight_gbs": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def router_side(dev, seed, reps):
    """The router projection before the path (x . W_r^T, fp32 weights
    896 x 7168): one token streams W_r (25.7 MB, HBM-bound); 512 tokens are
    2*T*E*H flops against the fp32 peak."""
    import numpy as np
    import torch

    from mxfp4_routed_expert_02_amd import router_logits, synth

    out = {}
    for name, T in (("decode", 1), ("prefill512", 512)):
        wl = synth.Workload("router", E=896, H=7168, I=1536, k=16, T=T, sub=8)
        V = 4  # rotating weight matrices (103 MB) so the last-level cache does not serve W_r
        wrs = [torch.from_numpy(synth.router_weights(seed, wl, layer=v)).to(dev) for v in range(V)]
        x = torch.from_numpy(synth.activations_bf16(seed, wl).view(np.int16)).to(dev).view(torch.bfloat16)
        logits = torch.empty((T, wl.E), dtype=torch.float32, device=dev)
        for v in range(V):
            router_logits(x, wrs[v], logits)
        stream = torch.cuda.current_stream(dev)
        each = per_call_us(lambda i: router_logits(x, wrs[i % V], logits), reps, stream)
        us = float(np.median(each))
        wbytes = wl.E * wl.H * 4
        flops = 2.0 * T * wl.E * wl.H
        out[name] = {"us": pct(each), "weight_gbs": round(wbytes / (us * 1e-6) / 1e9, 1),
                     "tflops": round(flops / (us * 1e-6) / 1e12, 2),
                     "frac_hbm_peak": round(wbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "frac_fp32_peak": round(flops / (us * 1e-6) / 1e12 / FP32_PEAK_TFLOPS, 4)}
        log(f"router {name}: {us:.1f} us (median), {out[name]['weight_gbs']} GB/s of W_r, "
            f"{out[name]['tflops']} TFLOP/s")
    return out


def prefill_side(dev, pool, seed, reps, name):
    """512-token expert-major prefill on the same pool: algorithmic TFLOP/s
    (2 * R * 3 * H * I per layer) against the FP4 peak and the binding roofline."""
    import numpy as np
    import torch

    from mxfp4_routed_expert_02_amd import synth
    from mxfp4_routed_expert_02_amd.layer import RoutedExpertLayer

    wl = synth.WORKLOADS[name]
    x = torch.from_numpy(synth.activations_bf16(seed, wl).view(np.int16)).to(dev).view(torch.bfloat16)
    logits = torch.from_numpy(synth.router_logits(seed, wl)).to(dev)
    layer = RoutedExpertLayer(wl.E, wl.H, wl.I, wl.k, wl.T, dev)
    for _ in range(2):
        layer(x, logits, pool)
    torch.cuda.synchronize()
    offs = layer.grp.expert_offsets.cpu().numpy()
    touched = int((np.diff(offs) > 0).sum())
    stream = torch.cuda.current_stream(dev)
    each = per_call_us(lambda i: layer(x, logits, pool), reps, stream)
    ms = float(np.median(each)) * 1e-3
    flops = 2.0 * wl.R * 3 * wl.H * wl.I
    tflops = flops / (ms * 1e-3) / 1e12
    bytes_touched = touched * synth.slab_bytes(wl.H, wl.I)
    floor_ms = max(bytes_touched / (HBM_PEAK_GBS * 1e9), flops / (FP4_PEAK_TFLOPS * 1e12)) * 1e3
    log(f"{name}: {ms:.3f} ms/layer (median), {tflops:.1f} TFLOP/s, {touched} experts touched")
    return {"ms_per_layer": round(ms, 4), "us_per_layer": pct(each), "tflops": round(tflops, 2),
            "frac_fp4_peak": round(tflops / FP4_PEAK_TFLOPS, 4), "experts_touched": touched,
            "binding_floor_ms": round(floor_ms, 4), "frac_binding_roofline": round(floor_ms / ms, 4)}


def stack_side(dev, seed, reps):
    """Batch-1 decode through the 92-layer stack (96 experts per layer, 155 GB
    resident), RMS rescale between layers; the token step (92 x 2 launches:
    rescale + top-k + gate/up, then down + combine; one final rescale) is
    captured once in a HIP graph and replayed."""
    import numpy as np
    import torch

    from mxfp4_routed_expert_02_amd import ExpertPool, rms_rescale_bf16, synth
    from mxfp4_routed_expert_02_amd.layer import RoutedExpertLayer

    wl = synth.WORKLOADS["stack92"]
    t0 = time.time()
    pools = [ExpertPool(synth.device_pool_slabs(seed, wl.pool, l, wl.E, wl.H, wl.I, dev), wl.H, wl.I)
             for l in range(wl.layers)]
    torch.cuda.synchronize()
    log(f"stack92: {wl.layers} pools generated on the device in {time.time() - t0:.1f} s")
    layer = RoutedExpertLayer(wl.E, wl.H, wl.I, wl.k, 1, dev)
    x0 = torch.from_numpy(synth.activations_bf16(seed, wl).view(np.int16)).to(dev).view(torch.bfloat16)
    logits = torch.stack([torch.from_numpy(synth.router_logits(seed, wl, layer=l)) for l in range(wl.layers)]).to(dev)
    xbuf = torch.empty((2, 1, wl.H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((1, wl.H), dtype=torch.float32, device=dev)

    def token():
        # layer 0 from the token's bf16 input; layers 1..91 from the previous
        # layer's output (RMS rescale inside the gate/up launch): 2 launches a
        # layer, then the rescale that would feed the next token
        layer(x0, logits[0], pools[0], out)
        for l in range(1, wl.layers):
            layer.step_rms(out, logits[l], pools[l], out, xbuf[l & 1], 1e-6)
        rms_rescale_bf16(out, 1e-6, xbuf[wl.layers & 1])

    token()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    eager = per_call_us(lambda i: token(), 3, stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        token()
    g.replay()
    torch.cuda.synchronize()
    each = per_call_us(lambda i: g.replay(), reps, stream)
    bytes_token = wl.layers * wl.k * synth.slab_bytes(wl.H, wl.I)
    ms = float(np.median(each)) * 1e-3
    gbs = bytes_token / (ms * 1e-3) / 1e9
    log(f"stack92: {ms:.3f} ms/token in a graph (median), {gbs:.0f} GB/s; eager {np.median(eager) * 1e-3:.3f} ms")
    del g, pools
    torch.cuda.empty_cache()
    return {"ms_per_token": round(ms, 4), "us_per_token": pct(each), "weight_gbs": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "weight_bytes_per_token": bytes_token,
            "eager_ms_per_token": round(float(np.median(eager)) * 1e-3, 4), "graph": True}


def cpu_baseline(args, wl):
    """The CPU oracle (as it stands) on the host cores: whole decode896 layers
    for successive variants until about --cpu-seconds have passed on
    --cpu-threads threads, then one more layer on a single thread."""
    import numpy as np

    import oracle
    from mxfp4_routed_expert_02_amd import synth

    host_cores = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = host_cores
    threads = max(1, min(args.cpu_threads, affinity))
    sb = synth.slab_bytes(wl.H, wl.I)

    def one_layer(v, nthreads):
        x = synth.activations_bf16(args.seed, wl, variant=v)
        logits = synth.router_logits(args.seed, wl, variant=v)
        ids, _ = oracle.route_topk(logits, wl.k)
        slabs = np.zeros((wl.E, sb), np.uint8)
        for e in ids.reshape(-1):
            synth.expert_slabs(args.seed, wl.pool, 0, int(e), 1, wl.H, wl.I, out=slabs[e:e + 1])
        hp = oracle.Pool(slabs, wl.H, wl.I)
        t = time.perf_counter()
        oracle.layer(x, logits, wl.k, hp, nthreads=nthreads)
        return time.perf_counter() - t

    done, t_acc = 0, 0.0
    while t_acc < args.cpu_seconds and done < args.variants:
        t_acc += one_layer(done, threads)
        done += 1
    gbs = done * wl.T * wl.k * sb / t_acc / 1e9
    t1 = one_layer(done % args.variants, 1)
    gbs1 = wl.T * wl.k * sb / t1 / 1e9
    log(f"cpu oracle: {done} decode896 layers in {t_acc:.1f} s on {threads} threads, {gbs:.3f} GB/s; "
        f"1 thread {gbs1:.4f} GB/s; host has {host_cores} cores ({affinity} in this process's affinity mask)")
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} whole decode896 layers (1 token, 16 of 896 experts each, variants 0..{done - 1}), "
                      f"{t_acc:.1f} s of oracle time on {threads} threads",
            "threads_used": threads, "host_cores": host_cores, "affinity_cpus": affinity,
            "single_thread": {"value": round(gbs1, 5), "unit": "GB/s", "threads": 1,
                              "sample": f"1 whole decode896 layer (variant {done % args.variants}), {t1:.1f} s"}}


if __name__ == "__main__":
    main()
