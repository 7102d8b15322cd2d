"""Batch-1 decode through the 92-layer stack (96 resident experts per layer,
155 GB of MXFP4 weights on the device), with the RMS rescale between layers.

The token step runs exactly as the benchmark times it: layer 0 through
moe_decode_layer_mxfp4, layers 1..91 through moe_decode_layer_rms_mxfp4 (the
RMS rescale inside the gate/up launch, output written in place), once
eagerly with every layer's results copied out, then captured in a HIP graph
whose replays must give the eager bits.  Each layer's output is checked
against the oracle run on the GPU's own input to that layer (bf16, so both
sides see identical bytes), and each in-launch rescale against the oracle's
rescale of the GPU's previous output.

Free-running chains cannot be compared at the output bar: a random stack of
this depth amplifies a one-ulp bf16 difference about 1.4x per layer until
the chains are unrelated (about layer 22).  So the GPU's chain is instead
held to the oracle chain's own sensitivity: at every layer its distance from
the oracle's chain may not exceed four times the distance between the
oracle's chain and the oracle's chain with one bf16 ulp changed in one
element of the layer-0 input (plus the output bar)."""
import numpy as np
import pytest
import torch

import oracle
from mxfp4_routed_expert_02_amd import ExpertPool, rms_rescale_bf16, synth
from mxfp4_routed_expert_02_amd.layer import RoutedExpertLayer
from tests.gpu_common import REL_L2, assert_close, say

pytestmark = pytest.mark.gpu
NTH = 16
EPS = 1e-6


def _host_pool(wl, layer, ids):
    sb = synth.slab_bytes(wl.H, wl.I)
    slabs = np.zeros((wl.E, sb), np.uint8)
    for e in sorted(set(int(e) for e in ids.reshape(-1))):
        synth.expert_slabs(0, wl.pool, layer, e, 1, wl.H, wl.I, out=slabs[e:e + 1])
    return oracle.Pool(slabs, wl.H, wl.I)


def _token_step(L, x0, logits_d, pools, out, xbuf, record=None):
    """One token through the stack exactly as the benchmark runs it: layer 0
    from the token's bf16 input (moe_decode_layer_mxfp4), layers 1..91 from
    the previous layer's fp32 output with the RMS rescale inside the gate/up
    launch, writing in place (moe_decode_layer_rms_mxfp4), then the rescale
    that would feed the next token.  `record(l, ...)` copies a layer's
    results out (eager runs only)."""
    n = len(pools)
    L(x0, logits_d[0], pools[0], out)
    if record:
        record(0, None)
    for l in range(1, n):
        L.step_rms(out, logits_d[l], pools[l], out, xbuf[l & 1], EPS)
        if record:
            record(l, xbuf[l & 1])
    rms_rescale_bf16(out, EPS, xbuf[n & 1])


def test_stack92_decode():
    wl = synth.WORKLOADS["stack92"]
    dev = torch.device("cuda", 0)
    say(f"generating {wl.layers} pools of {wl.E} experts on the device "
        f"({wl.layers * wl.E * synth.slab_bytes(wl.H, wl.I) / 1e9:.1f} GB)")
    pools = [ExpertPool(synth.device_pool_slabs(0, wl.pool, l, wl.E, wl.H, wl.I, dev), wl.H, wl.I)
             for l in range(wl.layers)]
    torch.cuda.synchronize()
    L = RoutedExpertLayer(wl.E, wl.H, wl.I, wl.k, 1, dev)
    x0 = synth.activations_bf16(0, wl)
    xd = torch.from_numpy(x0.view(np.int16)).to(dev).view(torch.bfloat16)
    logits = [synth.router_logits(0, wl, layer=l) for l in range(wl.layers)]
    logits_d = torch.stack([torch.from_numpy(a) for a in logits]).to(dev)
    out = torch.empty((1, wl.H), dtype=torch.float32, device=dev)
    xbuf = torch.empty((2, 1, wl.H), dtype=torch.bfloat16, device=dev)
    xs, ids, outs = [x0], [], []

    def record(l, x_used):
        torch.cuda.synchronize()
        if x_used is not None:
            xs.append(x_used.view(torch.int16).cpu().numpy().view(np.uint16).copy())
        ids.append(L.ids[:1].cpu().numpy().copy())
        outs.append(out.cpu().numpy().copy())

    say("  eager token step (the benchmark's launches), every layer recorded")
    _token_step(L, xd, logits_d, pools, out, xbuf, record)
    torch.cuda.synchronize()
    xs.append(xbuf[wl.layers & 1].view(torch.int16).cpu().numpy().view(np.uint16).copy())
    final_out, final_x = out.clone(), xbuf[wl.layers & 1].clone()

    say("  the same token step captured in a HIP graph, replayed")
    stream = torch.cuda.Stream(dev)
    stream.wait_stream(torch.cuda.current_stream(dev))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            _token_step(L, xd, logits_d, pools, out, xbuf)
    torch.cuda.current_stream(dev).wait_stream(stream)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()  # eager work between replays
        xbuf.zero_()
        L.ids.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), final_out.view(torch.int32)), f"replay {rep}: layer-91 out"
        assert torch.equal(xbuf[wl.layers & 1].view(torch.int16), final_x.view(torch.int16)), f"replay {rep}: x"
        assert np.array_equal(L.ids[:1].cpu().numpy(), ids[-1]), f"replay {rep}: layer-91 ids"
    del graph, pools
    torch.cuda.empty_cache()

    x_free = x0
    x_pert = x0.copy()
    x_pert[0, 0] ^= 1  # one bf16 ulp on one element of the layer-0 input
    drift, sens = [], []
    for l in range(wl.layers):
        ref_ids, _ = oracle.route_topk(logits[l], wl.k)
        assert np.array_equal(ids[l], ref_ids), f"layer {l}: top-k ids differ"
        hp = _host_pool(wl, l, ref_ids)
        ref = oracle.layer(xs[l], logits[l], wl.k, hp, nthreads=NTH)["out"]
        assert_close(outs[l], ref, f"layer {l} out (GPU input)")
        # the rescale that fed layer l+1 (inside its gate/up launch), and the final one
        ref_x = oracle.rms_rescale_bf16(outs[l], EPS)
        diff = np.abs(ref_x.astype(np.int32) - xs[l + 1].astype(np.int32))
        assert diff.max() <= 1, f"layer {l}: rescale more than one bf16 ulp off"
        # the oracle's own chain
        free_out = oracle.layer(x_free, logits[l], wl.k, hp, nthreads=NTH)["out"]
        x_free = oracle.rms_rescale_bf16(free_out, EPS)
        pert_out = oracle.layer(x_pert, logits[l], wl.k, hp, nthreads=NTH)["out"]
        x_pert = oracle.rms_rescale_bf16(pert_out, EPS)
        drift.append(float(np.linalg.norm(outs[l] - free_out) / np.linalg.norm(free_out)))
        sens.append(float(np.linalg.norm(pert_out - free_out) / np.linalg.norm(free_out)))
        if l % 10 == 9 or l == wl.layers - 1:
            say(f"  checked layers 0..{l}")
    say("  GPU chain vs oracle chain, rel-L2 by layer: " + " ".join(f"{d:.1e}" for d in drift))
    say("  oracle chain vs itself with one ulp changed in x0: " + " ".join(f"{d:.1e}" for d in sens))
    assert drift[0] <= REL_L2, "layer 0 (identical inputs) beyond the bar"
    for l in range(wl.layers):
        assert drift[l] <= 4 * sens[l] + REL_L2, f"layer {l}: chain drift {drift[l]:.2e} vs sensitivity {sens[l]:.2e}"
