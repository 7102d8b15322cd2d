"""The fused one-token calls on the GPU: moe_route_group_one against the
separate moe_route_topk + moe_group_rows and against the oracle's top-k and
grouping; moe_combine_rms_bf16 against the separate moe_combine +
moe_rms_rescale_bf16 and against the oracle's combine and rescale.

Against the separate GPU calls the fused outputs must be bit for bit the
same.  The fused expert-FFN and decode-layer calls are also compared with
the oracle directly: routing bit for bit, y_rows and out at the parity bar
(the RMS variant on the GPU's own bf16 input, its rescale within one ulp).  Against the oracle: ids and grouping bit for bit, routing weights
within 1e-6; the combine within the layer's tolerance (the GPU sums with
fused multiply-adds, the oracle without), the rescale within one bf16 ulp of
the oracle's rescale of the GPU's own combine.
"""
import numpy as np
import pytest
import torch

import oracle
from mxfp4_routed_expert_02_amd import (Grouping, combine, combine_rms_bf16, group_rows, rms_rescale_bf16,
                                        route_group_one, route_topk, synth)
from tests.gpu_common import assert_close, oracle_outputs, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)

ROUTE_CASES = [  # E, k, logits kind: every register-top-k width, the fallback above 2048, ties
    (896, 16, "normal"), (96, 16, "normal"), (8, 2, "normal"), (2048, 32, "normal"), (4096, 16, "normal"),
    (896, 16, "ties"), (96, 1, "normal"), (300, 32, "ties"), (1, 1, "normal"),
]


def _logits(E, kind, seed):
    wl = synth.Workload("fused", E=E, H=32, I=32, k=1, T=1, sub=seed)
    lg = synth.router_logits(0, wl)
    if kind == "ties":
        lg = np.floor(np.abs(lg) * 2.0).astype(np.float32) % 4  # values in {0, 1, 2, 3}
    elif kind == "stride16":  # experts 0, 16, 32, ... far above the rest: the top k share one residue mod 16
        lg = lg.copy()
        lg.reshape(-1)[::16] += 10.0
    return np.ascontiguousarray(lg, dtype=np.float32)


def _grouping(E, R):
    z = lambda n: torch.empty(n, dtype=torch.int32, device=DEV)  # noqa: E731
    return Grouping(z(E + 1), z(R), z(R), z(E + 1))


@pytest.mark.parametrize("E,k,kind", ROUTE_CASES, ids=[f"E{e}_k{k}_{c}" for e, k, c in ROUTE_CASES])
def test_route_group_one(E, k, kind):
    say(f"route_group_one E={E} k={k} {kind}")
    lg = _logits(E, kind, 50 + E % 7)
    lgd = torch.from_numpy(lg).to(DEV)
    ids = torch.empty((1, k), dtype=torch.int32, device=DEV)
    w = torch.empty((1, k), dtype=torch.float32, device=DEV)
    fused = route_group_one(lgd, k, ids, w, _grouping(E, k))
    ids2, w2 = route_topk(lgd, k)
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    sep = group_rows(ids2, E, ws)
    torch.cuda.synchronize()
    n = int(sep.active[0].item())
    assert n == k
    assert torch.equal(ids, ids2) and torch.equal(w.view(torch.int32), w2.view(torch.int32))
    for name in ("expert_offsets", "sorted_rows", "row_pos"):
        assert torch.equal(getattr(fused, name), getattr(sep, name)), name
    assert torch.equal(fused.active[:1 + n], sep.active[:1 + n])
    # against the oracle
    rid, rw = oracle.route_topk(lg, k)
    rg = oracle.group_rows(rid, E)
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    assert np.abs(w.cpu().numpy() - rw).max() <= 1e-6
    np.testing.assert_array_equal(fused.expert_offsets.cpu().numpy(), rg["expert_offsets"])
    np.testing.assert_array_equal(fused.sorted_rows.cpu().numpy(), rg["sorted_rows"])
    np.testing.assert_array_equal(fused.row_pos.cpu().numpy(), rg["row_pos"])
    np.testing.assert_array_equal(fused.active.cpu().numpy()[:1 + n], rg["active"][:1 + n])


COMBINE_CASES = [(1, 16, 7168), (3, 16, 7168), (1, 1, 32), (2, 32, 16384), (5, 4, 96), (0, 16, 7168)]


@pytest.mark.parametrize("T,k,H", COMBINE_CASES, ids=[f"T{t}_k{k}_H{h}" for t, k, h in COMBINE_CASES])
def test_combine_rms_bf16(T, k, H):
    say(f"combine_rms T={T} k={k} H={H}")
    rng = np.random.default_rng(1000 + 7 * T + k + H)
    R = T * k
    y = (rng.standard_normal((R, H)) * 300.0).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    row_pos = rng.permutation(R).astype(np.int32)
    yd, wd, rpd = (torch.from_numpy(a).to(DEV) for a in (y, w, row_pos))
    out = torch.empty((T, H), dtype=torch.float32, device=DEV)
    xn = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    combine_rms_bf16(yd, wd, rpd, out, xn, 1e-6)
    out2 = combine(yd, wd, rpd)
    xn2 = rms_rescale_bf16(out2, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), out2.view(torch.int32))
    assert torch.equal(xn.view(torch.int16), xn2.view(torch.int16))
    if T == 0:
        return
    ref = oracle.combine(y, w, row_pos, T, k, H)
    got = out.cpu().numpy()
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    rms = np.sqrt(np.mean(ref.astype(np.float64) ** 2))
    assert rel <= 2e-3 and np.abs(got - ref).max() <= 1e-2 * rms
    ref_x = oracle.rms_rescale_bf16(got, 1e-6).astype(np.int32)
    got_x = xn.view(torch.int16).cpu().numpy().astype(np.uint16).astype(np.int32)
    assert np.abs(got_x - ref_x).max() <= 1, "rescale more than one bf16 ulp off"


# moe_expert_ffn_combine_mxfp4 against moe_expert_ffn_mxfp4 + moe_combine:
# the fused one-token down + combine launch (decode shape, k <= 16, with and
# without repeated ids) and the shapes that fall back to the two calls
FFN_COMBINE_CASES = [  # name, E, H, I, k, T, ids (None: routed from logits)
    ("decode896", 896, 7168, 1536, 16, 1, None),
    ("decode896_k8", 896, 7168, 1536, 8, 1, None),
    ("decode896_k1", 896, 7168, 1536, 1, 1, None),
    ("repeated_ids", 896, 7168, 1536, 16, 1, [7, 300, 7, 895, 0, 300, 7, 41, 42, 43, 500, 501, 0, 650, 651, 7]),
    ("odd_hidden", 64, 4096, 1536, 16, 1, None),
    ("k32_two_calls", 96, 7168, 1536, 32, 1, None),
    ("tiny_two_calls", 8, 256, 128, 2, 4, None),
    ("verify_two_calls", 64, 7168, 1536, 16, 3, None),
]


@pytest.mark.parametrize("case", FFN_COMBINE_CASES, ids=[c[0] for c in FFN_COMBINE_CASES])
def test_ffn_combine_matches_two_calls(case):
    from mxfp4_routed_expert_02_amd import expert_ffn_combine_mxfp4, expert_ffn_mxfp4, workspace_bytes
    from tests.gpu_common import device_pool

    name, E, H, I, k, T, ids_list = case
    say(f"ffn_combine {name}: E={E} H={H} I={I} k={k} T={T}")
    wl = synth.Workload(name, E=E, H=H, I=I, k=k, T=T, pool=40, sub=40)
    pool = device_pool(wl)
    x = torch.from_numpy(synth.activations_bf16(0, wl).view(np.int16)).to(DEV).view(torch.bfloat16)
    if ids_list is None:
        ids, w = route_topk(torch.from_numpy(synth.router_logits(0, wl)).to(DEV), k)
    else:
        ids = torch.tensor([ids_list], dtype=torch.int32, device=DEV)
        w = torch.softmax(torch.arange(k, dtype=torch.float32, device=DEV), 0).view(1, k)
    ws = torch.empty(workspace_bytes(T, k, E, H, I), dtype=torch.uint8, device=DEV)
    g = group_rows(ids, E, ws)
    y1 = expert_ffn_mxfp4(x, k, pool, g, ws)
    out1 = combine(y1, w, g.row_pos)
    y2 = torch.full_like(y1, float("nan"))
    out2 = torch.full_like(out1, float("nan"))
    expert_ffn_combine_mxfp4(x, k, pool, g, w, ws, y2, out2)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32)), "y_rows bits differ"
    assert torch.equal(out1.view(torch.int32), out2.view(torch.int32)), "out bits differ"
    # against the oracle on the same ids and weights
    ids_np, w_np = ids.cpu().numpy(), w.cpu().numpy()
    ref_g = oracle.group_rows(ids_np, E)
    np.testing.assert_array_equal(g.sorted_rows.cpu().numpy(), ref_g["sorted_rows"])
    out_ref, y_ref = oracle_outputs(synth.activations_bf16(0, wl), ids_np, w_np, ref_g["sorted_rows"], wl)
    assert_close(y2.cpu().numpy(), y_ref, "y_rows vs oracle")
    assert_close(out2.cpu().numpy(), out_ref, "out vs oracle")


def _against_oracle(lg_np, x_np, k, wl, ids, w, g, y_rows, out):
    """One token's fused-call outputs against the oracle: top-k ids and
    grouping bit for bit, routing weights within 1e-6, y_rows and out at the
    parity bar."""
    rid, rw = oracle.route_topk(lg_np.reshape(1, -1), k)
    rg = oracle.group_rows(rid, wl.E)
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    assert np.abs(w.cpu().numpy() - rw).max() <= 1e-6
    for nm in ("expert_offsets", "sorted_rows", "row_pos"):
        np.testing.assert_array_equal(getattr(g, nm).cpu().numpy(), rg[nm])
    out_ref, y_ref = oracle_outputs(x_np.reshape(1, -1), rid, rw, rg["sorted_rows"], wl)
    assert_close(y_rows.cpu().numpy(), y_ref, "y_rows vs oracle")
    assert_close(out.cpu().numpy(), out_ref, "out vs oracle")


# moe_decode_layer_mxfp4 against moe_route_group_one + moe_expert_ffn_combine_mxfp4:
# routing inside the gate/up launch (the wide top-k at 1, 2, 4 and 8 experts
# per thread; ties; the top k all in one 16-lane row; fewer experts than the
# 16 rows, where every expert is a candidate; k = 1) and the shapes that run
# the separate calls
DECODE_LAYER_CASES = [  # name, E, H, I, k, logits kind
    ("E896_k16", 896, 7168, 1536, 16, "normal"),
    ("E96_k16", 96, 7168, 1536, 16, "normal"),
    ("E2048_k16", 2048, 7168, 1536, 16, "normal"),
    ("E896_ties", 896, 7168, 1536, 16, "ties"),
    ("E896_stride16", 896, 7168, 1536, 16, "stride16"),
    ("E300_k1", 300, 7168, 1536, 1, "normal"),
    ("E40_k16", 40, 7168, 1536, 16, "normal"),
    ("E16_k16", 16, 7168, 1536, 16, "normal"),
    ("E8_k4", 8, 7168, 1536, 4, "normal"),
    ("E5_k5_ties", 5, 7168, 1536, 5, "ties"),
    ("E4096_separate", 4096, 7168, 1536, 16, "normal"),
    ("k32_separate", 96, 7168, 1536, 32, "normal"),
    ("small_separate", 8, 256, 128, 2, "normal"),
]


@pytest.mark.parametrize("case", DECODE_LAYER_CASES, ids=[c[0] for c in DECODE_LAYER_CASES])
def test_decode_layer_matches_calls(case):
    from mxfp4_routed_expert_02_amd import decode_layer_mxfp4, expert_ffn_combine_mxfp4, workspace_bytes
    from tests.gpu_common import device_pool

    name, E, H, I, k, kind = case
    say(f"decode_layer {name}: E={E} H={H} I={I} k={k} {kind}")
    wl = synth.Workload(name, E=E, H=H, I=I, k=k, T=1, pool=41, sub=41)
    pool = device_pool(wl)
    x = torch.from_numpy(synth.activations_bf16(0, wl).view(np.int16)).to(DEV).view(torch.bfloat16)
    lg = torch.from_numpy(_logits(E, kind, 60 + E % 5)).to(DEV)
    ws = torch.empty(workspace_bytes(1, k, E, H, I), dtype=torch.uint8, device=DEV)
    # separate calls
    ids1 = torch.empty((1, k), dtype=torch.int32, device=DEV)
    w1 = torch.empty((1, k), dtype=torch.float32, device=DEV)
    g1 = route_group_one(lg, k, ids1, w1, _grouping(E, k))
    y1 = torch.empty((k, H), dtype=torch.float32, device=DEV)
    out1 = torch.empty((1, H), dtype=torch.float32, device=DEV)
    expert_ffn_combine_mxfp4(x, k, pool, g1, w1, ws, y1, out1)
    # one call, outputs pre-filled with garbage
    ids2 = torch.full((1, k), -7, dtype=torch.int32, device=DEV)
    w2 = torch.full((1, k), float("nan"), dtype=torch.float32, device=DEV)
    g2 = _grouping(E, k)
    for t in (g2.expert_offsets, g2.sorted_rows, g2.row_pos, g2.active):
        t.fill_(-5)
    y2 = torch.full_like(y1, float("nan"))
    out2 = torch.full_like(out1, float("nan"))
    decode_layer_mxfp4(lg, x, k, pool, ids2, w2, g2, ws, y2, out2)
    torch.cuda.synchronize()
    assert torch.equal(ids1, ids2), "ids differ"
    assert torch.equal(w1.view(torch.int32), w2.view(torch.int32)), "weights differ"
    for nm in ("expert_offsets", "sorted_rows", "row_pos"):
        assert torch.equal(getattr(g1, nm), getattr(g2, nm)), nm
    assert torch.equal(g1.active[:1 + k], g2.active[:1 + k]), "active differs"
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32)), "y_rows bits differ"
    assert torch.equal(out1.view(torch.int32), out2.view(torch.int32)), "out bits differ"
    # against the oracle: routing bit for bit, then the layer on its ids and weights
    _against_oracle(lg.cpu().numpy(), synth.activations_bf16(0, wl), k, wl, ids2, w2, g2, y2, out2)


# moe_decode_layer_rms_mxfp4 against moe_rms_rescale_bf16 + moe_decode_layer_mxfp4,
# including the stack's use with out in y_prev's own buffer
DECODE_RMS_CASES = [  # name, E, H, I, k, out aliases y_prev
    ("E96_k16", 96, 7168, 1536, 16, False),
    ("E16_k16", 16, 7168, 1536, 16, False),
    ("E896_k16_in_place", 896, 7168, 1536, 16, True),
    ("E4096_separate", 4096, 7168, 1536, 16, False),
    ("small_separate_in_place", 8, 256, 128, 2, True),
]


@pytest.mark.parametrize("case", DECODE_RMS_CASES, ids=[c[0] for c in DECODE_RMS_CASES])
def test_decode_layer_rms_matches_calls(case):
    from mxfp4_routed_expert_02_amd import decode_layer_mxfp4, decode_layer_rms_mxfp4, workspace_bytes
    from tests.gpu_common import device_pool

    name, E, H, I, k, in_place = case
    say(f"decode_layer_rms {name}: E={E} H={H} I={I} k={k} in_place={in_place}")
    wl = synth.Workload(name, E=E, H=H, I=I, k=k, T=1, pool=42, sub=42)
    pool = device_pool(wl)
    y_prev = torch.from_numpy(synth.normal_f32(synth.key(0, 62), H, stddev=900.0).reshape(1, H)).to(DEV)
    lg = torch.from_numpy(_logits(E, "normal", 70 + E % 3)).to(DEV)
    ws = torch.empty(workspace_bytes(1, k, E, H, I), dtype=torch.uint8, device=DEV)
    # separate calls
    x1 = rms_rescale_bf16(y_prev, 1e-6)
    ids1 = torch.empty((1, k), dtype=torch.int32, device=DEV)
    w1 = torch.empty((1, k), dtype=torch.float32, device=DEV)
    g1 = _grouping(E, k)
    y1 = torch.empty((k, H), dtype=torch.float32, device=DEV)
    out1 = torch.empty((1, H), dtype=torch.float32, device=DEV)
    decode_layer_mxfp4(lg, x1, k, pool, ids1, w1, g1, ws, y1, out1)
    # one call
    x2 = torch.zeros((1, H), dtype=torch.bfloat16, device=DEV)
    ids2 = torch.full((1, k), -7, dtype=torch.int32, device=DEV)
    w2 = torch.full((1, k), float("nan"), dtype=torch.float32, device=DEV)
    g2 = _grouping(E, k)
    y2 = torch.full_like(y1, float("nan"))
    yp = y_prev.clone()
    out2 = yp if in_place else torch.full_like(out1, float("nan"))
    decode_layer_rms_mxfp4(lg, yp, 1e-6, x2, k, pool, ids2, w2, g2, ws, y2, out2)
    torch.cuda.synchronize()
    assert torch.equal(x1.view(torch.int16), x2.view(torch.int16)), "x_next bits differ"
    assert torch.equal(ids1, ids2) and torch.equal(w1.view(torch.int32), w2.view(torch.int32)), "routing differs"
    for nm in ("expert_offsets", "sorted_rows", "row_pos"):
        assert torch.equal(getattr(g1, nm), getattr(g2, nm)), nm
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32)), "y_rows bits differ"
    assert torch.equal(out1.view(torch.int32), out2.view(torch.int32)), "out bits differ"
    # against the oracle: the rescale within one bf16 ulp of the oracle's, then
    # the layer on the GPU's own bf16 input
    x_gpu = x2.view(torch.int16).cpu().numpy().view(np.uint16)
    x_ref = oracle.rms_rescale_bf16(y_prev.cpu().numpy(), 1e-6)
    assert np.abs(x_gpu.astype(np.int32) - x_ref.astype(np.int32)).max() <= 1, "rescale more than one ulp off"
    _against_oracle(lg.cpu().numpy(), x_gpu, k, wl, ids2, w2, g2, y2, out2)


def test_decode_layer_graph_replays_match_eager():
    """A stacked step (moe_decode_layer_rms_mxfp4 then moe_decode_layer_mxfp4)
    captured in a HIP graph: every replay, with eager work and
    synchronizations between them, gives the eager bits."""
    from mxfp4_routed_expert_02_amd import decode_layer_mxfp4, decode_layer_rms_mxfp4, workspace_bytes
    from tests.gpu_common import device_pool

    E, H, I, k = 96, 7168, 1536, 16
    wl = synth.Workload("graph", E=E, H=H, I=I, k=k, T=1, pool=43, sub=43)
    pool = device_pool(wl)
    y_prev = torch.from_numpy(synth.normal_f32(synth.key(0, 63), H, stddev=900.0).reshape(1, H)).to(DEV)
    lg0 = torch.from_numpy(_logits(E, "normal", 80)).to(DEV)
    lg1 = torch.from_numpy(_logits(E, "normal", 81)).to(DEV)
    ws = torch.empty(workspace_bytes(1, k, E, H, I), dtype=torch.uint8, device=DEV)
    ids = torch.empty((1, k), dtype=torch.int32, device=DEV)
    w = torch.empty((1, k), dtype=torch.float32, device=DEV)
    g = _grouping(E, k)
    y = torch.empty((k, H), dtype=torch.float32, device=DEV)
    x1 = torch.empty((1, H), dtype=torch.bfloat16, device=DEV)
    out1 = torch.empty((1, H), dtype=torch.float32, device=DEV)
    out2 = torch.empty((1, H), dtype=torch.float32, device=DEV)

    def step():
        decode_layer_rms_mxfp4(lg0, y_prev, 1e-6, x1, k, pool, ids, w, g, ws, y, out1)
        decode_layer_mxfp4(lg1, x1, k, pool, ids, w, g, ws, y, out2)

    step()
    torch.cuda.synchronize()
    ref = (x1.clone(), out1.clone(), out2.clone(), ids.clone())
    stream = torch.cuda.Stream(DEV)
    stream.wait_stream(torch.cuda.current_stream(DEV))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            step()
    torch.cuda.current_stream(DEV).wait_stream(stream)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (x1, out1, out2):
            t.zero_()  # eager work between replays
        ids.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(x1.view(torch.int16), ref[0].view(torch.int16)), f"replay {rep}: x_next"
        assert torch.equal(out1.view(torch.int32), ref[1].view(torch.int32)), f"replay {rep}: out of layer 1"
        assert torch.equal(out2.view(torch.int32), ref[2].view(torch.int32)), f"replay {rep}: out of layer 2"
        assert torch.equal(ids, ref[3]), f"replay {rep}: ids"
