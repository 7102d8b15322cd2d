"""Helpers of the GPU parity tests: device inputs from the seeded generator,
the HIP layer through the C ABI, and the parity bar."""
import numpy as np
import torch

import oracle
from mxfp4_routed_expert_02_amd import ExpertPool, synth
from mxfp4_routed_expert_02_amd.layer import RoutedExpertLayer

REL_L2 = 2e-3  # bar on the whole [T][H] fp32 output
MAX_ABS_RMS = 1e-2  # max-abs error bar as a fraction of rms(ref)
W_ATOL = 1e-6  # routing weights


def say(*a):
    print(*a, flush=True)


def assert_close(got: np.ndarray, ref: np.ndarray, what: str):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    nref = np.linalg.norm(ref)
    rms = nref / np.sqrt(max(ref.size, 1))
    rel = np.linalg.norm(got - ref) / max(nref, 1e-30)
    mab = np.abs(got - ref).max() / max(rms, 1e-30) if ref.size else 0.0
    say(f"  {what}: rel-L2 {rel:.3e}  max-abs/rms {mab:.3e}")
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.3e} > {REL_L2}"
    assert mab <= MAX_ABS_RMS, f"{what}: max-abs/rms {mab:.3e} > {MAX_ABS_RMS}"


def device_pool(wl, layer=0, seed=0):
    """The workload's pool generated on the device (the same bytes as the
    host generator, which test_gpu_synth checks)."""
    dev = torch.device("cuda", 0)
    slabs = synth.device_pool_slabs(seed, wl.pool, layer, wl.E, wl.H, wl.I, dev)
    torch.cuda.synchronize()
    return ExpertPool(slabs, wl.H, wl.I)


def host_pool_subset(wl, experts, layer=0, seed=0):
    """Host pool holding only the listed experts (others zero), as the oracle needs."""
    sb = synth.slab_bytes(wl.H, wl.I)
    slabs = np.zeros((wl.E, sb), np.uint8)
    for e in sorted(set(int(e) for e in experts)):
        synth.expert_slabs(seed, wl.pool, layer, e, 1, wl.H, wl.I, out=slabs[e:e + 1])
    return oracle.Pool(slabs, wl.H, wl.I)


def run_gpu_layer(wl, pool, x_np, logits_np, layer_obj=None):
    dev = torch.device("cuda", 0)
    T = x_np.shape[0]
    x = torch.from_numpy(x_np.view(np.int16)).to(dev).view(torch.bfloat16)
    logits = torch.from_numpy(logits_np).to(dev)
    L = layer_obj or RoutedExpertLayer(wl.E, wl.H, wl.I, wl.k, max(T, 1), dev)
    out = L(x, logits, pool)
    torch.cuda.synchronize()
    R = T * wl.k
    return dict(ids=L.ids[:T].cpu().numpy(), w=L.weights[:T].cpu().numpy(),
                expert_offsets=L.grp.expert_offsets.cpu().numpy(),
                sorted_rows=L.grp.sorted_rows[:R].cpu().numpy(), row_pos=L.grp.row_pos[:R].cpu().numpy(),
                active=L.grp.active.cpu().numpy(), y_rows=L.y_rows[:R].cpu().numpy(),
                out=out.cpu().numpy())


def check_routing(gpu, ref, E):
    assert np.array_equal(gpu["ids"], ref["ids"]), "top-k ids differ"
    assert np.abs(gpu["w"] - ref["w"]).max() <= W_ATOL, "routing weights differ"
    assert np.array_equal(gpu["expert_offsets"], ref["expert_offsets"]), "expert_offsets differ"
    assert np.array_equal(gpu["sorted_rows"], ref["sorted_rows"]), "sorted_rows differ"
    assert np.array_equal(gpu["row_pos"], ref["row_pos"]), "row_pos differ"
    na = int(ref["active"][0])
    assert gpu["active"][0] == na and np.array_equal(gpu["active"][1:1 + na], ref["active"][1:1 + na])


def oracle_rows(x_np, tokens, experts, hpool, nthreads=16):
    """The oracle's y for arbitrary (token, expert) pairs: y[i] = FFN of expert
    experts[i] on token tokens[i], computed through the oracle's own grouped
    steps on a sub-batch with k = 1 (each row's arithmetic is the one the
    full layer gives it)."""
    tokens = np.asarray(tokens, np.int64)
    ids = np.asarray(experts, np.int32).reshape(-1, 1)
    xs = np.ascontiguousarray(x_np[tokens])
    grp = oracle.group_rows(ids, hpool.E)
    h = oracle.gateup(xs, 1, hpool, grp, nthreads)
    y = oracle.down(h, hpool, grp, nthreads)
    return y[grp["row_pos"]]


def tile_edge_positions(offsets, tile=128):
    """Sorted positions of the first and last routed row of every
    (expert, tile-row) chunk of each expert's rows: every (expert, token
    tile) pair of the grouped GEMM and every GEMV expert is represented."""
    pos = []
    offsets = np.asarray(offsets)
    for e in range(offsets.size - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        for s in range(a, b, tile):
            pos += [s, min(s + tile, b) - 1]
    return np.array(sorted(set(pos)), np.int64)


def host_pool_compact(wl, experts, layer=0, seed=0, pool_id=None):
    """Host pool holding just the listed experts, packed: returns (pool, map)
    where map[e] is expert e's index in the packed pool (for pools too large
    to mirror on the host, e.g. 4096 experts at the real shape)."""
    uniq = sorted(set(int(e) for e in np.asarray(experts).reshape(-1)))
    sb = synth.slab_bytes(wl.H, wl.I)
    slabs = np.zeros((max(len(uniq), 1), sb), np.uint8)
    for i, e in enumerate(uniq):
        synth.expert_slabs(seed, wl.pool if pool_id is None else pool_id, layer, e, 1, wl.H, wl.I, out=slabs[i:i + 1])
    return oracle.Pool(slabs, wl.H, wl.I), {e: i for i, e in enumerate(uniq)}


def oracle_outputs(x_np, ids_np, w_np, sorted_rows_np, wl, layer=0, seed=0, nthreads=16):
    """The oracle's out[T][H] (per-token layer on the given ids and weights)
    and y_rows[R][H] in the grouped order that sorted_rows gives, from a
    packed host pool of just the routed experts."""
    ids_np = np.asarray(ids_np, np.int32)
    T, k = ids_np.shape
    hp, m = host_pool_compact(wl, ids_np, layer, seed)
    cid = np.vectorize(lambda e: m[int(e)], otypes=[np.int32])(ids_np).reshape(T, k)
    out = oracle.token_layers_parallel(x_np, cid, np.asarray(w_np, np.float32), hp, range(T), nthreads)
    rows = np.asarray(sorted_rows_np, np.int64).reshape(-1)
    y = oracle_rows(x_np, rows // k, cid.reshape(-1)[rows], hp, nthreads)
    return out, y
