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
