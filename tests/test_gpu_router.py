"""The router projection on the GPU against the oracle.

Both sides accumulate in fp32 in different orders, so neither is bit-exact;
each lies within the recursive-summation bound g(H + 1) * sum |x w| of the
exact value (g(n) = n u / (1 - n u), u = 2^-24), so the two lie within twice
that of each other.  The exact value here is a float64 matmul.  Top-k taken
on the GPU's logits matches the oracle's top-k of the same logits bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from mxfp4_routed_expert_02_amd import route_topk, router_logits, synth
from tests.gpu_common import say

pytestmark = pytest.mark.gpu

CASES = [  # E, H, T: GEMV (T <= 4) and tiled paths, ragged tiles, the ranges' ends
    (8, 256, 4), (896, 7168, 1), (896, 7168, 3), (896, 7168, 8), (896, 7168, 512), (100, 96, 37),
    (4096, 32, 5), (64, 16384, 2), (64, 16384, 5), (1, 32, 1), (896, 7168, 0), (896, 7168, 4), (33, 224, 2),
    (130, 128, 65),
]


@pytest.mark.parametrize("E,H,T", CASES, ids=[f"E{e}_H{h}_T{t}" for e, h, t in CASES])
def test_router_logits_match_oracle(E, H, T):
    say(f"router E={E} H={H} T={T}")
    wl = synth.Workload("router", E=E, H=H, I=32, k=min(16, E), T=T, sub=40)
    wr = synth.router_weights(0, wl)
    x = synth.activations_bf16(0, wl)
    dev = torch.device("cuda", 0)
    xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    got = router_logits(xd, torch.from_numpy(wr).to(dev))
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    assert got.shape == (T, E)
    if T == 0:
        return
    ref = oracle.router_logits(x, wr, nthreads=16)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    exact = xf @ wr.astype(np.float64).T
    mag = np.abs(xf) @ np.abs(wr.astype(np.float64)).T
    u = 2.0 ** -24
    g = (H + 1) * u / (1 - (H + 1) * u)
    err = np.abs(got.astype(np.float64) - exact)
    say(f"  max |gpu - exact| / bound = {(err / np.maximum(g * mag, 1e-300)).max():.3e}")
    assert np.all(err <= g * mag)
    assert np.all(np.abs(got.astype(np.float64) - ref) <= 2 * g * mag)
    # the routing decision on these logits, GPU and oracle taking it on the same values
    k = min(16, E)
    ids, _ = route_topk(torch.from_numpy(got).to(dev), k)
    ref_ids, _ = oracle.route_topk(got, k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
