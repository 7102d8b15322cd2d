"""moe_decode_layer_mxfp4_noalloc (the library's static device scratch in
place of a workspace) against moe_decode_layer_mxfp4 with a caller
workspace: every output bit for bit, on calls in a row that reuse the same
scratch, each later call with a smaller input than the one before."""
import numpy as np
import pytest
import torch

from mxfp4_routed_expert_02_amd import Grouping, decode_layer_mxfp4, decode_layer_mxfp4_noalloc, synth, workspace_bytes
from tests.gpu_common import assert_close, device_pool, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _bufs(E, H, k):
    z = lambda n, dt=torch.int32: torch.full((n,), -3, dtype=dt, device=DEV)  # noqa: E731
    return dict(ids=torch.full((1, k), -7, dtype=torch.int32, device=DEV),
                w=torch.full((1, k), float("nan"), dtype=torch.float32, device=DEV),
                g=Grouping(z(E + 1), z(k), z(k), z(E + 1)),
                y=torch.full((k, H), float("nan"), dtype=torch.float32, device=DEV),
                out=torch.full((1, H), float("nan"), dtype=torch.float32, device=DEV))


# one token each, largest first: the decode shape (fused launches), the same
# with fewer experts and picks, then a small shape (separate launches)
CASES = [("E896_k16", 896, 7168, 1536, 16), ("E96_k8", 96, 7168, 1536, 8), ("E8_k2_small", 8, 256, 128, 2)]


def test_noalloc_decode_layer_matches_workspace_call():
    results = []
    for name, E, H, I, k in CASES:
        say(f"noalloc {name}: E={E} H={H} I={I} k={k}")
        wl = synth.Workload(name, E=E, H=H, I=I, k=k, T=1, pool=45, sub=45)
        pool = device_pool(wl)
        x = torch.from_numpy(synth.activations_bf16(0, wl).view(np.int16)).to(DEV).view(torch.bfloat16)
        lg = torch.from_numpy(synth.router_logits(0, wl)).to(DEV)
        a, b = _bufs(E, H, k), _bufs(E, H, k)
        ws = torch.empty(workspace_bytes(1, k, E, H, I), dtype=torch.uint8, device=DEV)
        decode_layer_mxfp4(lg, x, k, pool, a["ids"], a["w"], a["g"], ws, a["y"], a["out"])
        decode_layer_mxfp4_noalloc(lg, x, k, pool, b["ids"], b["w"], b["g"], b["y"], b["out"])
        torch.cuda.synchronize()
        assert torch.equal(a["ids"], b["ids"]), "ids"
        assert torch.equal(a["w"].view(torch.int32), b["w"].view(torch.int32)), "weights"
        for nm in ("expert_offsets", "sorted_rows", "row_pos"):
            assert torch.equal(getattr(a["g"], nm), getattr(b["g"], nm)), nm
        assert torch.equal(a["g"].active[:1 + k], b["g"].active[:1 + k]), "active"
        assert_close(b["y"].cpu().numpy(), a["y"].cpu().numpy(), "y_rows")
        assert_close(b["out"].cpu().numpy(), a["out"].cpu().numpy(), "out")
        assert torch.equal(a["y"].view(torch.int32), b["y"].view(torch.int32)), "y_rows bits"
        assert torch.equal(a["out"].view(torch.int32), b["out"].view(torch.int32)), "out bits"
        results.append((pool, lg, x, b["out"].clone(), k, E, H))
        del ws
    # the first (largest) case again after the smaller ones: nothing left in
    # the shared scratch changes its result
    pool, lg, x, want, k, E, H = results[0]
    c = _bufs(E, H, k)
    decode_layer_mxfp4_noalloc(lg, x, k, pool, c["ids"], c["w"], c["g"], c["y"], c["out"])
    torch.cuda.synchronize()
    assert torch.equal(c["out"].view(torch.int32), want.view(torch.int32)), "repeat of the first call"
