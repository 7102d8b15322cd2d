"""The grouped GEMM's tile classes and stage counts against the oracle.

A tile of 128 token slots runs as one of three classes by the rows it
holds (1..32, 33..64, 65..128), each with its own LDS ring: 3 slots of
256-value stages for the first, 4 and 3 slots of 128-value stages for the
others.  Of the K / stage stages the first R are loaded before the loop,
the steady loop takes the rest that still have a stage R ahead to load
(two stages per trip on the 128-value rings), and the last R drain.
The prefill workloads reach every class only at K = 7168 and 1536.  Here
expert row counts hit each class and its edges (32/33, 64/65, 128/129 and
several tiles of one expert) at K = 512, 1024, 1536 and 2048 on both GEMMs
(gate/up: K = H, down: K = I), so that the loop runs with no steady stage
(drain only, also with exactly R stages), one, an odd and an even number.
Each case compares the whole y_rows and output with the oracle at the
task's bar, and the routing and grouping bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from mxfp4_routed_expert_02_amd import ExpertPool, synth
from tests.gpu_common import assert_close, check_routing, run_gpu_layer, say

pytestmark = pytest.mark.gpu

# rows per expert: a one-row expert (the register GEMV), then GEMM experts
# whose token tiles fall in each class and at its edges
COUNTS = [1, 20, 32, 33, 40, 64, 65, 100, 128, 129, 200, 300]
K_TOPK = 2


def _inputs(H, I, seed):
    """Tokens routed to exact row counts: the 2T rows sorted by expert are
    paired i with i + T (no expert holds T rows, so a token's two picks
    differ), then the tokens are shuffled, so the GEMM gathers its B rows
    from scattered tokens."""
    rng = np.random.default_rng(seed)
    E = len(COUNTS)
    rows = np.repeat(np.arange(E), COUNTS)
    R = rows.size
    assert R % K_TOPK == 0
    T = R // K_TOPK
    assert max(COUNTS) < T
    pairs = np.stack([rows[:T], rows[T:]], axis=1)[rng.permutation(T)]
    logits = (0.1 * rng.standard_normal((T, E))).astype(np.float32)
    logits[np.arange(T), pairs[:, 0]] = 10.0
    logits[np.arange(T), pairs[:, 1]] = 9.0
    wl = synth.Workload("gemm_classes", E=E, H=H, I=I, k=K_TOPK, T=T, pool=20 + H // 512 + I // 512, sub=20)
    x = synth.activations_bf16(seed, wl)
    slabs = synth.expert_slabs(seed, wl.pool, 0, 0, E, H, I)
    return wl, x, logits, slabs


@pytest.mark.parametrize("H,I", [(512, 1024), (1024, 512), (2048, 1536), (1536, 2048)],
                         ids=["H512_I1024", "H1024_I512", "H2048_I1536", "H1536_I2048"])
def test_gemm_tile_classes_and_stage_counts(H, I):
    wl, x, logits, slabs = _inputs(H, I, seed=H + I)
    say(f"gemm classes H={H} I={I}: T={wl.T} k={wl.k} rows per expert {COUNTS}")
    pool = ExpertPool(torch.from_numpy(slabs).to(torch.device("cuda", 0)), H, I)
    got = run_gpu_layer(wl, pool, x, logits)
    ref = oracle.layer(x, logits, wl.k, oracle.Pool(slabs, H, I), nthreads=16)
    check_routing(got, ref, wl.E)
    assert np.array_equal(np.diff(ref["expert_offsets"]), COUNTS)
    offs = ref["expert_offsets"]
    for e, c in enumerate(COUNTS):
        sl = slice(int(offs[e]), int(offs[e + 1]))
        assert_close(got["y_rows"][sl], ref["y_rows"][sl], f"expert {e} ({c} rows) y_rows")
    assert_close(got["y_rows"], ref["y_rows"], "y_rows")
    assert_close(got["out"], ref["out"], "out")
