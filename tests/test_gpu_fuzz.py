"""Seeded random layer configurations against the oracle.

Each case draws the expert count, top-k, token count, hidden and
intermediate sizes and the logit recipe from a fixed seed, half of them on
shapes the grouped GEMM takes (H and I multiples of 512) and half on any
multiple of 32 (the register GEMVs and their LDS fallbacks).  The oracle's
work per case is capped so the whole file runs in seconds.  The bar is the
task's: routing and grouping bit for bit, y_rows and the output within
rel-L2 2e-3 and max-abs 1e-2 * rms(ref).
"""
import numpy as np
import pytest

import oracle
from mxfp4_routed_expert_02_amd import synth
from tests.gpu_common import assert_close, check_routing, device_pool, run_gpu_layer, say

pytestmark = pytest.mark.gpu
N_CASES = 16
MAX_MACS = 3e9  # oracle multiply-adds per case (GEMM cases may exceed it to reach 17 tokens)


def _case(i):
    rng = np.random.default_rng(7000 + i)
    if i % 2 == 0:
        H = 512 * int(rng.integers(1, 5))
        I = 512 * int(rng.integers(1, 4))
    else:
        H = 32 * int(rng.integers(1, 97))
        I = 32 * int(rng.integers(1, 65))
    E = int(rng.integers(1, 301))
    k = int(rng.integers(1, min(E, 32) + 1))
    kinds = ["normal", "zipf", "ties", "shared_bias"] + (["dense16"] if E >= 16 and k <= 16 else [])
    kind = kinds[int(rng.integers(0, len(kinds)))]
    t_cap = max(1, int(MAX_MACS / (3.0 * H * I * k)))
    t_min = 17 if i % 2 == 0 else 1  # the GEMM takes experts of 2+ rows only above 16 tokens
    T = int(rng.integers(t_min, max(t_min, min(600, t_cap)) + 1))
    return synth.Workload(f"fuzz{i}", E=E, H=H, I=I, k=k, T=T, logits=kind, pool=200 + i, sub=200 + i)


CASES = [_case(i) for i in range(N_CASES)]


@pytest.mark.parametrize("wl", CASES, ids=[f"{w.name}_E{w.E}_k{w.k}_T{w.T}_H{w.H}_I{w.I}_{w.logits}" for w in CASES])
def test_fuzz_layer(wl):
    say(f"case {wl.name}: E={wl.E} H={wl.H} I={wl.I} k={wl.k} T={wl.T} logits={wl.logits}")
    x = synth.activations_bf16(0, wl)
    logits = synth.router_logits(0, wl)
    pool = device_pool(wl)
    hpool = oracle.Pool(synth.expert_slabs(0, wl.pool, 0, 0, wl.E, wl.H, wl.I), wl.H, wl.I)
    ref = oracle.layer(x, logits, wl.k, hpool, nthreads=16)
    gpu = run_gpu_layer(wl, pool, x, logits)
    check_routing(gpu, ref, wl.E)
    assert_close(gpu["y_rows"], ref["y_rows"], "y_rows")
    assert_close(gpu["out"], ref["out"], "out")
