"""The device twin of the slab generator gives the host generator's bytes.

The HIP layer reads pools generated on the device; the oracle reads slabs
generated on the host.  Both must be the same bytes, so every workload's
parity rests on this comparison (tiny shape in full, real-shape experts at
both ends of a pool, another seed, layer and pool id)."""
import numpy as np
import pytest
import torch

from mxfp4_routed_expert_02_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed,pool,layer,first,n,H,I", [
    (0, 1, 0, 0, 8, 256, 128),        # tiny pool, every expert
    (0, 0, 0, 0, 2, 7168, 1536),      # real shape, first experts of the 896 pool
    (0, 0, 0, 894, 2, 7168, 1536),    # real shape, last experts
    (7, 3, 91, 94, 2, 7168, 1536),    # other seed, stack pool, last layer
    (3, 23, 2, 5, 3, 288, 96),        # odd shape
])
def test_device_slabs_equal_host_slabs(seed, pool, layer, first, n, H, I):
    dev = torch.device("cuda", 0)
    got = synth.device_pool_slabs(seed, pool, layer, n, H, I, dev, first=first).cpu().numpy()
    ref = synth.expert_slabs(seed, pool, layer, first, n, H, I)
    assert got.shape == ref.shape
    assert np.array_equal(got, ref)
