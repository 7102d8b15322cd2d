"""Grouping of many routed rows against the oracle, bit for bit.

Above 512 rows the grouping runs in 256-row chunks: per chunk the expert
counts and each row's rank, then a scan in which 32 lanes share an expert's
chunks (8 experts a block), then a scatter in which every block scans the
expert totals.  The cases put the chunk count on both sides of the 32-lane
split (one chunk per lane, several per lane, a ragged last run), the expert
count on both sides of a scan block's 8 experts, and the ids on skewed
recipes: most rows on a few experts, empty experts between busy ones, one
expert taking every row, and ids repeated inside a token (the call takes any
ids in range).  expert_offsets, sorted_rows, row_pos and the active list must
equal the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_common import say

pytestmark = pytest.mark.gpu

# (rows, experts, recipe)
CASES = [
    (513, 1, "uniform"),
    (600, 5, "skewed"),
    (32 * 256, 8, "uniform"),
    (32 * 256 + 1, 9, "skewed"),
    (33 * 256 - 7, 13, "holes"),
    (64 * 256, 896, "zipf"),
    (65 * 256 + 100, 896, "holes"),
    (100 * 256 + 3, 4096, "zipf"),
    (257 * 256, 17, "one"),
    (3 * 256 + 5, 4096, "uniform"),
]


def _ids(R, E, recipe, rng):
    if recipe == "uniform":
        return rng.integers(0, E, R)
    if recipe == "skewed":  # 90% of rows on the first two experts
        hot = rng.integers(0, min(2, E), R)
        return np.where(rng.random(R) < 0.9, hot, rng.integers(0, E, R))
    if recipe == "holes":  # only every third expert is used
        used = np.arange(0, E, 3)
        return used[rng.integers(0, used.size, R)]
    if recipe == "zipf":
        return np.minimum(rng.zipf(1.1, R) - 1, E - 1)
    if recipe == "one":
        return np.full(R, E // 2)
    raise ValueError(recipe)


@pytest.mark.parametrize("R,E,recipe", CASES, ids=[f"R{r}_E{e}_{c}" for r, e, c in CASES])
def test_group_rows_chunked(R, E, recipe):
    from mxfp4_routed_expert_02_amd import group_rows, workspace_bytes

    rng = np.random.default_rng(R * 7 + E)
    ids = _ids(R, E, recipe, rng).astype(np.int32).reshape(R, 1)
    say(f"grouping R={R} E={E} ({recipe}): {(R + 255) // 256} chunks")
    ref = oracle.group_rows(ids, E)
    ws = torch.empty(workspace_bytes(R, 1, E, 32, 32), dtype=torch.uint8, device="cuda")
    g = group_rows(torch.from_numpy(ids).cuda(), E, ws)
    torch.cuda.synchronize()
    assert np.array_equal(g.expert_offsets.cpu().numpy(), ref["expert_offsets"])
    assert np.array_equal(g.sorted_rows.cpu().numpy(), ref["sorted_rows"])
    assert np.array_equal(g.row_pos.cpu().numpy(), ref["row_pos"])
    act = g.active.cpu().numpy()
    assert np.array_equal(act[: 1 + act[0]], ref["active"][: 1 + ref["active"][0]])
