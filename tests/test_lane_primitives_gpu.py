"""The cross-lane helpers every kernel builds on (gla_lane_selftest): DPP group
reductions, the strided exclusive scans, the 64-lane scan, the row broadcast and
row sum, and the gfx950 row-pair and half-wave swaps, each held against its
definition on one wavefront of 64 lanes (lane l of row l // 16)."""
import numpy as np
import pytest
import torch

import chunked_linear_attention_gla_amd as gla
from gpu_util import device

pytestmark = pytest.mark.gpu


def run(values):
    out = gla.lane_selftest(torch.tensor(values, dtype=torch.float32, device=device()))
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("seed", [0, 1])
def test_lane_layouts(seed):
    # small integers: every sum below is exact in fp32, so the comparisons are exact
    x = np.random.default_rng(seed).integers(-50, 50, 64).astype(np.float64)
    o = run(x)
    lanes = np.arange(64)
    rows = x.reshape(4, 16)
    for n, slot_max, slot_sum in ((8, 0, 2), (16, 1, 3)):
        grp = x.reshape(64 // n, n)
        assert (o[slot_max] == np.repeat(grp.max(1), n)).all(), n
        assert (o[slot_sum] == np.repeat(grp.sum(1), n)).all(), n
    for slot, s in ((4, 4), (5, 8), (6, 16)):
        ref = np.array([sum(x[l - k * s] for k in range(1, l // s + 1)) for l in lanes])
        assert (o[slot] == ref).all(), s
    assert (o[7] == np.cumsum(x)).all()
    for r in range(4):
        assert (o[8 + r] == np.tile(rows[r], 4)).all(), r
    assert (o[12] == np.tile(rows.sum(0), 4)).all()
    y = (x + 100.0).reshape(4, 16)
    # row-pair swap: odd rows of a trade places with even rows of b
    assert (o[13] == np.concatenate([rows[0], y[0], rows[2], y[2]])).all()
    assert (o[14] == np.concatenate([rows[1], y[1], rows[3], y[3]])).all()
    # half-wave swap: the high half of a trades places with the low half of b
    assert (o[15] == np.concatenate([x[:32], (x + 100.0)[:32]])).all()
    assert (o[16] == np.concatenate([x[32:], (x + 100.0)[32:]])).all()
