"""GPU tests of the work-list step on its own (fva_schedule) over synthetic row
lengths, bit for bit against the oracle's work list.

FVAttn S3.2: placement changes where work runs, never which blocks are
computed; on one GPU it is the heaviest-first list of work items, with tiles
heavier than a compute unit's mean load cut in two.  The list is ordered by
item length (descending), then tile, then part.  The length distributions
below reach every case of the kernel's sort: lengths spread over the whole
1 .. 2048 range (three 4-bit digits of the length field differ), lengths all
equal (no digit differs), two values, many split tiles, and the largest tile
count.  fva_schedule reads only the CSR row offsets, so no column ids are
needed.
"""

import zlib

import numpy as np
import pytest
import torch

import adaptive_block_sparse_fva_amd as F
import oracle as O
from gpu_helpers import say

pytestmark = pytest.mark.gpu

# name, heads, grid (T, H, W) with B = 128 tokens per block, length generator
CASES = [
    ("uniform_nb2048_16384tiles", 8, (16, 128, 128), "uniform"),
    ("uniform_nb256", 5, (21, 30, 52), "uniform"),
    ("equal_nb256", 5, (21, 30, 52), "equal"),
    ("two_values_nb256", 5, (21, 30, 52), "two_values"),
    ("split_heavy_nb64", 1, (2, 64, 64), "split_heavy"),
    ("split_mixed_nb64", 3, (2, 64, 64), "split_mixed"),
]


def _lengths(kind, rows, nb, rng):
    if kind == "uniform":
        return rng.integers(1, nb + 1, size=rows)
    if kind == "equal":
        return np.full(rows, 37)
    if kind == "two_values":
        return rng.choice([8, 200], size=rows)
    if kind == "split_heavy":
        return rng.integers(nb // 2, nb + 1, size=rows)
    if kind == "split_mixed":
        lens = rng.integers(1, 9, size=rows)
        heavy = rng.choice(rows, size=rows // 4, replace=False)
        lens[heavy] = rng.integers(nb // 2, nb + 1, size=len(heavy))
        return lens
    raise ValueError(kind)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_schedule_matches_oracle_work_list(case):
    name, H, grid, kind = case
    N = grid[0] * grid[1] * grid[2]
    prob = F.make_problem(H, N, 128, grid, 128, (8, 16), 0.9, 8)
    sz = F.sizes(prob)
    rows = int(sz.num_rows)
    nb = rows // H
    assert rows == H * nb and nb == -(-N // 128)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    lens = _lengths(kind, rows, nb, rng).astype(np.int64)
    assert lens.min() >= 1 and lens.max() <= nb
    row_ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu = F.compute_units()
    work, slot, nsplit = O.work_items(lens, cu)
    say(f"[gpu] schedule {name}: {rows} tiles, lengths {lens.min()}..{lens.max()}, "
        f"{nsplit} split tiles, {len(work)} items")

    dev = dict(dtype=torch.int32, device="cuda")
    rp = torch.from_numpy(row_ptr).cuda()
    work_order = torch.full((sz.work_order_elems,), -5, **dev)
    plan_meta = torch.full((sz.plan_meta_elems,), -5, **dev)
    counter = torch.full((sz.tile_counter_elems,), 7, **dev)
    F.fva.schedule(prob, rp, work_order, plan_meta, counter)
    torch.cuda.synchronize()

    wo, meta = work_order.cpu().numpy(), plan_meta.cpu().numpy()
    items = rows + nsplit
    assert meta[0] == items and meta[1] == nsplit
    np.testing.assert_array_equal(wo[:items], work)
    np.testing.assert_array_equal(meta[2: 2 + rows], slot)
    split_tiles = np.flatnonzero(slot >= 0)[np.argsort(slot[slot >= 0])]
    np.testing.assert_array_equal(meta[2 + rows: 2 + rows + nsplit], split_tiles)
    np.testing.assert_array_equal(counter.cpu().numpy(), [0, 0])
    # the row offsets are an input here and stay as they were
    np.testing.assert_array_equal(rp.cpu().numpy(), row_ptr)
