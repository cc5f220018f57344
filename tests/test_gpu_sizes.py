"""GPU parity at the size limits and at the ranking widths the named workloads
do not reach.

The routing's per-row sort keeps 64 E keys per wave (E = 1, 2, 4, 8, 16, 32
for nb up to 64, 128, 256, 512, 1024, 2048); the workloads of the other tests
cover E = 1, 4 and 16.  These cases cover E = 2, 8 and 32, the largest key-block
count (nb = 2048) and the largest tile count (H * nb = 16384, the plan's
longest sort), with the same bar: integer outputs bit-exact against the oracle
on the GPU's fp32 scores, attention within tolerance on sampled tiles.
"""

import numpy as np
import pytest
import torch

import adaptive_block_sparse_fva_amd as F
import oracle.fva_gsrs as G
from gpu_helpers import device_inputs, problem_for, run_chain, sample_tiles, say
from synth import Workload, make_inputs
from test_gpu_parity import check_attention, check_routing_and_plan

pytestmark = pytest.mark.gpu

SIZES = [
    # name, heads, d, grid, block, p, k_min, refill
    ("nb128_E2", 2, 128, (2, 64, 64), 64, 0.9, 4, 0),
    ("nb384_E8", 2, 128, (8, 64, 96), 128, 0.95, 8, 50),
    ("nb2048_E32", 1, 128, (16, 128, 128), 128, 0.9, 8, 0),
    ("tiles16384", 8, 64, (8, 128, 128), 64, 0.8, 2, 0),
]


@pytest.mark.parametrize("case", SIZES, ids=[c[0] for c in SIZES])
def test_size_limits(case):
    name, H, d, grid, block, p, kmin, refill = case
    wl = Workload(name, H, d, grid, block, (p,), kmin, refill, seed=41, heads="lograndom")
    say(f"[gpu] size {name} H={H} N={wl.seq_len} nb={wl.num_blocks} tiles={H * wl.num_blocks}")
    inp = make_inputs(wl, cache=False)
    q, k, v = device_inputs(inp)
    prob = problem_for(wl, p, refill)
    buf, res = run_chain(prob, q, k, v)
    check_routing_and_plan(wl, inp, res, p, refill)
    tiles = sample_tiles(res["row_ptr"], H, res["nb"], per_head=max(2, 24 // H), seed=9)
    check_attention(wl, inp, res, tiles, label=f"{len(tiles)} sampled tiles:")

    if name == "nb2048_E32":
        # re-selection at the widest sort: precise importance of the kept
        # blocks, then Top-p inside them
        sz = F.sizes(prob)
        nnz = int(res["row_ptr"][-1])
        block_lse = torch.empty(nnz * block, dtype=torch.float32, device="cuda")
        buf.attn(q, block_lse=block_lse)
        imp = buf.importance(block_lse)
        ranked = torch.empty(sz.ranked_elems, dtype=torch.int16, device="cuda")
        count = torch.empty(sz.num_rows, dtype=torch.int32, device="cuda")
        head = torch.empty(H, dtype=torch.int32, device="cuda")
        sp = problem_for(wl, 0.8, 0)
        F.reselect(sp, buf.row_ptr, buf.col_idx, imp, ranked, count, head)
        torch.cuda.synchronize()
        nb = res["nb"]
        ref_ranked, ref_count, ref_head = G.select_from_importance(
            imp.cpu().numpy(), res["row_ptr"], res["col_idx"], 0.8, kmin)
        np.testing.assert_array_equal(ranked.cpu().numpy().astype(np.int64).reshape(H * nb, nb), ref_ranked)
        np.testing.assert_array_equal(count.cpu().numpy(), ref_count)
        np.testing.assert_array_equal(head.cpu().numpy(), ref_head)
        say(f"  re-selection: {int(ref_count.sum())} of {nnz} kept blocks")
