"""GPU tests of the boundary's separable calls: attention on the caller's K/V
and a caller-built mask (no routing in between), routing without the K/V
re-layout, and the traced attention launch.

FVAttn S2.1 states the problem per head over Q, K, V and a block mask; the
routing is one way to produce that mask, and the attention must give the
masked softmax for any mask it is handed.
"""

import math

import numpy as np
import pytest
import torch

import adaptive_block_sparse_fva_amd as F
import oracle as O
from gpu_helpers import (LSE_MAX_ABS, O_MAX_ABS, O_MEAN_ABS, device_inputs, f64_inputs, host,
                         problem_for, run_chain, sample_tiles, say, tile_rows)
from synth import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def _random_mask(rows, nb, seed):
    """Seeded CSR mask: each row keeps a uniform count in [1, nb] of distinct
    blocks, ascending; row 0 keeps every block and row 1 a single one."""
    rng = np.random.default_rng(seed)
    counts = rng.integers(1, nb + 1, size=rows)
    counts[0], counts[1] = nb, 1
    cols = [np.sort(rng.choice(nb, int(c), replace=False)) for c in counts]
    row_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return row_ptr, np.concatenate(cols).astype(np.int64), counts.astype(np.int64)


@pytest.mark.parametrize("name", ["two_head", "rank480p"])
def test_attention_on_caller_kv_and_caller_mask(name):
    """fva_kv_layout + fva_schedule + fva_sparse_attn_fwd on a mask the
    routing never saw, against the fp64 masked softmax."""
    wl = WORKLOADS[name]
    say(f"[gpu] caller K/V + caller mask {name}")
    inp = make_inputs(wl)
    q, k, v = device_inputs(inp)
    prob = problem_for(wl, wl.top_p[0])
    buf = F.Buffers.allocate(prob)
    H, nb = wl.num_heads, buf.nb
    rows = H * nb
    row_ptr, col_idx, counts = _random_mask(rows, nb, seed=23)
    buf.row_ptr.copy_(torch.from_numpy(row_ptr.astype(np.int32)))
    buf.col_idx[: len(col_idx)].copy_(torch.from_numpy(col_idx.astype(np.int32)))
    buf.kv_layout(k, v)
    buf.schedule()
    buf.attn(q)
    torch.cuda.synchronize()
    res = host(buf)
    order = O.token_order(wl.grid, wl.tile_hw)
    np.testing.assert_array_equal(res["order"], O.padded_order(order, wl.block))
    np.testing.assert_array_equal(res["row_ptr"], row_ptr)
    np.testing.assert_array_equal(res["col_idx"], col_idx)
    work, slot, nsplit = O.work_items(counts, F.compute_units())
    meta = res["plan_meta"]
    assert meta[0] == rows + nsplit and meta[1] == nsplit
    np.testing.assert_array_equal(meta[2: 2 + rows], slot)
    np.testing.assert_array_equal(res["work_order"], work)
    np.testing.assert_array_equal(res["tile_counter"], [0, 0])

    q64, k64, v64 = f64_inputs(inp)
    tiles = None if rows <= 256 else sample_tiles(row_ptr, H, nb, per_head=64, seed=4)
    o_ref, lse_ref = O.masked_attention(q64, k64, v64, order, wl.block, row_ptr, col_idx,
                                        1.0 / math.sqrt(wl.head_dim), tiles)
    if tiles is None:
        do, dl = np.abs(res["o"] - o_ref), np.abs(res["lse"] - lse_ref)
    else:
        sel = tile_rows(order, wl.block, wl.seq_len, tiles, nb)
        do = np.concatenate([np.abs(res["o"][h, r] - o_ref[h, r]).ravel() for h, r in sel.items()])
        dl = np.concatenate([np.abs(res["lse"][h, r] - lse_ref[h, r]).ravel() for h, r in sel.items()])
    say(f"  {'all' if tiles is None else len(tiles)} tiles, density {len(col_idx) / (rows * nb):.3f}, "
        f"split tiles {nsplit}: O max-abs {do.max():.3e} mean-abs {do.mean():.3e}; "
        f"LSE max-abs {dl.max():.3e}")
    assert np.all(np.isfinite(do))
    assert do.max() <= O_MAX_ABS and do.mean() <= O_MEAN_ABS and dl.max() <= LSE_MAX_ABS


@pytest.mark.parametrize("name", ["two_head", "rank480p", "rank720p"])
def test_routing_alone_and_kv_layout_match_the_fused_pass(name):
    """fva_route without v/kv (and without exported scores) decides exactly
    what the fused pass decides; fva_kv_layout writes exactly the fused
    pass's K/V re-layout and order table."""
    wl = WORKLOADS[name]
    say(f"[gpu] routing alone vs fused {name}")
    inp = make_inputs(wl)
    q, k, v = device_inputs(inp)
    prob = problem_for(wl, wl.top_p[0])
    fused = F.Buffers.allocate(prob)
    fused.route(q, k, v)
    alone = F.Buffers.allocate(prob)
    alone.order.fill_(-7)
    alone.route(q, k, with_scores=False)
    layout = F.Buffers.allocate(prob)
    layout.kv_layout(k, v)
    torch.cuda.synchronize()
    for key in ("ranked", "row_count", "head_count", "order"):
        assert torch.equal(getattr(fused, key), getattr(alone, key)), key
    assert torch.equal(fused.order, layout.order)
    assert torch.equal(fused.kv.view(torch.int16), layout.kv.view(torch.int16))


def test_traced_attention_is_the_same_call():
    """The traced launch writes the same O and LSE bit for bit, and one trace
    record per work item: workgroup w starts with item w, clocks advance."""
    wl = WORKLOADS["rank480p"]
    say("[gpu] traced attention rank480p")
    inp = make_inputs(wl)
    q, k, v = device_inputs(inp)
    buf, res = run_chain(problem_for(wl, wl.top_p[0]), q, k, v)
    items = int(res["plan_meta"][0])
    trace = torch.full((items, F.fva.FVA_TRACE_FIELDS), -1, dtype=torch.int64, device="cuda")
    buf.attn(q, item_trace=trace)
    torch.cuda.synchronize()
    assert torch.equal(buf.o.view(torch.int16).cpu(),
                       torch.from_numpy(res["o"].astype(np.float32)).to(torch.bfloat16).view(torch.int16))
    np.testing.assert_array_equal(buf.lse.cpu().numpy(), res["lse"].astype(np.float32))
    tr = trace.cpu().numpy()
    grid = F.attn_workgroups(buf.prob)
    assert (tr[:, 1] >= tr[:, 0]).all() and (tr[:, 3] >= tr[:, 2]).all()
    assert (tr[:, 0] > 0).all()
    assert ((tr[:, 5] >= 0) & (tr[:, 5] < grid)).all()
    first = min(items, grid)
    np.testing.assert_array_equal(tr[:first, 5], np.arange(first))
    span_us = (tr[:, 1].max() - tr[:, 0].min()) / 100.0
    say(f"  {items} items on {grid} workgroups, {len(np.unique(tr[:, 4]))} distinct placements, "
        f"span {span_us:.1f} us")
