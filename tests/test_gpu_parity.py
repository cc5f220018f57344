"""GPU parity: the HIP chain (through the C ABI) against the fp64 oracle.

Routing and plan outputs are integers and must match bit for bit (the oracle
selects from the GPU's exported fp32 scores, so both sides decide from the
same numbers); scores match the oracle's fp64 scores to 1e-4 relative;
attention outputs are within max-abs 2e-2 / mean-abs 2e-3 of an fp64 masked
softmax, LSE within 1e-3.
"""

import math

import numpy as np
import pytest
import torch

import adaptive_block_sparse_fva_amd as F
import oracle as O
from gpu_helpers import (LSE_MAX_ABS, O_MAX_ABS, O_MEAN_ABS, S_REL, device_inputs, f64_inputs,
                         problem_for, run_chain, sample_tiles, say, tile_rows)
from synth import WORKLOADS, Workload, make_inputs
from synth.workloads import WORKLOAD_ORDER

pytestmark = pytest.mark.gpu

CASES = [(name, p) for name in WORKLOAD_ORDER for p in WORKLOADS[name].top_p]
# attention compared on every tile (the 480p share: 1,280 tiles, ~20 s of fp64
# on the host); the two larger workloads on >= 64 seeded tiles per head plus
# each head's heaviest, lightest and last tile
FULL_ATTENTION = {"tiny", "two_head", "rank480p"}
SAMPLED_PER_HEAD = 64


def _oracle_scores(wl, inp, order=None):
    q64, k64, _ = f64_inputs(inp)
    order = O.token_order(wl.grid, wl.tile_hw) if order is None else order
    return O.block_scores(O.pool(q64, order, wl.block), O.pool(k64, order, wl.block),
                          1.0 / math.sqrt(wl.head_dim))


def check_routing_and_plan(wl, inp, res, p, refill, order=None, kind="tiles"):
    H, nb = wl.num_heads, res["nb"]
    order = O.token_order(wl.grid, wl.tile_hw) if order is None else order
    # order: closed form on the GPU vs enumeration in the oracle
    np.testing.assert_array_equal(res["order"], O.padded_order(order, wl.block))
    # scores: fp32 MFMA vs fp64
    s64 = _oracle_scores(wl, inp, order)
    err = np.abs(res["scores"].astype(np.float64) - s64).max()
    assert err <= S_REL * np.abs(s64).max(), f"score error {err}"
    # ranking, counts: bit-exact from the GPU's own fp32 scores
    S32 = res["scores"]
    for r in range(H * nb):
        h, i = divmod(r, nb)
        np.testing.assert_array_equal(res["ranked"][r], O.ranking(S32[h, i]), err_msg=f"row {r}")
    rc, hc = O.select_counts(S32, p, wl.k_min)
    np.testing.assert_array_equal(res["row_count"], rc)
    np.testing.assert_array_equal(res["head_count"], hc)
    # the oracle's own scores rounded to fp32 give the same counts except on rows
    # whose cutoff sits within rounding of p (reported, expected zero or near)
    rc_own, _ = O.select_counts(s64.astype(np.float32), p, wl.k_min)
    say(f"  rows whose count differs under the oracle's own scores: {int((rc_own != rc).sum())}"
        f" of {H * nb}")
    pl = O.plan(S32, rc, refill)
    np.testing.assert_array_equal(res["row_ptr"], pl["row_ptr"])
    np.testing.assert_array_equal(res["col_idx"], pl["col_idx"])
    np.testing.assert_array_equal(res["head_count_final"], pl["head_count"])
    # placement: split tiles and the heaviest-first work list, for the
    # device's compute-unit count
    rows = H * nb
    work, slot, nsplit = O.work_items(pl["kept"], F.compute_units())
    meta = res["plan_meta"]
    assert meta[0] == rows + nsplit and meta[1] == nsplit
    np.testing.assert_array_equal(meta[2: 2 + rows], slot)
    np.testing.assert_array_equal(meta[2 + rows: 2 + rows + nsplit], np.flatnonzero(slot >= 0))
    np.testing.assert_array_equal(res["work_order"], work)
    np.testing.assert_array_equal(res["tile_counter"], [0, 0])
    return pl


def check_attention(wl, inp, res, tiles=None, label="", order=None):
    q64, k64, v64 = f64_inputs(inp)
    order = O.token_order(wl.grid, wl.tile_hw) if order is None else order
    scale = 1.0 / math.sqrt(wl.head_dim)
    o_ref, lse_ref = O.masked_attention(q64, k64, v64, order, wl.block, res["row_ptr"],
                                        res["col_idx"], scale, tiles)
    if tiles is None:
        do = np.abs(res["o"] - o_ref)
        dl = np.abs(res["lse"] - lse_ref)
    else:
        rows = tile_rows(order, wl.block, wl.seq_len, tiles, res["nb"])
        do = np.concatenate([np.abs(res["o"][h, r] - o_ref[h, r]).ravel() for h, r in rows.items()])
        dl = np.concatenate([np.abs(res["lse"][h, r] - lse_ref[h, r]).ravel() for h, r in rows.items()])
    say(f"  {label} O max-abs {do.max():.3e} mean-abs {do.mean():.3e}; LSE max-abs {dl.max():.3e}")
    assert np.all(np.isfinite(do))
    assert do.max() <= O_MAX_ABS
    assert do.mean() <= O_MEAN_ABS
    assert dl.max() <= LSE_MAX_ABS


@pytest.mark.parametrize("name,p", CASES, ids=[f"{n}-p{p}" for n, p in CASES])
def test_chain_matches_oracle(name, p):
    wl = WORKLOADS[name]
    say(f"[gpu] chain {name} p={p} H={wl.num_heads} N={wl.seq_len} d={wl.head_dim} B={wl.block}")
    inp = make_inputs(wl)
    q, k, v = device_inputs(inp)
    _, res = run_chain(problem_for(wl, p), q, k, v)
    check_routing_and_plan(wl, inp, res, p, wl.refill_per_mille)
    if name in FULL_ATTENTION:
        check_attention(wl, inp, res, label="all tiles:")
    else:
        tiles = sample_tiles(res["row_ptr"], wl.num_heads, res["nb"], per_head=SAMPLED_PER_HEAD, seed=7)
        assert len(tiles) >= SAMPLED_PER_HEAD * wl.num_heads
        check_attention(wl, inp, res, tiles, label=f"{len(tiles)} sampled tiles:")


# the two rank shares at thresholds and refills their workload entries do not
# use: a sparse mask (p = 0.5), the refill at 100 per mille, a near-dense mask
# (p = 0.99); integer outputs in full, attention on sampled tiles
MORE_P = [("rank480p", 0.5, 0), ("rank480p", 0.8, 100), ("rank480p", 0.99, 0), ("rank720p", 0.8, 0)]


@pytest.mark.parametrize("name,p,refill", MORE_P, ids=[f"{n}-p{p}-r{r}" for n, p, r in MORE_P])
def test_rank_shares_at_other_thresholds(name, p, refill):
    wl = WORKLOADS[name]
    say(f"[gpu] chain {name} p={p} refill={refill}")
    inp = make_inputs(wl)
    q, k, v = device_inputs(inp)
    _, res = run_chain(problem_for(wl, p, refill), q, k, v)
    check_routing_and_plan(wl, inp, res, p, refill)
    tiles = sample_tiles(res["row_ptr"], wl.num_heads, res["nb"], per_head=SAMPLED_PER_HEAD, seed=11)
    check_attention(wl, inp, res, tiles, label=f"{len(tiles)} sampled tiles:")


@pytest.mark.parametrize("name", ["tiny", "two_head"])
def test_p_one_is_dense_attention(name):
    wl = WORKLOADS[name]
    say(f"[gpu] dense p=1 {name}")
    inp = make_inputs(wl)
    q, k, v = device_inputs(inp)
    _, res = run_chain(problem_for(wl, 1.0), q, k, v)
    nb = res["nb"]
    assert np.all(res["row_count"] == nb)
    q64, k64, v64 = f64_inputs(inp)
    o_ref, lse_ref = O.dense_attention(q64, k64, v64, 1.0 / math.sqrt(wl.head_dim))
    do = np.abs(res["o"] - o_ref)
    say(f"  dense O max-abs {do.max():.3e} mean-abs {do.mean():.3e}")
    assert do.max() <= O_MAX_ABS and do.mean() <= O_MEAN_ABS
    assert np.abs(res["lse"] - lse_ref).max() <= LSE_MAX_ABS


def test_p_zero_is_pure_top_k():
    wl = WORKLOADS["two_head"]
    say("[gpu] p=0 -> Top-k_min")
    inp = make_inputs(wl)
    q, k, v = device_inputs(inp)
    _, res = run_chain(problem_for(wl, 0.0), q, k, v)
    assert np.all(res["row_count"] == wl.k_min)
    check_routing_and_plan(wl, inp, res, 0.0, 0)
    check_attention(wl, inp, res, label="top-k:")


@pytest.mark.parametrize("name,has_splits", [("two_head", True), ("rank480p", False)])
def test_work_order_changes_placement_only(name, has_splits):
    """Any queue order gives bitwise the same output (placement, not computation).
    two_head's 128 tiles are few for 256 compute units, so its heavy tiles are
    cut in two; at the 480p share no tile outweighs a compute unit's mean load."""
    wl = WORKLOADS[name]
    say(f"[gpu] LPT vs natural tile order {name}")
    inp = make_inputs(wl)
    q, k, v = device_inputs(inp)
    buf, res = run_chain(problem_for(wl, wl.top_p[0]), q, k, v)
    items = res["work_order"]
    assert (res["plan_meta"][1] > 0) == has_splits, f"split tiles: {res['plan_meta'][1]}"
    by_tile = torch.from_numpy(np.sort(items).astype(np.int32)).cuda()
    reverse = torch.flip(by_tile, [0])
    for alt in (by_tile, reverse):
        buf.attn(q, work_order=alt)
        torch.cuda.synchronize()
        assert torch.equal(buf.o.view(torch.int16).cpu(), torch.from_numpy(
            res["o"].astype(np.float32)).to(torch.bfloat16).view(torch.int16))
        np.testing.assert_array_equal(buf.lse.cpu().numpy(), res["lse"].astype(np.float32))
        assert buf.tile_counter.cpu().tolist() == [0, 0]


def test_repeat_calls_are_deterministic():
    wl = WORKLOADS["rank480p"]
    say("[gpu] determinism rank480p")
    inp = make_inputs(wl)
    q, k, v = device_inputs(inp)
    _, a = run_chain(problem_for(wl, wl.top_p[0]), q, k, v)
    _, b = run_chain(problem_for(wl, wl.top_p[0]), q, k, v)
    for key in ("order", "scores", "ranked", "row_count", "row_ptr", "col_idx", "work_order",
                "o", "lse"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)


EDGE = [
    # name, heads, d, grid, block, tile, p, k_min, refill, recipe
    ("one_short_block", 2, 64, (1, 5, 7), 64, (8, 8), 0.9, 2, 0, "tau1"),
    ("ragged_tail", 2, 128, (3, 9, 11), 64, (8, 8), 0.8, 1, 0, "conc_flat"),
    ("raster_order", 1, 64, (2, 10, 20), 128, (0, 0), 0.9, 1, 0, "tau1"),
    ("d64_b128", 3, 64, (4, 24, 32), 128, (8, 16), 0.95, 3, 250, "lograndom"),
    ("kmin_above_nb", 2, 128, (2, 16, 16), 64, (8, 8), 0.5, 100, 0, "conc_flat"),
    ("refill_full", 2, 128, (4, 16, 24), 64, (8, 8), 0.7, 2, 1000, "lograndom"),
    ("odd_tiles", 2, 128, (3, 13, 29), 64, (5, 7), 0.9, 2, 100, "lograndom"),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_edge_shapes(case):
    name, H, d, grid, block, tile, p, kmin, refill, recipe = case
    wl = Workload(name, H, d, grid, block, (p,), kmin, refill, seed=11, heads=recipe, tile=tile)
    say(f"[gpu] edge {name} N={wl.seq_len} nb={wl.num_blocks}")
    inp = make_inputs(wl, cache=False)
    q, k, v = device_inputs(inp)
    _, res = run_chain(problem_for(wl, p), q, k, v)
    check_routing_and_plan(wl, inp, res, p, refill)
    check_attention(wl, inp, res, label=name)


def test_token_major_layout_matches_head_major():
    """q/k/v/o given as [N][H][d] (heads interleaved, as a DiT projection emits)."""
    wl = WORKLOADS["two_head"]
    say("[gpu] token-major strides")
    inp = make_inputs(wl)
    q, k, v = device_inputs(inp)
    _, ref = run_chain(problem_for(wl, wl.top_p[0]), q, k, v)
    H, N, d = q.shape
    qt, kt, vt = (x.permute(1, 0, 2).contiguous() for x in (q, k, v))
    prob = problem_for(wl, wl.top_p[0], stride_head=d, stride_token=H * d)
    import adaptive_block_sparse_fva_amd as F
    buf = F.Buffers.allocate(prob)
    assert buf.o.stride() == (d, H * d, 1)  # o allocated with the problem's strides
    buf.run(qt, kt, vt)
    torch.cuda.synchronize()
    got = buf.o.float().cpu().numpy()
    np.testing.assert_array_equal(got, ref["o"])
    np.testing.assert_array_equal(buf.row_ptr.cpu().numpy(), ref["row_ptr"])


def _vt_key(j):
    # column j of a V^T sub-tile holds this key position (the layout fva.h documents)
    return 16 * (j // 16) + 8 * ((j % 8) // 4) + 4 * ((j // 8) % 2) + j % 4


@pytest.mark.parametrize("name", ["two_head", "rank480p"])
def test_kv_relayout_is_the_documented_permutation(name):
    """fva_route's kv output: K rows and transposed V sub-tiles in position order, bit-exact."""
    wl = WORKLOADS[name]
    say(f"[gpu] kv re-layout {name}")
    inp = make_inputs(wl)
    q, k, v = device_inputs(inp)
    buf, res = run_chain(problem_for(wl, wl.top_p[0]), q, k, v)
    H, N, d, B, nb = wl.num_heads, wl.seq_len, wl.head_dim, wl.block, res["nb"]
    npad = nb * B
    order = O.padded_order(O.token_order(wl.grid, wl.tile_hw), B)
    kv = buf.kv.view(torch.int16).cpu().numpy().view(np.uint16).reshape(2, H, npad, d)
    valid = order >= 0
    kp_ref = np.zeros((H, npad, d), np.uint16)
    kp_ref[:, valid] = inp.k[:, order[valid]]
    np.testing.assert_array_equal(kv[0], kp_ref)
    vp = np.zeros((H, npad, d), np.uint16)
    vp[:, valid] = inp.v[:, order[valid]]
    cols = np.array([_vt_key(j) for j in range(64)])
    vt_ref = vp.reshape(H, npad // 64, 64, d)[:, :, cols, :].transpose(0, 1, 3, 2)
    np.testing.assert_array_equal(kv[1].reshape(H, npad // 64, d, 64), vt_ref)


def test_mfma_probe_reports_a_rate():
    """The MFMA-rate diagnostic runs and reports a plausible FLOP count."""
    say("[gpu] mfma probe")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(2 * cus * 256, dtype=torch.float32, device="cuda")
    flops = F.mfma_probe(10, True, sink)
    torch.cuda.synchronize()
    assert flops == 2 * cus * 4 * 10 * 4 * 32768
    assert torch.isfinite(sink).all()
    with pytest.raises(F.FvaError):
        F.mfma_probe(10, True, sink[:16])


IMPORTANCE_ABS = 1e-4  # fp32 exponentials and sums of at most B keys vs fp64


@pytest.mark.parametrize("name,refill", [("two_head", 0), ("rank480p", 0), ("edge_ragged_split", 250)])
def test_precise_block_importance_matches_oracle(name, refill):
    """GSRS S5.3: per-block LSE recorded in the attention kernel, normalised by
    the row LSE afterwards, against the oracle's mean attention weight per kept
    block."""
    if name == "edge_ragged_split":
        wl = Workload(name, 2, 128, (3, 9, 11), 64, (0.8,), 1, refill, seed=13, heads="conc_flat",
                      tile=(8, 8))
        inp = make_inputs(wl, cache=False)
    else:
        wl = WORKLOADS[name]
        inp = make_inputs(wl)
    say(f"[gpu] precise importance {name}")
    q, k, v = device_inputs(inp)
    prob = problem_for(wl, wl.top_p[0], refill)
    buf = F.Buffers.allocate(prob)
    buf.route(q, k, v)
    buf.plan()
    torch.cuda.synchronize()
    nnz = int(buf.row_ptr[-1].item())
    block_lse = torch.empty(nnz * wl.block, dtype=torch.float32, device="cuda")
    buf.attn(q, block_lse=block_lse)
    imp = buf.importance(block_lse)
    torch.cuda.synchronize()
    got = imp.cpu().numpy().astype(np.float64)
    res = gpu_host = __import__("gpu_helpers").host(buf)
    H, nb = wl.num_heads, res["nb"]
    np.testing.assert_allclose(got.sum(axis=2), 1.0, atol=IMPORTANCE_ABS)
    q64, k64, _ = f64_inputs(inp)
    order = O.token_order(wl.grid, wl.tile_hw)
    tiles = None if H * nb <= 256 else sample_tiles(res["row_ptr"], H, nb, per_head=10, seed=3)
    ref = O.precise_block_importance(q64, k64, order, wl.block, res["row_ptr"], res["col_idx"],
                                     1.0 / math.sqrt(wl.head_dim), tiles)
    rows = [divmod(int(t), nb) for t in (range(H * nb) if tiles is None else tiles)]
    err = max(np.abs(got[h, i] - ref[h, i]).max() for h, i in rows)
    say(f"  importance max-abs {err:.2e} over {len(rows)} rows; split tiles {int(res['plan_meta'][1])}")
    assert err <= IMPORTANCE_ABS


HILBERT = [
    # name, heads, d, grid, block, p, k_min, refill, recipe
    ("rank480p_hilbert", 5, 128, (21, 30, 52), 128, 0.95, 8, 0, "lograndom"),
    ("odd_hilbert", 2, 128, (3, 13, 29), 64, 0.9, 2, 100, "lograndom"),
    ("pow2_hilbert", 2, 64, (2, 32, 32), 128, 0.9, 2, 0, "tau1"),
    ("strip_hilbert", 1, 128, (2, 5, 61), 64, 0.8, 1, 0, "conc_flat"),
]


@pytest.mark.parametrize("case", HILBERT, ids=[c[0] for c in HILBERT])
def test_hilbert_order_chain(case):
    """FVAttn S3.1 / GSRS A.6 Hilbert reordering: the GPU's index-to-cell
    descent vs the oracle's enumeration, and the whole chain on that order."""
    name, H, d, grid, block, p, kmin, refill, recipe = case
    wl = Workload(name, H, d, grid, block, (p,), kmin, refill, seed=17, heads=recipe, tile=(0, 0))
    say(f"[gpu] hilbert {name} N={wl.seq_len} nb={wl.num_blocks}")
    inp = make_inputs(wl, cache=False)
    q, k, v = device_inputs(inp)
    order = O.hilbert_order(grid)
    _, res = run_chain(problem_for(wl, p, refill, order="hilbert"), q, k, v)
    check_routing_and_plan(wl, inp, res, p, refill, order=order, kind="hilbert")
    tiles = None if H * res["nb"] <= 256 else sample_tiles(res["row_ptr"], H, res["nb"], per_head=8, seed=5)
    check_attention(wl, inp, res, tiles, label=name, order=order)
