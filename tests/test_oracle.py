"""Pins for the CPU oracle: hand-derived fixtures, closed forms, brute force and
library special cases.  None of these tests reads the HIP path."""

import itertools
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O
from synth import WORKLOADS, get_workload, make_inputs, bf16_bits_to_f64
from synth.workloads import WORKLOAD_ORDER


# ---------------------------------------------------------------------------
# Video-aware order
# ---------------------------------------------------------------------------

def test_order_golden(golden):
    g = golden("order_T2_H3_W5_tile2x2.txt")
    grid = tuple(int(x) for x in g["grid"][0])
    tile = tuple(int(x) for x in g["tile"][0])
    expected = np.array([int(x) for x in g["order"][0]])
    np.testing.assert_array_equal(O.token_order(grid, tile), expected)


@pytest.mark.parametrize("grid", [(2, 3, 5), (4, 16, 16), (1, 7, 9)])
def test_order_identity_cases(grid):
    n = grid[0] * grid[1] * grid[2]
    np.testing.assert_array_equal(O.token_order(grid, (0, 0)), np.arange(n))
    # one tile covering the whole frame is plain raster order
    np.testing.assert_array_equal(O.token_order(grid, (grid[1], grid[2])), np.arange(n))
    # 1-row tiles as wide as the frame: also raster order
    np.testing.assert_array_equal(O.token_order(grid, (1, grid[2])), np.arange(n))


def _closed_form_order(grid, tile):
    """Position -> token by arithmetic on the position (independent of the
    enumeration in the oracle): split the position into frame, tile-row band,
    tile inside the band, row and column inside the tile."""
    T, H, W = grid
    th, tw = tile
    pos = np.arange(T * H * W)
    t, r = np.divmod(pos, H * W)
    band, r2 = np.divmod(r, th * W)
    band_h = np.minimum(th, H - band * th)
    col_tile, r3 = np.divmod(r2, band_h * tw)
    tile_w = np.minimum(tw, W - col_tile * tw)
    y_in, x_in = np.divmod(r3, tile_w)
    return t * H * W + (band * th + y_in) * W + col_tile * tw + x_in


@pytest.mark.parametrize("name", WORKLOAD_ORDER)
def test_order_bijection_and_closed_form(name):
    wl = WORKLOADS[name]
    order = O.token_order(wl.grid, wl.tile_hw)
    n = wl.seq_len
    assert len(order) == n
    np.testing.assert_array_equal(np.sort(order), np.arange(n))
    np.testing.assert_array_equal(order, _closed_form_order(wl.grid, wl.tile_hw))


def test_order_full_tiles_are_blocks():
    # 4 x 16 x 16 grid, block 64, tiles 8 x 8: every block is one 8 x 8 square of one frame
    wl = WORKLOADS["tiny"]
    order = O.token_order(wl.grid, wl.tile_hw)
    T, H, W = wl.grid
    for b in range(wl.num_blocks):
        toks = order[b * 64:(b + 1) * 64]
        t, r = np.divmod(toks, H * W)
        y, x = np.divmod(r, W)
        assert len(set(t)) == 1
        assert y.max() - y.min() == 7 and x.max() - x.min() == 7
        assert len(set(zip(y, x))) == 64


def test_padded_order():
    order = np.arange(10)
    p = O.padded_order(order, 4)
    np.testing.assert_array_equal(p, [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, -1, -1])


# ---------------------------------------------------------------------------
# Pooling and scores
# ---------------------------------------------------------------------------

def test_pool_closed_forms():
    # ramp: token n holds value n in every feature; block means are midpoints and
    # the short last block divides by its own size
    N, d = 10, 3
    x = np.repeat(np.arange(N, dtype=np.float64)[None, :, None], d, axis=2)
    got = O.pool(x, np.arange(N), 4)
    np.testing.assert_allclose(got[0, :, 0], [1.5, 5.5, 8.5], rtol=0, atol=1e-15)
    # constants pool to the constant
    c = np.full((2, 7, 4), 3.25)
    np.testing.assert_allclose(O.pool(c, np.arange(7), 3), 3.25, rtol=0, atol=0)


def test_pool_follows_order(golden):
    g = golden("order_T2_H3_W5_tile2x2.txt")
    order = np.array([int(v) for v in g["order"][0]])
    x = np.arange(30, dtype=np.float64)[None, :, None]
    got = O.pool(x, order, 4)[0, :, 0]
    # blocks of 4 consecutive positions: (0 1 5 6) (2 3 7 8) (4 9 10 11) ...
    assert got[0] == pytest.approx(3.0)
    assert got[1] == pytest.approx(5.0)
    assert got[2] == pytest.approx((4 + 9 + 10 + 11) / 4)
    assert got[-1] == pytest.approx((28 + 29) / 2)  # 30 = 7*4 + 2 -> last block has 2
    assert len(got) == 8


def test_block_scores_hand_example():
    d = 4
    qbar = np.zeros((1, 2, d)); qbar[0, 0, 0] = 2.0; qbar[0, 1, 1] = -1.0
    kbar = np.zeros((1, 3, d)); kbar[0, 0, 0] = 3.0; kbar[0, 1, 1] = 4.0; kbar[0, 2, :] = 1.0
    s = O.block_scores(qbar, kbar, 1 / math.sqrt(d))
    np.testing.assert_allclose(s[0], [[3.0, 0.0, 1.0], [0.0, -2.0, -0.5]], atol=1e-15)


def test_importance_rows_sum_to_one_and_shift_invariant():
    rng = np.random.default_rng(0)
    s = rng.normal(size=(2, 5, 7)) * 3
    imp = O.block_importance(s)
    np.testing.assert_allclose(imp.sum(-1), 1.0, atol=1e-15)
    np.testing.assert_allclose(O.block_importance(s + 11.0), imp, atol=1e-14)
    np.testing.assert_allclose(imp, scipy.special.softmax(s, axis=-1), atol=1e-15)


# ---------------------------------------------------------------------------
# Ranking, Top-p and the floor
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fixture", ["topp_row.txt", "topp_exact_tie.txt"])
def test_topp_golden(golden, fixture):
    g = golden(fixture)
    s = np.array([float(v) for v in g["scores"][0]], dtype=np.float32)
    np.testing.assert_array_equal(O.ranking(s), [int(v) for v in g["ranking"][0]])
    kmin = int(g["kmin"][0][0])
    for p, kp, kf in g["p"]:
        assert O.topp_count(s, float(p)) == int(kp), p
        rc, hc = O.select_counts(s[None, None, :].repeat(1, axis=1), float(p), kmin)
        assert int(rc[0]) == int(kf), p


def test_ranking_ties_and_signed_zero():
    s = np.array([1.0, 3.0, 3.0, 2.0, 3.0, -0.0, 0.0], dtype=np.float32)
    np.testing.assert_array_equal(O.ranking(s), [1, 2, 4, 3, 0, 5, 6])
    s2 = np.array([0.0, -0.0, 0.0], dtype=np.float32)
    np.testing.assert_array_equal(O.ranking(s2), [0, 1, 2])


def _normalised(s32):
    e = np.exp(s32.astype(np.float64) - s32.max())
    return e / e.sum()


def test_topp_brute_force_minimal_subsets():
    """Over all 2^16 subsets of 16 key blocks: the smallest subset whose
    normalised importance reaches p has exactly k_p blocks."""
    rng = np.random.default_rng(1)
    nb = 16
    masks = np.array(list(itertools.product([0, 1], repeat=nb)), dtype=np.float64)
    sizes = masks.sum(axis=1)
    checked = 0
    for trial in range(24):
        s = (rng.normal(size=nb) * rng.uniform(0.3, 3.0)).astype(np.float32)
        imp = _normalised(s)
        mass = masks @ imp
        for p in (0.3, 0.5, 0.8, 0.9, 0.95, 0.99):
            if np.min(np.abs(mass - p)) < 1e-9:
                continue  # knife edge: the fixed-point cutoff may legitimately differ
            k_brute = int(sizes[mass >= p].min())
            assert O.topp_count(s, p) == k_brute, (trial, p)
            checked += 1
    assert checked >= 140


def test_topp_fixed_point_matches_float_cumsum():
    rng = np.random.default_rng(2)
    for trial in range(200):
        nb = int(rng.integers(1, 300))
        s = (rng.normal(size=nb) * rng.uniform(0.1, 10.0)).astype(np.float32)
        order = O.ranking(s)
        cum = np.cumsum(_normalised(s)[order])
        for p in (0.5, 0.9, 0.95):
            if np.min(np.abs(cum - p)) < 1e-9:
                continue
            k_float = int(np.argmax(cum >= p)) + 1
            assert O.topp_count(s, p) == k_float


def test_topp_kept_mass_and_minimality():
    rng = np.random.default_rng(3)
    for trial in range(100):
        nb = int(rng.integers(2, 400))
        s = (rng.normal(size=nb) * 4).astype(np.float32)
        imp = _normalised(s)[O.ranking(s)]
        for p in (0.6, 0.9, 0.95):
            k = O.topp_count(s, p)
            assert imp[:k].sum() >= p - 1e-9
            assert imp[:k - 1].sum() < p + 1e-9


def test_topp_degenerate_p():
    rng = np.random.default_rng(4)
    s = rng.normal(size=37).astype(np.float32)
    assert O.topp_count(s, 1.0) == 37
    assert O.topp_count(s, 1.5) == 37
    assert O.topp_count(s, 0.0) == 0
    assert O.topp_count(s, -0.2) == 0
    # p just below 1 keeps every block that carries weight
    assert O.topp_count(s, float(np.nextafter(np.float32(1), np.float32(0)))) == 37


def test_pure_topk_when_p_nonpositive():
    """p <= 0 reduces the router to textbook Top-k with k = k_min."""
    rng = np.random.default_rng(5)
    S = rng.normal(size=(2, 9, 9)).astype(np.float32)
    S[0, 3, [1, 4, 6]] = 0.75  # ties resolved by index
    for kmin in (1, 3, 9, 20):
        rc, hc = O.select_counts(S, 0.0, kmin)
        k = min(kmin, 9)
        assert np.all(rc == k)
        for h in range(2):
            for i in range(9):
                textbook = np.sort(np.argsort(-S[h, i].astype(np.float64), kind="stable")[:k])
                np.testing.assert_array_equal(O.kept_blocks(S[h, i], k), textbook)


def test_floor_and_all_blocks():
    rng = np.random.default_rng(6)
    S = (rng.normal(size=(3, 12, 12)) * 8).astype(np.float32)
    rc, hc = O.select_counts(S, 0.5, 5)
    assert rc.min() >= 5
    rc, _ = O.select_counts(S, 1.0, 2)
    assert np.all(rc == 12)
    rc, _ = O.select_counts(S, 0.5, 50)  # floor clamps to nb
    assert np.all(rc == 12)
    np.testing.assert_array_equal(hc, O.select_counts(S, 0.5, 5)[0].reshape(3, 12).sum(1))


# ---------------------------------------------------------------------------
# Plan: refill, CSR, LPT order, Eq 1 / Eq 2
# ---------------------------------------------------------------------------

def _random_routing(seed, H=3, nb=20, p=0.8, kmin=2):
    rng = np.random.default_rng(seed)
    S = (rng.normal(size=(H, nb, nb)) * rng.uniform(0.5, 6, size=(H, 1, 1))).astype(np.float32)
    rc, hc = O.select_counts(S, p, kmin)
    return S, rc, hc


@pytest.mark.parametrize("refill", [0, 100, 333, 1000])
def test_plan_refill_is_ranking_prefix(refill):
    S, rc, hc = _random_routing(7)
    H, nb, _ = S.shape
    pl = O.plan(S, rc, refill)
    kept = pl["kept"]
    extra = kept - rc
    assert np.all(extra >= 0)
    assert np.all(extra <= (rc * refill) // 1000)
    assert np.all(kept <= nb)
    if refill == 1000:
        np.testing.assert_array_equal(kept, np.minimum(2 * rc, nb))
    for t in range(H * nb):
        h, i = divmod(t, nb)
        cols = pl["col_idx"][pl["row_ptr"][t]:pl["row_ptr"][t + 1]]
        rank = O.ranking(S[h, i])
        np.testing.assert_array_equal(cols, np.sort(rank[:kept[t]]))
        base = set(rank[:rc[t]].tolist())
        assert base <= set(cols.tolist())  # refill only adds blocks


def test_plan_csr_and_counts():
    S, rc, hc = _random_routing(8)
    H, nb, _ = S.shape
    pl = O.plan(S, rc, 100)
    rp = pl["row_ptr"]
    assert rp[0] == 0 and np.all(np.diff(rp) == pl["kept"])
    for t in range(H * nb):
        cols = pl["col_idx"][rp[t]:rp[t + 1]]
        assert np.all(np.diff(cols) > 0) and cols.min() >= 0 and cols.max() < nb
    np.testing.assert_array_equal(pl["head_count"], pl["kept"].reshape(H, nb).sum(1))


def test_plan_lpt_order():
    S, rc, hc = _random_routing(9, H=4, nb=16, p=0.7)
    pl = O.plan(S, rc, 0)
    order = pl["tile_order"]
    np.testing.assert_array_equal(np.sort(order), np.arange(64))
    k = pl["kept"][order]
    assert np.all(np.diff(k) <= 0)
    for a, b in zip(order[:-1], order[1:]):
        if pl["kept"][a] == pl["kept"][b]:
            assert a < b  # equal counts: head, then query block


def test_work_items_hand_example():
    # k' = [5, 1, 3, 8], 4 compute units: S = 2, total 17, a = ceil(17/2) = 9,
    # so tiles with 2k' > 9 (tiles 0 and 3) are cut: 5 -> 3 + 2, 8 -> 4 + 4.
    # Items (length, tile, part): (4,3,0) (4,3,1) (3,0,0) (3,2,0) (2,0,1) (1,1,0).
    order, slot, nsplit = O.work_items(np.array([5, 1, 3, 8]), 4)
    np.testing.assert_array_equal(order, [6, 7, 0, 4, 1, 2])
    np.testing.assert_array_equal(slot, [0, -1, -1, 1])
    assert nsplit == 2
    # 2 compute units: S = 1, a = 17, no tile has 2k' > 17: four whole tiles,
    # longest first
    order, slot, nsplit = O.work_items(np.array([5, 1, 3, 8]), 2)
    np.testing.assert_array_equal(order, [6, 0, 4, 2])
    np.testing.assert_array_equal(slot, [-1, -1, -1, -1])
    assert nsplit == 0
    # 256 compute units (S = 128) and the 480p-share shape: 1,280 tiles of at
    # most 256 kept blocks, 104,448 in total: a = 816, no tile has 2k' > 816
    kept = np.full(1280, 38)
    kept[:256] = 256
    order, slot, nsplit = O.work_items(kept, 256)
    assert nsplit == 0 and len(order) == 1280


def test_work_items_invariants():
    rng = np.random.default_rng(5)
    for trial in range(40):
        rows = int(rng.integers(1, 300))
        kept = rng.integers(1, 200, rows)
        if trial % 3 == 0:
            kept[: rows // 4] = 200  # a heavy head
        cus = int(rng.integers(1, 1400))
        order, slot, nsplit = O.work_items(kept, cus)
        S = min(max(cus // 2, 1), O.MAX_SPLITS // 2)
        assert nsplit < 2 * S and nsplit <= O.MAX_SPLITS
        tiles, parts = order // 2, order % 2
        # every tile once, split tiles twice (parts 0 and 1)
        counts = np.bincount(tiles, minlength=rows)
        np.testing.assert_array_equal(counts, np.where(slot >= 0, 2, 1))
        assert np.all(parts[slot[tiles] < 0] == 0)
        # split slots number the split tiles in tile-id order
        np.testing.assert_array_equal(slot[np.flatnonzero(slot >= 0)], np.arange(nsplit))
        # item lengths cover every kept block and never increase along the list
        length = np.where(slot[tiles] < 0, kept[tiles],
                          np.where(parts == 0, (kept[tiles] + 1) // 2, kept[tiles] // 2))
        assert length.sum() == kept.sum()
        assert np.all(np.diff(length) <= 0)
        # with the heavy tiles cut, no item exceeds a = ceil(total / S) (about
        # twice a compute unit's mean load) unless a single tile is more than
        # twice a
        mean = -(-kept.sum() // S)
        assert length.max() <= max(mean, (kept.max() + 1) // 2)


def _tiny_routing(seed, H=2, grid=(2, 8, 8), block=32, d=16, p=0.6, k_min=1):
    rng = np.random.default_rng(seed)
    N = grid[0] * grid[1] * grid[2]
    q, k = rng.standard_normal((H, N, d)), rng.standard_normal((H, N, d))
    order = O.token_order(grid, (4, 8))
    S = O.block_scores(O.pool(q, order, block), O.pool(k, order, block), 1 / math.sqrt(d)).astype(np.float32)
    rc, _ = O.select_counts(S, p, k_min)
    pl = O.plan(S, rc, 0)
    return q, k, order, block, d, pl


def test_precise_importance_rows_sum_to_one_over_kept_blocks():
    q, k, order, block, d, pl = _tiny_routing(3)
    imp = O.precise_block_importance(q, k, order, block, pl["row_ptr"], pl["col_idx"], 1 / math.sqrt(d))
    H, nb, _ = imp.shape
    np.testing.assert_allclose(imp.sum(axis=2), 1.0, atol=1e-12)
    for t in range(H * nb):
        h, i = divmod(t, nb)
        kept = set(pl["col_idx"][pl["row_ptr"][t]: pl["row_ptr"][t + 1]].tolist())
        for j in range(nb):
            assert (imp[h, i, j] > 0) == (j in kept)


def test_precise_importance_matches_torch_dense_probabilities():
    # with every block kept, the importance is the block average of the dense
    # attention map (torch's softmax, independent of the oracle's arithmetic)
    import torch
    rng = np.random.default_rng(4)
    H, grid, block, d = 1, (1, 8, 12), 16, 8
    N = grid[0] * grid[1] * grid[2]
    q, k = rng.standard_normal((H, N, d)), rng.standard_normal((H, N, d))
    order = O.token_order(grid, (0, 0))
    nb = O.num_blocks(N, block)
    row_ptr = np.arange(nb + 1) * nb
    col_idx = np.tile(np.arange(nb), nb)
    imp = O.precise_block_importance(q, k, order, block, row_ptr, col_idx, 0.3)
    P = torch.softmax(0.3 * torch.from_numpy(q[0]) @ torch.from_numpy(k[0]).T, dim=1).numpy()
    ref = P.reshape(nb, block, nb, block).sum(axis=3).mean(axis=1)
    np.testing.assert_allclose(imp[0], ref, atol=1e-12)


def test_precise_importance_single_kept_block_is_one():
    q, k, order, block, d, pl = _tiny_routing(5, p=0.0, k_min=1)
    imp = O.precise_block_importance(q, k, order, block, pl["row_ptr"], pl["col_idx"], 1 / math.sqrt(d))
    assert np.all(np.diff(pl["row_ptr"]) == 1)
    np.testing.assert_allclose(imp.max(axis=2), 1.0, atol=1e-12)


def _textbook_hilbert_d2xy(n, d):
    # the classic bit-by-bit index -> point conversion of Hilbert's curve on an
    # n x n grid (n a power of two)
    x = y = 0
    s, t = 1, d
    while s < n:
        rx = 1 & (t // 2)
        ry = 1 & (t ^ rx)
        if ry == 0:
            if rx == 1:
                x, y = s - 1 - x, s - 1 - y
            x, y = y, x
        x += s * rx
        y += s * ry
        t //= 4
        s *= 2
    return x, y


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32])
def test_hilbert_order_is_the_textbook_curve_on_power_of_two_squares(n):
    order = O.hilbert_order((1, n, n))
    ref = [_textbook_hilbert_d2xy(n, d) for d in range(n * n)]
    np.testing.assert_array_equal(order, [y * n + x for x, y in ref])


@pytest.mark.parametrize("grid", [(1, 30, 52), (2, 45, 80), (1, 55, 64), (3, 5, 7), (1, 1, 9), (1, 9, 1),
                                  (1, 2, 13), (1, 13, 2), (1, 3, 3)])
def test_hilbert_order_is_a_local_permutation(grid):
    T, H, W = grid
    order = O.hilbert_order(grid)
    np.testing.assert_array_equal(np.sort(order), np.arange(T * H * W))
    # frame-major, and inside a frame almost every step moves to a grid neighbour
    frame = order[: H * W]
    assert np.all(order.reshape(T, H * W) - np.arange(T)[:, None] * H * W == frame)
    y, x = frame // W, frame % W
    step = np.abs(np.diff(y)) + np.abs(np.diff(x))
    assert step[0] <= 1 if len(step) else True
    assert np.mean(step <= 2) >= 0.95
    if min(H, W) >= 8:
        assert np.mean(step == 1) >= 0.85
    # 128-token blocks are compact: their bounding boxes have about half the
    # height + width of the thin full-width strips that raster order gives
    if H * W >= 1024:
        hw = [np.ptp(y[i:i + 128]) + np.ptp(x[i:i + 128]) + 2 for i in range(0, H * W - 127, 128)]
        raster = [np.ptp(np.arange(i, i + 128) // W) + 1 + min(W, 128) for i in range(0, H * W - 127, 128)]
        assert np.mean(hw) < 0.6 * np.mean(raster)


def test_eq1_eq2_hand_examples():
    np.testing.assert_allclose(O.head_workload(np.array([32, 8]), 16), [2.0, 0.5])
    assert O.imbalance([3, 1, 1, 3]) == pytest.approx(1.5)
    assert O.imbalance([2, 2, 2]) == pytest.approx(1.0)


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def test_attention_golden(golden):
    g = golden("attention_two_tokens.txt")
    q = np.array([float(v) for v in g["q"][0]])[None, :, None]
    k = np.array([float(v) for v in g["k"][0]])[None, :, None]
    v = np.array([float(v) for v in g["v"][0]])[None, :, None]
    order = np.arange(2)
    full_rp = np.array([0, 2, 4]); full_ci = np.array([0, 1, 0, 1])
    o, lse = O.masked_attention(q, k, v, order, 1, full_rp, full_ci, 1.0)
    np.testing.assert_allclose(o[0, :, 0], [float(x) for x in g["full_o"][0]], atol=1e-14)
    np.testing.assert_allclose(lse[0], [float(x) for x in g["full_lse"][0]], atol=1e-14)
    od, lsed = O.dense_attention(q, k, v, 1.0)
    np.testing.assert_allclose(od[0, :, 0], [float(x) for x in g["full_o"][0]], atol=1e-14)
    mcols = np.array([int(x) for x in g["masked_cols"][0]])
    o, lse = O.masked_attention(q, k, v, order, 1, np.array([0, 1, 2]), mcols, 1.0)
    np.testing.assert_allclose(o[0, :, 0], [float(x) for x in g["masked_o"][0]], atol=1e-14)
    np.testing.assert_allclose(lse[0], [float(x) for x in g["masked_lse"][0]], atol=1e-14)


def _sdpa(q, k, v, scale):
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None], scale=scale)
    return out[0].numpy()


def _small_inputs():
    wl = WORKLOADS["tiny"]
    inp = make_inputs(wl)
    return wl, bf16_bits_to_f64(inp.q), bf16_bits_to_f64(inp.k), bf16_bits_to_f64(inp.v)


def test_all_blocks_kept_is_dense_attention():
    wl, q, k, v = _small_inputs()
    nb = wl.num_blocks
    order = O.token_order(wl.grid, wl.tile_hw)
    rp = np.arange(nb + 1) * nb
    ci = np.tile(np.arange(nb), nb)
    scale = 1 / math.sqrt(wl.head_dim)
    o, lse = O.masked_attention(q, k, v, order, wl.block, rp, ci, scale)
    ref = _sdpa(q, k, v, scale)
    np.testing.assert_allclose(o, ref, atol=1e-12)
    od, lsed = O.dense_attention(q, k, v, scale)
    np.testing.assert_allclose(od, ref, atol=1e-12)
    logits = scale * np.einsum("hnd,hmd->hnm", q, k)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(logits, axis=-1), atol=1e-11)
    np.testing.assert_allclose(O.attention_recall(lse, lsed), 1.0, atol=1e-12)


def test_single_kept_block_is_attention_on_that_block():
    wl, q, k, v = _small_inputs()
    nb, B = wl.num_blocks, wl.block
    order = O.token_order(wl.grid, wl.tile_hw)
    rng = np.random.default_rng(10)
    cols = rng.integers(0, nb, size=nb)
    rp = np.arange(nb + 1)
    scale = 1 / math.sqrt(wl.head_dim)
    o, lse = O.masked_attention(q, k, v, order, B, rp, cols, scale)
    for i in range(nb):
        qt = order[i * B:(i + 1) * B]
        kt = order[cols[i] * B:(cols[i] + 1) * B]
        ref = _sdpa(q[:, qt], k[:, kt], v[:, kt], scale)
        np.testing.assert_allclose(o[:, qt], ref, atol=1e-12)


def test_masked_attention_ragged_last_block():
    # N = 10 tokens, block 4: the last block has 2 tokens and must count only them
    rng = np.random.default_rng(11)
    q, k, v = (rng.normal(size=(1, 10, 8)) for _ in range(3))
    order = rng.permutation(10)
    rp = np.array([0, 3, 6, 9]); ci = np.array([0, 1, 2] * 3)
    o, lse = O.masked_attention(q, k, v, order, 4, rp, ci, 0.3)
    qs = order  # all keys kept -> dense attention in natural order
    ref = _sdpa(q, k, v, 0.3)
    np.testing.assert_allclose(o, ref, atol=1e-12)
    assert O.kept_flops(rp, ci, 10, 4, 8) == 4 * 8 * 10 * 10


# ---------------------------------------------------------------------------
# The synthetic workloads themselves
# ---------------------------------------------------------------------------

def test_inputs_deterministic_and_shaped():
    wl = get_workload("two_head")
    a = make_inputs(wl, cache=False)
    b = make_inputs(wl, cache=False)
    assert a.q.shape == (2, 4096, 128) and a.q.dtype == np.uint16
    np.testing.assert_array_equal(a.q, b.q)
    np.testing.assert_array_equal(a.v, b.v)
    assert a.amps[1] == 0.0 and a.amps[0] > 0


def test_route_end_to_end_small():
    wl, q, k, v = _small_inputs()
    r = O.route(q, k, wl.grid, wl.tile_hw, wl.block, wl.top_p[0], wl.k_min)
    nb = wl.num_blocks
    assert r["scores32"].shape == (1, nb, nb)
    assert r["row_count"].min() >= wl.k_min
    assert r["head_count"][0] == r["row_count"].sum()
    # the self block of a local head ranks first for most rows
    first = np.array([O.ranking(r["scores32"][0, i])[0] for i in range(nb)])
    assert np.mean(first == np.arange(nb)) > 0.8
