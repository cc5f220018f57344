"""Pins for the growing-sparsity / reduced-search oracle (GSRS S5.1, S5.2,
A.2, A.4, A.5, S6.1): hand-worked rows with dyadic importances (exact in
float32 and in the 2^-40 fixed point), the defining properties of the
shortest reaching prefix on random rows, and the paper's default schedule."""

import numpy as np
import pytest

import oracle.fva_gsrs as G


def _one_row(vals, cand, nb, p, k_min):
    """Row 0 of a one-head problem as given; the other rows evaluate every
    block with equal importance."""
    imp = np.full((1, nb, nb), 1.0 / nb, np.float32)
    imp[0, 0] = 0.0
    imp[0, 0, cand] = vals
    cols = list(cand) + list(range(nb)) * (nb - 1)
    row_ptr = np.concatenate([[0], len(cand) + nb * np.arange(nb)])
    ranked, count, head = G.select_from_importance(imp, row_ptr, np.array(cols), p, k_min)
    return ranked[0].tolist(), int(count[0])


def test_hand_rows():
    # candidates 0..3 with importance 1/2, 1/4, 1/8, 1/8: p = 0.75 is reached
    # exactly by two blocks, p = 0.76 needs three; ties (1/8) by lower id
    cand = [0, 1, 2, 3]
    vals = [0.5, 0.25, 0.125, 0.125]
    assert _one_row(vals, cand, 4, 0.75, 1) == ([0, 1, 2, 3], 2)
    assert _one_row(vals, cand, 4, 0.76, 1) == ([0, 1, 2, 3], 3)
    assert _one_row(vals, cand, 4, 0.5, 1) == ([0, 1, 2, 3], 1)
    # out-of-order candidates among 8 blocks: evaluated ones first by
    # importance, the rest by ascending id
    ranked, k = _one_row([0.125, 0.5, 0.375], [6, 2, 4], 8, 0.8, 1)
    assert ranked == [2, 4, 6, 0, 1, 3, 5, 7] and k == 2
    # the floor never reaches past the evaluated set
    ranked, k = _one_row([0.75, 0.25], [5, 1], 8, 0.1, 6)
    assert ranked[:2] == [5, 1] and k == 2
    # p >= 1 keeps every evaluated block, p <= 0 only the floor
    assert _one_row(vals, cand, 4, 1.0, 1)[1] == 4
    assert _one_row(vals, cand, 4, 0.0, 3)[1] == 3
    # equal importance everywhere: ids decide
    assert _one_row([0.25] * 4, [3, 2, 1, 0], 4, 0.5, 1) == ([0, 1, 2, 3], 2)


def test_prefix_is_the_shortest_reaching_p():
    rng = np.random.default_rng(31)
    H, nb = 3, 17
    imp = np.zeros((H, nb, nb), np.float32)
    row_ptr = [0]
    cols = []
    for r in range(H * nb):
        c = int(rng.integers(1, nb + 1))
        cand = np.sort(rng.choice(nb, c, replace=False))
        x = rng.exponential(size=c) ** 3
        imp[r // nb, r % nb, cand] = (x / x.sum()).astype(np.float32)
        cols.extend(cand.tolist())
        row_ptr.append(len(cols))
    row_ptr, cols = np.array(row_ptr), np.array(cols)
    for p in (0.3, 0.8, 0.95):
        ranked, count, head = G.select_from_importance(imp, row_ptr, cols, p, 2)
        assert np.array_equal(head, count.reshape(H, nb).sum(axis=1))
        for r in range(H * nb):
            cand = cols[row_ptr[r]: row_ptr[r + 1]]
            c, k = len(cand), int(count[r])
            sel = ranked[r][:k]
            assert set(sel) <= set(cand.tolist())                      # inside the evaluated set
            assert sorted(ranked[r].tolist()) == list(range(nb))       # a permutation
            v = imp[r // nb, r % nb]
            vals = v[ranked[r][:c]].astype(np.float64)
            assert np.all(np.diff(vals) <= 0)                          # descending
            tot = vals.sum()
            if k > min(2, c):                                          # not set by the floor
                assert vals[:k].sum() >= p * tot - 1e-9 * tot          # reaches p
                assert vals[:k - 1].sum() < p * tot + 1e-9 * tot       # and is the shortest
            assert k >= min(2, c)


def test_default_schedule():
    steps, warm, at, ps = 50, 10, [10, 20, 30, 40], [0.95, 0.9, 0.85, 0.8]
    acts = [G.gsrs_action(s, steps, warm, at, ps) for s in range(steps)]
    assert all(a == (G.ACT_DENSE, 1.0) for a in acts[:10])
    assert acts[10] == (G.ACT_FULL_SEARCH, 0.95)
    assert acts[20] == (G.ACT_CANDIDATE_SEARCH, 0.9)
    assert acts[30] == (G.ACT_CANDIDATE_SEARCH, 0.85)
    assert acts[40] == (G.ACT_CANDIDATE_SEARCH, 0.8)
    assert all(acts[s][0] == G.ACT_REUSE for s in range(11, 50) if s not in at)
    full = [G.gsrs_action(s, steps, warm, at, ps, reduced=False) for s in at]
    assert [a[0] for a in full] == [G.ACT_FULL_SEARCH] * 4
    # searches scheduled inside the warm-up are dense; no search -> dense throughout
    assert G.gsrs_action(3, 10, 5, [3, 6], [0.9, 0.8]) == (G.ACT_DENSE, 1.0)
    assert G.gsrs_action(6, 10, 5, [3, 6], [0.9, 0.8]) == (G.ACT_FULL_SEARCH, 0.8)
    assert G.gsrs_action(7, 10, 2, [], []) == (G.ACT_DENSE, 1.0)
    with pytest.raises(ValueError):
        G.gsrs_action(10, 10, 2, [], [])
