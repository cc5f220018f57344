"""Pins for the RLB / SASA oracle (FVAttn S3.2 Eq 5-6, S3.3 Eq 7-10, gating).

Each check ties the oracle to something other than itself: hand-worked
examples, the count of involutions (telephone numbers), a pure-Python
enumeration over all permutations on tiny inputs, invariants every plan
must satisfy, and a linear scan for the budget-to-refill conversion.
"""

import itertools

import numpy as np
import pytest

import oracle.fva_balance as B


def test_involution_counts_are_the_telephone_numbers():
    # number of self-inverse permutations of R items: 1, 2, 4, 10, 26, 76, 232, 764, 2620
    expect = [1, 2, 4, 10, 26, 76, 232, 764, 2620]
    assert [len(B.involutions(R)) for R in range(1, 10)] == expect
    for sig in B.involutions(5):
        assert all(sig[sig[r]] == r for r in range(5))
    assert len(set(B.involutions(6))) == 76


def test_pairs_hand_example():
    # loads 12, 2, 8, 8: swapping a 6-head of rank 0 with a 1-head of rank 1
    # gives 7, 7, 8, 8 (max 8, the best any plan reaches: ranks 2 and 3 can
    # only trade equal heads).  A second swap between 2 and 3 ties on (max,
    # sum of squares) but moves more heads; head ids tie -> lowest.
    w = np.array([[6, 6], [1, 1], [4, 4], [4, 4]])
    r = B.rlb_search(w, "pairs")
    assert r["sigma"].tolist() == [1, 0, 2, 3]
    assert r["send"].tolist() == [0, 0, -1, -1]
    assert r["loads_new"].tolist() == [7, 7, 8, 8]
    assert r["moves"] == 2


def test_pairs_picks_the_right_heads():
    # rank 0 = {9, 3}, rank 1 = {1, 2}: loads 12, 3.  Options (send0, send1):
    # (9,1): 4, 11; (9,2): 5, 10; (3,1): 10, 5; (3,2): 11, 4; none: 12, 3.
    # Best max is 10, twice; sums of squares 125 both; heads (0,1) < (1,0).
    w = np.array([[9, 3], [1, 2]])
    r = B.rlb_search(w, "pairs")
    assert r["loads_new"].tolist() == [5, 10]
    assert r["send"].tolist() == [0, 1]
    assert r["sigma"].tolist() == [1, 0]


def test_ring_hand_example():
    # ring 0 -> 1 -> 2 -> 0 with loads 8, 2, 4: rank 0 passes a 4, rank 1 a 1,
    # rank 2 a 2, so 8-4+2 = 6, 2-1+4 = 5, 4-2+1 = 3 (max 6 < 8).
    w = np.array([[4, 4], [1, 1], [2, 2]])
    r = B.rlb_search(w, "ring")
    assert r["sigma"].tolist() == [1, 2, 0]
    assert r["send"].tolist() == [0, 0, 0]
    assert r["loads_new"].tolist() == [6, 5, 3]


def test_ring_keeps_identity_when_no_ring_helps():
    # every ring plan pushes the 9-head onto rank 1 or keeps rank 0 at 11
    w = np.array([[9, 1], [2, 2], [2, 2]])
    r = B.rlb_search(w, "ring")
    assert r["sigma"].tolist() == [0, 1, 2]
    assert r["send"].tolist() == [-1, -1, -1]
    assert r["loads_new"].tolist() == [10, 4, 4]


def _slow_search(w, topology):
    """Pure-Python enumeration over itertools.permutations, filtered to the
    topology, and over every vector of sent heads."""
    R, Hl = w.shape
    ring = tuple((r + 1) % R for r in range(R))
    best = None
    for sigma in itertools.permutations(range(R)):
        if topology == "pairs" and any(sigma[sigma[r]] != r for r in range(R)):
            continue
        if topology == "ring" and sigma not in (tuple(range(R)), ring):
            continue
        movers = [r for r in range(R) if sigma[r] != r]
        for heads in itertools.product(range(Hl), repeat=len(movers)):
            send = [-1] * R
            for r, h in zip(movers, heads):
                send[r] = h
            L = [int(sum(w[r])) for r in range(R)]
            for r in movers:
                L[r] -= int(w[r][send[r]])
                L[sigma[r]] += int(w[r][send[r]])
            key = (max(L), sum(x * x for x in L), len(movers), tuple(sigma), tuple(send))
            if best is None or key < best:
                best = key
    return best


@pytest.mark.parametrize("topology", ["pairs", "ring"])
def test_search_matches_enumeration_over_all_permutations(topology):
    rng = np.random.default_rng(5)
    for R in range(1, 6):
        for Hl in (1, 2, 3):
            for _ in range(4):
                hi = int(rng.choice([3, 20, 1000]))
                w = rng.integers(0, hi, (R, Hl))
                r = B.rlb_search(w, topology)
                key = B.plan_key(r["loads_new"], r["sigma"].tolist(), r["send"].tolist())
                assert key == _slow_search(w, topology), (R, Hl, w.tolist())


@pytest.mark.parametrize("topology", ["pairs", "ring"])
def test_plan_invariants(topology):
    rng = np.random.default_rng(6)
    for _ in range(20):
        R = int(rng.integers(2, 7))
        Hl = int(rng.integers(1, 4))
        w = rng.integers(0, 500, (R, Hl))
        r = B.rlb_search(w, topology)
        sig, send, new = r["sigma"], r["send"], r["loads_new"]
        L = w.sum(axis=1)
        assert sorted(sig.tolist()) == list(range(R))            # a permutation
        assert new.sum() == L.sum()                                # work is moved, not changed
        assert new.max() <= L.max()                                # identity is a candidate
        assert np.array_equal(new, B.migrate(w, sig, send))        # Eq 5
        for x in range(R):
            moving = sig[x] != x
            assert (send[x] >= 0) == moving and send[x] < Hl     # one send ...
        assert len(set(sig.tolist())) == R                         # ... one receive
        if topology == "pairs":
            assert all(sig[sig[x]] == x for x in range(R))
        else:
            assert sig.tolist() in (list(range(R)), [(x + 1) % R for x in range(R)])


def test_gate_thresholds_are_inclusive_lower_bounds():
    assert B.gate([104, 100, 96, 100]) == B.MODE_NONE        # rho = 1.04
    assert B.gate([105, 100, 100, 95]) == B.MODE_SASA        # rho = 1.05 exactly
    assert B.gate([109, 100, 91, 100]) == B.MODE_SASA        # rho = 1.09
    assert B.gate([110, 100, 90, 100]) == B.MODE_RLB_SASA    # rho = 1.10 exactly
    assert B.gate([0, 0, 0]) == B.MODE_NONE
    assert B.gate([7]) == B.MODE_NONE                         # one rank: rho = 1


def test_sasa_hand_example():
    # L_new = 100, 90, 50, 95: slack 0, 10, 50, 5; trigger slack > 0.07 * 100;
    # budget floor(0.8 * slack) where triggered.
    slack, budget = B.sasa_budgets([100, 90, 50, 95])
    assert slack.tolist() == [0, 10, 50, 5]
    assert budget.tolist() == [0, 8, 40, 0]
    # exactly at the trigger (slack 7 of 100) nothing is added
    assert B.sasa_budgets([100, 93])[1].tolist() == [0, 0]


def test_budget_never_creates_a_new_straggler():
    # Eq 10: with n1 <= 1 the augmented loads stay within the critical path
    rng = np.random.default_rng(7)
    for _ in range(50):
        L = rng.integers(0, 10000, int(rng.integers(1, 9)))
        slack, budget = B.sasa_budgets(L)
        assert (L + budget).max() == L.max()
        assert np.all(budget <= slack)


def test_balance_modes():
    w_flat = np.full((4, 3), 10)
    r = B.balance(w_flat)
    assert r["mode"] == B.MODE_NONE and r["moves"] == 0 and not r["budget"].any()
    w_mid = np.array([[36, 36, 36], [35, 35, 35], [33, 33, 33], [36, 36, 36]])  # 108,105,99,108: rho 1.029
    assert B.balance(w_mid)["mode"] == B.MODE_NONE
    w_sasa = np.array([[40, 37, 35], [35, 35, 35], [30, 30, 30], [35, 35, 35]])  # 112,105,90,105: rho 1.087
    r = B.balance(w_sasa)
    assert r["mode"] == B.MODE_SASA and r["moves"] == 0
    assert r["loads_new"].tolist() == [112, 105, 90, 105]
    assert r["budget"].tolist() == [0, 0, 17, 0]   # only rank 2's slack 22 > 0.07 * 112; floor(0.8 * 22)
    w_rlb = np.array([[60, 50, 40], [10, 10, 10], [30, 30, 30], [30, 30, 30]])  # 150,30,90,90: rho 1.67
    r = B.balance(w_rlb)
    assert r["mode"] == B.MODE_RLB_SASA and r["moves"] >= 2
    assert r["loads_new"].max() < 150


def test_refill_from_budget_hand_example():
    # one rank, one head, nb = 8 rows with k = 2, 4 and six full rows:
    # A(f) = min(6, 2f/1000) + min(4, 4f/1000);
    # A(500) = 1 + 2 = 3, A(749) = 1 + 2, A(750) = 1 + 3 = 4 > 3  ->  f = 500, 3 blocks
    refill, added = B.refill_from_budget(np.array([[2, 4, 8, 8, 8, 8, 8, 8]]), 8, 1, 1, [-1], [3])
    assert refill.tolist() == [500] and added.tolist() == [3]
    refill, added = B.refill_from_budget(np.array([[2, 4, 8, 8, 8, 8, 8, 8]]), 8, 1, 1, [-1], [0])
    assert refill.tolist() == [0] and added.tolist() == [0]
    # a budget past saturation fills every row: 6 + 4 = 10 blocks, first at f = 3000
    refill, added = B.refill_from_budget(np.array([[2, 4, 8, 8, 8, 8, 8, 8]]), 8, 1, 1, [-1], [1000])
    assert refill.tolist() == [3000] and added.tolist() == [10]


def test_refill_from_budget_matches_a_linear_scan():
    rng = np.random.default_rng(8)
    for _ in range(30):
        R, Hl, nb = int(rng.integers(1, 4)), int(rng.integers(1, 4)), int(rng.integers(1, 7))
        rc = rng.integers(1, nb + 1, (R * Hl, nb))
        send = [int(rng.integers(-1, Hl)) for _ in range(R)]
        budget = rng.integers(0, 3 * nb * Hl, R)
        refill, added = B.refill_from_budget(rc, nb, R, Hl, send, budget)
        for r in range(R):
            heads = [r * Hl + j for j in range(Hl) if j != send[r]]
            rows = rc[heads].reshape(-1)
            table = [int(np.minimum(nb - rows, rows * f // 1000).sum()) for f in range(1000 * (nb - 1) + 1)]
            best = max(a for a in table if a <= budget[r])
            f = table.index(best)
            assert added[r] == best and all(refill[h] == f for h in heads)
            if 0 <= send[r]:
                assert refill[r * Hl + send[r]] == 0


def test_per_head_refill_plan_is_the_per_head_single_value_plan():
    import oracle as O
    rng = np.random.default_rng(9)
    H, nb = 3, 9
    S = rng.standard_normal((H, nb, nb)).astype(np.float32)
    rc, _ = O.select_counts(S, 0.7, 2)
    f = [0, 350, 4000]
    both = O.plan(S, rc, 0, head_refill=f)
    for h in range(H):
        one = O.plan(S[h:h + 1], rc[h * nb:(h + 1) * nb], f[h])
        a, b = both["row_ptr"][h * nb], both["row_ptr"][(h + 1) * nb]
        assert np.array_equal(both["kept"][h * nb:(h + 1) * nb], one["kept"])
        assert np.array_equal(both["col_idx"][a:b], one["col_idx"])
    same = O.plan(S, rc, 350, head_refill=[350] * H)
    ref = O.plan(S, rc, 350)
    assert all(np.array_equal(same[k], ref[k]) for k in ref)
