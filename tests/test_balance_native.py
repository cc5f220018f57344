"""The library's host RLB / SASA search against the oracle (FVAttn S3.2 Eq 5-6,
S3.3 Eq 7-10 and gating).  Host code only: these run without a GPU, and every
integer output must match the exhaustive oracle exactly."""

import ctypes
import time

import numpy as np
import pytest

import adaptive_block_sparse_fva_amd as F
from adaptive_block_sparse_fva_amd import fva
import oracle.fva_balance as B


def _compare(w, topology, k1=1050, k2=1100, n1=800, n2=70):
    R, Hl = w.shape
    got = F.balance(F.balance_params(R, Hl, topology, k1, k2, n1, n2), w)
    ref = B.balance(w, topology, k1, k2, n1, n2)
    ctx = (topology, w.tolist())
    assert got["mode"] == ref["mode"], ctx
    for key in ("sigma", "send", "loads_new", "slack", "budget"):
        assert got[key].tolist() == ref[key].tolist(), (key, ctx)
    assert got["moves"] == ref["moves"]
    assert got["load_total"] == int(w.sum())
    assert got["load_max"] == int(w.sum(axis=1).max())
    assert got["load_new_max"] == int(ref["loads_new"].max())
    assert got["load_aug_max"] == int((ref["loads_new"] + ref["budget"]).max())
    return got


def _cases(rng, R, Hl, n):
    for i in range(n):
        kind = i % 4
        if kind == 0:
            w = rng.integers(0, 4, (R, Hl))          # many ties
        elif kind == 1:
            w = rng.integers(100, 3000, (R, Hl))     # generic
        elif kind == 2:                              # density spread like routed heads
            w = np.round(np.exp(rng.uniform(np.log(300), np.log(6000), (R, Hl)))).astype(np.int64)
        else:
            w = np.full((R, Hl), 50)
            w[rng.integers(0, R), rng.integers(0, Hl)] = int(rng.integers(51, 2000))
        yield w


@pytest.mark.parametrize("topology", ["pairs", "ring"])
def test_search_matches_oracle_small(topology):
    rng = np.random.default_rng(21)
    for R in range(1, 7):
        for Hl in range(1, 5):
            for w in _cases(rng, R, Hl, 4):
                _compare(w, topology, k1=0, k2=0)     # force the search
                _compare(w, topology)                 # the paper's gating


def test_ring_matches_oracle_at_larger_world_sizes():
    rng = np.random.default_rng(22)
    for R, Hl in ((8, 5), (8, 5), (12, 3), (16, 2), (9, 4)):
        for w in _cases(rng, R, Hl, 2):
            _compare(w, "ring", k1=0, k2=0)


def test_pairs_matches_oracle_at_eight_ranks_of_five_heads():
    # the paper's setting: 8 ranks, 5 heads each, one head moved per rank
    rng = np.random.default_rng(23)
    w = np.round(np.exp(rng.uniform(np.log(300), np.log(6000), (8, 5)))).astype(np.int64)
    got = _compare(w, "pairs", k1=0, k2=0)
    assert got["load_new_max"] < got["load_max"]
    for w in _cases(rng, 7, 3, 4):
        _compare(w, "pairs", k1=0, k2=0)


def test_gating_thresholds_and_parameters_match_oracle():
    rng = np.random.default_rng(24)
    for _ in range(40):
        R, Hl = int(rng.integers(2, 6)), int(rng.integers(1, 4))
        w = rng.integers(80, 120, (R, Hl))
        k1 = int(rng.integers(1000, 1150))
        k2 = k1 + int(rng.integers(0, 80))
        _compare(w, "pairs", k1, k2, int(rng.integers(0, 1001)), int(rng.integers(0, 200)))


def test_refill_matches_oracle():
    rng = np.random.default_rng(25)
    for _ in range(40):
        R, Hl, nb = int(rng.integers(1, 6)), int(rng.integers(1, 5)), int(rng.integers(1, 40))
        rc = rng.integers(1, nb + 1, (R * Hl, nb))
        send = np.array([int(rng.integers(-1, Hl)) for _ in range(R)])
        budget = rng.integers(0, 3 * nb * Hl, R)
        prm = F.balance_params(R, Hl)
        got_f, got_a = F.sasa_refill(prm, nb, rc, send, budget)
        ref_f, ref_a = B.refill_from_budget(rc, nb, R, Hl, send, budget)
        assert got_f.tolist() == ref_f.tolist() and got_a.tolist() == ref_a.tolist()
        assert np.all(got_a <= budget)


def test_refill_at_routed_size():
    # 8 ranks x 5 heads x 256 query blocks, kept counts spread like routed rows
    rng = np.random.default_rng(26)
    R, Hl, nb = 8, 5, 256
    dens = np.exp(rng.uniform(np.log(0.03), np.log(0.6), R * Hl))
    rc = np.clip(np.round(dens[:, None] * nb * rng.uniform(0.5, 1.5, (R * Hl, nb))), 8, nb).astype(np.int64)
    w = rc.sum(axis=1).reshape(R, Hl)
    prm = F.balance_params(R, Hl)
    bal = F.balance(prm, w)
    got_f, got_a = F.sasa_refill(prm, nb, rc, bal["send"], bal["budget"])
    ref_f, ref_a = B.refill_from_budget(rc, nb, R, Hl, bal["send"], bal["budget"])
    assert got_f.tolist() == ref_f.tolist() and got_a.tolist() == ref_a.tolist()


def test_balance_rejects_bad_arguments():
    lib = F.load_library()
    w = np.ones((4, 2), np.int32)
    good = F.balance_params(4, 2)
    F.balance(good, w)
    bad = [
        (F.balance_params(0, 2), fva.FVA_ERR_ARG),
        (F.balance_params(4, 0), fva.FVA_ERR_ARG),
        (F.balance_params(13, 2), fva.FVA_ERR_UNSUPPORTED),
        (F.balance_params(65, 2, "ring"), fva.FVA_ERR_UNSUPPORTED),
        (F.balance_params(4, 65), fva.FVA_ERR_UNSUPPORTED),
        (F.balance_params(4, 2, k1_per_mille=1200, k2_per_mille=1100), fva.FVA_ERR_ARG),
        (F.balance_params(4, 2, n1_per_mille=1001), fva.FVA_ERR_ARG),
        (F.balance_params(4, 2, n2_per_mille=-1), fva.FVA_ERR_ARG),
        (F.balance_params(4, 2, k2_per_mille=2_000_000), fva.FVA_ERR_ARG),
    ]
    for prm, status in bad:
        R, Hl = max(prm.num_ranks, 1), max(prm.heads_per_rank, 1)
        with pytest.raises(fva.FvaError) as ei:
            F.balance(prm, np.ones((R, Hl), np.int32))
        assert ei.value.status == status
    prm = F.balance_params(4, 2)
    prm.reserved = 1
    with pytest.raises(fva.FvaError):
        F.balance(prm, w)
    prm.topology = 7
    prm.reserved = 0
    with pytest.raises(fva.FvaError):
        F.balance(prm, w)
    for load in (-1, fva.FVA_RLB_MAX_HEAD_LOAD + 1):
        ww = w.copy()
        ww[1, 1] = load
        with pytest.raises(fva.FvaError):
            F.balance(good, ww)
    assert lib.fva_balance(ctypes.byref(good), *([None] * 7)) == fva.FVA_ERR_ARG
    assert lib.fva_sasa_refill(ctypes.byref(good), 4, *([None] * 5)) == fva.FVA_ERR_ARG


def test_refill_rejects_bad_arguments():
    prm = F.balance_params(2, 2)
    rc = np.full(2 * 2 * 4, 2)
    F.sasa_refill(prm, 4, rc, [-1, 0], [3, 3])
    for nb, rcv, send, bud in ((0, rc[:0], [-1, -1], [1, 1]),
                               (4, np.where(np.arange(16) == 3, 5, rc), [-1, -1], [1, 1]),
                               (4, rc, [2, -1], [1, 1]),
                               (4, rc, [-2, -1], [1, 1]),
                               (4, rc, [-1, -1], [-1, 1])):
        with pytest.raises(fva.FvaError):
            F.sasa_refill(prm, nb, rcv, send, bud)


def test_search_time_at_eight_ranks():
    # the paper reports its constrained search in the hundreds of microseconds
    rng = np.random.default_rng(27)
    w = rng.integers(300, 6000, (8, 5))
    prm = F.balance_params(8, 5, k1_per_mille=0, k2_per_mille=0)
    F.balance(prm, w)
    t0 = time.perf_counter()
    for _ in range(50):
        F.balance(prm, w)
    per_call = (time.perf_counter() - t0) / 50
    assert per_call < 5e-3, per_call
