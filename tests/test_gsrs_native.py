"""The library's GSRS step schedule (host only) against the oracle."""

import ctypes

import numpy as np
import pytest

import adaptive_block_sparse_fva_amd as F
from adaptive_block_sparse_fva_amd import fva
import oracle.fva_gsrs as G


def _check(num_steps, warmup, at, ps, reduced):
    sched = F.gsrs_schedule(num_steps, warmup, at, ps, reduced)
    for t in range(num_steps):
        got = F.gsrs_action(sched, t)
        act, p = G.gsrs_action(t, num_steps, warmup, at, ps, reduced)
        assert got[0] == act and got[1] == float(np.float32(p)), (t, got, act, p)


def test_default_schedule_matches_oracle():
    for reduced in (True, False):
        _check(50, 10, [10, 20, 30, 40], [0.95, 0.9, 0.85, 0.8], reduced)


def test_random_schedules_match_oracle():
    rng = np.random.default_rng(41)
    for _ in range(200):
        S = int(rng.integers(1, 40))
        warm = int(rng.integers(0, S + 2))
        n = int(rng.integers(0, min(S, 16) + 1))
        at = sorted(rng.choice(S, n, replace=False).tolist())
        ps = rng.uniform(0.5, 1.0, n).round(3).tolist()
        _check(S, warm, at, ps, bool(rng.integers(0, 2)))


def test_schedule_rejects_bad_arguments():
    lib = F.load_library()
    ok = F.gsrs_schedule(10, 2, [2, 5], [0.9, 0.8])
    F.gsrs_action(ok, 9)
    for step in (-1, 10):
        with pytest.raises(fva.FvaError):
            F.gsrs_action(ok, step)
    for bad in (F.gsrs_schedule(10, 2, [5, 5], [0.9, 0.8]),       # not increasing
                F.gsrs_schedule(10, 2, [2, 10], [0.9, 0.8]),      # past the last step
                F.gsrs_schedule(0, 0, [], []),                    # no steps
                F.gsrs_schedule(10, -1, [], []),
                F.gsrs_schedule(10, 2, [3], [float("nan")])):
        with pytest.raises(fva.FvaError):
            F.gsrs_action(bad, 0)
    s = F.gsrs_schedule(10, 2, [2], [0.9])
    s.reduced = 2
    with pytest.raises(fva.FvaError):
        F.gsrs_action(s, 0)
    s.reduced, s.num_searches = 1, 17
    with pytest.raises(fva.FvaError):
        F.gsrs_action(s, 0)
    with pytest.raises(fva.FvaError):
        F.gsrs_schedule(10, 2, [1, 2], [0.9])
    assert lib.fva_gsrs_action(None, 0, None, None) == fva.FVA_ERR_ARG


def test_reselect_rejects_null_pointers_without_a_device():
    lib = F.load_library()
    p = F.make_problem(2, 4096, 128, (4, 32, 32), 64, (8, 8), 0.9, 4)
    assert lib.fva_reselect(ctypes.byref(p), *([None] * 7)) == fva.FVA_ERR_ARG
    bad = F.make_problem(2, 4096, 96, (4, 32, 32), 64, (8, 8), 0.9, 4)
    assert lib.fva_reselect(ctypes.byref(bad), *([None] * 7)) == fva.FVA_ERR_UNSUPPORTED
